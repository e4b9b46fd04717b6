"""Plain CPU float64 oracle for softmax attention on padded batches: the
comparison workload that sigmoid attention replaces.

TEST INFRASTRUCTURE.  Only the tests and the bench's CPU leg may import this
module; the library never calls it and the two share no code.  Dense
matrices per (sequence, head), no tiling, no online normalisation.

Sources (facts restated, not quoted):

* "Transformer Attention機構の効率化と最新派生モデル", the vanilla
  self-attention pseudo code: scores are Q K^T / sqrt(d), masked positions
  are excluded, the weights are a softmax along each query's row, and the
  output is the weights times V.  Its FlashAttention section: the same result
  computed tile by tile, keeping per query a log-sum-exp normaliser instead of
  the n x n weight matrix.
* "Better Models, Faster Training: Sigmoid Attention for single-cell
  Foundation Models", technical summary §1: softmax makes each row of weights
  sum to 1; §2B: its Jacobian with respect to the scores is dense (each
  weight depends on every score of its row).

Readings (each one is a choice, mirroring the sigmoid oracle's):

* bidirectional: no causal mask; padding on the right (rows 0..n_b-1 valid);
  padded keys are excluded from every row's normalisation;
* padded query rows of O and dQ and padded key rows of dK and dV are 0; a
  sequence with n_b = 0 gives zeros;
* the per-row normaliser handed from the forward to the backward is the
  natural-log log-sum-exp of the row's scaled scores (0 on padded rows).

Backward of l = sum(O * dO): with P = softmax(X) along rows, the row Jacobian
is diag(p) - p p^T, so dX_ij = P_ij (dP_ij - sum_k P_ik dP_ik), dP = dO V^T.
"""
from __future__ import annotations

import math

import numpy as np


def row_softmax(x):
    """Softmax along the last axis, shifted by the row maximum (no overflow)."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def row_logsumexp(x):
    """ln(sum_j exp(x_ij)) per row, shifted by the row maximum."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=-1, keepdims=True)
    return (m + np.log(np.sum(np.exp(x - m), axis=-1, keepdims=True)))[..., 0]


def _masked(x, causal):
    """Scores with keys after the query set to -inf (causal variant)."""
    if not causal:
        return x
    n = x.shape[0]
    return np.where(np.tril(np.ones((n, n))) > 0, x, -np.inf)


def head_forward(q, k, v, causal=False):
    """One (sequence, head) on its valid rows: (O, lse).  q, k, v: [n, d]."""
    x = _masked((q @ k.T) / math.sqrt(q.shape[1]), causal)
    p = row_softmax(x)
    return p @ v, row_logsumexp(x)


def head_backward(q, k, v, do, causal=False):
    """dQ, dK, dV of l = sum(O * dO) on the valid rows, through the dense row
    Jacobian of the softmax: dX = P (dP - sum_k P_ik dP_ik)."""
    s = 1.0 / math.sqrt(q.shape[1])
    x = _masked(s * (q @ k.T), causal)
    p = row_softmax(x)
    dv = p.T @ do
    dp = do @ v.T
    row = np.sum(p * dp, axis=-1, keepdims=True)
    dx = p * (dp - row)
    return s * (dx @ k), s * (dx.T @ q), dv


def attention(q, k, v, seqlens, do=None, causal=False):
    """Whole padded batch, float64 [B, H, Lmax, d] inputs.  Returns "o" and
    "lse" ([B, H, Lmax]) and, with do, "dq", "dk", "dv"; padded rows 0.
    causal: query i sees keys 0..i only."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, d = q.shape
    seqlens = np.asarray(seqlens).astype(np.int64)
    if seqlens.shape != (B,) or (seqlens < 0).any() or (seqlens > L).any():
        raise ValueError("seqlens must hold B values in [0, Lmax]")
    out = {"o": np.zeros((B, H, L, d)), "lse": np.zeros((B, H, L))}
    if do is not None:
        do = np.asarray(do, dtype=np.float64)
        for key in ("dq", "dk", "dv"):
            out[key] = np.zeros((B, H, L, d))
    for bi in range(B):
        n = int(seqlens[bi])
        if n == 0:
            continue
        for h in range(H):
            qv, kv, vv = q[bi, h, :n], k[bi, h, :n], v[bi, h, :n]
            out["o"][bi, h, :n], out["lse"][bi, h, :n] = head_forward(qv, kv, vv, causal)
            if do is not None:
                dq, dk, dv = head_backward(qv, kv, vv, do[bi, h, :n], causal)
                out["dq"][bi, h, :n], out["dk"][bi, h, :n], out["dv"][bi, h, :n] = dq, dk, dv
    return out
