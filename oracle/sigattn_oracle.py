"""Plain CPU float64 oracle for bidirectional sigmoid attention on padded batches.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
baseline leg may import this module.  The library (``sigmoid_attention_amd``)
never calls it, and the two share no code: this file is written from the pages
alone, in their order and notation, with dense matrices and no tiling.

Sources (the pages' own words are not quoted; the facts are restated):

* "Better Models, Faster Training: Sigmoid Attention for single-cell Foundation
  Models", technical summary, §2A (Sigmoid Attention mechanism): the attention
  weights are the logistic function sigma(x) = 1/(1 + e^-x) applied to each
  scaled dot-product score independently, with an added bias b = -log(n); the
  output is the weight matrix times V.  Scores are never normalised along a row.
* same summary, §2B (theoretical stability): sigma'(x) = sigma(x)(1 - sigma(x)),
  bounded by 1/4, and the Jacobian of the weights with respect to the scores is
  diagonal.  So the backward is dX = dP * sigma'(X) elementwise, with no
  row-sum (normaliser) term.
* paperdance card of the same paper, English abstract: the models use
  bidirectional attention, hence no causal mask.
* same summary, §1 and §2C: sequences are padded to the longest in the batch
  and fully padded blocks on both the query and the key side are skipped, so
  padding carries no information into valid outputs.

Readings where the pages are silent or ambiguous (each one is a choice):

* n in b = -log(n) is the sequence's own valid length (mode "seqlen"); a fixed
  n ("fixed_n", b = -log(arg)) and a constant b ("const", b = arg) are offered
  because the pages do not pin it.
* log is the natural logarithm: then sigma(-log n) = 1/(n + 1), the
  softmax-like scale the summary motivates the bias with.
* d in sqrt(d) is the head dimension.
* padding is on the right: sequence b holds rows 0..n_b-1.
* padded query rows of O and dQ, and padded key rows of dK and dV, are 0;
  padded rows of dO are ignored; a sequence with n_b = 0 gives all-zero outputs
  and no logarithm is evaluated for it.
* the bias is a constant by default.  The learnable variant ("per_head": one
  trained value per head) also reports the gradient of the bias: per key, the
  sum over queries of dX (see attention()).

Every function here is pinned by tests that do not re-run this code's own
formulas: closed forms, a textbook logistic, finite differences, automatic
differentiation and brute force on tiny inputs.
"""
from __future__ import annotations

import math

import numpy as np

BIAS_MODES = ("seqlen", "fixed_n", "const", "per_head")


def logistic(x):
    """sigma(x) = 1/(1 + exp(-x)) (summary §2A), evaluated without overflow.

    For x >= 0 the textbook form is used; for x < 0 the equal form
    exp(x)/(1 + exp(x)), so exp never sees a large positive argument.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def score_scale(d: int) -> float:
    """The 1/sqrt(d) of the SigmoidAttn formula (summary §2A); d = head dim."""
    return 1.0 / math.sqrt(d)


def bias(n: int, mode: str = "seqlen", arg=None) -> float:
    """The additive bias b of summary §2A.  Default: b = -ln(n_b)."""
    if mode == "seqlen":
        return -math.log(n)
    if mode == "fixed_n":
        if arg is None or not arg > 0:
            raise ValueError("fixed_n bias needs arg > 0")
        return -math.log(arg)
    if mode == "const":
        if arg is None or not math.isfinite(arg):
            raise ValueError("const bias needs a finite arg")
        return float(arg)
    raise ValueError(f"unknown bias mode {mode!r}")


def per_head_bias(values, h: int) -> float:
    """The learnable variant: one bias value per head, b = values[h] (the
    summary's additive bias term made a trained parameter, one per head)."""
    vals = np.asarray(values, dtype=np.float64)
    if vals.ndim != 1 or not np.all(np.isfinite(vals)):
        raise ValueError("per_head bias needs a 1-D array of finite values, one per head")
    return float(vals[h])


def causal_mask(n: int):
    """1 where key j <= query i, else 0 (the causal variant; see attention())."""
    return np.tril(np.ones((n, n)))


def head_forward(q, k, v, b, causal: bool = False):
    """One (sequence, head) on its valid block: O = sigma(Q K^T / sqrt(d) + b) V.

    q, k, v: float64 arrays [n, d] holding only the valid rows.  causal: weights
    of keys after the query are 0.
    """
    s = score_scale(q.shape[1])
    x = s * (q @ k.T) + b          # scores, n x n (query i, key j)
    p = logistic(x)                # weights; each one independent (§2A)
    if causal:
        p = p * causal_mask(q.shape[0])
    return p @ v


def head_backward(q, k, v, do, b, intermediates: bool = False, causal: bool = False):
    """Gradients of l = sum(O * dO) for one (sequence, head) on its valid block.

    With X = s Q K^T + b, P = sigma(X), O = P V (summary §2A) and the diagonal
    Jacobian of §2B:
        dV = P^T dO
        dP = dO V^T
        dX = dP * sigma'(X),  sigma'(X) = sigma(X)(1 - sigma(X)) = sigma(X) sigma(-X)
        dQ = s dX K
        dK = s dX^T Q
    The sigma(-X) form of the derivative avoids the cancellation of 1 - sigma(X)
    when sigma(X) is close to 1; it is the same quantity.
    """
    s = score_scale(q.shape[1])
    x = s * (q @ k.T) + b
    p = logistic(x)
    if causal:  # masked weights are constants 0: no gradient through them
        p = p * causal_mask(q.shape[0])
    dv = p.T @ do
    dp = do @ v.T
    dx = dp * (p * logistic(-x))
    dq = s * (dx @ k)
    dk = s * (dx.T @ q)
    if intermediates:
        return dq, dk, dv, {"x": x, "p": p, "dp": dp, "dx": dx}
    return dq, dk, dv


def attention(q, k, v, seqlens, do=None, bias_mode: str = "seqlen", bias_arg=None, causal: bool = False):
    """Whole padded batch.  q, k, v, do: float64 [B, H, Lmax, d]; seqlens: [B].

    Returns {"o": ...} and, if do is given, also "dq", "dk", "dv"; every output
    is [B, H, Lmax, d] float64 with padded rows set to 0.  With do, "dbias"
    ([B, H, Lmax]) holds for every valid key j the sum over queries i of dX_ij:
    since each score is X_ij = s q_i.k_j + b, the derivative of l with respect
    to that (sequence, head)'s bias is the sum of this row, and a per-head bias
    gets the sum over sequences and keys.  Padded entries are 0.

    bias_mode "per_head": bias_arg is an array of H values, b = bias_arg[h].

    causal: the variant for autoregressive use (the language experiments of
    "Theory, Analysis, and Best Practices for Sigmoid Self-Attention", abstract),
    where query i sees keys 0..i only; the single-cell models of the summary
    are bidirectional, which is the default.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, L, d = q.shape
    seqlens = np.asarray(seqlens).astype(np.int64)
    if seqlens.shape != (B,) or (seqlens < 0).any() or (seqlens > L).any():
        raise ValueError("seqlens must hold B values in [0, Lmax]")
    out = {"o": np.zeros((B, H, L, d))}
    if do is not None:
        do = np.asarray(do, dtype=np.float64)
        for key in ("dq", "dk", "dv"):
            out[key] = np.zeros((B, H, L, d))
        out["dbias"] = np.zeros((B, H, L))
    if bias_mode == "per_head":
        per_head_bias(bias_arg, H - 1)  # validates the array (and that it holds H values)
    for bi in range(B):
        n = int(seqlens[bi])
        if n == 0:
            continue
        b = bias(n, bias_mode, bias_arg) if bias_mode != "per_head" else None
        for h in range(H):
            bh = b if b is not None else per_head_bias(bias_arg, h)
            qv, kv, vv = q[bi, h, :n], k[bi, h, :n], v[bi, h, :n]
            out["o"][bi, h, :n] = head_forward(qv, kv, vv, bh, causal)
            if do is not None:
                dq, dk, dv, it = head_backward(qv, kv, vv, do[bi, h, :n], bh, intermediates=True, causal=causal)
                out["dq"][bi, h, :n] = dq
                out["dk"][bi, h, :n] = dk
                out["dv"][bi, h, :n] = dv
                out["dbias"][bi, h, :n] = it["dx"].sum(axis=0)  # over queries i, per key j
    return out


def head(q, k, v, do, n: int, bias_mode: str = "seqlen", bias_arg=None):
    """One (sequence, head) sampled from a large batch.

    q, k, v, do: [Lmax, d] arrays of that head (any float dtype).  Returns
    (o, dq, dk, dv), each [Lmax, d] float64 with padded rows 0; do may be None,
    in which case the gradients are None.
    """
    q = np.asarray(q, dtype=np.float64)
    L, d = q.shape
    o = np.zeros((L, d))
    grads = None if do is None else tuple(np.zeros((L, d)) for _ in range(3))
    if n == 0:
        return (o,) + (grads if grads is not None else (None, None, None))
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    b = bias(n, bias_mode, bias_arg)
    o[:n] = head_forward(q[:n], k[:n], v[:n], b)
    if do is None:
        return o, None, None, None
    do = np.asarray(do, dtype=np.float64)
    dq, dk, dv = head_backward(q[:n], k[:n], v[:n], do[:n], b)
    grads[0][:n], grads[1][:n], grads[2][:n] = dq, dk, dv
    return (o,) + grads
