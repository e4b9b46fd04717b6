"""PyTorch autograd and module face of libsigattn.

A drop-in attention core for models: ``sigmoid_attention(q, k, v, seqlens)``
differentiates through the library's three calls (forward; dQ; dK and dV),
and ``SigmoidAttention`` wraps it as an ``nn.Module`` that also accepts a key
padding mask.  Inputs may be strided views — [B, Lmax, H, d] activations,
slices of a fused QKV projection, a K/V head broadcast over the query heads —
so no transposes or copies are made.  All arithmetic runs in the HIP kernels
(argument marshalling only here).

"Better Models, Faster Training: Sigmoid Attention for single-cell Foundation
Models", technical summary §2C: the forward is one fused pass, the backward
recomputes P and is split into a dQ kernel and a dK/dV kernel.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

from . import _binding


def _host_lengths(seqlens, B: int) -> np.ndarray:
    if isinstance(seqlens, torch.Tensor):
        seqlens = seqlens.detach().to("cpu")  # synchronises if the lengths live on the GPU
    lens = np.asarray(seqlens, dtype=np.int32).reshape(-1)
    if lens.shape[0] != B:
        raise ValueError(f"expected {B} sequence lengths, got {lens.shape[0]}")
    return lens


def _usable(t: torch.Tensor, layout: str) -> torch.Tensor:
    """t itself if the library accepts its strides, else a contiguous copy
    (e.g. a gradient that autograd hands over expanded or misaligned)."""
    pos = _binding.LAYOUTS[layout]
    d = t.shape[3]
    st = [t.stride(pos[i]) for i in range(3)]
    ok = (t.stride(3) == 1 and t.data_ptr() % 16 == 0 and all(s >= 0 and s % 8 == 0 for s in st)
          and st[2] >= d)
    return t if ok else t.contiguous()


class _SigmoidAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, head_bias, lens, layout, bias_mode, bias_arg, precision, causal):
        arg = head_bias if head_bias is not None else bias_arg
        o = _binding.fwd(q, k, v, lens, bias_mode=bias_mode, bias_arg=arg, precision=precision,
                         layout=layout, causal=causal)
        ctx.save_for_backward(q, k, v, head_bias)
        ctx.cfg = (lens, layout, bias_mode, bias_arg, precision, causal)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, head_bias = ctx.saved_tensors
        lens, layout, bias_mode, bias_arg, precision, causal = ctx.cfg
        do = _usable(do, layout)
        arg = head_bias if head_bias is not None else bias_arg
        kw = dict(bias_mode=bias_mode, bias_arg=arg, precision=precision, layout=layout, causal=causal)
        dq = dk = dv = db = None
        want_db = head_bias is not None and ctx.needs_input_grad[3]
        want_kv = ctx.needs_input_grad[1] or ctx.needs_input_grad[2] or want_db
        if ctx.needs_input_grad[0] and want_kv:  # both sides in one call (one fused launch at d = 64)
            out = _binding.bwd(q, k, v, do, lens, bias_rows=want_db, **kw)
            dq, dk, dv = out[:3]
            if want_db:
                db = _binding.bias_grad(out[3], lens)
        elif ctx.needs_input_grad[0]:
            dq = _binding.bwd_dq(q, k, v, do, lens, **kw)
        elif want_db:
            dk, dv, rows = _binding.bwd_dkdv_dbias(q, k, v, do, lens, **kw)
            db = _binding.bias_grad(rows, lens)
        elif want_kv:
            dk, dv = _binding.bwd_dkdv(q, k, v, do, lens, **kw)
        return dq, dk, dv, db, None, None, None, None, None, None


def sigmoid_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seqlens, layout: str = "bhld",
                      bias_mode: str = "seqlen", bias_arg=0.0, precision: str = "fast",
                      causal: bool = False) -> torch.Tensor:
    """O = sigma(Q K^T / sqrt(d) + b) V per sequence and head, differentiable.

    q, k, v: bf16 CUDA tensors, 4-d in `layout` order ("bhld" = [B, H, Lmax, d],
    "blhd" = [B, Lmax, H, d]), head dimension contiguous, d in {64, 128}.
    seqlens: B valid lengths (right padding), host sequence or tensor.  Rows at
    or beyond a sequence's length are ignored on input and zero on output (and
    in the gradients).  bias_mode / bias_arg / precision as in
    sigmoid_attention_amd.fwd.  causal: query i sees keys 0..i only.

    precision: "fast" (default) suits the method's regime, b = -ln n with
    scores of order one.  Scores that saturate the sigmoid (|x| >> 10, e.g.
    large-norm queries and keys) or a bias near 0 need precision="split":
    there "fast" exceeds the 2e-2 (1 + |exact|) error bound.
    bias_mode "per_head": bias_arg is a float32 tensor of H values on the
    device, b_h = bias_arg[h]; if it requires grad, its gradient (the sum of
    dX over each head's valid (query, key) pairs) is computed by the kernels.
    """
    B = q.shape[0]
    lens = _host_lengths(seqlens, B)
    if bias_mode == "per_head":
        return _SigmoidAttention.apply(q, k, v, bias_arg, lens, layout, bias_mode, 0.0, precision, bool(causal))
    return _SigmoidAttention.apply(q, k, v, None, lens, layout, bias_mode, bias_arg, precision, bool(causal))


class _SoftmaxAttention(torch.autograd.Function):
    """Softmax attention on the same schedule (the comparison path)."""

    @staticmethod
    def forward(ctx, q, k, v, lens, layout, precision, causal):
        o, lse2 = _binding.softmax_fwd(q, k, v, lens, precision=precision, layout=layout, causal=causal)
        ctx.save_for_backward(q, k, v, o, lse2)
        ctx.cfg = (lens, layout, precision, causal)
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse2 = ctx.saved_tensors
        lens, layout, precision, causal = ctx.cfg
        do = _usable(do, layout)
        dq, dk, dv = _binding.softmax_bwd(q, k, v, o, do, lse2, lens, precision=precision, layout=layout,
                                          causal=causal)
        return dq, dk, dv, None, None, None, None


def softmax_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, seqlens, layout: str = "bhld",
                      precision: str = "fast", causal: bool = False) -> torch.Tensor:
    """Differentiable softmax attention over each sequence's valid keys, on the
    same kernels' schedule: the mechanism sigmoid attention replaces, for
    like-for-like comparisons.  Arguments as for sigmoid_attention."""
    lens = _host_lengths(seqlens, q.shape[0])
    return _SoftmaxAttention.apply(q, k, v, lens, layout, precision, bool(causal))


def lengths_from_padding_mask(key_padding_mask: torch.Tensor) -> np.ndarray:
    """Valid lengths from a [B, Lmax] boolean mask (True = padding), which must
    pad on the right only."""
    m = key_padding_mask.detach().to("cpu").numpy().astype(bool)
    lens = (~m).sum(axis=1).astype(np.int32)
    expect = np.arange(m.shape[1])[None, :] >= lens[:, None]
    if not np.array_equal(m, expect):
        raise ValueError("key_padding_mask must mark a right-padded suffix of each row")
    return lens


class SigmoidAttention(torch.nn.Module):
    """Attention core (after the Q/K/V projections) with sigmoid weights and
    bias b = -ln(n), for bidirectional models on padded batches.

    forward(q, k, v, seqlens=None, key_padding_mask=None): give either the B
    valid lengths or a right-padding mask (True = pad); with neither, every
    row is valid.  Tensors are in `layout` order ([B, Lmax, H, d] by default,
    the usual layout after a projection and a view).

    bias_mode "per_head" makes the bias a trained parameter, one value per
    head (`heads` of them, initialised to `bias_arg`, e.g. -ln of a typical
    length); its gradient comes from the kernels.

    precision "fast" (default) is meant for b = -ln n and scores of order
    one; use precision="split" when scores saturate the sigmoid (|x| >> 10)
    or the bias is near 0, where "fast" exceeds the 2e-2 (1 + |exact|) bound.
    """

    def __init__(self, layout: str = "blhd", bias_mode: str = "seqlen", bias_arg: float = 0.0,
                 precision: str = "fast", causal: bool = False, heads: Optional[int] = None):
        super().__init__()
        if layout not in _binding.LAYOUTS:
            raise ValueError(f"layout must be one of {sorted(_binding.LAYOUTS)}")
        self.layout, self.bias_mode, self.bias_arg, self.precision = layout, bias_mode, bias_arg, precision
        self.causal = bool(causal)
        self.head_bias = None
        if bias_mode == "per_head":
            if not heads or heads < 1:
                raise ValueError("bias_mode per_head needs heads >= 1")
            self.head_bias = torch.nn.Parameter(torch.full((heads,), float(bias_arg), dtype=torch.float32))

    def forward(self, q, k, v, seqlens: Optional[Sequence[int]] = None,
                key_padding_mask: Optional[torch.Tensor] = None) -> torch.Tensor:
        if seqlens is None:
            if key_padding_mask is not None:
                seqlens = lengths_from_padding_mask(key_padding_mask)
            else:
                L = q.shape[_binding.LAYOUTS[self.layout][2]]
                seqlens = [L] * q.shape[0]
        arg = self.head_bias if self.head_bias is not None else self.bias_arg
        return sigmoid_attention(q, k, v, seqlens, self.layout, self.bias_mode, arg, self.precision, self.causal)

    def extra_repr(self) -> str:
        return (f"layout={self.layout}, bias_mode={self.bias_mode}, precision={self.precision}, "
                f"causal={self.causal}")
