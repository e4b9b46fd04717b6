"""Sigmoid attention on padded variable-length batches for AMD MI355X (gfx950).

Python face of the C-ABI library ``libsigattn`` (include/sigattn.h):

    o       = fwd(q, k, v, seqlens)
    dq      = bwd_dq(q, k, v, do, seqlens)
    dk, dv  = bwd_dkdv(q, k, v, do, seqlens)

q, k, v, do: bf16 CUDA tensors [B, H, Lmax, d] (d = 64 or 128), or
[B, Lmax, H, d] with layout="blhd", head dimension contiguous (other strides
are passed through); seqlens: B valid lengths (right padding).  Calls enqueue
on the current stream.  ``sigmoid_attention`` and ``SigmoidAttention`` add
autograd and an nn.Module on top.  All computation happens in the library's
HIP kernels; this package only marshals arguments and fails loudly if the
library is not built.
"""
from ._binding import (BIAS_MODES, DTYPES, EXPORTED, LAYOUTS, PASSES, PRECISIONS, SigattnError, bias_grad, bwd, bwd_dkdv,
                       bwd_dkdv_dbias, bwd_dq, fwd, lib_path, load, make_args, plan_stats, probe_mfma, softmax_bwd, softmax_bwd_dkdv, softmax_bwd_dq,
                       softmax_bwd_prep, softmax_fwd, status_str, tile_shape, validate)
from .function import SigmoidAttention, lengths_from_padding_mask, sigmoid_attention, softmax_attention

__all__ = ["BIAS_MODES", "DTYPES", "EXPORTED", "LAYOUTS", "PASSES", "PRECISIONS", "SigattnError", "SigmoidAttention",
           "bias_grad", "bwd", "bwd_dkdv", "bwd_dkdv_dbias", "bwd_dq", "fwd", "lengths_from_padding_mask", "lib_path", "load", "make_args",
           "plan_stats", "probe_mfma", "sigmoid_attention", "softmax_attention", "softmax_bwd", "softmax_bwd_dkdv", "softmax_bwd_dq", "softmax_bwd_prep", "softmax_fwd", "status_str", "tile_shape", "validate"]
