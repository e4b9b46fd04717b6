"""Sigmoid attention on padded variable-length batches for AMD MI355X (gfx950).

Python face of the C-ABI library ``libsigattn`` (include/sigattn.h):

    o       = fwd(q, k, v, seqlens)
    dq      = bwd_dq(q, k, v, do, seqlens)
    dk, dv  = bwd_dkdv(q, k, v, do, seqlens)

q, k, v, do: bf16 CUDA tensors [B, H, Lmax, d] (d = 64 or 128), contiguous;
seqlens: B valid lengths (right padding).  Calls enqueue on the current
stream.  All computation happens in the library's HIP kernels; this package
only marshals arguments and fails loudly if the library is not built.
"""
from ._binding import (BIAS_MODES, EXPORTED, PASSES, PRECISIONS, SigattnError, bwd_dkdv, bwd_dq, fwd, lib_path,
                       load, make_args, plan_stats, status_str, tile_shape)

__all__ = ["BIAS_MODES", "EXPORTED", "PASSES", "PRECISIONS", "SigattnError", "bwd_dkdv", "bwd_dq", "fwd",
           "lib_path", "load", "make_args", "plan_stats", "status_str", "tile_shape"]
