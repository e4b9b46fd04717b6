"""Helpers for the GPU parity tests: run the three C-ABI calls, compare with
the oracle under the elementwise bound |gpu - ref| <= 2e-2 * (1 + |ref|)."""
from __future__ import annotations

import numpy as np
import torch

import sigmoid_attention_amd as sa
from workloads import as_f64

ATOL_REL = 2e-2  # |gpu - ref| <= ATOL_REL * (1 + |ref|), elementwise, for O, dQ, dK, dV


def device():
    return torch.device("cuda:0")


def to_dev(case):
    dev = device()
    return {t: case[t].to(dev) for t in ("q", "k", "v", "do")}


def run_all(t, seqlens, precision="fast", bias_mode="seqlen", bias_arg=0.0, fused=False):
    """Forward, dQ and dK/dV through the library on the current stream: the
    separate backward calls, or (fused=True) the one-launch sigattn_bwd that
    bench.py times."""
    kw = dict(bias_mode=bias_mode, bias_arg=bias_arg, precision=precision)
    o = sa.fwd(t["q"], t["k"], t["v"], seqlens, **kw)
    if fused:
        dq, dk, dv = sa.bwd(t["q"], t["k"], t["v"], t["do"], seqlens, **kw)
    else:
        dq = sa.bwd_dq(t["q"], t["k"], t["v"], t["do"], seqlens, **kw)
        dk, dv = sa.bwd_dkdv(t["q"], t["k"], t["v"], t["do"], seqlens, **kw)
    torch.cuda.synchronize()
    return {"o": o, "dq": dq, "dk": dk, "dv": dv}


def worst_ratio(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max over elements of |gpu - ref| / (2e-2 * (1 + |ref|)); <= 1 passes."""
    if gpu.size == 0:
        return 0.0
    return float(np.max(np.abs(gpu - ref) / (ATOL_REL * (1.0 + np.abs(ref)))))


def host(x: torch.Tensor) -> np.ndarray:
    return as_f64(x)


def padded_rows_zero(out: torch.Tensor, seqlens) -> bool:
    L = out.shape[2]
    mask = torch.arange(L, device=out.device)[None, :] >= torch.as_tensor(
        np.asarray(seqlens, dtype=np.int64), device=out.device)[:, None]  # [B, L]
    pad = out.masked_select(mask[:, None, :, None].expand_as(out))
    return bool((pad == 0).all().item())
