"""ctypes binding of libsigattn (include/sigattn.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of the library.  PyTorch provides device memory and the current
stream.  There is no fallback: if the library is missing, loading fails with
an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsigattn.so")
_lib = None

BIAS_MODES = {"seqlen": 0, "fixed_n": 1, "const": 2, "per_head": 3}
PRECISIONS = {"fast": 0, "split": 1}
DTYPES = {"bf16": 0, "fp16": 1}
PASSES = {"fwd": 0, "bwd_dq": 1, "bwd_dkdv": 2, "bwd": 3}

STATUS_NAMES = {
    0: "SIGATTN_OK", 1: "SIGATTN_ERR_NULL", 2: "SIGATTN_ERR_SHAPE", 3: "SIGATTN_ERR_SEQLEN",
    4: "SIGATTN_ERR_ALIGN", 5: "SIGATTN_ERR_ALIAS", 6: "SIGATTN_ERR_BIAS", 7: "SIGATTN_ERR_PRECISION",
    8: "SIGATTN_ERR_HIP", 9: "SIGATTN_ERR_PASS", 10: "SIGATTN_ERR_STRIDE", 11: "SIGATTN_ERR_MASK",
    12: "SIGATTN_ERR_DTYPE",
}

# Index order of a 4-d tensor for each supported layout, as (b, h, l, d) positions.
LAYOUTS = {"bhld": (0, 1, 2, 3), "blhd": (0, 2, 1, 3)}

EXPORTED = ("sigattn_fwd", "sigattn_bwd_dq", "sigattn_bwd_dkdv", "sigattn_status_str",
            "sigattn_plan_stats", "sigattn_tile_shape", "sigattn_validate", "sigattn_softmax_fwd",
            "sigattn_softmax_bwd_prep", "sigattn_softmax_bwd_dq", "sigattn_softmax_bwd_dkdv",
            "sigattn_bwd_dkdv_dbias", "sigattn_bias_grad", "sigattn_bwd", "sigattn_softmax_bwd",
            "sigattn_probe_mfma")


class SigattnStrides(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("h", ctypes.c_int64), ("l", ctypes.c_int64)]


class SigattnArgs(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("H", ctypes.c_int32), ("Lmax", ctypes.c_int32), ("d", ctypes.c_int32),
        ("seqlens", ctypes.POINTER(ctypes.c_int32)),
        ("bias_mode", ctypes.c_int32), ("bias_arg", ctypes.c_float),
        ("precision", ctypes.c_int32),
        ("stream", ctypes.c_void_p),
        ("strides", ctypes.POINTER(SigattnStrides)),
        ("mask", ctypes.c_int32),
        ("head_bias", ctypes.c_void_p),
        ("dtype", ctypes.c_int32),
    ]


class SigattnError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS_NAMES.get(code, code)} ({status_str(code)})")


def lib_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load libsigattn.so (built in-tree); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(
            f"{_LIB_PATH} is not built; run `python -m sigmoid_attention_amd.build` "
            "(or __graft_entry__.build()) first. There is no fallback implementation.")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, ap = ctypes.c_void_p, ctypes.POINTER(SigattnArgs)
    lib.sigattn_fwd.argtypes = [ap, vp, vp, vp, vp]
    lib.sigattn_bwd_dq.argtypes = [ap, vp, vp, vp, vp, vp]
    lib.sigattn_bwd_dkdv.argtypes = [ap, vp, vp, vp, vp, vp, vp]
    for f in (lib.sigattn_fwd, lib.sigattn_bwd_dq, lib.sigattn_bwd_dkdv):
        f.restype = ctypes.c_int
    lib.sigattn_status_str.argtypes = [ctypes.c_int]
    lib.sigattn_status_str.restype = ctypes.c_char_p
    lib.sigattn_plan_stats.argtypes = [ap, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64),
                                       ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]
    lib.sigattn_plan_stats.restype = ctypes.c_int
    lib.sigattn_tile_shape.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                       ctypes.POINTER(ctypes.c_int32)]
    lib.sigattn_tile_shape.restype = ctypes.c_int
    lib.sigattn_validate.argtypes = [ap, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
    lib.sigattn_validate.restype = ctypes.c_int
    lib.sigattn_softmax_fwd.argtypes = [ap, vp, vp, vp, vp, vp]
    lib.sigattn_softmax_bwd_prep.argtypes = [ap, vp, vp, vp]
    lib.sigattn_softmax_bwd_dq.argtypes = [ap, vp, vp, vp, vp, vp, vp, vp]
    lib.sigattn_softmax_bwd_dkdv.argtypes = [ap, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sigattn_bwd_dkdv_dbias.argtypes = [ap, vp, vp, vp, vp, vp, vp, vp]
    lib.sigattn_bias_grad.argtypes = [ap, vp, vp]
    lib.sigattn_bwd.argtypes = [ap, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sigattn_softmax_bwd.argtypes = [ap, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.sigattn_bwd.restype = ctypes.c_int
    lib.sigattn_probe_mfma.argtypes = [ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
    lib.sigattn_probe_mfma.restype = ctypes.c_int
    lib.sigattn_softmax_bwd.restype = ctypes.c_int
    for f in (lib.sigattn_softmax_fwd, lib.sigattn_softmax_bwd_prep, lib.sigattn_softmax_bwd_dq,
              lib.sigattn_softmax_bwd_dkdv, lib.sigattn_bwd_dkdv_dbias, lib.sigattn_bias_grad):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(code: int) -> str:
    return load().sigattn_status_str(int(code)).decode()


def make_args(B, H, Lmax, d, seqlens, bias_mode="seqlen", bias_arg=0.0, precision="fast", stream=0,
              strides=None, causal=False, head_bias=None, dtype="bf16"):
    """Build a sigattn_args struct.  `strides`: None (every tensor contiguous
    [B, H, Lmax, d]) or one (b, h, l) element-stride triple per tensor
    argument, in argument order.  `head_bias`: device address of H fp32
    values (bias mode "per_head").  `dtype`: "bf16" or "fp16", the element
    type of every tensor of the call.  Returns (args, keepalive) — keep the
    second object alive for as long as the struct is used (it owns the
    lengths and strides)."""
    lens = np.ascontiguousarray(np.asarray(seqlens, dtype=np.int32))
    a = SigattnArgs()
    a.B, a.H, a.Lmax, a.d = int(B), int(H), int(Lmax), int(d)
    a.seqlens = lens.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)) if lens.size else None
    a.bias_mode = BIAS_MODES[bias_mode] if isinstance(bias_mode, str) else int(bias_mode)
    a.bias_arg = float(bias_arg)
    a.precision = PRECISIONS[precision] if isinstance(precision, str) else int(precision)
    a.stream = int(stream) if stream else None
    a.mask = int(causal) if not isinstance(causal, bool) else (1 if causal else 0)
    a.head_bias = int(head_bias) if head_bias else None
    a.dtype = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    st = None
    if strides is not None:
        st = (SigattnStrides * len(strides))(*[SigattnStrides(int(b), int(h), int(l)) for b, h, l in strides])
        a.strides = ctypes.cast(st, ctypes.POINTER(SigattnStrides))
    return a, (lens, st)


def _check(code: int, where: str):
    if code != 0:
        raise SigattnError(code, where)


def layout_strides(t, layout: str = "bhld"):
    """(B, H, Lmax, d) and the (b, h, l) element strides of a 4-d tensor in
    `layout` order."""
    pos = LAYOUTS[layout]
    return tuple(t.shape[i] for i in pos), (t.stride(pos[0]), t.stride(pos[1]), t.stride(pos[2]))


def _tensor_args(ts, seqlens, bias_mode, bias_arg, precision, stream, layout="bhld", causal=False):
    """Validate tensors and build the argument block.  Each tensor is 4-d in
    `layout` order ("bhld": [B, H, Lmax, d]; "blhd": [B, Lmax, H, d]) with a
    contiguous last dimension; any other strides (views of a fused projection,
    a broadcast K/V head) go to the library, which checks them."""
    import torch
    if layout not in LAYOUTS:
        raise ValueError(f"layout must be one of {sorted(LAYOUTS)}")
    pos = LAYOUTS[layout]
    q = ts[0]
    for t in ts:
        if not isinstance(t, torch.Tensor):
            raise TypeError("expected torch tensors")
        if t.dtype not in (torch.bfloat16, torch.float16) or t.dtype != q.dtype:
            raise TypeError(f"expected bfloat16 or float16 tensors of one type, got {t.dtype} and {q.dtype}")
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if t.dim() != 4:
            raise ValueError(f"expected 4-d tensors in {layout} order")
        if t.shape != q.shape or t.device != q.device:
            raise ValueError("all tensors must share shape and device")
        if t.stride(3) != 1:
            raise ValueError("the head dimension must be contiguous")
    (B, H, L, d), _ = layout_strides(q, layout)
    strides = [layout_strides(t, layout)[1] for t in ts]
    contiguous = all(s == (H * L * d, L * d, d) for s in strides)
    if stream is None:
        stream = torch.cuda.current_stream(q.device).cuda_stream
    head_bias = None
    if bias_mode == "per_head" or bias_mode == BIAS_MODES["per_head"]:
        hb = bias_arg
        if (not isinstance(hb, torch.Tensor) or hb.dtype != torch.float32 or tuple(hb.shape) != (H,)
                or not hb.is_contiguous() or hb.device != q.device):
            raise ValueError("bias mode per_head takes bias_arg = a contiguous float32 tensor of H values "
                             "on the tensors' device")
        head_bias, bias_arg = hb.data_ptr(), 0.0
    return make_args(B, H, L, d, seqlens, bias_mode, bias_arg, precision, stream,
                     None if contiguous else strides, causal, head_bias,
                     "fp16" if q.dtype == torch.float16 else "bf16")


def _new_like(t):
    """A fresh contiguous tensor of t's shape (t itself may be a strided view)."""
    import torch

    return torch.empty(t.shape, dtype=t.dtype, device=t.device)


def fwd(q, k, v, seqlens: Sequence[int], o=None, bias_mode="seqlen", bias_arg=0.0, precision="fast",
        stream: Optional[int] = None, layout: str = "bhld", causal: bool = False):
    """O = sigma(Q K^T / sqrt(d) + b) V, padded rows of O zero (causal: query i
    sees keys 0..i).  Enqueued on the
    current stream (or `stream`); returns O (a new O is contiguous in `layout`
    order).

    precision "fast" suits b = -ln n with scores of order one; "split" is
    required when scores saturate the sigmoid (|x| >> 10) or the bias is near
    0 (see sigattn_precision in include/sigattn.h)."""
    import torch

    if o is None:
        o = _new_like(q)
    args, keep = _tensor_args((q, k, v, o), seqlens, bias_mode, bias_arg, precision, stream, layout, causal)
    with torch.cuda.device(q.device):
        _check(load().sigattn_fwd(ctypes.byref(args), q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr()),
               "sigattn_fwd")
    del keep
    return o


def bwd_dq(q, k, v, dout, seqlens, dq=None, bias_mode="seqlen", bias_arg=0.0, precision="fast", stream=None,
           layout: str = "bhld", causal: bool = False):
    """dQ of sum(O * dO); padded rows zero.  Returns dQ."""
    import torch

    if dq is None:
        dq = _new_like(q)
    args, keep = _tensor_args((q, k, v, dout, dq), seqlens, bias_mode, bias_arg, precision, stream, layout, causal)
    with torch.cuda.device(q.device):
        _check(load().sigattn_bwd_dq(ctypes.byref(args), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                     dout.data_ptr(), dq.data_ptr()), "sigattn_bwd_dq")
    del keep
    return dq


def bwd_dkdv(q, k, v, dout, seqlens, dk=None, dv=None, bias_mode="seqlen", bias_arg=0.0, precision="fast",
             stream=None, layout: str = "bhld", causal: bool = False):
    """dK and dV of sum(O * dO); padded rows zero.  Returns (dK, dV)."""
    import torch

    if dk is None:
        dk = _new_like(k)
    if dv is None:
        dv = _new_like(v)
    args, keep = _tensor_args((q, k, v, dout, dk, dv), seqlens, bias_mode, bias_arg, precision, stream, layout,
                              causal)
    with torch.cuda.device(q.device):
        _check(load().sigattn_bwd_dkdv(ctypes.byref(args), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       dout.data_ptr(), dk.data_ptr(), dv.data_ptr()), "sigattn_bwd_dkdv")
    del keep
    return dk, dv


def bwd_dkdv_dbias(q, k, v, dout, seqlens, dk=None, dv=None, dbias=None, bias_mode="seqlen", bias_arg=0.0,
                   precision="fast", stream=None, layout: str = "bhld", causal: bool = False):
    """dK, dV and the bias gradient rows: dbias[b, h, j] = sum over valid
    queries i of dX_ij (fp32 [B, H, Lmax], 0 on padded rows).  Returns
    (dK, dV, dbias)."""
    import torch

    dk = _new_like(k) if dk is None else dk
    dv = _new_like(v) if dv is None else dv
    dbias = _rows_like(q, layout) if dbias is None else dbias
    _check_rows(dbias, q, layout)
    args, keep = _tensor_args((q, k, v, dout, dk, dv), seqlens, bias_mode, bias_arg, precision, stream, layout,
                              causal)
    with torch.cuda.device(q.device):
        _check(load().sigattn_bwd_dkdv_dbias(ctypes.byref(args), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             dout.data_ptr(), dk.data_ptr(), dv.data_ptr(), dbias.data_ptr()),
               "sigattn_bwd_dkdv_dbias")
    del keep
    return dk, dv, dbias


def bwd(q, k, v, dout, seqlens, dq=None, dk=None, dv=None, dbias=None, bias_rows=False, bias_mode="seqlen",
        bias_arg=0.0, precision="fast", stream=None, layout: str = "bhld", causal: bool = False):
    """The whole backward in one call (one fused launch at d = 64): returns
    (dQ, dK, dV), plus the bias-gradient rows if `bias_rows` or `dbias` is
    given.  Bitwise the results of bwd_dq and bwd_dkdv(_dbias), except when
    every sequence fits 256 rows (d = 64, fast precision, no mask): then one
    kernel computes dS once for all of them, dK, dV and the bias rows are
    still bitwise those of bwd_dkdv(_dbias), and dQ differs from bwd_dq by
    rounding only."""
    import torch

    dq = _new_like(q) if dq is None else dq
    dk = _new_like(k) if dk is None else dk
    dv = _new_like(v) if dv is None else dv
    want = bias_rows or dbias is not None
    if want:
        dbias = _rows_like(q, layout) if dbias is None else dbias
        _check_rows(dbias, q, layout)
    args, keep = _tensor_args((q, k, v, dout, dq, dk, dv), seqlens, bias_mode, bias_arg, precision, stream, layout,
                              causal)
    with torch.cuda.device(q.device):
        _check(load().sigattn_bwd(ctypes.byref(args), q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr(),
                                  dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dbias.data_ptr() if want else None),
               "sigattn_bwd")
    del keep
    return (dq, dk, dv, dbias) if want else (dq, dk, dv)


def probe_mfma(blocks=256, iters=20000, repeats=3):
    """Measurement helper: sustained bf16 MFMA TFLOP/s of this GPU (best of
    `repeats` timed launches of sigattn_probe_mfma) and the shader clock in
    GHz during the last one."""
    import torch

    dev = torch.device("cuda", torch.cuda.current_device())
    out = torch.empty(blocks * 1024, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    st = torch.cuda.current_stream(dev)
    lib = load()

    def launch():
        _check(lib.sigattn_probe_mfma(blocks, iters, out.data_ptr(), clocks.data_ptr(), st.cuda_stream),
               "sigattn_probe_mfma")
    launch()
    best = float("inf")
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        launch()
        e1.record(st)
        e1.synchronize()
        best = min(best, e0.elapsed_time(e1))
    ticks, real = (int(x) for x in clocks.cpu())
    flop = blocks * 16 * iters * 4 * 32768.0
    return {"tflops": flop / (best * 1e-3) / 1e12, "ms": best, "shader_clock_ghz": ticks / real * 0.1 if real else None,
            "blocks": blocks, "iters": iters}


def bias_grad(dbias, seqlens, db=None, stream=None):
    """db[h] = sum over sequences and rows of dbias[:, h, :] (fp32 [H]), the
    gradient of a per-head bias.  dbias as returned by bwd_dkdv_dbias."""
    import torch

    if dbias.dtype != torch.float32 or dbias.dim() != 3 or not dbias.is_contiguous() or not dbias.is_cuda:
        raise ValueError("dbias must be a contiguous float32 [B, H, Lmax] tensor on the GPU")
    B, H, L = dbias.shape
    db = torch.empty(H, dtype=torch.float32, device=dbias.device) if db is None else db
    if db.dtype != torch.float32 or tuple(db.shape) != (H,) or not db.is_contiguous() or db.device != dbias.device:
        raise ValueError("db must be a contiguous float32 [H] tensor on dbias's device")
    if stream is None:
        stream = torch.cuda.current_stream(dbias.device).cuda_stream
    # d is not used by this call (it is validated like the others)
    args, keep = make_args(B, H, L, 64, seqlens, stream=stream)
    with torch.cuda.device(dbias.device):
        _check(load().sigattn_bias_grad(ctypes.byref(args), dbias.data_ptr(), db.data_ptr()), "sigattn_bias_grad")
    del keep
    return db


def _rows_like(t, layout):
    """fp32 [B, H, Lmax] per-row array for a tensor in `layout` order."""
    import torch

    (B, H, L, d), _ = layout_strides(t, layout)
    return torch.empty((B, H, L), dtype=torch.float32, device=t.device)


def _check_rows(x, like, layout):
    import torch

    (B, H, L, _), _ = layout_strides(like, layout)
    if x.dtype != torch.float32 or tuple(x.shape) != (B, H, L) or not x.is_contiguous() or x.device != like.device:
        raise ValueError("per-row arrays must be contiguous float32 [B, H, Lmax] on the tensors' device")


def softmax_fwd(q, k, v, seqlens, o=None, lse2=None, precision="fast", stream=None, layout="bhld", causal=False):
    """Softmax attention forward on the same schedule (comparison path).
    Returns (O, lse2); lse2 is the base-2 log-sum-exp of each valid row's
    scores scaled by log2(e)/sqrt(d), fp32 [B, H, Lmax], 0 on padded rows."""
    import torch

    if o is None:
        o = _new_like(q)
    if lse2 is None:
        lse2 = _rows_like(q, layout)
    _check_rows(lse2, q, layout)
    args, keep = _tensor_args((q, k, v, o), seqlens, "seqlen", 0.0, precision, stream, layout, causal)
    with torch.cuda.device(q.device):
        _check(load().sigattn_softmax_fwd(ctypes.byref(args), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          o.data_ptr(), lse2.data_ptr()), "sigattn_softmax_fwd")
    del keep
    return o, lse2


def softmax_bwd_prep(o, dout, seqlens, delta=None, precision="fast", stream=None, layout="bhld"):
    """delta = rowsum(dO * O), fp32 [B, H, Lmax], 0 on padded rows."""
    import torch

    delta = _rows_like(o, layout) if delta is None else delta
    _check_rows(delta, o, layout)
    args, keep = _tensor_args((o, dout), seqlens, "seqlen", 0.0, precision, stream, layout)
    with torch.cuda.device(o.device):
        _check(load().sigattn_softmax_bwd_prep(ctypes.byref(args), o.data_ptr(), dout.data_ptr(), delta.data_ptr()),
               "sigattn_softmax_bwd_prep")
    del keep
    return delta


def softmax_bwd_dq(q, k, v, dout, lse2, delta, seqlens, dq=None, precision="fast", stream=None, layout="bhld",
                   causal=False):
    """dQ of the softmax path."""
    import torch

    dq = _new_like(q) if dq is None else dq
    for x in (lse2, delta):
        _check_rows(x, q, layout)
    args, keep = _tensor_args((q, k, v, dout, dq), seqlens, "seqlen", 0.0, precision, stream, layout, causal)
    with torch.cuda.device(q.device):
        _check(load().sigattn_softmax_bwd_dq(ctypes.byref(args), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             dout.data_ptr(), lse2.data_ptr(), delta.data_ptr(), dq.data_ptr()),
               "sigattn_softmax_bwd_dq")
    del keep
    return dq


def softmax_bwd_dkdv(q, k, v, dout, lse2, delta, seqlens, dk=None, dv=None, precision="fast", stream=None,
                     layout="bhld", causal=False):
    """dK and dV of the softmax path."""
    import torch

    dk = _new_like(k) if dk is None else dk
    dv = _new_like(v) if dv is None else dv
    for x in (lse2, delta):
        _check_rows(x, q, layout)
    args, keep = _tensor_args((q, k, v, dout, dk, dv), seqlens, "seqlen", 0.0, precision, stream, layout, causal)
    with torch.cuda.device(q.device):
        _check(load().sigattn_softmax_bwd_dkdv(ctypes.byref(args), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                               dout.data_ptr(), lse2.data_ptr(), delta.data_ptr(), dk.data_ptr(),
                                               dv.data_ptr()), "sigattn_softmax_bwd_dkdv")
    del keep
    return dk, dv


def softmax_bwd(q, k, v, o, dout, lse2, seqlens, dq=None, dk=None, dv=None, delta=None, precision="fast",
                stream=None, layout="bhld", causal=False):
    """Softmax attention backward: delta = rowsum(dO * O), then the dQ and
    dK/dV kernels (one fused launch at d = 64).  Returns (dQ, dK, dV)."""
    import torch

    delta = softmax_bwd_prep(o, dout, seqlens, delta, precision=precision, stream=stream, layout=layout)
    return softmax_bwd_fused(q, k, v, dout, lse2, delta, seqlens, dq, dk, dv, precision, stream, layout, causal)


def softmax_bwd_fused(q, k, v, dout, lse2, delta, seqlens, dq=None, dk=None, dv=None, precision="fast", stream=None,
                      layout="bhld", causal=False):
    """dQ, dK and dV of the softmax path (one fused launch at d = 64), given lse2 and
    delta (softmax_bwd_prep).  Returns (dQ, dK, dV)."""
    import torch

    dq = _new_like(q) if dq is None else dq
    dk = _new_like(k) if dk is None else dk
    dv = _new_like(v) if dv is None else dv
    for x in (lse2, delta):
        _check_rows(x, q, layout)
    args, keep = _tensor_args((q, k, v, dout, dq, dk, dv), seqlens, "seqlen", 0.0, precision, stream, layout,
                              causal)
    with torch.cuda.device(q.device):
        _check(load().sigattn_softmax_bwd(ctypes.byref(args), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                          dout.data_ptr(), lse2.data_ptr(), delta.data_ptr(), dq.data_ptr(),
                                          dk.data_ptr(), dv.data_ptr()), "sigattn_softmax_bwd")
    del keep
    return dq, dk, dv


def plan_stats(B, H, Lmax, d, seqlens, pass_="fwd", bias_mode="seqlen", bias_arg=0.0, precision="fast",
               causal=False):
    """Host-only: (work_items, tile_pairs, launches) the pass would run."""
    args, keep = make_args(B, H, Lmax, d, seqlens, bias_mode, bias_arg, precision, causal=causal)
    items, pairs, launches = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check(load().sigattn_plan_stats(ctypes.byref(args), PASSES[pass_], ctypes.byref(items), ctypes.byref(pairs),
                                     ctypes.byref(launches)), "sigattn_plan_stats")
    del keep
    return items.value, pairs.value, launches.value


def validate(args, pass_: str, pointers) -> int:
    """Status the compute call for `pass_` would return for these arguments
    and tensor addresses (host-only, nothing enqueued or dereferenced)."""
    arr = (ctypes.c_void_p * len(pointers))(*[int(p) for p in pointers])
    return load().sigattn_validate(ctypes.byref(args), PASSES[pass_], arr)


def tile_shape(pass_: str, d: int):
    """(outer_rows, inner_rows) of the tiles the pass uses at head dim d."""
    o, i = ctypes.c_int32(), ctypes.c_int32()
    _check(load().sigattn_tile_shape(PASSES[pass_], int(d), ctypes.byref(o), ctypes.byref(i)), "sigattn_tile_shape")
    return o.value, i.value
