"""C-ABI of libsigattn on the CPU: the library loads, exports every function
include/sigattn.h declares, and rejects bad arguments before touching the GPU.

No call here reaches a kernel launch: every argument set is invalid in at
least one way, and the library validates everything before it enqueues.
Pointers are fake, 16-byte aligned addresses far apart; they are never
dereferenced.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import sigmoid_attention_amd as sa
from sigmoid_attention_amd import _binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sigattn.h")

OK, NULL, SHAPE, SEQLEN, ALIGN, ALIAS, BIAS, PREC, HIP, PASS = range(10)
BIG = 1 << 40  # spacing between fake buffers: larger than any test tensor
P = [0x100000000000 + i * BIG for i in range(8)]  # fake device addresses


def declared_functions():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"\b(sigattn_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = sa.load()
    names = declared_functions()
    assert set(names) == set(_binding.EXPORTED)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings():
    for code in range(13):
        s = sa.status_str(code)
        assert isinstance(s, str) and s
    assert sa.status_str(0) == "ok"
    assert sa.status_str(1234) == "unknown status"


def fwd(args, q=P[0], k=P[1], v=P[2], o=P[3]):
    return sa.load().sigattn_fwd(ctypes.byref(args) if args is not None else None, q, k, v, o)


def dq(args, q=P[0], k=P[1], v=P[2], g=P[3], d=P[4]):
    return sa.load().sigattn_bwd_dq(ctypes.byref(args), q, k, v, g, d)


def dkdv(args, q=P[0], k=P[1], v=P[2], g=P[3], dk=P[4], dv=P[5]):
    return sa.load().sigattn_bwd_dkdv(ctypes.byref(args), q, k, v, g, dk, dv)


def args(B=2, H=2, L=128, d=64, lens=(128, 77), **kw):
    return sa.make_args(B, H, L, d, lens, **kw)


def test_null_pointers():
    assert fwd(None) == NULL
    a, keep = args()
    assert fwd(a, q=None) == NULL
    assert fwd(a, o=None) == NULL
    assert dq(a, g=None) == NULL
    assert dkdv(a, dv=None) == NULL
    a.seqlens = None
    assert fwd(a) == NULL


@pytest.mark.parametrize("shape", [(0, 2, 128, 64), (2, 0, 128, 64), (2, 2, 0, 64), (2, 2, 128, 32),
                                   (2, 2, 128, 96), (2, 2, 128, 256), (-1, 2, 128, 64)])
def test_bad_shapes(shape):
    B, H, L, d = shape
    a, keep = sa.make_args(B, H, L, d, [1] * max(B, 1))
    for f in (fwd, dq, dkdv):
        assert f(a) == SHAPE


def test_size_overflow_rejected():
    a, keep = sa.make_args(1 << 20, 1 << 20, 1 << 20, 128, [0] * 1)  # 2^67 elements
    a.B = 1 << 20
    # seqlens would be read after the shape check; the shape check fails first
    assert fwd(a) == SHAPE


@pytest.mark.parametrize("d", [64, 128])
def test_lmax_bound_for_32bit_slice_offsets(d):
    # largest accepted Lmax: (Lmax + 256) * d * 2 <= 2^31 - 1
    top = (2**31 - 1) // (2 * d) - 256
    a, keep = sa.make_args(1, 1, top + 1, d, [0])
    for f in (fwd, dq, dkdv):
        assert f(a) == SHAPE
    with pytest.raises(sa.SigattnError) as e:
        sa.plan_stats(1, 1, top + 1, d, [0])
    assert e.value.code == SHAPE
    assert sa.plan_stats(1, 1, top, d, [0])[0] == 0  # one empty sequence: no work
    a, keep = sa.make_args(1, 1, top, d, [0])
    # passes the shape check; the (fake) pointers then fail alignment
    assert fwd(a, q=P[0] + 8) == ALIGN


@pytest.mark.parametrize("lens", [(129, 77), (-1, 77), (128, 1 << 30)])
def test_bad_lengths(lens):
    a, keep = args(lens=lens)
    for f in (fwd, dq, dkdv):
        assert f(a) == SEQLEN


def test_misaligned_pointers():
    a, keep = args()
    assert fwd(a, q=P[0] + 8) == ALIGN
    assert fwd(a, o=P[3] + 2) == ALIGN
    assert dq(a, d=P[4] + 4) == ALIGN
    assert dkdv(a, dk=P[4] + 8) == ALIGN


def test_aliasing_outputs():
    a, keep = args()
    nbytes = 2 * 2 * 128 * 64 * 2
    assert fwd(a, o=P[0]) == ALIAS                    # O is Q
    assert fwd(a, o=P[1] + nbytes - 16) == ALIAS      # O overlaps the tail of K
    assert dq(a, d=P[3]) == ALIAS                     # dQ is dO
    assert dkdv(a, dk=P[4], dv=P[4] + 16) == ALIAS    # dK overlaps dV
    assert dkdv(a, dv=P[2]) == ALIAS                  # dV is V


def test_inputs_may_alias_each_other_but_output_checks_still_run():
    a, keep = args()
    # q == k == v is legal; the call still fails on the aliased output first.
    assert fwd(a, q=P[0], k=P[0], v=P[0], o=P[0]) == ALIAS


@pytest.mark.parametrize("mode,arg", [(4, 0.0), (-1, 0.0), (1, 0.0), (1, -5.0), (1, float("nan")),
                                      (2, float("inf")), (2, float("nan"))])
def test_bad_bias(mode, arg):
    a, keep = args(bias_mode=mode, bias_arg=arg)
    for f in (fwd, dq, dkdv):
        assert f(a) == BIAS


@pytest.mark.parametrize("prec", [2, -1, 99])
def test_bad_precision(prec):
    a, keep = args(precision=prec)
    for f in (fwd, dq, dkdv):
        assert f(a) == PREC


def test_validation_order_no_side_effects():
    """A bad length is reported even when pointers are also bad: all checks run
    on the host before anything is enqueued."""
    a, keep = args(lens=(500, 1))
    assert fwd(a, q=P[0] + 1) == SEQLEN


def expected_counts(H, lens, outer, inner):
    lens = np.asarray(lens, dtype=np.int64)
    return int((H * -(-lens // outer)).sum()), int((H * -(-lens // outer) * -(-lens // inner)).sum())


@pytest.mark.parametrize("pass_", ["fwd", "bwd_dq", "bwd_dkdv"])
@pytest.mark.parametrize("d", [64, 128])
def test_plan_stats_closed_forms(pass_, d):
    lens = [1124, 2023, 1379, 743, 0, 545, 1602, 2048]
    outer, inner = sa.tile_shape(pass_, d)
    items, pairs, launches = sa.plan_stats(8, 16, 2048, d, lens, pass_)
    assert (items, pairs) == expected_counts(16, lens, outer, inner)
    assert launches == 1  # one launch: compute workgroups plus trailing zero-fill workgroups
    items, pairs, launches = sa.plan_stats(2, 3, 256, d, [0, 0], pass_)
    assert (items, pairs, launches) == (0, 0, 1)  # nothing to compute, all rows zero-filled
    items, pairs, launches = sa.plan_stats(2, 3, 256, d, [256, 256], pass_)
    assert launches == 1  # no padding: no zero-fill launch


def test_plan_stats_errors():
    with pytest.raises(sa.SigattnError) as e:
        sa.plan_stats(2, 2, 128, 64, [128, 77], "fwd", bias_mode=7)
    assert e.value.code == BIAS
    lib = sa.load()
    a, keep = args()
    assert lib.sigattn_plan_stats(ctypes.byref(a), 5, None, None, None) == PASS
    assert lib.sigattn_tile_shape(0, 48, None, None) == SHAPE
    assert lib.sigattn_tile_shape(7, 64, None, None) == PASS


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(_binding, "_LIB_PATH", "/nonexistent/libsigattn.so")
    monkeypatch.setattr(_binding, "_lib", None)
    with pytest.raises(ImportError, match="not built"):
        _binding.load()


def test_no_oracle_in_product_path():
    """The library package never imports the oracle (test infrastructure)."""
    pkg = os.path.join(ROOT, "sigmoid_attention_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, re.M), f
                assert "oracle/" not in src, f


@pytest.mark.parametrize("pass_", ["fwd", "bwd_dq", "bwd_dkdv"])
def test_plan_stats_causal_closed_forms(pass_):
    """Causal: only tiles on the visible side of the diagonal are visited.  A
    query tile t (outer R rows) visits key tiles 0 .. ceil((t+1) R / r) - 1; a
    key tile t visits query tiles floor(t R / r) .. ceil(n / r) - 1."""
    lens = [1124, 2023, 0, 545, 64, 65, 2048]
    outer, inner = sa.tile_shape(pass_, 64)
    items, pairs, _ = sa.plan_stats(len(lens), 4, 2048, 64, lens, pass_, causal=True)
    want_items = want_pairs = 0
    for n in lens:
        nt, ni = -(-n // outer), -(-n // inner)
        want_items += 4 * nt
        for t in range(nt):
            if pass_ == "bwd_dkdv":
                want_pairs += 4 * (ni - t * outer // inner)
            else:
                want_pairs += 4 * min(ni, -(-(t + 1) * outer // inner))
    assert (items, pairs) == (want_items, want_pairs)
    full = sa.plan_stats(len(lens), 4, 2048, 64, lens, pass_)[1]
    assert pairs < full  # roughly half the tile pairs are skipped


def test_bad_mask_mode():
    a, keep = args()
    a.mask = 2
    for f in (fwd, dq, dkdv):
        assert f(a) == 11


def validate(a, pass_, ptrs):
    arr = (ctypes.c_void_p * len(ptrs))(*ptrs)
    return sa.load().sigattn_validate(ctypes.byref(a), pass_, arr)


def test_per_head_bias_checks():
    """Bias mode 3 reads H fp32 values from device memory: the pointer must be
    set and 4-byte aligned, and may overlap inputs but no output."""
    hb = P[6]
    a, keep = args(bias_mode=3, head_bias=hb)
    assert validate(a, 0, P[:4]) == OK
    assert validate(a, 2, P[:6]) == OK
    a0, keep0 = args(bias_mode=3)  # no head_bias pointer
    for f in (fwd, dq, dkdv):
        assert f(a0) == NULL
    a2, keep2 = args(bias_mode=3, head_bias=hb + 2)
    for f in (fwd, dq, dkdv):
        assert f(a2) == ALIGN
    a4, keep4 = args(bias_mode=3, head_bias=hb + 4)  # 4-byte alignment suffices
    assert validate(a4, 1, P[:5]) == OK
    a5, keep5 = args(bias_mode=3, head_bias=P[0] + 64)  # inside the q input: allowed
    assert validate(a5, 0, P[:4]) == OK
    a6, keep6 = args(bias_mode=3, head_bias=P[3] + 64)  # inside the o output
    assert validate(a6, 0, P[:4]) == ALIAS
    assert fwd(a6) == ALIAS
    a7, keep7 = args(bias_mode=3, head_bias=P[5] + 64)  # inside dv
    assert dkdv(a7) == ALIAS


def dkdv_db(a, db, q=P[0], k=P[1], v=P[2], g=P[3], dk=P[4], dv=P[5]):
    return sa.load().sigattn_bwd_dkdv_dbias(ctypes.byref(a), q, k, v, g, dk, dv, db)


def test_dbias_rows_checks():
    a, keep = args()
    assert dkdv_db(a, None) == NULL
    assert dkdv_db(a, P[6] + 8) == ALIGN
    assert dkdv_db(a, P[4] + 64) == ALIAS   # inside dk
    assert dkdv_db(a, P[0] + 64) == ALIAS   # inside q (an output may overlap nothing)
    ab, keepb = args(lens=(129, 77))
    assert dkdv_db(ab, P[6]) == SEQLEN
    a3, keep3 = args(bias_mode=3, head_bias=P[6] + 256)  # bias values inside the dbias rows
    assert dkdv_db(a3, P[6]) == ALIAS


def test_bias_grad_checks():
    lib = sa.load()
    a, keep = args()
    assert lib.sigattn_bias_grad(ctypes.byref(a), None, P[7]) == NULL
    assert lib.sigattn_bias_grad(ctypes.byref(a), P[6], None) == NULL
    assert lib.sigattn_bias_grad(ctypes.byref(a), P[6] + 4, P[7]) == ALIGN
    assert lib.sigattn_bias_grad(ctypes.byref(a), P[6], P[7] + 2) == ALIGN
    assert lib.sigattn_bias_grad(ctypes.byref(a), P[6], P[6] + 4 * 2 * 2 * 128 - 4) == ALIAS
    ab, keepb = args(lens=(5, -1))
    assert lib.sigattn_bias_grad(ctypes.byref(ab), P[6], P[7]) == SEQLEN


@pytest.mark.parametrize("dtype", [2, -1, 7])
def test_bad_dtype(dtype):
    a, keep = args(dtype=dtype)
    for f in (fwd, dq, dkdv):
        assert f(a) == 12  # SIGATTN_ERR_DTYPE
    assert validate(a, 0, P[:4]) == 12


def test_fp16_dtype_validates():
    a, keep = args(dtype="fp16")
    assert validate(a, 0, P[:4]) == OK
    assert validate(a, 2, P[:6]) == OK


def bwd_all(a, q=P[0], k=P[1], v=P[2], g=P[3], dq_=P[4], dk=P[5], dv=P[6], db=None):
    return sa.load().sigattn_bwd(ctypes.byref(a), q, k, v, g, dq_, dk, dv, db)


def test_fused_backward_checks():
    """sigattn_bwd validates like the separate calls before launching."""
    a, keep = args()
    assert bwd_all(a, q=None) == NULL
    assert bwd_all(a, dv=None) == NULL
    assert bwd_all(a, dk=P[4]) == ALIAS            # dk on top of dq
    assert bwd_all(a, dq_=P[0]) == ALIAS           # dq on top of q
    assert bwd_all(a, dv=P[6] + 8) == ALIGN
    assert bwd_all(a, db=P[7] + 4) == ALIGN
    assert bwd_all(a, db=P[5] + 64) == ALIAS       # rows inside dk
    ab, keepb = args(lens=(200, 1))
    assert bwd_all(ab) == SEQLEN
    ah, keeph = args(bias_mode=3, head_bias=P[4] + 64)  # bias values inside dq
    assert bwd_all(ah) == ALIAS
    lib = sa.load()
    assert lib.sigattn_softmax_bwd(ctypes.byref(a), P[0], P[1], P[2], P[3], None, P[5], P[6], P[7], 0) == NULL


def test_probe_checks():
    lib = sa.load()
    assert lib.sigattn_probe_mfma(1, 1, None, P[1], None) == NULL
    assert lib.sigattn_probe_mfma(1, 1, P[0], None, None) == NULL
    assert lib.sigattn_probe_mfma(1, 1, P[0] + 2, P[1], None) == ALIGN
    assert lib.sigattn_probe_mfma(1, 1, P[0], P[1] + 4, None) == ALIGN
    assert lib.sigattn_probe_mfma(0, 1, P[0], P[1], None) == SHAPE
    assert lib.sigattn_probe_mfma(1, 0, P[0], P[1], None) == SHAPE
    assert lib.sigattn_probe_mfma(2, 1, P[0], P[0] + 4096, None) == ALIAS


def test_fused_backward_pass_in_validate_and_plan_stats():
    lens = (128, 77)
    a, keep = args(lens=lens)
    assert validate(a, 3, P[:7]) == OK
    assert validate(a, 3, P[:4] + [P[4], P[4], P[6]]) == ALIAS     # dk on top of dq
    assert validate(a, 3, P[:4] + [P[4], P[5], P[0]]) == ALIAS     # dv on top of q
    kv = sa.plan_stats(2, 2, 128, 64, lens, "bwd_dkdv")
    q = sa.plan_stats(2, 2, 128, 64, lens, "bwd_dq")
    both = sa.plan_stats(2, 2, 128, 64, lens, "bwd")
    assert both[0] == kv[0] + q[0] and both[1] == kv[1] + q[1] and both[2] == 1
    # at d = 128 the two sides run at different occupancies: two launches
    assert sa.plan_stats(2, 2, 128, 128, lens, "bwd")[2] == 2
    # beyond one launch's length table (4096 sequences): each side runs two
    # launches and the backward runs them in turn instead of one fused launch
    many = [64] * 5000
    for lmax, prec in ((300, "fast"), (96, "split")):
        kv_l = sa.plan_stats(5000, 1, lmax, 64, many, "bwd_dkdv", precision=prec)[2]
        q_l = sa.plan_stats(5000, 1, lmax, 64, many, "bwd_dq", precision=prec)[2]
        assert kv_l == 2 and sa.plan_stats(5000, 1, lmax, 64, many, "bwd", precision=prec)[2] == kv_l + q_l
    # every sequence within 256 rows (fast precision, d = 64): the
    # short-sequence backward, one launch per length table
    assert sa.plan_stats(5000, 1, 96, 64, many, "bwd")[2] == 2
    assert sa.plan_stats(5000, 1, 256, 64, many, "bwd")[2] == 2
    assert sa.plan_stats(5000, 1, 257, 64, many, "bwd")[2] == 4
    assert sa.plan_stats(2, 2, 128, 64, lens, "bwd", precision="split")[2] == 1  # fused


@pytest.mark.parametrize("B,n,Lmax", [(1024, 256, 256), (4096, 128, 128), (1024, 200, 256), (300, None, 96)])
def test_many_short_sequences_one_launch(B, n, Lmax):
    """Batches of many short sequences (single cells of a few hundred genes)
    run every pass as one launch: pieces span many sequences and the lengths
    travel in a table of the kernel arguments."""
    lens = [n] * B if n is not None else list(np.random.default_rng(5).integers(0, Lmax + 1, size=B))
    for pass_ in ("fwd", "bwd_dq", "bwd_dkdv", "bwd"):
        items, pairs, launches = sa.plan_stats(B, 16, Lmax, 64, lens, pass_)
        assert launches == 1, (pass_, launches)
    items, pairs, _ = sa.plan_stats(B, 16, Lmax, 64, lens, "fwd")
    ln = np.asarray(lens, dtype=np.int64)
    assert items == int((16 * -(-ln // 128)).sum()) and pairs == int((16 * -(-ln // 128) * -(-ln // 64)).sum())


def test_long_padded_length_uses_wide_table():
    """Lmax above 65535 needs 32-bit lengths: a launch then holds 2048 sequences."""
    lens = [100] * 2500
    assert sa.plan_stats(2500, 1, 70000, 64, lens, "fwd")[2] == 2
    assert sa.plan_stats(2048, 1, 70000, 64, lens[:2048], "fwd")[2] == 1
    assert sa.plan_stats(2500, 1, 65535, 64, lens, "fwd")[2] == 1
