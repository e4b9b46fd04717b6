"""The short-sequence backward: when every sequence fits 256 rows (sigmoid,
fast precision, head dim 64, no mask, no bias gradient), sigattn_bwd runs one
workgroup per (sequence, head) (4 waves for Lmax <= 128, 8 waves up to 256)
that computes S, dP and dS once for dQ, dK and dV.  Its dK and dV take the
dK/dV kernel's arithmetic in the same order (bitwise equal to
sigattn_bwd_dkdv); its dQ uses that side's dS (scores from the prescaled K
rather than the prescaled Q), so it is checked against the CPU fp64 oracle,
element by element, with the padded rows zero."""
import numpy as np
import pytest
import torch

import oracle
import sigmoid_attention_amd as sa
import workloads
from gpu_util import host, padded_rows_zero, worst_ratio

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DEV = torch.device("cuda:0")
CASES = [
    # B, H, Lmax, lengths, bias_mode, bias_arg, dtype
    (5, 3, 128, [128, 77, 1, 0, 64], "seqlen", 0.0, torch.bfloat16),
    (4, 2, 96, [96, 50, 17, 33], "per_head", [-4.0, -2.5], torch.bfloat16),
    (3, 4, 128, [128, 128, 100], "fixed_n", 200.0, torch.float16),
    (6, 1, 16, [16, 3, 0, 16, 9, 1], "const", -1.5, torch.bfloat16),
    (2, 2, 40, [0, 0], "seqlen", 0.0, torch.bfloat16),
    # 8 waves: two 128-row tiles, dQ in two 128-query pairs
    (5, 3, 256, [256, 129, 128, 1, 0], "seqlen", 0.0, torch.bfloat16),
    (4, 2, 200, [200, 77, 150, 33], "per_head", [-4.0, -2.5], torch.bfloat16),
    (3, 2, 256, [255, 256, 193], "fixed_n", 300.0, torch.float16),
    (3, 1, 129, [129, 0, 65], "const", -2.0, torch.bfloat16),
]
IDS = [f"B{c[0]}H{c[1]}L{c[2]}-{c[4]}-{str(c[6])[6:]}" for c in CASES]


def _bias(mode, arg):
    if mode == "per_head":
        return torch.tensor(arg, dtype=torch.float32, device=DEV), np.asarray(arg, dtype=np.float64)
    return arg, arg


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_one_tile_backward(case):
    B, H, L, lens, mode, arg, dt = case
    print(f"[one-tile] {case}", flush=True)
    assert sa.plan_stats(B, H, L, 64, lens, "bwd")[2] == sa.plan_stats(B, H, L, 64, lens, "bwd_dkdv")[2]
    c = workloads.random_case(B, H, 64, L, lens, seed=71 + B, dtype=dt)
    t = {x: c[x].to(DEV) for x in ("q", "k", "v", "do")}
    n = c["seqlens"]
    barg, oarg = _bias(mode, arg)
    kw = dict(bias_mode=mode, bias_arg=barg)
    # outputs start as NaN: every element must be written
    dq, dk, dv = (torch.full_like(t["q"], float("nan")) for _ in range(3))
    sa.bwd(t["q"], t["k"], t["v"], t["do"], n, dq=dq, dk=dk, dv=dv, **kw)
    dk0, dv0 = sa.bwd_dkdv(t["q"], t["k"], t["v"], t["do"], n, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0)
    ref = oracle.attention(host(c["q"]), host(c["k"]), host(c["v"]), n, do=host(c["do"]), bias_mode=mode,
                           bias_arg=oarg)
    ratios = {name: worst_ratio(host(g), ref[name]) for name, g in (("dq", dq), ("dk", dk), ("dv", dv))}
    print(f"[one-tile] ratios={ratios}", flush=True)
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        assert ratios[name] <= 1.0, (name, ratios)
        assert padded_rows_zero(g, n), name


def test_one_tile_strided_fused_qkv_layout():
    """[B, L, 3, H, d] projection slices in, one [B, L, 3, H, d] gradient buffer out."""
    B, H, L, lens = 3, 4, 240, [240, 60, 129]
    c = workloads.random_case(B, H, 64, L, lens, seed=81)
    qkv = torch.stack([c[x].permute(0, 2, 1, 3) for x in ("q", "k", "v")], dim=2).contiguous().to(DEV)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    do = c["do"].permute(0, 2, 1, 3).contiguous().to(DEV)
    g = torch.full_like(qkv, float("nan"))
    n = c["seqlens"]
    sa.bwd(q, k, v, do, n, dq=g[:, :, 0], dk=g[:, :, 1], dv=g[:, :, 2], layout="blhd")
    dq, dk, dv = sa.bwd(c["q"].to(DEV), c["k"].to(DEV), c["v"].to(DEV), c["do"].to(DEV), n)
    torch.cuda.synchronize()
    for i, ref in enumerate((dq, dk, dv)):
        assert torch.equal(g[:, :, i].permute(0, 2, 1, 3), ref), i


@pytest.mark.parametrize("L,lens", [(128, [128, 100, 64, 1, 127, 90, 33, 128]),
                                    (256, [256, 200, 129, 1, 255, 128, 64, 17])], ids=["L128", "L256"])
def test_one_tile_matches_two_kernel_route_closely(L, lens):
    """The same batch at Lmax L (short-sequence kernel) and 257 (the fused
    two-kernel launch; the extra rows are padding in every sequence): dK and
    dV agree bitwise, dQ to the rounding of the prescaled operand."""
    B, H = len(lens), 2
    c = workloads.random_case(B, H, 64, L, lens, seed=82 + L)
    t = {x: c[x].to(DEV) for x in ("q", "k", "v", "do")}
    pad = {x: torch.nn.functional.pad(t[x], (0, 0, 0, 257 - L)) for x in t}
    n = c["seqlens"]
    assert sa.plan_stats(B, H, 257, 64, n, "bwd")[2] == 1
    dq, dk, dv = sa.bwd(t["q"], t["k"], t["v"], t["do"], n)
    dq1, dk1, dv1 = sa.bwd(pad["q"], pad["k"], pad["v"], pad["do"], n)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk1[:, :, :L]) and torch.equal(dv, dv1[:, :, :L])
    a, b = host(dq), host(dq1[:, :, :L])
    assert np.max(np.abs(a - b) / (1e-2 * (1.0 + np.abs(b)))) <= 1.0


@pytest.mark.parametrize("L,lens", [(128, [128, 77, 0, 1]), (256, [256, 129, 100, 0])], ids=["L128", "L256"])
def test_one_tile_bias_rows(L, lens):
    """With the bias-gradient rows (a learnable per-head bias): the rows, dK
    and dV bitwise those of sigattn_bwd_dkdv_dbias, every output against the
    oracle, padded rows 0 (outputs pre-filled with NaN)."""
    B, H = len(lens), 3
    c = workloads.random_case(B, H, 64, L, lens, seed=90 + L)
    t = {x: c[x].to(DEV) for x in ("q", "k", "v", "do")}
    n = c["seqlens"]
    vals = [-float(np.log(x)) for x in (60.0, 250.0, 700.0)]  # -ln n for lengths in the workloads' range
    kw = dict(bias_mode="per_head", bias_arg=torch.tensor(vals, dtype=torch.float32, device=DEV))
    dq, dk, dv = (torch.full_like(t["q"], float("nan")) for _ in range(3))
    rows = torch.full((B, H, L), float("nan"), dtype=torch.float32, device=DEV)
    sa.bwd(t["q"], t["k"], t["v"], t["do"], n, dq=dq, dk=dk, dv=dv, dbias=rows, **kw)
    dk0, dv0, rows0 = sa.bwd_dkdv_dbias(t["q"], t["k"], t["v"], t["do"], n, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0) and torch.equal(rows, rows0)
    ref = oracle.attention(host(c["q"]), host(c["k"]), host(c["v"]), n, do=host(c["do"]), bias_mode="per_head",
                           bias_arg=np.asarray(vals))
    got = {"dq": dq, "dk": dk, "dv": dv, "dbias": rows}
    ratios = {k_: worst_ratio(host(g), ref[k_]) for k_, g in got.items()}
    print(f"[one-tile] bias rows L={L} ratios={ratios}", flush=True)
    for k_, r in ratios.items():
        assert r <= 1.0, (k_, ratios)
    for b, nb in enumerate(n):
        assert bool((rows[b, :, nb:] == 0).all())
        for g in (dq, dk, dv):
            assert bool((g[b, :, nb:] == 0).all())
