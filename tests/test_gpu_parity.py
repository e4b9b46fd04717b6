"""Parity of the HIP path (through the C-ABI) with the CPU fp64 oracle.

Bound, elementwise for O, dQ, dK and dV:  |gpu - oracle| <= 2e-2 * (1 + |oracle|).
Padded output rows must be exactly 0.

* Small cases (the tiny workload and ragged edge cases spanning several tiles
  and a partial last tile): every element is compared.
* Full-size workloads, called exactly as the bench calls them: sampled heads
  (the longest and the shortest sequence, plus a random one) are computed by
  the oracle one by one and compared row by row; every padded row of every
  head is checked to be 0 and every output to be finite.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_util import host, padded_rows_zero, run_all, to_dev, worst_ratio

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

OUTS = ("o", "dq", "dk", "dv")


def check_full(case, precision="fast", bias_mode="seqlen", bias_arg=0.0, label=""):
    t = to_dev(case)
    n = case["seqlens"]
    got = run_all(t, n, precision, bias_mode, bias_arg)
    ref = oracle.attention(host(case["q"]), host(case["k"]), host(case["v"]), n, do=host(case["do"]),
                           bias_mode=bias_mode, bias_arg=bias_arg)
    ratios = {k: worst_ratio(host(got[k]), ref[k]) for k in OUTS}
    print(f"[parity] {label} precision={precision} ratios={ratios}", flush=True)
    for k in OUTS:
        assert ratios[k] <= 1.0, (k, ratios)
        assert padded_rows_zero(got[k], n), f"{k}: padded rows not zero"
    return ratios


@pytest.mark.parametrize("precision", ["fast", "split"])
def test_tiny_workload_every_element(precision):
    case = workloads.make(workloads.TINY)
    check_full(case, precision, label=workloads.TINY)


EDGE = [
    # (B, H, d, Lmax, lengths)
    (3, 2, 64, 300, [300, 1, 0]),
    (5, 2, 64, 200, [127, 128, 129, 64, 65]),
    (2, 3, 128, 192, [192, 100]),
    (1, 1, 64, 64, [64]),
    (2, 2, 64, 1, [1, 0]),
    (1, 2, 128, 130, [130]),
    (2, 1, 64, 520, [520, 257]),
    (4, 1, 128, 260, [0, 0, 0, 0]),
]


@pytest.mark.parametrize("precision", ["fast", "split"])
@pytest.mark.parametrize("shape", EDGE, ids=lambda s: f"B{s[0]}H{s[1]}d{s[2]}L{s[3]}")
def test_edge_cases_every_element(shape, precision):
    B, H, d, L, lens = shape
    case = workloads.random_case(B, H, d, L, lens, seed=sum(lens) + d)
    check_full(case, precision, label=str(shape))


@pytest.mark.parametrize("mode,arg,precision", [("fixed_n", 4096.0, "fast"), ("const", -2.5, "fast"),
                                                ("fixed_n", 4096.0, "split"), ("const", -2.5, "split"),
                                                ("const", 0.0, "split")])
def test_bias_modes_every_element(mode, arg, precision):
    """A constant bias of 0 makes every weight about 1/2: hundreds of O(1)
    weights per row then sum with bf16 rounding errors of 2^-9 each, beyond
    the bound, so that case needs the split (hi + lo) precision."""
    case = workloads.random_case(3, 2, 64, 200, [200, 77, 130], seed=5)
    check_full(case, precision, mode, arg, label=f"bias {mode} {arg}")


def test_saturated_scores_split_every_element():
    """Scores scaled x4 (|x| >> 10) on a ragged batch: split precision keeps
    the many small saturated weights accurate."""
    case = workloads.random_case(2, 2, 64, 700, [700, 333], seed=9, scale_qkv=4.0)
    check_full(case, "split", label="x4 ragged")


FULL = [
    ("cells_b8h16d64_l2048", "fast"),
    ("sweep_b16h16d64_l4096_pad00", "fast"),
    ("sweep_b16h16d64_l4096_pad25", "fast"),
    ("sweep_b16h16d64_l4096_pad50", "fast"),
    ("dense_b4h16d128_l8192", "fast"),
    ("cells8k_b8h12d64_l8192_x4", "split"),
]


def sampled_heads(seqlens, H, seed=0):
    lens = np.asarray(seqlens)
    nz = np.flatnonzero(lens > 0)
    picks = {(int(nz[np.argmax(lens[nz])]), 0), (int(nz[np.argmin(lens[nz])]), H - 1)}
    rng = np.random.default_rng(seed)
    picks.add((int(rng.choice(nz)), int(rng.integers(H))))
    return sorted(picks)


@pytest.mark.parametrize("name,precision", FULL, ids=[f[0] for f in FULL])
def test_full_size_workload_sampled_heads(name, precision):
    """Full-size workloads in the launch configuration the bench times (the
    fused backward)."""
    case = workloads.make(name)
    w = case["workload"]
    n = case["seqlens"]
    t = to_dev(case)
    got = run_all(t, n, precision, fused=True)
    for k in OUTS:
        assert bool(torch.isfinite(got[k]).all().item()), f"{k} has non-finite values"
        assert padded_rows_zero(got[k], n), f"{k}: padded rows not zero"
    for b, h in sampled_heads(n, w.H):
        ref = oracle.head(host(case["q"][b, h]), host(case["k"][b, h]), host(case["v"][b, h]),
                          host(case["do"][b, h]), int(n[b]))
        ratios = {k: worst_ratio(host(got[k][b, h]), r) for k, r in zip(OUTS, ref)}
        print(f"[parity] {name} b={b} h={h} n={n[b]} precision={precision} ratios={ratios}", flush=True)
        for k in OUTS:
            assert ratios[k] <= 1.0, (name, b, h, k, ratios)
