"""Parity of the HIP path (through the C-ABI) with the CPU fp64 oracle.

Bound, elementwise for O, dQ, dK and dV:  |gpu - oracle| <= 2e-2 * (1 + |oracle|).
Padded output rows must be exactly 0.

* Small cases (the tiny workload and ragged edge cases spanning several tiles
  and a partial last tile): every element is compared.
* Full-size workloads: every (sequence, head) is compared in
  test_gpu_zfull_parity.py.
"""
import numpy as np
import pytest
import torch

import oracle
import sigmoid_attention_amd as sa
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


@pytest.mark.parametrize("B,H,Lmax,lo", [(1024, 2, 256, 1), (4096, 1, 128, 100), (1536, 3, 512, 1)],
                         ids=["B1024", "B4096", "B1536-mixed"])
def test_many_short_sequences_every_element(B, H, Lmax, lo):
    """Single-cell batches of many short cells: every pass is one launch
    (pieces span many sequences; the lengths travel in the kernel arguments),
    and the fused backward is the call the bench times.  The mixed batch has
    1 to 4 tiles per sequence and 3 heads, so the sequences of one piece
    carry different item counts (up to 12) for the kernels' wave-wide
    search."""
    rng = np.random.default_rng(B)
    lens = rng.integers(lo, Lmax + 1, size=B)
    lens[: B // 8] = Lmax  # some full-length cells: no padding to zero there
    for pass_ in ("fwd", "bwd"):
        assert sa.plan_stats(B, H, Lmax, 64, lens, pass_)[2] == 1, pass_
    case = workloads.random_case(B, H, 64, Lmax, lens, seed=B + 1)
    t = to_dev(case)
    got = run_all(t, lens, "fast", fused=True)
    ref = oracle.attention(host(case["q"]), host(case["k"]), host(case["v"]), lens, do=host(case["do"]))
    ratios = {k: worst_ratio(host(got[k]), ref[k]) for k in OUTS}
    print(f"[parity] many short B={B} H={H} Lmax={Lmax} ratios={ratios}", flush=True)
    for k in OUTS:
        assert ratios[k] <= 1.0, (k, ratios)
        assert padded_rows_zero(got[k], lens), f"{k}: padded rows not zero"
