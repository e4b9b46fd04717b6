"""fp16 tensors (args dtype = fp16: the fp16 build of the kernels, fp16 MFMA,
P and dX rounded to fp16) against the CPU fp64 oracle on the same fp16
inputs widened exactly: |gpu - oracle| <= 2e-2 (1 + |oracle|) elementwise,
padded rows 0, for the sigmoid path (both precisions, causal, per-head bias
with its gradient) and the softmax path."""
import math

import numpy as np
import pytest
import torch

import oracle
import sigmoid_attention_amd as sa
import workloads
from gpu_util import host, worst_ratio
from oracle import softmax_oracle

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DEV = torch.device("cuda:0")
SHAPES = [
    (2, 2, 64, 128, [128, 77]),
    (3, 2, 64, 300, [300, 1, 0]),
    (2, 2, 128, 260, [260, 131]),
    (1, 2, 64, 700, [700]),
]
IDS = [f"B{s[0]}H{s[1]}d{s[2]}L{s[3]}" for s in SHAPES]


def case16(shape, seed):
    B, H, d, L, lens = shape
    return workloads.random_case(B, H, d, L, lens, seed=seed, dtype=torch.float16)


def check(got, ref, n, label):
    ratios = {k: worst_ratio(host(got[k]), ref[k]) for k in got}
    print(f"[fp16] {label} ratios={ratios}", flush=True)
    for k, r in ratios.items():
        assert r <= 1.0, (label, k, ratios)
        for b, nb in enumerate(n):
            assert bool((got[k][b, :, nb:] == 0).all()), (label, k, b)
    return ratios


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("precision", ["fast", "split"])
@pytest.mark.parametrize("shape", SHAPES, ids=IDS)
def test_fp16_sigmoid(shape, precision, causal):
    c = case16(shape, seed=51)
    t = {x: c[x].to(DEV) for x in ("q", "k", "v", "do")}
    n = c["seqlens"]
    kw = dict(precision=precision, causal=causal)
    got = {"o": sa.fwd(t["q"], t["k"], t["v"], n, **kw), "dq": sa.bwd_dq(t["q"], t["k"], t["v"], t["do"], n, **kw)}
    got["dk"], got["dv"] = sa.bwd_dkdv(t["q"], t["k"], t["v"], t["do"], n, **kw)
    torch.cuda.synchronize()
    for x in got.values():
        assert x.dtype == torch.float16
    ref = oracle.attention(host(c["q"]), host(c["k"]), host(c["v"]), n, do=host(c["do"]), causal=causal)
    check(got, ref, n, f"sigmoid {shape} {precision} causal={causal}")


def test_fp16_rounds_p_finer_than_bf16():
    """fp16 keeps 11 significant bits of P against bf16's 8, so on the same
    float32 draws (rounded each way) the fast forward's worst error ratio is
    several times smaller in fp16."""
    shape = (2, 4, 64, 512, [512, 400])
    r = {}
    for dt in (torch.bfloat16, torch.float16):
        B, H, d, L, lens = shape
        c = workloads.random_case(B, H, d, L, lens, seed=52, dtype=dt)
        o = sa.fwd(c["q"].to(DEV), c["k"].to(DEV), c["v"].to(DEV), c["seqlens"])
        torch.cuda.synchronize()
        ref = oracle.attention(host(c["q"]), host(c["k"]), host(c["v"]), c["seqlens"])
        r[dt] = worst_ratio(host(o), ref["o"])
    print(f"[fp16] worst ratio bf16 {r[torch.bfloat16]:.4f} fp16 {r[torch.float16]:.4f}", flush=True)
    assert r[torch.float16] < 0.5 * r[torch.bfloat16]


def test_fp16_per_head_bias_gradient():
    shape = (2, 3, 64, 260, [260, 99])
    c = case16(shape, seed=53)
    vals = np.array([-5.0, -6.5, -3.0])
    hb = torch.tensor(vals, dtype=torch.float32, device=DEV)
    t = {x: c[x].to(DEV) for x in ("q", "k", "v", "do")}
    n = c["seqlens"]
    kw = dict(bias_mode="per_head", bias_arg=hb, causal=True)
    got = {"o": sa.fwd(t["q"], t["k"], t["v"], n, **kw), "dq": sa.bwd_dq(t["q"], t["k"], t["v"], t["do"], n, **kw)}
    got["dk"], got["dv"], got["dbias"] = sa.bwd_dkdv_dbias(t["q"], t["k"], t["v"], t["do"], n, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention(host(c["q"]), host(c["k"]), host(c["v"]), n, do=host(c["do"]), bias_mode="per_head",
                           bias_arg=vals, causal=True)
    check(got, ref, n, "per-head bias causal")


@pytest.mark.parametrize("shape", SHAPES[:3], ids=IDS[:3])
def test_fp16_softmax(shape):
    c = case16(shape, seed=54)
    t = {x: c[x].to(DEV) for x in ("q", "k", "v", "do")}
    n = c["seqlens"]
    o, lse2 = sa.softmax_fwd(t["q"], t["k"], t["v"], n)
    dq, dk, dv = sa.softmax_bwd(t["q"], t["k"], t["v"], o, t["do"], lse2, n)
    torch.cuda.synchronize()
    ref = softmax_oracle.attention(host(c["q"]), host(c["k"]), host(c["v"]), n, do=host(c["do"]))
    ref["lse2"] = ref.pop("lse") / math.log(2.0)
    check({"o": o, "lse2": lse2, "dq": dq, "dk": dk, "dv": dv}, ref, n, f"softmax {shape}")


def test_mixed_dtypes_rejected():
    c = case16(SHAPES[0], seed=55)
    q = c["q"].to(DEV)
    k = c["k"].to(DEV).to(torch.bfloat16)
    with pytest.raises(TypeError):
        sa.fwd(q, k, c["v"].to(DEV), c["seqlens"])
