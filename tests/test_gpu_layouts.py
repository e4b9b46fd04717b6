"""Strided layouts, autograd and the nn.Module face, on the GPU, against the
CPU fp64 oracle (bound |gpu - oracle| <= 2e-2 (1 + |oracle|), elementwise).

The oracle always sees contiguous [B, H, Lmax, d] copies; the library sees
the strided views ([B, Lmax, H, d] activations, slices of a fused QKV
buffer, a K/V head broadcast over query heads) and writes strided outputs.
Memory around strided outputs that belongs to no output element must be left
untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import sigmoid_attention_amd as sa
import workloads
from gpu_util import host, worst_ratio

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DEV = torch.device("cuda:0")
OUTS = ("o", "dq", "dk", "dv")


def reference(case):
    return oracle.attention(host(case["q"]), host(case["k"]), host(case["v"]), case["seqlens"],
                            do=host(case["do"]))


def assert_close(got_bhld: dict, ref: dict, label: str):
    ratios = {k: worst_ratio(host(got_bhld[k].contiguous()), ref[k]) for k in got_bhld}
    print(f"[layouts] {label} ratios={ratios}", flush=True)
    for k, r in ratios.items():
        assert r <= 1.0, (label, k, ratios)


def blhd(t):  # [B, H, L, d] CPU tensor -> [B, L, H, d] contiguous device tensor
    return t.permute(0, 2, 1, 3).contiguous().to(DEV)


def bhld(t):  # [B, L, H, d] view -> [B, H, L, d] view
    return t.permute(0, 2, 1, 3)


@pytest.mark.parametrize("d", [64, 128])
def test_blhd_layout_matches_oracle(d):
    case = workloads.random_case(3, 4, d, 200, [200, 130, 1], seed=11)
    q, k, v, do = (blhd(case[x]) for x in ("q", "k", "v", "do"))
    n = case["seqlens"]
    o = sa.fwd(q, k, v, n, layout="blhd")
    dq = sa.bwd_dq(q, k, v, do, n, layout="blhd")
    dk, dv = sa.bwd_dkdv(q, k, v, do, n, layout="blhd")
    torch.cuda.synchronize()
    for t in (o, dq, dk, dv):
        assert t.shape == q.shape and t.is_contiguous()
    got = {"o": bhld(o), "dq": bhld(dq), "dk": bhld(dk), "dv": bhld(dv)}
    assert_close(got, reference(case), f"blhd d={d}")
    for name, t in got.items():  # padded rows zero
        for b, nb in enumerate(n):
            assert bool((t[b, :, nb:] == 0).all()), name


def test_fused_qkv_views_and_fused_gradient_buffer():
    B, H, d, L = 2, 3, 64, 160
    case = workloads.random_case(B, H, d, L, [160, 97], seed=5)
    n = case["seqlens"]
    qkv = torch.stack([case[x].permute(0, 2, 1, 3) for x in ("q", "k", "v")], dim=2).contiguous().to(DEV)
    q, k, v = qkv.unbind(2)  # [B, L, H, d] views, row stride 3*H*d
    do = blhd(case["do"])
    sentinel = -7.0
    dqkv = torch.full((B, L, 3, H, d), sentinel, dtype=torch.bfloat16, device=DEV)
    o = sa.fwd(q, k, v, n, layout="blhd")
    sa.bwd_dq(q, k, v, do, n, dq=dqkv[:, :, 0], layout="blhd")
    sa.bwd_dkdv(q, k, v, do, n, dk=dqkv[:, :, 1], dv=dqkv[:, :, 2], layout="blhd")
    torch.cuda.synchronize()
    got = {"o": bhld(o), "dq": bhld(dqkv[:, :, 0]), "dk": bhld(dqkv[:, :, 1]), "dv": bhld(dqkv[:, :, 2])}
    assert_close(got, reference(case), "fused qkv")
    assert not bool((dqkv == sentinel).any()), "every element of the fused gradient is an output element"


def test_strided_output_leaves_gaps_untouched():
    B, H, d, L = 2, 2, 64, 130
    case = workloads.random_case(B, H, d, L, [130, 70], seed=9)
    n = case["seqlens"]
    t = {x: case[x].to(DEV) for x in ("q", "k", "v", "do")}
    sentinel = 3.0
    wide = torch.full((B, H, L, 2 * d), sentinel, dtype=torch.bfloat16, device=DEV)
    o = wide[..., :d]  # row stride 2d: the other half of each row is not ours
    sa.fwd(t["q"], t["k"], t["v"], n, o=o)
    torch.cuda.synchronize()
    assert bool((wide[..., d:] == sentinel).all())
    ref = reference(case)
    assert worst_ratio(host(o.contiguous()), ref["o"]) <= 1.0
    assert bool((o[1, :, 70:] == 0).all())


def test_broadcast_kv_head():
    B, H, d, L = 2, 4, 64, 150
    case = workloads.random_case(B, H, d, L, [150, 33], seed=3)
    n = case["seqlens"]
    k1 = case["k"][:, :1].to(DEV)
    v1 = case["v"][:, :1].to(DEV)
    k, v = k1.expand(B, H, L, d), v1.expand(B, H, L, d)  # head stride 0
    q, do = case["q"].to(DEV), case["do"].to(DEV)
    o = sa.fwd(q, k, v, n)
    dq = sa.bwd_dq(q, k, v, do, n)
    dk, dv = sa.bwd_dkdv(q, k, v, do, n)  # per-head gradients
    torch.cuda.synchronize()
    kk = case["k"][:, :1].expand(B, H, L, d).contiguous()
    vv = case["v"][:, :1].expand(B, H, L, d).contiguous()
    ref = oracle.attention(host(case["q"]), host(kk), host(vv), n, do=host(case["do"]))
    assert_close({"o": o, "dq": dq, "dk": dk, "dv": dv}, ref, "broadcast K/V head")


def test_autograd_matches_oracle_gradients():
    B, H, d, L = 2, 2, 64, 200
    case = workloads.random_case(B, H, d, L, [200, 121], seed=21)
    n = case["seqlens"]
    q, k, v = (blhd(case[x]).requires_grad_(True) for x in ("q", "k", "v"))
    w = blhd(case["do"])
    o = sa.sigmoid_attention(q, k, v, n, layout="blhd")
    (o.float() * w.float()).sum().backward()  # dL/dO = w
    torch.cuda.synchronize()
    got = {"o": bhld(o.detach()), "dq": bhld(q.grad), "dk": bhld(k.grad), "dv": bhld(v.grad)}
    assert_close(got, reference(case), "autograd")


def test_module_with_padding_mask_and_fused_projection_grad():
    B, H, d, L = 3, 2, 64, 96
    torch.manual_seed(0)
    lens = [96, 50, 1]
    mask = torch.arange(L)[None, :] >= torch.tensor(lens)[:, None]
    x = torch.randn(B, L, 3 * H * d, device=DEV, dtype=torch.bfloat16, requires_grad=True)
    attn = sa.SigmoidAttention()
    q, k, v = x.view(B, L, 3, H, d).unbind(2)
    o = attn(q, k, v, key_padding_mask=mask.to(DEV))
    o.float().sum().backward()
    torch.cuda.synchronize()
    # same computation through contiguous copies and explicit lengths
    x2 = x.detach().clone().requires_grad_(True)
    q2, k2, v2 = (t.contiguous() for t in x2.view(B, L, 3, H, d).unbind(2))
    o2 = sa.sigmoid_attention(q2, k2, v2, lens, layout="blhd")
    o2.float().sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(o, o2), "strided and contiguous inputs give identical results"
    assert torch.equal(x.grad, x2.grad)
    assert sa.lengths_from_padding_mask(mask).tolist() == lens
    with pytest.raises(ValueError):
        sa.lengths_from_padding_mask(torch.tensor([[False, True, False]]))
