"""The learnable per-head bias (bias mode "per_head") and the bias gradient
on the GPU against the CPU fp64 oracle: outputs and gradients elementwise
within |gpu - oracle| <= 2e-2 (1 + |oracle|).

The per-key bias-gradient rows are sums of fp32 dX values that the kernel
forms from fp32 scores; they are held to the same elementwise bound.  The
per-head totals are fp32 sums of B * Lmax of those rows (each of 1024
threads adds at most B * ceil(Lmax / 1024) terms in order, then a 10-level
tree), so they are checked against the float64 sum of the rows the GPU
returned with the standard summation bound (terms per chain) * 2^-24 *
sum |rows|, and against the oracle's total with the row bound summed over
the rows."""
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
CASES = [
    # (B, H, d, Lmax, lengths, causal, precision)
    (2, 3, 64, 200, [200, 77], False, "fast"),
    (3, 2, 64, 300, [300, 1, 0], True, "fast"),
    (2, 2, 128, 260, [260, 131], False, "split"),
    (2, 4, 64, 520, [520, 333], True, "split"),
    (3, 2, 64, 203, [203, 100, 64], False, "fast"),  # Lmax not a multiple of 4: scalar reduction loads
]
IDS = [f"B{c[0]}H{c[1]}d{c[2]}L{c[3]}{'-causal' if c[5] else ''}-{c[6]}" for c in CASES]


def head_values(H, seed):
    g = np.random.default_rng(seed)
    return -np.log(g.uniform(50.0, 800.0, size=H))  # -ln of lengths in the workloads' range


def check_db(got_db, got_rows, rows_ref):
    """db against the GPU's own rows (fp32 summation bound) and against the
    oracle (the elementwise row bound, summed)."""
    B, H, L = got_rows.shape
    own = got_rows.sum(axis=(0, 2))
    chain = B * ((L + 1023) // 1024) + 10
    tol_own = chain * 2.0 ** -24 * np.abs(got_rows).sum(axis=(0, 2)) + 1e-30
    want = rows_ref.sum(axis=(0, 2))
    tol_ref = 2e-2 * (1.0 + np.abs(rows_ref)).sum(axis=(0, 2))
    print(f"[bias] db {got_db} own {own} oracle {want}", flush=True)
    assert np.all(np.abs(got_db - own) <= tol_own), (got_db, own, tol_own)
    assert np.all(np.abs(got_db - want) <= tol_ref), (got_db, want, tol_ref)


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_per_head_bias_and_gradient(case):
    B, H, d, L, lens, causal, precision = case
    c = workloads.random_case(B, H, d, L, lens, seed=31 + H)
    vals = head_values(H, seed=H + d)
    hb = torch.tensor(vals, dtype=torch.float32, device=DEV)
    t = {x: c[x].to(DEV) for x in ("q", "k", "v", "do")}
    n = c["seqlens"]
    kw = dict(bias_mode="per_head", bias_arg=hb, precision=precision, causal=causal)
    o = sa.fwd(t["q"], t["k"], t["v"], n, **kw)
    dq = sa.bwd_dq(t["q"], t["k"], t["v"], t["do"], n, **kw)
    dk, dv, rows = sa.bwd_dkdv_dbias(t["q"], t["k"], t["v"], t["do"], n, **kw)
    dk0, dv0 = sa.bwd_dkdv(t["q"], t["k"], t["v"], t["do"], n, **kw)
    db = sa.bias_grad(rows, n)
    torch.cuda.synchronize()
    ref = oracle.attention(host(c["q"]), host(c["k"]), host(c["v"]), n, do=host(c["do"]),
                           bias_mode="per_head", bias_arg=vals, causal=causal)
    got = {"o": o, "dq": dq, "dk": dk, "dv": dv, "dbias": rows}
    ratios = {k_: worst_ratio(host(got[k_]), ref[k_]) for k_ in got}
    print(f"[bias] {case} ratios={ratios}", flush=True)
    for k_, r in ratios.items():
        assert r <= 1.0, (k_, ratios)
    for b, nb in enumerate(n):
        assert bool((rows[b, :, nb:] == 0).all())
    # the bias-gradient variant computes dK and dV exactly as the plain call
    assert torch.equal(dk, dk0) and torch.equal(dv, dv0)
    check_db(host(db), host(rows), ref["dbias"])


def test_dbias_rows_in_constant_modes():
    """The rows are reported in any bias mode: the default b = -ln n_b and a
    constant, against the oracle's rows in the same modes."""
    c = workloads.random_case(3, 2, 64, 200, [200, 130, 1], seed=37)
    t = {x: c[x].to(DEV) for x in ("q", "k", "v", "do")}
    n = c["seqlens"]
    for mode, arg in (("seqlen", 0.0), ("const", -2.5)):
        _, _, rows = sa.bwd_dkdv_dbias(t["q"], t["k"], t["v"], t["do"], n, bias_mode=mode, bias_arg=arg)
        torch.cuda.synchronize()
        ref = oracle.attention(host(c["q"]), host(c["k"]), host(c["v"]), n, do=host(c["do"]),
                               bias_mode=mode, bias_arg=arg if mode == "const" else None)
        assert worst_ratio(host(rows), ref["dbias"]) <= 1.0, mode


def test_learnable_bias_autograd_and_module():
    """A trained per-head bias through autograd (the [B, L, H, d] layout of a
    model) and through the module: gradients of q, k, v and of the bias."""
    B, H, d, L, lens = 2, 4, 64, 260, [260, 190]
    c = workloads.random_case(B, H, d, L, lens, seed=41)
    vals = head_values(H, seed=5)
    perm = (0, 2, 1, 3)
    q, k, v = (c[x].permute(*perm).contiguous().to(DEV).requires_grad_(True) for x in ("q", "k", "v"))
    w = c["do"].permute(*perm).contiguous().to(DEV)
    hb = torch.tensor(vals, dtype=torch.float32, device=DEV, requires_grad=True)
    o = sa.sigmoid_attention(q, k, v, c["seqlens"], layout="blhd", bias_mode="per_head", bias_arg=hb)
    (o.float() * w.float()).sum().backward()
    torch.cuda.synchronize()
    ref = oracle.attention(host(c["q"]), host(c["k"]), host(c["v"]), c["seqlens"], do=host(c["do"]),
                           bias_mode="per_head", bias_arg=vals)
    inv = (0, 2, 1, 3)
    for name, g in (("o", o.detach()), ("dq", q.grad), ("dk", k.grad), ("dv", v.grad)):
        assert worst_ratio(host(g.permute(*inv).contiguous()), ref[name]) <= 1.0, name
    _, _, rows = sa.bwd_dkdv_dbias(q.detach(), k.detach(), v.detach(), w, c["seqlens"], bias_mode="per_head",
                                   bias_arg=hb.detach(), layout="blhd")
    torch.cuda.synchronize()
    check_db(host(hb.grad), host(rows), ref["dbias"])

    mod = sa.SigmoidAttention(bias_mode="per_head", bias_arg=float(vals[0]), heads=H).to(DEV)
    with torch.no_grad():
        mod.head_bias.copy_(torch.tensor(vals, dtype=torch.float32))
    q.grad = k.grad = v.grad = None
    o2 = mod(q, k, v, seqlens=c["seqlens"])
    (o2.float() * w.float()).sum().backward()
    torch.cuda.synchronize()
    assert torch.equal(o2.detach(), o.detach())
    assert torch.equal(mod.head_bias.grad, hb.grad)
