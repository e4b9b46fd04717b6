"""Seeded random configurations on the GPU against the CPU fp64 oracle: shape
(B, H, d, Lmax), lengths (including 0, 1, Lmax and tile edges), precision,
mask, bias mode, element type, layout and backward route are drawn together,
so combinations no hand-written case covers are exercised.  Bound as
everywhere: |gpu - oracle| <= 2e-2 (1 + |oracle|) elementwise, padded rows 0;
the per-head bias gradient rows under the same bound."""
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
N_CASES = 24


def draw(seed):
    g = np.random.default_rng(1000 + seed)
    B = int(g.integers(1, 5))
    H = int(g.integers(1, 4))
    d = int(g.choice([64, 128]))
    L = int(g.choice([1, 63, 64, 65, 127, 128, 129, 200, 257, 320, 400]))
    special = [0, 1, L, max(1, L - 1), min(L, 64), min(L, 128)]
    lens = [int(g.choice(special)) if g.random() < 0.4 else int(g.integers(0, L + 1)) for _ in range(B)]
    return dict(B=B, H=H, d=d, L=L, lens=lens,
                precision=str(g.choice(["fast", "split"])),
                causal=bool(g.random() < 0.35),
                bias=str(g.choice(["seqlen", "const", "per_head"])),
                dtype=torch.float16 if g.random() < 0.3 else torch.bfloat16,
                layout=str(g.choice(["bhld", "blhd"])),
                fused=bool(g.random() < 0.5))


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(seed):
    c = draw(seed)
    print(f"[random] seed={seed} {c}", flush=True)
    case = workloads.random_case(c["B"], c["H"], c["d"], c["L"], c["lens"], seed=seed, dtype=c["dtype"])
    n = case["seqlens"]
    perm = (0, 2, 1, 3) if c["layout"] == "blhd" else (0, 1, 2, 3)
    t = {x: case[x].permute(*perm).contiguous().to(DEV) for x in ("q", "k", "v", "do")}
    kw = dict(precision=c["precision"], causal=c["causal"], layout=c["layout"])
    if c["bias"] == "const":
        kw.update(bias_mode="const", bias_arg=-3.0)
        ref_kw = dict(bias_mode="const", bias_arg=-3.0)
    elif c["bias"] == "per_head":
        vals = -np.log(np.random.default_rng(seed).uniform(20.0, 500.0, size=c["H"]))
        kw.update(bias_mode="per_head", bias_arg=torch.tensor(vals, dtype=torch.float32, device=DEV))
        ref_kw = dict(bias_mode="per_head", bias_arg=vals)
    else:
        ref_kw = {}
    got = {"o": sa.fwd(t["q"], t["k"], t["v"], n, **kw)}
    if c["fused"]:
        got["dq"], got["dk"], got["dv"], got["dbias"] = sa.bwd(t["q"], t["k"], t["v"], t["do"], n, bias_rows=True, **kw)
    else:
        got["dq"] = sa.bwd_dq(t["q"], t["k"], t["v"], t["do"], n, **kw)
        got["dk"], got["dv"], got["dbias"] = sa.bwd_dkdv_dbias(t["q"], t["k"], t["v"], t["do"], n, **kw)
    torch.cuda.synchronize()
    ref = oracle.attention(host(case["q"]), host(case["k"]), host(case["v"]), n, do=host(case["do"]),
                           causal=c["causal"], **ref_kw)
    inv = (0, 2, 1, 3) if c["layout"] == "blhd" else (0, 1, 2, 3)
    ratios = {}
    for name, g_ in got.items():
        x = g_ if name == "dbias" else g_.permute(*inv)
        x = host(x.contiguous())
        ratios[name] = worst_ratio(x, ref[name])
        for b, nb in enumerate(n):
            assert np.all(x[b, :, nb:] == 0), (name, b)
    print(f"[random] seed={seed} ratios={ratios}", flush=True)
    for name, r in ratios.items():
        assert r <= 1.0, (seed, name, ratios)
