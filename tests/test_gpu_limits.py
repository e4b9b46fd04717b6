"""The largest accepted Lmax (32-bit slice offsets: (Lmax + 256) * d * 2 <=
2^31 - 1) on the GPU: a short valid prefix is computed and compared with the
CPU fp64 oracle, and the millions of padded rows of every output are zero.
Runs the fused backward the bench times and the separate calls."""
import numpy as np
import pytest
import torch

import oracle
import sigmoid_attention_amd as sa
from gpu_util import worst_ratio

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DEV = torch.device("cuda:0")


@pytest.mark.parametrize("d", [64, 128])
def test_largest_lmax(d):
    L = (2**31 - 1) // (2 * d) - 256
    lens = [777]
    print(f"[limits] d={d} Lmax={L}", flush=True)
    g = torch.Generator().manual_seed(d)
    # only the valid rows hold data; the rest of each tensor is uninitialised
    t = {}
    for x in ("q", "k", "v", "do"):
        t[x] = torch.empty((1, 1, L, d), dtype=torch.bfloat16, device=DEV)
        t[x][:, :, :lens[0]] = torch.randn((1, 1, lens[0], d), generator=g).to(torch.bfloat16).to(DEV)
    o = sa.fwd(t["q"], t["k"], t["v"], lens)
    dq, dk, dv = sa.bwd(t["q"], t["k"], t["v"], t["do"], lens)
    dq0 = sa.bwd_dq(t["q"], t["k"], t["v"], t["do"], lens)
    torch.cuda.synchronize()
    assert torch.equal(dq, dq0)
    n = lens[0]
    host = {x: t[x][:, :, :n].float().cpu().double().numpy() for x in t}
    ref = oracle.attention(host["q"], host["k"], host["v"], lens, do=host["do"])
    for name, got in (("o", o), ("dq", dq), ("dk", dk), ("dv", dv)):
        r = worst_ratio(got[:, :, :n].float().cpu().double().numpy(), ref[name])
        assert r <= 1.0, (name, r)
        assert int(torch.count_nonzero(got[:, :, n:])) == 0, name
