"""The library's calls enqueue kernel launches only (no allocation, copy or
memset), so a forward + fused backward step can be captured in a HIP graph
and replayed.  The graph is replayed several times with new input values
copied in between (eager work and synchronisation between replays), and
every replay must equal the eager calls on the same inputs bitwise."""
import pytest
import torch

import sigmoid_attention_amd as sa
import workloads

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")]

DEV = torch.device("cuda:0")


# Lmax 300: the fused two-kernel backward; 200 without a mask: the
# short-sequence backward (one workgroup per (sequence, head))
@pytest.mark.parametrize("causal,L", [(False, 300), (True, 300), (False, 200)])
def test_graph_replays_match_eager(causal, L):
    B, H, d, lens = 3, 2, 64, [L, 129, 0]
    cases = [workloads.random_case(B, H, d, L, lens, seed=70 + i) for i in range(3)]
    q, k, v, do = (torch.empty((B, H, L, d), dtype=torch.bfloat16, device=DEV) for _ in range(4))
    o, dq, dk, dv = (torch.empty_like(q) for _ in range(4))
    n = cases[0]["seqlens"]

    def step():
        sa.fwd(q, k, v, n, o=o, causal=causal)
        sa.bwd(q, k, v, do, n, dq=dq, dk=dk, dv=dv, causal=causal)

    def load(c):
        for dst, name in ((q, "q"), (k, "k"), (v, "v"), (do, "do")):
            dst.copy_(c[name].to(DEV))

    load(cases[0])
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on the capture stream
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for c in cases:
        load(c)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [x.clone() for x in (o, dq, dk, dv)]
        step()  # eager on the same inputs
        torch.cuda.synchronize()
        for g, e in zip(got, (o, dq, dk, dv)):
            assert torch.equal(g, e)
