"""The whole step (pool, select, attention forward, level transposes,
backward) captured once as a HIP graph and replayed: every replay writes the
bytes of the eager step, also with other work and synchronisations between
the replays.  The library allocates nothing and records no memset, so its
calls capture as plain kernel launches."""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

from hierarchical_top_sparse_mean_amd import llsa as L  # noqa: E402

from parity_util import Case  # noqa: E402


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("b,h,N,L_,K,Le,dtype", [(1, 4, 16384, 2, 8, 1, torch.bfloat16),
                                                  (1, 2, 8192, 3, 4, 2, torch.bfloat16),
                                                  (1, 2, 8192, 2, 8, 1, torch.float32)])
def test_graph_replays_equal_eager(b, h, N, L_, K, Le, dtype):
    _log(f"[graph] {b} {h} {N} L{L_} K{K} Le{Le} {dtype}")
    c = Case(b, h, N, dtype, L_, K, Le, backward=True, sinus=round(N ** 0.5) ** 2 == N)
    q, k, v, do = c.q.cuda(), c.k.cuda(), c.v.cuda(), c.dout.cuda()
    B = L.Buffers(c.p, backward=True)

    def step():
        L.forward(B, q, k, v)
        L.backward(B, q, k, v, do)

    outs = lambda: [t.clone() for t in (B.o, B.lse, B.dq, B.dk, B.dv)]  # noqa: E731
    step()
    torch.cuda.synchronize()
    eager = outs()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for r in range(3):
        for t in (B.o, B.dq, B.dk, B.dv):
            t.fill_(float("nan"))
        scratch.mul_(1.5).add_(1.0)   # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, a, e in zip(("o", "lse", "dq", "dk", "dv"), outs(), eager):
            assert torch.equal(a, e), (r, name)
