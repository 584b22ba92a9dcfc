"""llsa_attn_bwd_noalloc, the backward entry point that allocates nothing
(its workspace is the library's static device scratch), against
llsa_attn_bwd with a caller workspace: the same bytes on two calls in a row,
the second on a smaller problem, so stale scratch contents must not matter.
"""
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


def _both(b, h, N, L_, K, Le, grad_dtype=torch.float32, dtype=torch.bfloat16):
    c = Case(b, h, N, dtype, L_, K, Le, backward=True, sinus=round(N ** 0.5) ** 2 == N,
             grad_dtype=grad_dtype)
    q, k, v, do = c.q.cuda(), c.k.cuda(), c.v.cuda(), c.dout.cuda()
    B = L.Buffers(c.p, backward=True)
    assert B.s.bwd_workspace_bytes <= L.NOALLOC_SCRATCH_BYTES
    L.llsa_pool(c.p, q, k, v, B.pyr_q, B.pyr_k, B.pyr_v)
    L.llsa_select(c.p, B.pyr_q, B.pyr_k, B.idx)
    L.llsa_attn_fwd(c.p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.o, B.lse)
    L.transpose_levels(B)
    B.ws.fill_(255)   # the caller's workspace starts with junk too
    L.llsa_attn_bwd(c.p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.csr_ptr, B.csr_col, B.o, B.lse, do,
                    B.dq, B.dk, B.dv, B.ws, B.ws.numel())
    want = [t.clone() for t in (B.dq, B.dk, B.dv)]
    for t in (B.dq, B.dk, B.dv):
        t.fill_(7.0)
    L.llsa_attn_bwd_noalloc(c.p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.csr_ptr, B.csr_col, B.o, B.lse,
                            do, B.dq, B.dk, B.dv)
    torch.cuda.synchronize()
    for name, a, w in zip(("dq", "dk", "dv"), (B.dq, B.dk, B.dv), want):
        assert torch.equal(a, w), name


def test_noalloc_backward_matches_workspace_backward_twice():
    # 65536 tokens x 16 heads (22 MiB of scratch), then a smaller problem
    _log("[no-alloc] 1x16x65536 K=8")
    _both(1, 16, 65536, 2, 8, 1)
    _log("[no-alloc] 2x4x16384 K=8, bfloat16 gradients")
    _both(2, 4, 16384, 2, 8, 1, torch.bfloat16)
    _log("[no-alloc] 1x2x8192 three levels")
    _both(1, 2, 8192, 3, 4, 2)
    _log("[no-alloc] 1x4x16384 float32 inputs")
    _both(1, 4, 16384, 2, 8, 1, dtype=torch.float32)


def test_noalloc_rejects_problems_beyond_the_scratch():
    # K = 32 at 65536 tokens x 16 heads needs 70 MiB: rejected on the host
    p = L.problem(1, 16, 65536, levels=2, topk=32, enrich=1)
    s = L.llsa_sizes_query(p)
    assert s.bwd_workspace_bytes > L.NOALLOC_SCRATCH_BYTES
    t = torch.zeros(16, dtype=torch.float32, device="cuda")   # never read: the call launches nothing
    with pytest.raises(L.LLSAError) as e:
        L.llsa_attn_bwd_noalloc(p, t, t, t, t, t, t, t, t, t, t, t, t, t, t)
    assert e.value.status == L.LLSA_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((t == 0).all())
