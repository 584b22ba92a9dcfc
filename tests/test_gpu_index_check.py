"""The debug index check on the GPU.

The device check alone runs on corrupt lists (it reads only inside the
lists' own buffers); the full path runs in debug mode on valid lists only,
and on lists whose fault keeps every value in range (rows out of order), so
that no kernel could read out of bounds even if the check let them through.
"""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

from hierarchical_top_sparse_mean_amd import llsa as L  # noqa: E402

from parity_util import Case  # noqa: E402
from test_index_check import SHAPES, _corrupt, oracle_lists  # noqa: E402


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _device_flags(p, idx, ptr, col):
    status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    L.llsa_check_indices(p, idx.cuda(), None if ptr is None else ptr.cuda(),
                         None if col is None else col.cuda(), status)
    torch.cuda.synchronize()
    return int(status.item())


@pytest.mark.parametrize("shape", SHAPES)
def test_device_check_passes_valid_lists(shape):
    _log(f"[index check] valid {shape}")
    p, _, idx, ptr, col = oracle_lists(*shape)
    assert _device_flags(p, idx, ptr, col) == 0
    assert _device_flags(p, idx, None, None) == 0


@pytest.mark.parametrize("what", ["range_high", "range_negative", "order", "duplicate", "parent",
                                  "ptr_start", "ptr_end", "ptr_decreasing", "col_range",
                                  "col_wrong_row", "col_order"])
def test_device_check_flags_equal_host_flags(what):
    _log(f"[index check] corrupt {what}")
    p, idx, ptr, col = _corrupt(SHAPES[0], what)
    want = L.llsa_check_indices_host(p, idx, ptr, col)
    assert want != 0
    assert _device_flags(p, idx, ptr, col) == want


@pytest.mark.parametrize("b,h,N,L_,K,Le,block", [(1, 4, 4096, 2, 8, 1, 16), (1, 2, 8192, 3, 4, 2, 16),
                                                 (1, 2, 16384, 2, 8, 1, 64)])
def test_debug_mode_full_path_matches_normal_path(b, h, N, L_, K, Le, block):
    # on valid lists the debug mode returns ok everywhere and writes the same bytes
    _log(f"[index check] debug path {b} {h} {N} L{L_} K{K} Le{Le} B{block}")
    c = Case(b, h, N, torch.bfloat16, L_, K, Le, backward=True, sinus=round(N ** 0.5) ** 2 == N,
             block=block)
    q, k, v, do = c.q.cuda(), c.k.cuda(), c.v.cuda(), c.dout.cuda()
    out = []
    for debug in (False, True):
        status = torch.full((1,), -1, dtype=torch.int32, device="cuda")
        p = L.problem(b, h, N, block=block, levels=L_, topk=K, enrich=Le,
                      index_status=status if debug else None)
        B = L.Buffers(p, backward=True)
        L.llsa_pool(p, q, k, v, B.pyr_q, B.pyr_k, B.pyr_v)
        L.llsa_select(p, B.pyr_q, B.pyr_k, B.idx)
        L.llsa_attn_fwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.o, B.lse)
        L.llsa_index_transpose_levels(p, B.idx, B.csr_ptr, B.csr_col, B.tws, B.tws_bytes)
        L.llsa_attn_bwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.csr_ptr, B.csr_col, B.o, B.lse, do,
                        B.dq, B.dk, B.dv, B.ws, B.ws.numel())
        torch.cuda.synchronize()
        if debug:
            assert status.item() == 0
            L.llsa_select_transpose(p, B.pyr_q, B.pyr_k, B.idx, B.csr_ptr, B.csr_col, B.tws, B.tws_bytes)
            torch.cuda.synchronize()
            assert status.item() == 0
        # the lists level by level (the padding between level segments is never written)
        lists = [B.index_level(l) for l in range(1, L_ + 1)]
        lists += [t for l in range(1, Le + 2) for t in B.csr_level(l)]
        out.append([t.clone() for t in lists + [B.o, B.lse, B.dq, B.dk, B.dv]])
    for a, b_ in zip(*out):
        assert torch.equal(a, b_)


def test_debug_mode_rejects_lists_before_any_gather():
    # rows out of order (every value in range): the debug check returns
    # LLSA_ERR_INDEX and the outputs stay untouched
    _log("[index check] debug rejection")
    b, h, N = 1, 2, 4096
    c = Case(b, h, N, torch.bfloat16, 2, 8, 1, backward=True, sinus=True)
    q, k, v, do = c.q.cuda(), c.k.cuda(), c.v.cuda(), c.dout.cuda()
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    p = L.problem(b, h, N, levels=2, topk=8, enrich=1, index_status=status)
    B = L.Buffers(p, backward=True)
    L.llsa_pool(p, q, k, v, B.pyr_q, B.pyr_k, B.pyr_v)
    _, idx_bad, _, _ = _corrupt(SHAPES[0], "order")
    B.idx.copy_(idx_bad.cuda())
    B.o.fill_(7.0)
    with pytest.raises(L.LLSAError) as e:
        L.llsa_attn_fwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.o, B.lse)
    assert e.value.status == L.LLSA_ERR_INDEX and status.item() == L.LLSA_IDX_ORDER
    assert bool((B.o == 7.0).all())
    with pytest.raises(L.LLSAError) as e:
        L.llsa_index_transpose_levels(p, B.idx, B.csr_ptr, B.csr_col, B.tws, B.tws_bytes)
    assert e.value.status == L.LLSA_ERR_INDEX
    # valid picks, a CSR with two rows of a segment swapped
    _, idx_ok, ptr_bad, col_bad = _corrupt(SHAPES[0], "col_order")
    B.idx.copy_(idx_ok.cuda())
    B.csr_ptr.copy_(ptr_bad.cuda())
    B.csr_col.copy_(col_bad.cuda())
    L.llsa_attn_fwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.o, B.lse)
    assert status.item() == 0
    B.dq.fill_(7.0)
    with pytest.raises(L.LLSAError) as e:
        L.llsa_attn_bwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.csr_ptr, B.csr_col, B.o, B.lse, do,
                        B.dq, B.dk, B.dv, B.ws, B.ws.numel())
    assert e.value.status == L.LLSA_ERR_INDEX and status.item() == L.LLSA_IDX_CSR_COL
    assert bool((B.dq == 7.0).all())
