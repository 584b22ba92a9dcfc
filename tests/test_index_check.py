"""The debug index check's rules, run on the CPU through the library's host
form (llsa_check_indices_host, the same checks the device kernels apply):
valid lists from the oracle pass, and each kind of corruption sets its flag.

The lists drive every gather of both passes (abstract: the operator is
driven by sparse indices alone), so each rule guards a class of bad input:
range, order, the hierarchy (a pick must be a child of a parent pick) and the
CSR being exactly the transpose of the pick lists (explainer, "Step 4")."""
import numpy as np
import pytest
import torch

from hierarchical_top_sparse_mean_amd import llsa as L
from hierarchical_top_sparse_mean_amd.inputs import make_inputs
from oracle import oracle as O


def oracle_lists(batch, heads, N, block, levels, K, enrich):
    """Pick lists of every level and CSR of levels 1..Le+1 from the oracle,
    packed in the library's layout (host int32 tensors)."""
    p = L.problem(batch, heads, N, block=block, levels=levels, topk=K, enrich=enrich)
    s = L.llsa_sizes_query(p)
    square = round(N ** 0.5) ** 2 == N
    q, k, _, _ = make_inputs(batch, heads, N, 64, torch.bfloat16, square, False, 1)
    bh = batch * heads
    q, k = (x.double().numpy().reshape(bh, N, 64) for x in (q, k))
    idx_l, _ = O.select(O.pool(q, block, levels), O.pool(k, block, levels), block, K)
    idx = np.zeros(s.index_elems, dtype=np.int32)
    ptr = np.zeros(s.csr_ptr_elems, dtype=np.int32)
    col = np.zeros(s.csr_col_elems, dtype=np.int32)
    for l in range(1, levels + 1):
        a = idx_l[l - 1].ravel()
        idx[s.index_offset[l]:s.index_offset[l] + a.size] = a
    for l in range(1, s.enrich + 2):
        pr, cl = O.transpose(idx_l[l - 1], s.level_tokens[l])
        ptr[s.csr_ptr_offset[l]:s.csr_ptr_offset[l] + pr.size] = pr.ravel()
        col[s.csr_col_offset[l]:s.csr_col_offset[l] + cl.size] = cl.ravel()
    return p, s, torch.from_numpy(idx), torch.from_numpy(ptr), torch.from_numpy(col)


SHAPES = [(1, 2, 4096, 16, 2, 8, 1), (2, 1, 8192, 16, 3, 4, 2), (1, 2, 16384, 64, 2, 5, 1),
          (1, 1, 336, 16, 1, 5, 0)]


@pytest.mark.parametrize("shape", SHAPES)
def test_valid_lists_pass(shape):
    p, _, idx, ptr, col = oracle_lists(*shape)
    assert L.llsa_check_indices_host(p, idx, ptr, col) == 0
    assert L.llsa_check_indices_host(p, idx) == 0


def _corrupt(shape, what):
    p, s, idx, ptr, col = oracle_lists(*shape)
    k1, n1 = s.level_k[1], s.level_tokens[1]
    o1, c1, p1 = s.index_offset[1], s.csr_col_offset[1], s.csr_ptr_offset[1]
    if what == "range_high":
        idx[o1 + 3 * k1 + 1] = n1
    elif what == "range_negative":
        idx[o1 + 5 * k1] = -1
    elif what == "order":            # two picks of a row swapped (values still in range)
        a, b = idx[o1 + 2].item(), idx[o1 + 3].item()
        idx[o1 + 2], idx[o1 + 3] = b, a
    elif what == "duplicate":
        idx[o1 + 1] = idx[o1]
    elif what == "parent":           # a level-1 pick that is no child of the parent's picks
        par = idx[s.index_offset[2]:s.index_offset[2] + s.level_k[2]].tolist()
        idx[o1 + k1 - 1] = max(c for c in range(n1) if c // p.block not in par)
    elif what == "ptr_start":
        ptr[p1] = 1
    elif what == "ptr_end":
        ptr[p1 + n1] = n1 * k1 - 1
    elif what == "ptr_decreasing":
        mid = p1 + n1 // 2
        ptr[mid] = ptr[mid + 1] + 1
    elif what == "col_range":
        col[c1 + 7] = n1 + 3
    elif what == "col_wrong_row":    # a listed row that did not pick the key
        seg0 = ptr[p1 + 1].item()
        rows = set(col[c1:c1 + seg0].tolist())
        col[c1] = next(r for r in range(n1) if r not in rows and r < (col[c1 + 1].item() if seg0 > 1 else n1))
    elif what == "col_order":        # two rows of one segment swapped
        c = next(c for c in range(n1) if ptr[p1 + c + 1] - ptr[p1 + c] >= 2)
        a = ptr[p1 + c].item()
        col[c1 + a], col[c1 + a + 1] = col[c1 + a + 1].item(), col[c1 + a].item()
    return p, idx, ptr, col


@pytest.mark.parametrize("what,flag", [
    ("range_high", L.LLSA_IDX_RANGE), ("range_negative", L.LLSA_IDX_RANGE),
    ("order", L.LLSA_IDX_ORDER), ("duplicate", L.LLSA_IDX_ORDER),
    ("parent", L.LLSA_IDX_PARENT),
    ("ptr_start", L.LLSA_IDX_CSR_PTR), ("ptr_end", L.LLSA_IDX_CSR_PTR),
    ("ptr_decreasing", L.LLSA_IDX_CSR_PTR),
    ("col_range", L.LLSA_IDX_CSR_COL), ("col_wrong_row", L.LLSA_IDX_CSR_COL),
    ("col_order", L.LLSA_IDX_CSR_COL),
])
def test_each_corruption_sets_its_flag(what, flag):
    p, idx, ptr, col = _corrupt(SHAPES[0], what)
    f = L.llsa_check_indices_host(p, idx, ptr, col)
    assert f & flag, (what, f)
    if flag < L.LLSA_IDX_CSR_PTR:
        assert L.llsa_check_indices_host(p, idx) & flag   # pick-list faults without the CSR too
    else:
        assert L.llsa_check_indices_host(p, idx) == 0     # CSR faults only with the CSR


def test_csr_rows_shifted_between_keys_are_rejected():
    # the same multiset of rows and the same ptr, every row moved one slot on:
    # rows land in segments of keys they did not pick
    p, s, idx, ptr, col = oracle_lists(*SHAPES[0])
    c1, n1, k1 = s.csr_col_offset[1], s.level_tokens[1], s.level_k[1]
    col[c1:c1 + n1 * k1] = torch.roll(col[c1:c1 + n1 * k1].clone(), 1)
    assert L.llsa_check_indices_host(p, idx, ptr, col) & L.LLSA_IDX_CSR_COL


def test_host_check_rejects_bad_arguments():
    with pytest.raises(L.LLSAError):   # 1000 tokens: not a whole number of coarsest blocks
        L.llsa_check_indices_host(L.problem(1, 2, 1000, levels=2, topk=8),
                                  torch.zeros(16, dtype=torch.int32))
    p = L.problem(1, 2, 4096, levels=2, topk=8)
    assert L.lib.llsa_check_indices_host(p, None, None, None, None) == L.LLSA_ERR_INVALID
