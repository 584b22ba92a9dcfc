"""GPU-vs-oracle comparison helpers used by the GPU parity tests.

The oracle sees the seeded inputs and, where a step consumes pick lists, the
GPU's own lists (teacher forcing), so every row and every output is checked:
  - pyramids: oracle pooling of the inputs;
  - selection, level by level: level L from the oracle's pyramids alone,
    level l < L with the GPU's level-(l+1) picks as parents.  A row must match
    exactly unless the oracle's gap between its K-th and (K+1)-th score is
    below GAP_BAND relative (a near-tie: exempt, counted);
  - O, LSE, dQ, dK, dV: the oracle's attention and backward over the GPU's
    pick lists, on every row;
  - CSR: the oracle's transpose of the GPU's pick lists, exactly.
The oracle's own unforced selection is also compared and the number of
equal rows reported.
"""
from __future__ import annotations

import numpy as np
import torch

from hierarchical_top_sparse_mean_amd import llsa as L
from oracle import oracle as O

GAP_BAND = 1e-5
PYR_TOL = 1e-5


def out_tol(dtype) -> float:
    """Max-abs tolerance for outputs and gradients: 1e-4 for float32 inputs,
    2e-2 for bfloat16 inputs (for bfloat16 gradients, on top of the rounding
    of the stored value, see grad_excess)."""
    return 1e-4 if dtype == torch.float32 else 2e-2


def to_np(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def patch_order(N):
    """Storage row (raster order of an S x S image) of every position of the
    nested-patch sequence: position t has x in its even bits and y in its odd
    bits (Z order), so 4^i consecutive positions form a 2^i x 2^i patch."""
    S = int(round(N ** 0.5))
    assert S * S == N and S & (S - 1) == 0
    t = np.arange(N, dtype=np.int64)
    x = np.zeros(N, dtype=np.int64)
    y = np.zeros(N, dtype=np.int64)
    for b in range(S.bit_length()):
        x |= ((t >> (2 * b)) & 1) << b
        y |= ((t >> (2 * b + 1)) & 1) << b
    return y * S + x


def seq_perm(c):
    """Storage row of each sequence position for case c."""
    return patch_order(c.N) if c.token_order else np.arange(c.N)


class Case:
    """One problem: seeded inputs on the host, a problem descriptor, flags."""

    def __init__(self, batch, heads, N, dtype, L_, K, Le=-1, q=None, k=None, v=None, dout=None,
                 backward=True, drop_covered=True, grad_dtype=torch.float32, seed=0, sinus=False,
                 token_order=0, block=16):
        from hierarchical_top_sparse_mean_amd.inputs import make_inputs
        self.batch, self.heads, self.N, self.dtype, self.L, self.K = batch, heads, N, dtype, L_, K
        self.B = block
        self.Le = L_ - 1 if Le < 0 else Le
        self.backward, self.drop = backward, drop_covered
        self.grad_dtype = grad_dtype
        gq, gk, gv, gd = make_inputs(batch, heads, N, 64, dtype, sinus, backward, seed)
        self.q = gq if q is None else q.to(dtype)
        self.k = gk if k is None else k.to(dtype)
        self.v = gv if v is None else v.to(dtype)
        self.dout = (gd if dout is None else dout.to(dtype)) if backward else None
        self.scale = 1.0 / 8.0
        self.token_order = token_order
        self.p = L.problem(batch, heads, N, 64, block, L_, K, Le, dtype, grad_dtype, 0.0, drop_covered,
                           token_order)

    @property
    def bh(self):
        return self.batch * self.heads


def check_index_lists(idx_levels, B_=16):
    """Host-side sanity of GPU pick lists before any kernel gathers with them:
    in range, ascending, and every pick a child of a parent pick."""
    Lv = len(idx_levels)
    for l in range(Lv, 0, -1):
        I = idx_levels[l - 1]
        n = I.shape[1]
        assert (I >= 0).all() and (I < n).all(), f"level {l}: index out of range"
        assert (np.diff(I, axis=-1) > 0).all(), f"level {l}: rows not ascending"
        if l < Lv:
            par = np.repeat(idx_levels[l], B_, axis=1)[:, :n]          # parent picks per row
            ok = (I[..., :, None] // B_ == par[..., None, :]).any(-1)
            assert ok.all(), f"level {l}: pick outside the parent's children"


def run_gpu(c: Case):
    B = L.Buffers(c.p, backward=c.backward)
    qd, kd, vd = c.q.cuda(), c.k.cuda(), c.v.cuda()
    s = B.s
    L.llsa_pool(B.p, qd, kd, vd, B.pyr_q, B.pyr_k, B.pyr_v)
    L.llsa_select(B.p, B.pyr_q, B.pyr_k, B.idx)
    torch.cuda.synchronize()
    check_index_lists([B.index_level(l).cpu().numpy() for l in range(1, c.L + 1)], c.B)
    L.llsa_attn_fwd(B.p, qd, kd, vd, B.pyr_k, B.pyr_v, B.idx, B.o, B.lse)
    res = {}
    if c.backward:
        L.transpose_levels(B)
        torch.cuda.synchronize()
        for l in range(1, s.enrich + 2):
            ptr, col = (t.cpu().numpy() for t in B.csr_level(l))
            n = s.level_tokens[l]
            assert (ptr[:, 0] == 0).all() and (np.diff(ptr, axis=1) >= 0).all()
            assert (ptr[:, -1] == n * s.level_k[l]).all()
            assert (col >= 0).all() and (col < n).all(), f"csr level {l}: row out of range"
        L.llsa_attn_bwd(B.p, qd, kd, vd, B.pyr_k, B.pyr_v, B.idx, B.csr_ptr, B.csr_col, B.o, B.lse,
                        c.dout.cuda(), B.dq, B.dk, B.dv, B.ws, B.ws.numel())
    torch.cuda.synchronize()
    bh, N = c.bh, c.N
    perm = seq_perm(c)   # token tensors are compared in sequence order
    res["pyr_q"] = [to_np(B.pyramid_level(B.pyr_q, l)) for l in range(1, c.L + 1)]
    res["pyr_k"] = [to_np(B.pyramid_level(B.pyr_k, l)) for l in range(1, c.L + 1)]
    res["pyr_v"] = [to_np(B.pyramid_level(B.pyr_v, l)) for l in range(1, c.L + 1)]
    res["idx"] = [B.index_level(l).cpu().numpy() for l in range(1, c.L + 1)]
    res["o"] = to_np(B.o).reshape(bh, N, 64)[:, perm]
    res["lse"] = to_np(B.lse).reshape(bh, N)[:, perm]
    if c.backward:
        res["csr"] = [tuple(t.cpu().numpy() for t in B.csr_level(l)) for l in range(1, s.enrich + 2)]
        res["dq"] = to_np(B.dq).reshape(bh, N, 64)[:, perm]
        res["dk"] = to_np(B.dk).reshape(bh, N, 64)[:, perm]
        res["dv"] = to_np(B.dv).reshape(bh, N, 64)[:, perm]
    return res


def bf16_half_ulp(x):
    """Half the spacing of bfloat16 numbers at |x| (8 significant bits): the
    largest error of rounding x to bfloat16 by round-to-nearest-even."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.maximum(a, np.finfo(np.float64).tiny)))
    return np.where(a > 0, 2.0 ** (e - 8), 0.0)


def grad_excess(c: Case, got, want):
    """Error of a gradient against the bar.  float32 gradients: |got - want|.
    bfloat16 gradients: |got - want| less the rounding of the stored value
    (half a bfloat16 ulp at max(|got|, |want|)), which no arithmetic can
    avoid; the stated bar applies to what is left."""
    err = np.abs(got - want)
    if c.grad_dtype == torch.bfloat16:
        err = np.maximum(err - bf16_half_ulp(np.maximum(np.abs(got), np.abs(want))), 0.0)
    return err


def oracle_inputs(c: Case):
    """The seeded inputs as float64 [bh, N, 64] in sequence order (patch order:
    permuted rows), and dO when the case has a backward pass."""
    bh, N = c.bh, c.N
    perm = seq_perm(c)
    f = lambda t: t.double().numpy().reshape(bh, N, 64)[:, perm]   # noqa: E731
    return f(c.q), f(c.k), f(c.v), (f(c.dout) if c.backward else None)


def forced_select(c: Case, pq, pk, gpu_idx):
    """Teacher-forced selection: level L from the oracle's pyramids alone,
    every finer level l from the GPU's own level-(l+1) picks as parents.
    Returns (idx list, relgap list), level 1 first."""
    idx, gap = [None] * c.L, [None] * c.L
    for l in range(c.L, 0, -1):
        parent = None if l == c.L else gpu_idx[l]
        idx[l - 1], gap[l - 1] = O.select_level(pq[l - 1], pk[l - 1], c.B, c.K, parent)
    return idx, gap


def compare_indices(gi, oi, og):
    """Status of every row of every level: 0 agree, 1 exempt near-tie (the
    oracle's relative gap between its K-th and (K+1)-th score in (0, 1e-5)),
    3 failure.  oi / og come from forced_select, so every row has the same
    candidates on both sides and no row is left unchecked.  Returns
    (status per level, counts)."""
    status = []
    for g, o, gap in zip(gi, oi, og):
        same = (g == o).all(axis=-1)
        status.append(np.where(same, 0, np.where((gap > 0) & (gap < GAP_BAND), 1, 3)))
    counts = {s: sum(int((st == k_).sum()) for st in status) for k_, s in
              ((0, "agree"), (1, "exempt"), (3, "fail"))}
    return status, counts


def run_oracle(c: Case, gpu_idx):
    """The oracle on the seeded inputs: pyramids, the teacher-forced selection,
    and attention (and gradients) over the GPU's own pick lists, so that every
    query row and every key is compared.  Also the oracle's own untied
    selection (not forced), for the end-to-end agreement count."""
    q, k, v, d = oracle_inputs(c)
    pq, pk, pv = O.pool(q, c.B, c.L), O.pool(k, c.B, c.L), O.pool(v, c.B, c.L)
    r = dict(pyr_q=pq, pyr_k=pk, pyr_v=pv)
    r["idx"], r["gap"] = forced_select(c, pq, pk, gpu_idx)
    r["idx_free"], _ = O.select(pq, pk, c.B, c.K)
    r["o"], r["lse"] = O.attn_fwd(q, k, v, pk, pv, gpu_idx, c.B, c.K, c.Le, c.scale, c.drop)
    if c.backward:
        r["dq"], r["dk"], r["dv"] = O.attn_bwd(q, k, v, pk, pv, gpu_idx, d, c.B, c.K, c.Le, c.scale,
                                               c.drop)
        r["csr"] = [O.transpose(gpu_idx[l - 1], c.N // c.B ** l) for l in range(1, c.Le + 2)]
    return r


def check_case(c: Case, report=None):
    """Runs GPU and oracle and asserts parity.  Returns a summary dict."""
    g = run_gpu(c)
    o = run_oracle(c, g["idx"])
    tol = out_tol(c.dtype)
    summ = {}
    for name in ("pyr_q", "pyr_k", "pyr_v"):
        err = max(float(np.abs(a - b).max()) for a, b in zip(g[name], o[name]))
        summ[name] = err
        assert err <= PYR_TOL, (name, err)
    _, counts = compare_indices(g["idx"], o["idx"], o["gap"])
    summ.update(counts)
    assert counts["fail"] == 0, counts
    # end to end, without forcing: rows whose picks equal the oracle's own
    summ["rows_equal_unforced"] = sum(int((a == b).all(axis=-1).sum())
                                      for a, b in zip(g["idx"], o["idx_free"]))
    summ["rows"] = sum(int(np.prod(a.shape[:-1])) for a in g["idx"])
    for name in ("o", "lse"):
        err = float(np.abs(g[name] - o[name]).max())
        summ[name] = err
        assert err <= tol, (name, err, tol)
    if c.backward:
        for name in ("dq", "dk", "dv"):
            summ[name] = float(np.abs(g[name] - o[name]).max())
            ex = float(grad_excess(c, g[name], o[name]).max())
            if c.grad_dtype == torch.bfloat16:
                summ[name + "_beyond_storage_rounding"] = ex
            assert ex <= tol, (name, ex, tol)
        # CSR: exactly the oracle's transpose of the GPU's pick lists
        for l, ((gp, gc), (op, oc)) in enumerate(zip(g["csr"], o["csr"]), start=1):
            assert np.array_equal(gp, op) and np.array_equal(gc, oc), ("csr", l)
    if report is not None:
        report.update(summ)
    return summ


def check_csr_valid(idx, ptr, col):
    """ptr / col is exactly the key-major form of idx (ascending rows per key)."""
    nb, rows, k = idx.shape
    cols = ptr.shape[1] - 1
    for b in range(nb):
        cnt = np.bincount(idx[b].ravel(), minlength=cols)
        assert ptr[b, 0] == 0 and (np.diff(ptr[b]) == cnt).all()
        r_of = np.repeat(np.arange(rows), k)
        order = np.lexsort((r_of, idx[b].ravel()))
        assert (col[b] == r_of[order]).all()
