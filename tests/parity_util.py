"""GPU-vs-oracle comparison helpers used by the GPU parity tests.

The oracle only ever sees the seeded inputs; the GPU results are compared to
its outputs.  Index lists are compared level by level, coarse to fine:
a row whose parent row agrees must match exactly unless the oracle's gap
between the K-th and (K+1)-th score is below GAP_BAND relative (a near-tie:
exempt, counted); rows below a differing parent are excluded ("cascade",
counted).  Outputs are compared on every query block whose attended set is
defined by agreeing rows only, and gradients of keys reached only from such
blocks.
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
    2e-2 for bfloat16 inputs."""
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


def run_oracle(c: Case):
    bh, N = c.bh, c.N
    perm = seq_perm(c)   # the oracle runs on the sequence (patch order: permuted rows)
    q = c.q.double().numpy().reshape(bh, N, 64)[:, perm]
    k = c.k.double().numpy().reshape(bh, N, 64)[:, perm]
    v = c.v.double().numpy().reshape(bh, N, 64)[:, perm]
    r = O.forward_all(q, k, v, c.B, c.L, c.K, c.Le, c.scale, c.drop)
    if c.backward:
        d = c.dout.double().numpy().reshape(bh, N, 64)[:, perm]
        r["dq"], r["dk"], r["dv"] = O.attn_bwd(q, k, v, r["pyr_k"], r["pyr_v"], r["idx"], d, c.B,
                                               c.K, c.Le, c.scale, c.drop)
        r["csr"] = [O.transpose(r["idx"][l - 1], N // c.B ** l) for l in range(1, c.Le + 2)]
    return r


def compare_indices(gi, oi, og, B_=16):
    """Level-by-level status of every row: 0 agree, 1 exempt near-tie,
    2 cascade (parent differs), 3 failure.  Returns (status per level, counts)."""
    Lv = len(gi)
    status = [None] * Lv
    parent_ok = None
    for l in range(Lv, 0, -1):
        g, o, gap = gi[l - 1], oi[l - 1], og[l - 1]
        same = (g == o).all(axis=-1)
        st = np.where(same, 0, np.where((gap > 0) & (gap < GAP_BAND), 1, 3))
        if parent_ok is not None:
            bh, n = same.shape
            inherit = np.repeat(parent_ok, B_, axis=1)[:, :n]
            st = np.where(inherit, st, 2)
        status[l - 1] = st
        parent_ok = st == 0
    counts = {s: sum(int((st == k_).sum()) for st in status) for k_, s in
              enumerate(("agree", "exempt", "cascade", "fail"))}
    return status, counts


def clean_blocks(status, Le, B_=16):
    """Query blocks whose fine row and every enriching ancestor row agree."""
    ok = status[0] == 0
    n1 = ok.shape[1]
    for l in range(2, Le + 2):
        anc = status[l - 1] == 0
        ok = ok & np.repeat(anc, B_ ** (l - 1), axis=1)[:, :n1]
    return ok


def clean_keys(gi, oi, blocks_ok, Le, N, B_=16):
    """Tokens whose gradient only comes from clean query blocks (under either
    side's picks)."""
    bh, n1 = blocks_ok.shape
    bad = np.zeros((bh, N), dtype=bool)
    for h, i in zip(*np.nonzero(~blocks_ok)):
        for side in (gi, oi):
            for f in side[0][h, i]:
                bad[h, f * B_:(f + 1) * B_] = True
            for l in range(2, Le + 2):
                span = B_ ** l
                for c in side[l - 1][h, i // B_ ** (l - 1)]:
                    bad[h, c * span:(c + 1) * span] = True
    return ~bad


def check_case(c: Case, report=None):
    """Runs GPU and oracle and asserts parity.  Returns a summary dict."""
    g = run_gpu(c)
    o = run_oracle(c)
    tol = out_tol(c.dtype)
    summ = {}
    for name in ("pyr_q", "pyr_k", "pyr_v"):
        err = max(float(np.abs(a - b).max()) for a, b in zip(g[name], o[name]))
        summ[name] = err
        assert err <= PYR_TOL, (name, err)
    status, counts = compare_indices(g["idx"], o["idx"], o["gap"], c.B)
    summ.update(counts)
    assert counts["fail"] == 0, counts
    ok_blocks = clean_blocks(status, c.Le, c.B)
    summ["clean_blocks"] = int(ok_blocks.sum())
    rows = np.repeat(ok_blocks, c.B, axis=1)
    for name in ("o", "lse"):
        err = float(np.abs(g[name] - o[name])[rows].max())
        summ[name] = err
        assert err <= tol, (name, err, tol)
    if c.backward:
        err = float(np.abs(g["dq"] - o["dq"])[rows].max())
        summ["dq"] = err
        assert err <= tol, ("dq", err, tol)
        keys = clean_keys(g["idx"], o["idx"], ok_blocks, c.Le, c.N, c.B)
        for name in ("dk", "dv"):
            err = float(np.abs(g[name] - o[name])[keys].max())
            summ[name] = err
            assert err <= tol, (name, err, tol)
        # CSR: exact where the index lists agree; always a valid transpose of the GPU lists
        for l, ((gp, gc), (op, oc)) in enumerate(zip(g["csr"], o["csr"]), start=1):
            if (g["idx"][l - 1] == o["idx"][l - 1]).all():
                assert (gp == op).all() and (gc == oc).all(), ("csr", l)
            check_csr_valid(g["idx"][l - 1], gp, gc)
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
