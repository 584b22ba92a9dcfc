"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Bar: pyramids within 1e-5; indices bit-exact level by level with the GPU's
parent picks fed to the oracle, except near-ties of the oracle (gap below
1e-5 relative, counted); outputs and gradients, computed by the oracle over
the GPU's pick lists, within 1e-4 (float32 inputs) / 2e-2 (bfloat16 inputs)
max-abs on every row (bfloat16 gradients: beyond the rounding of the stored
value); the CSR transpose exact.
"""
import sys

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU-only hosts, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

from hierarchical_top_sparse_mean_amd import llsa as L  # noqa: E402
from hierarchical_top_sparse_mean_amd.inputs import WORKLOADS  # noqa: E402
from oracle import oracle as O  # noqa: E402

from parity_util import (Case, check_case, check_csr_valid, compare_indices,  # noqa: E402
                         forced_select, oracle_inputs, run_gpu, to_np)


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _workload_case(name):
    w = WORKLOADS[name]
    return Case(w.batch, w.heads, w.seq_len, w.dtype, w.levels, w.topk, w.enrich,
                backward=w.backward, sinus=w.sinusoid)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_parity(name):
    _log(f"[parity] workload {name}")
    summ = check_case(_workload_case(name))
    _log(f"[parity] {name}: {summ}")


@pytest.mark.parametrize("name", ["n16384_bf16", "n65536_bf16"])
def test_workload_parity_bf16_gradients(name):
    # the backward workloads at full size with dQ, dK, dV stored in bfloat16:
    # gradients of magnitude 4..8 and above round by up to 0.016..0.031 when
    # stored, so the bar applies beyond that rounding (the plain max-abs
    # error is logged)
    _log(f"[parity] workload {name} with bfloat16 gradients")
    w = WORKLOADS[name]
    c = Case(w.batch, w.heads, w.seq_len, w.dtype, w.levels, w.topk, w.enrich,
             backward=True, sinus=w.sinusoid, grad_dtype=torch.bfloat16)
    summ = check_case(c)
    _log(f"[parity] {name} bf16 gradients: {summ}")


# ------------------------------------------------------------- edge cases --
EDGE = [
    # (batch, heads, N, dtype, L, K, Le, backward, extra)
    (1, 2, 768, torch.bfloat16, 2, 2, 1, True, {}),        # 3 coarsest tokens: ragged dense tile
    (1, 3, 16 * 21, torch.bfloat16, 1, 5, 0, True, {}),    # single level, 21 blocks, odd K
    (2, 1, 16 * 21, torch.float32, 1, 3, 0, True, {}),     # single level, f32
    (1, 2, 8192, torch.bfloat16, 3, 2, 2, True, {}),       # three pooling steps, two coarse levels
    (1, 2, 8192, torch.float32, 3, 2, 2, True, {}),
    (1, 2, 4096, torch.bfloat16, 2, 8, 0, True, {}),       # no enrichment
    (1, 2, 4096, torch.bfloat16, 2, 1, 1, True, {}),       # K = 1
    (1, 2, 4096, torch.bfloat16, 2, 16, 1, True, {}),      # K = 16
    (1, 2, 4096, torch.bfloat16, 1, 20, 0, True, {}),      # single level, K = 20
    (1, 2, 4096, torch.bfloat16, 1, 32, 0, True, {}),      # single level, K = 32 (largest)
    (1, 16, 16384, torch.bfloat16, 1, 8, 0, True, {}),     # single level, 1024 row groups: one wave each
    (1, 16, 16384, torch.bfloat16, 1, 20, 0, True, {}),    # the same with K = 20 (32-key sorted groups)
    (1, 2, 4096, torch.bfloat16, 2, 20, 1, True, {}),      # K = 20 and one coarse tile: 3 forward chunks
    (1, 2, 4096, torch.bfloat16, 2, 32, 1, True, {}),      # K = 32 with enrichment (16 coarse: 1 tile)
    (1, 2, 16384, torch.bfloat16, 2, 32, 1, True, {}),     # 32 coarse entries: 2 coarse tiles
    (1, 2, 8192, torch.bfloat16, 3, 16, 2, True, {}),      # 16 + 2 coarse entries: 2 coarse tiles
    (1, 1, 2048, torch.float32, 2, 24, 1, True, {}),
    (1, 4, 16384, torch.float32, 2, 8, 1, True, {}),        # float32 matrix-core path at size
    (1, 2, 16384, torch.float32, 2, 32, 1, True, {}),       # float32, 32 coarse entries: 2 tiles
    (1, 2, 2048, torch.float32, 2, 4, 1, True, {"grad_dtype": torch.bfloat16}),
    (1, 2, 4096, torch.bfloat16, 2, 3, 1, True, {"drop_covered": False}),
    (2, 2, 2048, torch.bfloat16, 2, 4, 1, True, {"grad_dtype": torch.bfloat16}),
    (1, 2, 4096, torch.bfloat16, 2, 8, 1, True, {"token_order": 1}),   # 2D patch order
    (1, 2, 4096, torch.bfloat16, 2, 16, 1, True, {"token_order": 1}),  # patch order, generic path
    (1, 2, 1024, torch.float32, 2, 2, 1, True, {"token_order": 1}),
    (1, 2, 4096, torch.bfloat16, 3, 2, 2, True, {"token_order": 1}),
    (1, 1, 256, torch.bfloat16, 2, 16, 1, True, {}),       # K = all blocks (dense reduction)
    (1, 1, 256, torch.float32, 2, 16, 1, True, {}),
    # blocks of 64 tokens (4 MFMA tiles per block)
    (1, 2, 8192, torch.bfloat16, 1, 8, 0, True, {"block": 64}),     # single level, 128 blocks
    (1, 2, 64 * 37, torch.bfloat16, 1, 5, 0, True, {"block": 64}),  # 37 blocks: ragged tile groups
    (1, 2, 64 * 37, torch.float32, 1, 5, 0, True, {"block": 64}),   # float32, ragged last tile group
    (1, 2, 16384, torch.bfloat16, 2, 8, 1, True, {"block": 64}),    # 16384 -> 256 -> 4
    (1, 2, 8192, torch.float32, 2, 2, 1, True, {"block": 64}),
    (1, 1, 2048, torch.bfloat16, 1, 32, 0, True, {"block": 64}),    # K = all 32 blocks
    (2, 1, 8192, torch.bfloat16, 1, 8, 0, True, {"block": 64, "grad_dtype": torch.bfloat16}),
    (1, 2, 16384, torch.bfloat16, 1, 4, 0, True, {"block": 64, "token_order": 1}),
    (1, 2, 16384, torch.bfloat16, 2, 8, 0, True, {"block": 64}),                      # no enrichment
    (1, 2, 16384, torch.bfloat16, 2, 3, 1, True, {"block": 64, "token_order": 1}),   # 128x128 image
    (1, 1, 17 * 4096, torch.bfloat16, 2, 17, 1, True, {"block": 64}),  # 17 coarse entries: 2 tiles
]


@pytest.mark.parametrize("case", EDGE, ids=[f"b{e[0]}h{e[1]}N{e[2]}{str(e[3])[6:]}L{e[4]}K{e[5]}Le{e[6]}{'-'.join(f'{k}{v}' for k, v in e[8].items())}" for e in EDGE])
def test_edge_parity(case):
    b, h, N, dt, L_, K, Le, bwd, extra = case
    _log(f"[parity] edge {case}")
    c = Case(b, h, N, dt, L_, K, Le, backward=bwd, **extra)
    summ = check_case(c)
    _log(f"[parity] edge done {summ}")


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_all_blocks_is_dense_attention(dtype):
    # K = every level-1 block: covered coarse picks are dropped and the result
    # is plain softmax attention (checked against a float64 textbook formula)
    _log(f"[parity] dense reduction {dtype}")
    c = Case(1, 2, 256, dtype, 2, 16, 1, backward=False)
    g = run_gpu(c)
    q = c.q.double().numpy().reshape(2, 256, 64)
    k = c.k.double().numpy().reshape(2, 256, 64)
    v = c.v.double().numpy().reshape(2, 256, 64)
    s = np.einsum("hqd,hkd->hqk", q, k) / 8.0
    p = np.exp(s - s.max(-1, keepdims=True))
    want = np.einsum("hqk,hkd->hqd", p / p.sum(-1, keepdims=True), v)
    assert np.abs(g["o"] - want).max() <= (1e-4 if dtype == torch.float32 else 2e-2)


def test_q_zero_closed_form_bitexact_picks():
    # Q = 0: every score is 0 in any precision, ties go to the lowest index at
    # every level, O is the mean of V over the attended multiset of tokens
    _log("[parity] q=0 closed form")
    N, K = 4096, 8
    base = Case(1, 2, N, torch.bfloat16, 2, K, 1, backward=False)
    c = Case(1, 2, N, torch.bfloat16, 2, K, 1, q=torch.zeros(1, 2, N, 64), k=base.k, v=base.v,
             backward=False)
    g = run_gpu(c)
    for lv in g["idx"]:
        assert (lv == np.arange(K)).all()
    v = c.v.double().numpy().reshape(2, N, 64)
    toks = list(range(K * 16)) + list(range(K * 256))
    want = v[:, toks].mean(axis=1)
    assert np.abs(g["o"] - want[:, None, :]).max() <= 2e-2
    assert np.abs(g["lse"] - np.log(len(toks))).max() <= 1e-5


def test_constant_values_give_that_value():
    _log("[parity] constant V")
    N = 4096
    base = Case(1, 2, N, torch.bfloat16, 2, 8, 1, backward=False)
    vals = torch.randn(64, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    c = Case(1, 2, N, torch.bfloat16, 2, 8, 1, q=base.q, k=base.k,
             v=vals.float().expand(1, 2, N, 64).contiguous(), backward=False)
    g = run_gpu(c)
    assert np.abs(g["o"] - vals.double().numpy()).max() <= 2e-2


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_deterministic_bitwise(dtype):
    # two runs of the whole path give identical bytes (no float atomics)
    _log(f"[parity] determinism {dtype}")
    c = Case(1, 4, 4096, dtype, 2, 8, 1, backward=True, sinus=True)
    a = run_gpu(c)
    b = run_gpu(c)
    for key in ("o", "lse", "dq", "dk", "dv"):
        assert np.array_equal(a[key], b[key]), key
    for x, y in zip(a["idx"], b["idx"]):
        assert np.array_equal(x, y)


# ------------------------------------------------------------- transpose --
@pytest.mark.parametrize("nb,rows,k,cols", [(3, 100, 8, 100), (2, 4096, 8, 4096), (1, 37, 5, 23),
                                            (4, 64, 1, 64), (1, 16384, 8, 32768), (2, 50, 16, 1000),
                                            (1, 4096, 8, 70000), (3, 2000, 8, 9000), (2, 9000, 3, 4097),
                                            (4, 65536, 8, 65536)])   # level 1 of 1M tokens: two passes
def test_transpose_parity(nb, rows, k, cols):
    _log(f"[parity] transpose {nb} {rows} {k} {cols}")
    rng = np.random.default_rng(rows * 31 + k)
    # skewed picks: half of the rows favour a few hot keys -> long and empty segments
    idx = np.empty((nb, rows, k), dtype=np.int32)
    hot = rng.choice(cols, size=min(cols, 2 * k), replace=False)
    if rows * cols > 10 ** 8:
        # large shapes, drawn vectorised: pick j of a row lies in the j-th of k
        # equal windows after a random start (so a row's picks are distinct)
        step = cols // k
        start = rng.integers(0, cols, size=(nb, rows, 1))
        jit = rng.integers(0, step, size=(nb, rows, k))
        idx[:] = np.sort((start + np.arange(k) * step + jit) % cols, axis=-1)
        idx[:, ::2] = np.sort(hot[:k])
    else:
        for b in range(nb):
            for r in range(rows):
                pool = hot if (r % 2 == 0 and len(hot) >= k) else np.arange(cols)
                idx[b, r] = np.sort(rng.choice(pool, size=k, replace=False))
    ptr_o, col_o = O.transpose(idx, cols)
    d_idx = torch.from_numpy(idx).cuda()
    ptr = torch.empty((nb, cols + 1), dtype=torch.int32, device="cuda")
    col = torch.empty((nb, rows * k), dtype=torch.int32, device="cuda")
    ws_bytes = L.llsa_index_transpose_workspace(nb, rows, k, cols)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    L.llsa_index_transpose(nb, rows, k, cols, d_idx, ptr, col, ws, ws_bytes)
    torch.cuda.synchronize()
    assert np.array_equal(ptr.cpu().numpy(), ptr_o)
    assert np.array_equal(col.cpu().numpy(), col_o)
    check_csr_valid(idx, ptr.cpu().numpy(), col.cpu().numpy())


@pytest.mark.parametrize("b,h,N,L_,K,Le,block", [
    (1, 16, 65536, 2, 8, 1, 16),    # the measured workload: level-1 count fused into selection
    (2, 4, 16384, 2, 8, 1, 16),
    (1, 2, 768, 2, 2, 1, 16),       # 48 level-1 rows: not four 16-row groups per workgroup
    (1, 2, 4096, 1, 8, 0, 16),      # single level, few groups: the split selection, no fusion
    (4, 16, 4096, 1, 5, 0, 16),     # single level with 1024 row groups: fused dense level
    (1, 4, 8192, 3, 4, 2, 16),      # three levels, two coarse transposes
    (1, 2, 16384, 2, 8, 1, 64),
])
def test_select_transpose_fused_matches_separate_and_oracle(b, h, N, L_, K, Le, block):
    # one fused call gives bit for bit the picks and key-major lists of
    # llsa_select followed by the transposes of every level, and both match
    # the oracle
    _log(f"[parity] fused select+transpose {b} {h} {N} L{L_} K{K} Le{Le} B{block}")
    c = Case(b, h, N, torch.bfloat16, L_, K, Le, backward=True, sinus=round(N ** 0.5) ** 2 == N,
             block=block)
    B = L.Buffers(c.p, backward=True)
    L.llsa_pool(c.p, c.q.cuda(), c.k.cuda(), c.v.cuda(), B.pyr_q, B.pyr_k, B.pyr_v)
    L.llsa_select(c.p, B.pyr_q, B.pyr_k, B.idx)
    L.transpose_levels(B)
    torch.cuda.synchronize()
    idx0 = [B.index_level(l).clone() for l in range(1, L_ + 1)]
    csr0 = [tuple(t.clone() for t in B.csr_level(l)) for l in range(1, Le + 2)]
    B.idx.fill_(-7)
    B.csr_ptr.fill_(-7)
    B.csr_col.fill_(-7)
    L.llsa_select_transpose(c.p, B.pyr_q, B.pyr_k, B.idx, B.csr_ptr, B.csr_col, B.tws, B.tws_bytes)
    torch.cuda.synchronize()
    for l in range(1, L_ + 1):
        assert torch.equal(B.index_level(l), idx0[l - 1]), l
    for l in range(1, Le + 2):
        ptr, col = B.csr_level(l)
        assert torch.equal(ptr, csr0[l - 1][0]) and torch.equal(col, csr0[l - 1][1]), l
    # and against the oracle: the picks level by level (teacher-forced, near-ties
    # exempt and counted), each level's key-major lists as the oracle's transpose
    gi = [B.index_level(l).cpu().numpy() for l in range(1, L_ + 1)]
    q, k, _, _ = oracle_inputs(c)
    pq, pk = O.pool(q, block, L_), O.pool(k, block, L_)
    oi, og = forced_select(c, pq, pk, gi)
    _, counts = compare_indices(gi, oi, og)
    _log(f"[parity]   picks vs oracle: {counts}")
    assert counts["fail"] == 0, counts
    for l in range(1, Le + 2):
        ptr, col = (t.cpu().numpy() for t in B.csr_level(l))
        ptr_o, col_o = O.transpose(gi[l - 1], B.s.level_tokens[l])
        assert np.array_equal(ptr, ptr_o) and np.array_equal(col, col_o), l


@pytest.mark.parametrize("b,h,N,L_,K,Le,block", [
    (1, 16, 65536, 2, 8, 1, 16),    # both levels in one launch
    (1, 4, 8192, 3, 4, 2, 16),      # three levels in one launch
    (1, 2, 65536, 1, 32, 0, 16),    # 131072 picks: the largest one-launch matrix
    (1, 2, 262144, 3, 8, 2, 16),    # level 1 has 16384 keys: two passes, levels 2-3 one launch
    (2, 2, 16384, 2, 8, 1, 64),
])
def test_transpose_levels_matches_per_level(b, h, N, L_, K, Le, block):
    # llsa_index_transpose_levels writes, bit for bit, what one
    # llsa_index_transpose per level writes, and both equal the oracle's lists
    _log(f"[parity] transpose levels {b} {h} {N} L{L_} K{K} Le{Le} B{block}")
    c = Case(b, h, N, torch.bfloat16, L_, K, Le, backward=True, sinus=round(N ** 0.5) ** 2 == N,
             block=block)
    B = L.Buffers(c.p, backward=True)
    L.llsa_pool(c.p, c.q.cuda(), c.k.cuda(), c.v.cuda(), B.pyr_q, B.pyr_k, B.pyr_v)
    L.llsa_select(c.p, B.pyr_q, B.pyr_k, B.idx)
    B.csr_ptr.fill_(-7)
    B.csr_col.fill_(-7)
    L.llsa_index_transpose_levels(c.p, B.idx, B.csr_ptr, B.csr_col, B.tws, B.tws_bytes)
    torch.cuda.synchronize()
    got = [tuple(t.cpu().numpy() for t in B.csr_level(l)) for l in range(1, Le + 2)]
    s, bh = B.s, b * h
    for l in range(1, Le + 2):
        ptr, col = B.csr_level(l)
        ptr.fill_(-5)
        col.fill_(-5)
        L.llsa_index_transpose(bh, s.level_tokens[l], s.level_k[l], s.level_tokens[l],
                               B.index_level(l), ptr, col, B.tws, B.tws_bytes)
    torch.cuda.synchronize()
    for l in range(1, Le + 2):
        ptr, col = (t.cpu().numpy() for t in B.csr_level(l))
        assert np.array_equal(got[l - 1][0], ptr) and np.array_equal(got[l - 1][1], col), l
        ptr_o, col_o = O.transpose(B.index_level(l).cpu().numpy(), s.level_tokens[l])
        assert np.array_equal(ptr, ptr_o) and np.array_equal(col, col_o), l


@pytest.mark.parametrize("cols", [100, 9000])
def test_transpose_skips_out_of_range(cols):
    # indices outside [0, cols) are not listed (one pass and two passes)
    nb, rows, k = 2, 300, 6
    rng = np.random.default_rng(cols)
    idx = np.stack([np.stack([np.sort(rng.choice(cols, k, replace=False)) for _ in range(rows)])
                    for _ in range(nb)]).astype(np.int32)
    bad = rng.random(idx.shape) < 0.1
    idx[bad] = np.where(rng.random(int(bad.sum())) < 0.5, -1, cols + 7)
    d_idx = torch.from_numpy(idx).cuda()
    ptr = torch.empty((nb, cols + 1), dtype=torch.int32, device="cuda")
    col = torch.full((nb, rows * k), -5, dtype=torch.int32, device="cuda")
    ws_bytes = L.llsa_index_transpose_workspace(nb, rows, k, cols)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    L.llsa_index_transpose(nb, rows, k, cols, d_idx, ptr, col, ws, ws_bytes)
    torch.cuda.synchronize()
    ptr, col = ptr.cpu().numpy(), col.cpu().numpy()
    for b in range(nb):
        r_of = np.repeat(np.arange(rows), k)
        key = idx[b].ravel()
        ok = (key >= 0) & (key < cols)
        order = np.lexsort((r_of[ok], key[ok]))   # by key, then row
        n = int(ok.sum())
        assert ptr[b, cols] == n and ptr[b, 0] == 0
        assert np.array_equal(np.diff(ptr[b]), np.bincount(key[ok], minlength=cols))
        assert np.array_equal(col[b, :n], r_of[ok][order])


@pytest.mark.parametrize("nb,rows,k,cols", [(3, 100, 8, 100), (2, 4096, 8, 4096), (1, 37, 5, 23),
                                            (1, 4096, 8, 32768)])
def test_mask_transpose_baseline_matches_oracle(nb, rows, k, cols):
    # the dense-mask baseline must build exactly the same key-major lists
    _log(f"[parity] mask transpose {nb} {rows} {k} {cols}")
    rng = np.random.default_rng(rows * 7 + k)
    idx = np.stack([np.stack([np.sort(rng.choice(cols, k, replace=False)) for _ in range(rows)])
                    for _ in range(nb)]).astype(np.int32)
    ptr_o, col_o = O.transpose(idx, cols)
    d_idx = torch.from_numpy(idx).cuda()
    ptr = torch.empty((nb, cols + 1), dtype=torch.int32, device="cuda")
    col = torch.empty((nb, rows * k), dtype=torch.int32, device="cuda")
    ws_bytes = L.llsa_index_transpose_mask_workspace(nb, rows, cols)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    L.llsa_index_transpose_mask(nb, rows, k, cols, d_idx, ptr, col, ws, ws_bytes)
    torch.cuda.synchronize()
    assert np.array_equal(ptr.cpu().numpy(), ptr_o)
    assert np.array_equal(col.cpu().numpy(), col_o)


def test_patch_order_pools_image_patches():
    # in 2D patch order a level-1 token is the mean of a 4x4 pixel patch and a
    # level-2 token of a 16x16 patch, read from the raster-stored image
    _log("[parity] patch-order pooling")
    from parity_util import patch_order
    N, S = 4096, 64
    c = Case(1, 2, N, torch.float32, 2, 2, 1, backward=False, token_order=1)
    B = L.Buffers(c.p, backward=False)
    L.llsa_pool(c.p, c.q.cuda(), c.k.cuda(), c.v.cuda(), B.pyr_q, B.pyr_k, B.pyr_v)
    torch.cuda.synchronize()
    img = c.k.double().numpy().reshape(2, S, S, 64)
    for l, side in ((1, 4), (2, 16)):
        n = N // 16 ** l
        pos = patch_order(n)            # position -> raster index in the (S/side)^2 grid
        grid = img.reshape(2, S // side, side, S // side, side, 64).mean(axis=(2, 4))
        want = grid.reshape(2, n, 64)[:, pos]
        got = to_np(B.pyramid_level(B.pyr_k, l)).reshape(2, n, 64)
        assert np.abs(got - want).max() <= 1e-5, l


def test_dense_comparator_matches_oracle_dense():
    # the full-attention comparator against K = all blocks in the oracle
    _log("[parity] dense comparator")
    N = 1024
    c = Case(1, 2, N, torch.bfloat16, 2, N // 16, 1, backward=False, sinus=True)
    p = L.problem(1, 2, N, dtype=torch.bfloat16)
    o = torch.empty(1, 2, N, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(2 * N, dtype=torch.float32, device="cuda")
    L.llsa_dense_attn_fwd(p, c.q.cuda(), c.k.cuda(), c.v.cuda(), o, lse)
    torch.cuda.synchronize()
    q = c.q.double().numpy().reshape(2, N, 64)
    k = c.k.double().numpy().reshape(2, N, 64)
    v = c.v.double().numpy().reshape(2, N, 64)
    s = np.einsum("hqd,hkd->hqk", q, k) / 8.0
    m = s.max(-1, keepdims=True)
    pr = np.exp(s - m)
    want = np.einsum("hqk,hkd->hqd", pr / pr.sum(-1, keepdims=True), v)
    want_lse = (m[..., 0] + np.log(pr.sum(-1)))
    assert np.abs(o.float().cpu().numpy().reshape(2, N, 64) - want).max() <= 2e-2
    assert np.abs(lse.cpu().numpy().reshape(2, N) - want_lse).max() <= 2e-2


@pytest.mark.parametrize("N", [1024, 1040])
def test_dense_backward_comparator_matches_textbook_gradients(N):
    # the dense backward comparator against the textbook softmax-attention
    # gradients of <O, dO> in float64 (1040 tokens: a partial last tile step)
    _log(f"[parity] dense backward comparator N={N}")
    from hierarchical_top_sparse_mean_amd.inputs import make_inputs
    q, k, v, do = make_inputs(1, 2, N, 64, torch.bfloat16, N == 1024, True, 3)
    p = L.problem(1, 2, N, dtype=torch.bfloat16)
    dev = [x.cuda() for x in (q, k, v, do)]
    o = torch.empty(1, 2, N, 64, dtype=torch.bfloat16, device="cuda")
    lse = torch.empty(2 * N, dtype=torch.float32, device="cuda")
    L.llsa_dense_attn_fwd(p, dev[0], dev[1], dev[2], o, lse)
    grads = [torch.empty(1, 2, N, 64, dtype=torch.float32, device="cuda") for _ in range(3)]
    ws_bytes = L.llsa_dense_attn_bwd_workspace(p)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    L.llsa_dense_attn_bwd(p, dev[0], dev[1], dev[2], o, lse, dev[3], *grads, ws, ws_bytes)
    torch.cuda.synchronize()
    Q, K, V, dO = (x.double().numpy().reshape(2, N, 64) for x in (q, k, v, do))
    s = np.einsum("hqd,hkd->hqk", Q, K) / 8.0
    pr = np.exp(s - s.max(-1, keepdims=True))
    pr /= pr.sum(-1, keepdims=True)
    O = np.einsum("hqk,hkd->hqd", pr, V)
    dP = np.einsum("hqd,hkd->hqk", dO, V)
    dS = pr * (dP - (dO * O).sum(-1, keepdims=True))
    want = {"dq": np.einsum("hqk,hkd->hqd", dS, K) / 8.0,
            "dk": np.einsum("hqk,hqd->hkd", dS, Q) / 8.0,
            "dv": np.einsum("hqk,hqd->hkd", pr, dO)}
    for name, got in zip(("dq", "dk", "dv"), grads):
        err = np.abs(got.cpu().numpy().reshape(2, N, 64) - want[name]).max()
        _log(f"[parity]   {name} max abs err {err:.3g}")
        assert err <= 2e-2, name
