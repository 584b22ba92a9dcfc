"""Pins of the fp64 CPU oracle against facts fixed by the method description
and by mathematics (no GPU).  Each test names the passage it checks:
"Trainable Log-linear Sparse Attention for Efficient Diffusion Transformers",
howistudyai.com explainer, sections "Step 1" .. "Step 4" and the building
blocks "KV Reweighting" / "Sparse Index Transpose".
"""
import math
import os

import numpy as np
import pytest

from oracle import oracle as O


def _read_fixture(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


# ----------------------------------------------------------------- Step 1 --
def test_pool_worked_example(golden_dir):
    fx = _read_fixture(os.path.join(golden_dir, "pool_n8_b2.txt"))
    N, B, L = int(fx["N"][0]), int(fx["B"][0]), int(fx["levels"][0])
    x = np.array([float(v) for v in fx["input"]]).reshape(1, N, 1)
    lv = O.pool(x, B, L)
    assert [N] + [a.shape[1] for a in lv] == [int(s) for s in fx["sizes"]]
    np.testing.assert_array_equal(lv[0].ravel(), [float(v) for v in fx["level1"]])
    np.testing.assert_array_equal(lv[1].ravel(), [float(v) for v in fx["level2"]])


@pytest.mark.parametrize("B,L", [(2, 3), (4, 2), (16, 2), (3, 3)])
def test_pool_ramp_closed_form(B, L):
    # x[t, c] = t + 100 c  ->  level l token j = j B^l + (B^l - 1)/2 + 100 c
    N, d = B ** L * 4, 3
    t = np.arange(N, dtype=np.float64)[:, None] + 100.0 * np.arange(d)[None, :]
    lv = O.pool(np.stack([t, -t]), B, L)
    for l in range(1, L + 1):
        span = B ** l
        j = np.arange(N // span, dtype=np.float64)[:, None]
        want = j * span + (span - 1) / 2.0 + 100.0 * np.arange(d)[None, :]
        np.testing.assert_allclose(lv[l - 1][0], want, rtol=0, atol=1e-9)
        np.testing.assert_allclose(lv[l - 1][1], -want, rtol=0, atol=1e-9)


def test_pool_equals_direct_block_mean():
    # repeated pooling by B equals one mean over the B^l tokens under a token
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 4 ** 3 * 2, 5))
    lv = O.pool(x, 4, 3)
    for l in range(1, 4):
        span = 4 ** l
        direct = x.reshape(3, -1, span, 5).mean(axis=2)
        np.testing.assert_allclose(lv[l - 1], direct, rtol=1e-13, atol=1e-13)


# ----------------------------------------------------------------- Step 2 --
def test_select_worked_example(golden_dir):
    fx = _read_fixture(os.path.join(golden_dir, "select_toy_n8_b2_k1.txt"))
    N, B, K = int(fx["N"][0]), int(fx["B"][0]), int(fx["K"][0])
    k = np.array([float(v) for v in fx["keys"]]).reshape(1, N, 1)
    q = np.array([float(v) for v in fx["queries"]]).reshape(1, N, 1)
    pq, pk = O.pool(q, B, 2), O.pool(k, B, 2)
    idx, _ = O.select(pq, pk, B, K)
    np.testing.assert_array_equal(idx[1].ravel(), [int(v) for v in fx["level2"]])
    np.testing.assert_array_equal(idx[0].ravel(), [int(v) for v in fx["level1"]])


def _brute_topk(scores, cand, K):
    """Full stable sort: higher score first, lower index first on ties."""
    order = np.lexsort((cand, -scores))
    keep = np.sort(cand[order[:K]])
    return keep


@pytest.mark.parametrize("integer_valued", [False, True])
def test_select_dense_level_matches_brute_force(integer_valued):
    rng = np.random.default_rng(2)
    bh, n, d, K = 3, 40, 6, 7
    if integer_valued:   # many exact ties
        q = rng.integers(-1, 2, (bh, n, d)).astype(np.float64)
        k = rng.integers(-1, 2, (bh, n, d)).astype(np.float64)
    else:
        q = rng.standard_normal((bh, n, d))
        k = rng.standard_normal((bh, n, d))
    idx, gap = O.select_level(q, k, 4, K, None)
    for h in range(bh):
        for i in range(n):
            s = k[h] @ q[h, i]
            want = _brute_topk(s, np.arange(n), K)
            np.testing.assert_array_equal(idx[h, i], want)
            srt = np.sort(s)[::-1]
            m = max(abs(srt[K - 1]), abs(srt[K]))
            g = 0.0 if m == 0 else (srt[K - 1] - srt[K]) / m
            assert gap[h, i] == pytest.approx(g, abs=1e-12)


def test_select_sparse_level_matches_brute_force():
    # level-l candidates are the B children of the parent's picks (Step 2)
    rng = np.random.default_rng(3)
    bh, n, d, B, K, kp = 2, 32, 5, 4, 3, 2
    q = rng.standard_normal((bh, n, d))
    k = rng.standard_normal((bh, n, d))
    parent = np.stack([np.sort(rng.choice(n // B, kp, replace=False)) for _ in range(bh * n // B)])
    parent = parent.reshape(bh, n // B, kp)
    idx, _ = O.select_level(q, k, B, K, parent)
    for h in range(bh):
        for i in range(n):
            cand = np.array([c * B + t for c in parent[h, i // B] for t in range(B)])
            s = k[h, cand] @ q[h, i]
            np.testing.assert_array_equal(idx[h, i], _brute_topk(s, cand, K))


def test_select_constant_inputs_pick_lowest_indices():
    # all scores equal -> the tie-break alone decides: lowest indices everywhere
    B, L, K, N = 4, 3, 2, 4 ** 3 * 2
    x = np.ones((2, N, 3))
    idx, gap = O.select(O.pool(x, B, L), O.pool(x, B, L), B, K)
    np.testing.assert_array_equal(idx[2], np.broadcast_to(np.arange(K), idx[2].shape))
    for l in range(L - 1, 0, -1):
        # parent picks {0..K-1}: children 0..K*B-1, lowest K of them
        np.testing.assert_array_equal(idx[l - 1], np.broadcast_to(np.arange(K), idx[l - 1].shape))
    assert (gap[2] == -1).all()          # 2 coarsest tokens, both kept: no (K+1)-th
    assert (gap[0] == 0).all() and (gap[1] == 0).all()   # exact ties below


def test_select_full_coarse_picks_reduce_to_single_level():
    # with every coarse token picked, level 1 sees all blocks: the hierarchy
    # reduces to a single-level dense Top-K over level-1 blocks
    rng = np.random.default_rng(4)
    B, N, d, K = 4, 64, 5, 3
    q = rng.standard_normal((2, N, d))
    k = rng.standard_normal((2, N, d))
    pq, pk = O.pool(q, B, 2), O.pool(k, B, 2)
    n2 = N // B ** 2
    full_parent = np.broadcast_to(np.arange(n2), (2, n2, n2)).copy()
    sparse, _ = O.select_level(pq[0], pk[0], B, K, full_parent)
    dense, _ = O.select_level(pq[0], pk[0], B, K, None)
    np.testing.assert_array_equal(sparse, dense)


def test_select_invariants_random():
    rng = np.random.default_rng(5)
    B, L, K, N, d = 4, 3, 3, 4 ** 3 * 2, 4
    q = rng.standard_normal((2, N, d))
    k = rng.standard_normal((2, N, d))
    pq, pk = O.pool(q, B, L), O.pool(k, B, L)
    idx, _ = O.select(pq, pk, B, K)
    for l in range(1, L + 1):
        I = idx[l - 1]
        assert (np.diff(I, axis=-1) > 0).all()            # ascending, distinct
        if l < L:
            par = idx[l]
            for h in range(2):
                for i in range(I.shape[1]):
                    allowed = set(int(c) * B + t for c in par[h, i // B] for t in range(B))
                    assert set(int(c) for c in I[h, i]) <= allowed


# ----------------------------------------------------------------- Step 3 --
def _dense_attention(q, k, v, scale, extra_k=None, extra_v=None, extra_w=None):
    """Textbook softmax attention, optionally over extra weighted keys."""
    s = scale * q @ k.T
    vals = v
    if extra_k is not None:
        s = np.concatenate([s, scale * q @ extra_k.T + np.log(extra_w)[None, :]], axis=1)
        vals = np.concatenate([v, extra_v], axis=0)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    z = p.sum(axis=1, keepdims=True)
    return (p / z) @ vals, (m + np.log(z)).ravel()


def test_attn_q_zero_closed_form():
    # Q = 0: every score is exactly 0, all levels pick {0..K-1}; each query
    # block attends to tokens 0..K*B-1 (weight 1) plus level-l tokens 0..K-1
    # (weight B^l), i.e. to B^l copies of the mean of the B^l tokens under
    # each: O = mean of V over that multiset of tokens.
    rng = np.random.default_rng(6)
    B, L, K, Le, N, d = 4, 3, 2, 2, 4 ** 3 * 2, 5
    q = np.zeros((2, N, d))
    k = rng.standard_normal((2, N, d))
    v = rng.standard_normal((2, N, d))
    r = O.forward_all(q, k, v, B, L, K, Le, 0.3)
    for h in range(2):
        toks = list(range(K * B))
        for l in range(2, Le + 2):
            toks += list(range(K * B ** l))
        want = v[h, toks].mean(axis=0)
        np.testing.assert_allclose(r["o"][h], np.broadcast_to(want, (N, d)), rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["lse"][h], math.log(len(toks)), rtol=0, atol=1e-12)


def test_attn_reweight_worked_example(golden_dir):
    fx = _read_fixture(os.path.join(golden_dir, "reweight_16.txt"))
    B, L, N, K, Le = (int(fx[x][0]) for x in ("B", "levels", "N", "K", "Le"))
    assert B ** 2 == int(fx["weight_level2"][0])
    rng = np.random.default_rng(7)
    q = np.zeros((1, N, 3))
    k = rng.standard_normal((1, N, 3))
    v = rng.standard_normal((1, N, 3))
    r = O.forward_all(q, k, v, B, L, K, Le, 1.0)
    np.testing.assert_allclose(r["lse"], math.log(float(fx["lse_exp"][0])), rtol=0, atol=1e-12)


def test_attn_constant_values_give_that_value():
    rng = np.random.default_rng(8)
    B, L, K, Le, N, d = 4, 2, 3, 1, 4 ** 2 * 4, 6
    q = rng.standard_normal((2, N, d))
    k = rng.standard_normal((2, N, d))
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, (2, N, d)).copy()
    r = O.forward_all(q, k, v, B, L, K, Le, 0.4)
    np.testing.assert_allclose(r["o"], np.broadcast_to(c, r["o"].shape), rtol=0, atol=1e-12)


@pytest.mark.parametrize("B,L,Le", [(4, 2, 1), (4, 3, 2), (4, 3, 0), (4, 1, 0)])
def test_attn_all_blocks_is_dense_attention(B, L, Le):
    # K = every level-1 block: all coarse picks are fully covered and left
    # out, and the attended set is every token -> textbook softmax attention
    rng = np.random.default_rng(9)
    N, d = B ** L * 2, 5
    K = N // B
    q = rng.standard_normal((2, N, d))
    k = rng.standard_normal((2, N, d))
    v = rng.standard_normal((2, N, d))
    r = O.forward_all(q, k, v, B, L, K, Le, 0.37)
    for h in range(2):
        want, lse = _dense_attention(q[h], k[h], v[h], 0.37)
        np.testing.assert_allclose(r["o"][h], want, rtol=0, atol=1e-12)
        np.testing.assert_allclose(r["lse"][h], lse, rtol=0, atol=1e-12)


def test_attn_all_blocks_without_drop_is_augmented_dense():
    # keeping every coarse pick: the attended set is all tokens (weight 1)
    # plus all level-l tokens (weight B^l) for l = 2..Le+1
    rng = np.random.default_rng(10)
    B, L, Le, N, d = 4, 3, 2, 4 ** 3 * 2, 5
    K = N // B
    q = rng.standard_normal((1, N, d))
    k = rng.standard_normal((1, N, d))
    v = rng.standard_normal((1, N, d))
    r = O.forward_all(q, k, v, B, L, K, Le, 0.21, drop_covered=False)
    ek, ev, ew = [], [], []
    for l in range(2, Le + 2):
        span = B ** l
        ek.append(k[0].reshape(-1, span, d).mean(axis=1))
        ev.append(v[0].reshape(-1, span, d).mean(axis=1))
        ew.append(np.full(N // span, float(span)))
    want, lse = _dense_attention(q[0], k[0], v[0], 0.21, np.concatenate(ek),
                                 np.concatenate(ev), np.concatenate(ew))
    np.testing.assert_allclose(r["o"][0], want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"][0], lse, rtol=0, atol=1e-12)


def test_attn_single_query_block_by_hand():
    # one query block, explicit attended set written out here from Step 3
    rng = np.random.default_rng(11)
    B, L, K, Le, N, d = 4, 2, 2, 1, 64, 3
    q = rng.standard_normal((1, N, d))
    k = rng.standard_normal((1, N, d))
    v = rng.standard_normal((1, N, d))
    r = O.forward_all(q, k, v, B, L, K, Le, 0.5)
    i = 5                                   # query block 5 -> tokens 20..23
    fine = r["idx"][0][0, i]
    coarse = r["idx"][1][0, i // B]         # ancestor at level 2
    toks = [int(f) * B + t for f in fine for t in range(B)]
    ck = np.stack([k[0, int(c) * 16:(int(c) + 1) * 16].mean(axis=0) for c in coarse])
    cv = np.stack([v[0, int(c) * 16:(int(c) + 1) * 16].mean(axis=0) for c in coarse])
    want, lse = _dense_attention(q[0, 20:24], k[0, toks], v[0, toks], 0.5, ck, cv,
                                 np.full(len(coarse), 16.0))
    np.testing.assert_allclose(r["o"][0, 20:24], want, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["lse"][0, 20:24], lse, rtol=0, atol=1e-12)


# ------------------------------------------------------------ backward ----
def _loss(q, k, v, dout, idx, B, L, K, Le, scale):
    pk, pv = O.pool(k, B, L), O.pool(v, B, L)
    o, _ = O.attn_fwd(q, k, v, pk, pv, idx, B, K, Le, scale)
    return float((o * dout).sum())


@pytest.mark.parametrize("L,Le", [(2, 1), (3, 2), (2, 0)])
def test_bwd_finite_differences(L, Le):
    rng = np.random.default_rng(12 + L + Le)
    B, K, d, scale = 4, 2, 4, 0.45
    N = B ** L * 2
    q = rng.standard_normal((2, N, d))
    k = rng.standard_normal((2, N, d))
    v = rng.standard_normal((2, N, d))
    dout = rng.standard_normal((2, N, d))
    pq, pk, pv = O.pool(q, B, L), O.pool(k, B, L), O.pool(v, B, L)
    idx, _ = O.select(pq, pk, B, K)
    dq, dk, dv = O.attn_bwd(q, k, v, pk, pv, idx, dout, B, K, Le, scale)
    h = 1e-6
    probes = [(t, 0 if t == 1 else 1, i, e) for t in range(3)
              for i in rng.choice(N, 6, replace=False) for e in range(d)]
    for which, b, i, e in probes:
        args = [q, k, v]
        plus = [a.copy() for a in args]
        minus = [a.copy() for a in args]
        plus[which][b, i, e] += h
        minus[which][b, i, e] -= h
        # the picks are unchanged by the step (no gradient through Top-K)
        for pm in (plus, minus):
            idx2, _ = O.select(O.pool(pm[0], B, L), O.pool(pm[1], B, L), B, K)
            assert all((a == c).all() for a, c in zip(idx, idx2))
        num = (_loss(*plus, dout, idx, B, L, K, Le, scale)
               - _loss(*minus, dout, idx, B, L, K, Le, scale)) / (2 * h)
        ana = (dq, dk, dv)[which][b, i, e]
        assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (which, b, i, e, num, ana)


def test_bwd_value_gradient_is_linear_map():
    # O is linear in V for fixed picks: <O(V), dO> = <V, dV> exactly
    rng = np.random.default_rng(20)
    B, L, K, Le, N, d = 4, 3, 2, 2, 4 ** 3 * 2, 4
    q = rng.standard_normal((1, N, d))
    k = rng.standard_normal((1, N, d))
    v = rng.standard_normal((1, N, d))
    dout = rng.standard_normal((1, N, d))
    pk, pv = O.pool(k, B, L), O.pool(v, B, L)
    idx, _ = O.select(O.pool(q, B, L), pk, B, K)
    o, _ = O.attn_fwd(q, k, v, pk, pv, idx, B, K, Le, 0.3)
    _, _, dv = O.attn_bwd(q, k, v, pk, pv, idx, dout, B, K, Le, 0.3)
    assert float((o * dout).sum()) == pytest.approx(float((v * dv).sum()), rel=1e-12, abs=1e-12)


# ----------------------------------------------------------------- Step 4 --
def _brute_transpose(idx, cols):
    nb, rows, k = idx.shape
    out = []
    for b in range(nb):
        out.append([[r for r in range(rows) if c in set(idx[b, r].tolist())] for c in range(cols)])
    return out


def test_transpose_worked_example(golden_dir):
    fx = _read_fixture(os.path.join(golden_dir, "transpose_100x8.txt"))
    rows, k, pairs = int(fx["rows"][0]), int(fx["k"][0]), int(fx["pairs"][0])
    rng = np.random.default_rng(21)
    idx = np.stack([np.sort(rng.choice(100, k, replace=False)) for _ in range(rows)])[None]
    ptr, col = O.transpose(idx, 100)
    assert ptr[0, -1] == pairs and col.shape[1] == pairs


@pytest.mark.parametrize("rows,k,cols", [(37, 5, 23), (64, 8, 64), (5, 1, 9), (16, 16, 16)])
def test_transpose_brute_force_and_round_trip(rows, k, cols):
    rng = np.random.default_rng(rows * 7 + k)
    idx = np.stack([np.sort(rng.choice(cols, k, replace=False)) for _ in range(3 * rows)])
    idx = idx.reshape(3, rows, k)
    ptr, col = O.transpose(idx, cols)
    brute = _brute_transpose(idx, cols)
    for b in range(3):
        np.testing.assert_array_equal(np.diff(ptr[b]), np.bincount(idx[b].ravel(), minlength=cols))
        assert ptr[b, 0] == 0 and ptr[b, -1] == rows * k
        for c in range(cols):
            seg = col[b, ptr[b, c]:ptr[b, c + 1]].tolist()
            assert seg == brute[b][c]
        # round trip: key-major lists back to the query-major rows
        back = [[] for _ in range(rows)]
        for c in range(cols):
            for r in col[b, ptr[b, c]:ptr[b, c + 1]]:
                back[r].append(c)
        np.testing.assert_array_equal(np.array(back), idx[b])


def test_transpose_rejects_out_of_range():
    with pytest.raises(ValueError):
        O.transpose(np.array([[[0, 5]]], dtype=np.int32), 5)
