"""Seeded random problem shapes against the fp64 oracle.

The edge list in test_gpu_parity.py names the shapes each kernel path was
built for; this module draws a fixed list of further shapes from one seed
(block size, pooling steps, top-K, enrichment levels, dtypes, token order,
the drop rule, batch and heads), so that a path the edge list misses still
meets the oracle.  Each shape is small enough for the oracle to finish in a
second or two.  A second list draws shapes in the 2D patch order (N a power
of 4).  The lists are the same on every run.
"""
import sys

import numpy as np
import pytest
import torch

from hierarchical_top_sparse_mean_amd import llsa as L

N_CASES = 24
MAX_PAIRS = 1 << 24   # query-key pairs per head that the oracle visits


def _draw_cases():
    rng = np.random.default_rng(20261203)
    cases = []
    while len(cases) < N_CASES:
        B = 64 if rng.random() < 0.25 else 16
        Lv = int(rng.integers(1, 3 if B == 64 else 4))
        if Lv == 1:
            n1 = int(rng.integers(2, 65))
            N = n1 * B
        else:
            N = int(rng.integers(1, 9)) * B ** Lv
        if N > 65536:
            continue
        order = 0
        if rng.random() < 0.25:
            m = int(round(np.log(N) / np.log(4)))
            if 4 ** m == N:
                order = 1
        K = int(rng.integers(1, 33))
        Le = int(rng.integers(0, Lv)) if Lv > 1 else 0
        if K * B * N > MAX_PAIRS:
            continue
        dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
        grad = torch.bfloat16 if rng.random() < 0.2 else torch.float32
        drop = bool(rng.random() < 0.85)
        batch = int(rng.integers(1, 3))
        heads = int(rng.integers(1, 4))
        cases.append((batch, heads, N, dtype, Lv, K, Le, B, order, grad, drop))
    return cases


def _draw_patch_cases(n_cases=8):
    """Shapes in 2D patch order: N = 4^m pixels of a square image."""
    rng = np.random.default_rng(4096)
    cases = []
    while len(cases) < n_cases:
        B = 64 if rng.random() < 0.25 else 16
        N = int(4 ** rng.integers(4, 9))            # 256 .. 65536 pixels
        Lmax = 1
        while Lmax < 3 and N % (B ** (Lmax + 1)) == 0 and N // (B ** (Lmax + 1)) >= 1:
            Lmax += 1
        if N % B != 0:
            continue
        Lv = int(rng.integers(1, Lmax + 1))
        K = int(rng.integers(1, 33))
        Le = int(rng.integers(0, Lv)) if Lv > 1 else 0
        if K * B * N > MAX_PAIRS:
            continue
        dtype = torch.float32 if rng.random() < 0.25 else torch.bfloat16
        grad = torch.bfloat16 if rng.random() < 0.2 else torch.float32
        drop = bool(rng.random() < 0.85)
        batch = int(rng.integers(1, 3))
        heads = int(rng.integers(1, 4))
        cases.append((batch, heads, N, dtype, Lv, K, Le, B, 1, grad, drop))
    return cases


CASES = _draw_cases() + _draw_patch_cases()
IDS = [f"b{c[0]}h{c[1]}N{c[2]}{str(c[3])[6:]}L{c[4]}K{c[5]}Le{c[6]}B{c[7]}o{c[8]}g{str(c[9])[6:]}d{int(c[10])}"
       for c in CASES]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_random_shape_accepted(case):
    """Host side, no GPU: the library's validation accepts every drawn problem."""
    b, h, N, dt, Lv, K, Le, B, order, grad, drop = case
    p = L.problem(b, h, N, 64, B, Lv, K, Le, dt, grad, 0.0, drop, order)
    assert L.llsa_sizes_query(p) is not None


@pytest.mark.gpu
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_random_shape_parity(case):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from parity_util import Case, check_case
    b, h, N, dt, Lv, K, Le, B, order, grad, drop = case
    print(f"[parity] random shape {case}", flush=True)
    sys.stdout.flush()
    c = Case(b, h, N, dt, Lv, K, Le, backward=True, drop_covered=drop, grad_dtype=grad,
             token_order=order, block=B, sinus=(order == 1))
    summ = check_case(c)
    print(f"[parity] random shape done {summ}", flush=True)
