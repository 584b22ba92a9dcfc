"""C ABI checks that need no GPU: every symbol the header declares is
exported, sizes are derived as documented, and bad arguments are rejected on
the host before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

from hierarchical_top_sparse_mean_amd import llsa as L
from hierarchical_top_sparse_mean_amd.inputs import WORKLOADS, make_inputs, sinusoid

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "llsa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(llsa_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    syms = _declared_symbols()
    assert {"llsa_pool", "llsa_select", "llsa_attn_fwd", "llsa_index_transpose",
            "llsa_attn_bwd"} <= set(syms)
    lib = ctypes.CDLL(L._LIB_PATH)
    for s in syms:
        assert hasattr(lib, s), s


def _status(p):
    return L.lib.llsa_sizes_query(ctypes.byref(p), ctypes.byref(L.Sizes()))


def test_sizes_of_the_measured_workload():
    w = WORKLOADS["n65536_bf16"]
    p = L.problem(w.batch, w.heads, w.seq_len, levels=w.levels, topk=w.topk, enrich=w.enrich)
    s = L.llsa_sizes_query(p)
    assert s.levels == 2 and s.enrich == 1
    assert list(s.level_tokens)[:3] == [65536, 4096, 256]
    assert list(s.level_k)[1:3] == [8, 8]
    bh = 16
    assert s.pyramid_offset[1] == 0 and s.pyramid_offset[2] == bh * 4096 * 64
    assert s.pyramid_elems == bh * (4096 + 256) * 64
    assert s.index_offset[2] == bh * 4096 * 8 and s.index_elems == bh * (4096 + 256) * 8
    assert s.csr_ptr_offset[2] == 65552 and s.csr_ptr_elems == 65552 + 4112   # 16-element padding
    assert s.csr_col_elems == bh * (4096 + 256) * 8
    assert s.lse_elems == bh * 65536
    assert s.bwd_workspace_bytes > 0
    for arr in (s.pyramid_offset, s.index_offset, s.csr_ptr_offset, s.csr_col_offset):
        assert all(arr[l] % 16 == 0 for l in range(1, 4))


def test_sizes_block_64():
    p = L.problem(1, 2, 65536, block=64, levels=2, topk=8)
    s = L.llsa_sizes_query(p)
    assert list(s.level_tokens)[:3] == [65536, 1024, 16]
    assert list(s.level_k)[1:3] == [8, 8]
    assert s.pyramid_elems == 2 * (1024 + 16) * 64
    assert s.csr_col_elems == 2 * (1024 + 16) * 8
    p = L.problem(1, 1, 4096, block=64, levels=2, topk=8)   # 1 coarsest token -> 64 candidates
    assert list(L.llsa_sizes_query(p).level_k)[1:3] == [8, 1]


def test_picks_clamped_to_candidates():
    p = L.problem(1, 1, 1024, levels=2, topk=16)  # 4 coarsest tokens
    s = L.llsa_sizes_query(p)
    assert list(s.level_k)[1:3] == [16, 4]
    p = L.problem(1, 1, 256, levels=2, topk=3)    # 1 coarsest token -> 16 candidates below
    s = L.llsa_sizes_query(p)
    assert list(s.level_k)[1:3] == [3, 1]


@pytest.mark.parametrize("kw,status", [
    (dict(seq_len=1000), L.LLSA_ERR_INVALID),           # not divisible by 16^2
    (dict(seq_len=16, levels=2), L.LLSA_ERR_INVALID),   # fewer tokens than one coarsest token
    (dict(topk=0), L.LLSA_ERR_INVALID),
    (dict(enrich=2), L.LLSA_ERR_INVALID),               # Le > L-1
    (dict(enrich=-2), L.LLSA_ERR_INVALID),
    (dict(scale=-1.0), L.LLSA_ERR_INVALID),
    (dict(head_dim=128), L.LLSA_ERR_UNSUPPORTED),
    (dict(block=32, seq_len=32 * 32 * 4), L.LLSA_ERR_UNSUPPORTED),
    (dict(block=64, seq_len=4096 + 1024), L.LLSA_ERR_INVALID),   # not divisible by 64^2
    (dict(topk=33), L.LLSA_ERR_UNSUPPORTED),
    (dict(token_order=2), L.LLSA_ERR_INVALID),
    (dict(token_order=1, seq_len=2048), L.LLSA_ERR_INVALID),    # not a square image
    (dict(levels=7, seq_len=16 ** 5), L.LLSA_ERR_UNSUPPORTED),
    (dict(heads=1, seq_len=1 << 26), L.LLSA_ERR_UNSUPPORTED),    # one head beyond 2^25 tokens
    (dict(heads=1, seq_len=1 << 25), L.LLSA_ERR_UNSUPPORTED),    # 2^25 tokens: 4 GiB per head
])
def test_sizes_query_rejects(kw, status):
    args = dict(batch=1, heads=2, seq_len=4096, levels=2, topk=8)
    args.update(kw)
    assert _status(L.problem(**args)) == status


def test_bad_dtype_rejected():
    p = L.problem(1, 2, 4096)
    p.dtype = 7
    assert _status(p) == L.LLSA_ERR_INVALID


def test_entry_points_validate_before_launch():
    # no GPU needed: every call below fails host-side validation
    lib = L.lib
    good = L.problem(1, 2, 4096)
    bad = L.problem(1, 2, 4096, head_dim=32)
    fake = 1 << 20          # 16-byte aligned non-null "device" address, never dereferenced
    mis = fake + 4          # misaligned
    bp = ctypes.byref(bad)
    gp = ctypes.byref(good)
    assert lib.llsa_pool(bp, fake, fake, fake, fake, fake, fake, None) == L.LLSA_ERR_UNSUPPORTED
    assert lib.llsa_pool(gp, None, fake, fake, fake, fake, fake, None) == L.LLSA_ERR_INVALID
    assert lib.llsa_pool(gp, mis, fake, fake, fake, fake, fake, None) == L.LLSA_ERR_INVALID
    assert lib.llsa_select(gp, fake, None, fake, None) == L.LLSA_ERR_INVALID
    assert lib.llsa_attn_fwd(bp, *([fake] * 8), None) == L.LLSA_ERR_UNSUPPORTED
    assert lib.llsa_attn_fwd(gp, *([fake] * 7), mis, None) == L.LLSA_ERR_INVALID
    assert lib.llsa_index_transpose(1, 10, 2, 1 << 25, fake, fake, fake, None, 0, None) == L.LLSA_ERR_UNSUPPORTED
    assert lib.llsa_index_transpose(0, 10, 2, 10, fake, fake, fake, None, 0, None) == L.LLSA_ERR_INVALID
    assert lib.llsa_index_transpose(1, 10, 2, 10, None, fake, fake, None, 0, None) == L.LLSA_ERR_INVALID
    # transposes of every level: nothing fits the one-launch kernel at 262144
    # tokens on level 1 (16384 keys), so that level needs a workspace
    assert L.llsa_index_transpose_levels_workspace(good) == 0
    big = L.problem(1, 2, 262144, levels=3)
    assert L.llsa_index_transpose_levels_workspace(big) > 0
    assert lib.llsa_index_transpose_levels(bp, fake, fake, fake, None, 0, None) == L.LLSA_ERR_UNSUPPORTED
    assert lib.llsa_index_transpose_levels(gp, mis, fake, fake, None, 0, None) == L.LLSA_ERR_INVALID
    assert lib.llsa_index_transpose_levels(ctypes.byref(big), fake, fake, fake, None, 0, None) == L.LLSA_ERR_WORKSPACE
    s = L.llsa_sizes_query(good)
    args = [fake] * 14
    assert lib.llsa_attn_bwd(gp, *args, None, 0, None) == L.LLSA_ERR_WORKSPACE
    assert lib.llsa_attn_bwd(gp, *args, fake, s.bwd_workspace_bytes - 1, None) == L.LLSA_ERR_WORKSPACE
    # 16 + 16 + 2 = 34 coarse entries per query block: more than the backward supports
    many = L.problem(1, 2, 16 ** 4 * 2, levels=4, topk=16, enrich=3)
    assert L.llsa_sizes_query(many).level_k[4] == 2
    assert lib.llsa_attn_bwd(ctypes.byref(many), *args, fake, 1 << 40, None) == L.LLSA_ERR_UNSUPPORTED
    dense_f32 = L.problem(1, 2, 4096, dtype=torch.float32)
    assert lib.llsa_dense_attn_fwd(ctypes.byref(dense_f32), *([fake] * 5), None) == L.LLSA_ERR_UNSUPPORTED


def test_strerror():
    assert L.lib.llsa_strerror(0) == b"ok"
    assert b"workspace" in L.lib.llsa_strerror(L.LLSA_ERR_WORKSPACE)
    assert L.lib.llsa_strerror(99) == b"unknown status"


# ---------------------------------------------------------------- inputs --
def test_inputs_are_seeded_and_shaped():
    a = make_inputs(1, 2, 256, 64, torch.bfloat16, True, True, seed=0)
    b = make_inputs(1, 2, 256, 64, torch.bfloat16, True, True, seed=0)
    for x, y in zip(a, b):
        assert x.shape == (1, 2, 256, 64) and x.dtype == torch.bfloat16
        assert torch.equal(x, y)
    c = make_inputs(1, 2, 256, 64, torch.bfloat16, True, True, seed=1)
    assert not torch.equal(a[0], c[0])


def test_sinusoid_values():
    s = sinusoid(256, 64).double()
    # channel 0: fy = 1 -> sin(2 pi y / 16), phase 0; token 20 is (y=1, x=4)
    assert s[20, 0].item() == pytest.approx(torch.sin(torch.tensor(2 * torch.pi / 16)).item(), abs=1e-6)
    # channel 1: fx = 1, phase 2 pi / 64
    assert s[20, 1].item() == pytest.approx(
        float(torch.sin(torch.tensor(2 * torch.pi * 4 / 16 + 2 * torch.pi / 64))), abs=1e-6)
    # constant along a raster row for the (0, 1) channels
    assert torch.allclose(s[16:32, 0], s[16, 0].expand(16))


def test_patch_order_is_a_nested_permutation():
    # the 2D patch order used by the parity tests: a permutation whose runs of
    # 4^i positions are 2^i x 2^i patches of the raster image
    from parity_util import patch_order
    N, S = 4096, 64
    perm = patch_order(N)
    assert sorted(perm.tolist()) == list(range(N))
    for side in (2, 4, 16):
        runs = perm.reshape(-1, side * side)
        ys, xs = runs // S, runs % S
        assert ((ys.max(1) - ys.min(1)) == side - 1).all()
        assert ((xs.max(1) - xs.min(1)) == side - 1).all()
    assert perm[:4].tolist() == [0, 1, S, S + 1]
