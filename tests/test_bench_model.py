"""The benchmark's byte and FLOP model, and its one-GPU contract (CPU only).

bench.py reports each call's HBM fraction from the compulsory bytes of the
call: every tensor it must read or write, counted once.  These tests check the
model against the closed forms for the 65536-token, 16-head workload (block
16, levels 65536 -> 4096 -> 256, K = 8, one coarse level; bf16 inputs):

  token tensor (one of Q, K, V, O, dO) = 16 * 65536 * 64 * 2 B = 134217728 B
  pool       = 3 inputs + 3 float32 pyramids of 4096 + 256 tokens
  backward   = Q, K, V, O, dO read + dQ, dK, dV written + LSE and D
  transpose  = per level 1..2: the picks read, the CSR pointers and columns written
  forward    = Q, K, V read, O written, LSE, the pick lists and the coarse pyramids
  attention FLOPs = 4 * tokens * heads * d * (keys per query block = 8 * 16 + 8)
"""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from hierarchical_top_sparse_mean_amd import llsa as L  # noqa: E402
from hierarchical_top_sparse_mean_amd.inputs import WORKLOADS  # noqa: E402

TOK = 16 * 65536 * 64 * 2


def _model(grad_bytes=4):
    w = WORKLOADS["n65536_bf16"]
    s = L.llsa_sizes_query(L.problem(w.batch, w.heads, w.seq_len, block=w.block, levels=w.levels,
                                     topk=w.topk, enrich=w.enrich, dtype=w.dtype))
    return bench.algorithmic(w, s, grad_bytes)


def test_pool_bytes():
    alg, _ = _model()
    assert alg["pool"]["bytes"] == 3 * TOK + 3 * 16 * (4096 + 256) * 64 * 4   # 456.1 MB


def test_backward_bytes_both_gradient_dtypes():
    alg, _ = _model(4)
    lse_d = 2 * 16 * 65536 * 4
    assert alg["attn_bwd"]["bytes"] == 5 * TOK + 3 * 16 * 65536 * 64 * 4 + lse_d   # 1484.8 MB
    alg2, _ = _model(2)
    assert alg2["attn_bwd"]["bytes"] == 5 * TOK + 3 * TOK + lse_d                  # 1082.1 MB


def test_transpose_bytes():
    alg, _ = _model()
    lv1 = 16 * 4096 * 8 * 4 * 2 + 16 * 4097 * 4
    lv2 = 16 * 256 * 8 * 4 * 2 + 16 * 257 * 4
    assert alg["transpose"]["bytes"] == lv1 + lv2                                  # 4.7 MB


def test_forward_bytes_and_flops():
    alg, nkv = _model()
    assert nkv == 8 * 16 + 8
    picks = 16 * (4096 + 256) * 8 * 4
    coarse = 2 * 16 * 256 * 64 * 4
    assert alg["attn_fwd"]["bytes"] == 4 * TOK + 16 * 65536 * 4 + picks + coarse   # 545.4 MB
    assert alg["attn_fwd"]["flops"] == 4 * 16 * 65536 * 64 * nkv                    # 36.5 GFLOP
    assert alg["attn_bwd"]["flops"] == int(2.5 * alg["attn_fwd"]["flops"])


def test_selection_bytes_and_flops():
    alg, _ = _model()
    coarsest = 2 * 16 * 256 * 64 * 4 + 16 * 256 * 8 * 4
    level1 = 2 * 16 * 4096 * 64 * 4 + 16 * 256 * 8 * 4 + 16 * 4096 * 8 * 4
    assert alg["select"]["bytes"] == coarsest + level1                            # 38.0 MB
    assert alg["select"]["flops"] == 2 * 64 * 16 * 256 * 256 + 2 * 64 * 16 * 4096 * 8 * 16


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
