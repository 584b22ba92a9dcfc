"""ctypes wrapper around the fp64 CPU oracle (``llsa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by ``__graft_entry__.smoke``
and by the CPU-baseline leg of ``bench.py``; never by the library.  The oracle
follows the method description "Trainable Log-linear Sparse Attention for
Efficient Diffusion Transformers" (howistudyai.com explainer, "Step 1"
through "Step 4"), in double precision, and shares no code with the HIP path.

Arrays are numpy; every floating input is converted to float64 exactly
(bf16 and fp32 values are representable in fp64).  Shapes use ``bh`` for
batch*heads.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "llsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        i, d = ctypes.c_int, ctypes.c_double
        lib.oracle_pool.argtypes = [i, i, i, i, i, _dp, _dp]
        lib.oracle_select_level.argtypes = [i, i, i, i, i, _dp, _dp, _ip, i, _ip, _dp]
        lib.oracle_select_level.restype = i
        lib.oracle_select.argtypes = [i, i, i, i, i, i, _dp, _dp, _ip, _dp]
        lib.oracle_attn_fwd.argtypes = [i, i, i, i, i, i, i, d, i, _dp, _dp, _dp, _dp, _dp,
                                        _ip, _dp, _dp]
        lib.oracle_attn_bwd.argtypes = [i, i, i, i, i, i, i, d, i, _dp, _dp, _dp, _dp, _dp,
                                        _ip, _dp, _dp, _dp, _dp]
        lib.oracle_transpose.argtypes = [i, i, i, i, _ip, _ip, _ip]
        lib.oracle_transpose.restype = i
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _p(a: np.ndarray, kind):
    return a.ctypes.data_as(kind)


def level_sizes(N: int, B: int, L: int):
    """Tokens per level l = 1..L (N / B^l)."""
    return [N // B ** l for l in range(1, L + 1)]


def level_k(N: int, B: int, L: int, K: int):
    """Picks per level l = 1..L: min(K, #candidates)."""
    n = level_sizes(N, B, L)
    kl = [0] * (L + 1)
    kl[L] = min(K, n[-1])
    for l in range(L - 1, 0, -1):
        kl[l] = min(K, kl[l + 1] * B)
    return kl[1:]


def pool(x, B: int, L: int):
    """Step 1: returns [level 1, ..., level L], level l of shape [bh, N/B^l, d]."""
    x = _f64(x)
    bh, N, d = x.shape
    sizes = level_sizes(N, B, L)
    out = np.zeros(sum(bh * n * d for n in sizes), dtype=np.float64)
    _load().oracle_pool(bh, N, d, B, L, _p(x, _dp), _p(out, _dp))
    res, off = [], 0
    for n in sizes:
        res.append(out[off:off + bh * n * d].reshape(bh, n, d))
        off += bh * n * d
    return res


def select_level(q_l, k_l, B: int, K: int, parent=None):
    """Step 2, one level.  q_l, k_l: [bh, n, d]; parent: [bh, n/B, kp] or None.

    Returns (idx [bh, n, kout], relgap [bh, n])."""
    q_l, k_l = _f64(q_l), _f64(k_l)
    bh, n, d = q_l.shape
    if parent is None:
        kp, ncand, pp = 0, n, None
    else:
        parent = _i32(parent)
        kp = parent.shape[-1]
        ncand = kp * B
        pp = _p(parent, _ip)
    kout = min(K, ncand)
    out = np.zeros((bh, n, kout), dtype=np.int32)
    gap = np.zeros((bh, n), dtype=np.float64)
    _load().oracle_select_level(bh, n, d, B, K, _p(q_l, _dp), _p(k_l, _dp), pp, kp,
                                _p(out, _ip), _p(gap, _dp))
    return out, gap


def select(pyr_q, pyr_k, B: int, K: int):
    """Step 2, all levels coarse to fine.  Returns (idx list, relgap list), level 1 first."""
    L = len(pyr_q)
    idx = [None] * L
    gap = [None] * L
    parent = None
    for l in range(L, 0, -1):
        idx[l - 1], gap[l - 1] = select_level(pyr_q[l - 1], pyr_k[l - 1], B, K, parent)
        parent = idx[l - 1]
    return idx, gap


def _flat_pyr(levels):
    return np.ascontiguousarray(np.concatenate([_f64(a).ravel() for a in levels]))


def _flat_idx(levels):
    return np.ascontiguousarray(np.concatenate([_i32(a).ravel() for a in levels]))


def attn_fwd(q, k, v, pyr_k, pyr_v, idx, B: int, K: int, Le: int, scale: float,
             drop_covered: bool = True):
    """Step 3.  q,k,v: [bh, N, d]; pyramids / idx: lists level 1..L.

    Returns (o [bh, N, d], lse [bh, N])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    bh, N, d = q.shape
    L = len(pyr_k)
    pk, pv, ii = _flat_pyr(pyr_k), _flat_pyr(pyr_v), _flat_idx(idx)
    o = np.zeros((bh, N, d))
    lse = np.zeros((bh, N))
    _load().oracle_attn_fwd(bh, N, d, B, L, K, Le, float(scale), int(drop_covered),
                            _p(q, _dp), _p(k, _dp), _p(v, _dp), _p(pk, _dp), _p(pv, _dp),
                            _p(ii, _ip), _p(o, _dp), _p(lse, _dp))
    return o, lse


def attn_bwd(q, k, v, pyr_k, pyr_v, idx, dout, B: int, K: int, Le: int, scale: float,
             drop_covered: bool = True):
    """Gradients of <O, dO> for fixed picks.  Returns (dq, dk, dv), each [bh, N, d]."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    bh, N, d = q.shape
    L = len(pyr_k)
    pk, pv, ii = _flat_pyr(pyr_k), _flat_pyr(pyr_v), _flat_idx(idx)
    dq = np.zeros((bh, N, d))
    dk = np.zeros((bh, N, d))
    dv = np.zeros((bh, N, d))
    _load().oracle_attn_bwd(bh, N, d, B, L, K, Le, float(scale), int(drop_covered),
                            _p(q, _dp), _p(k, _dp), _p(v, _dp), _p(pk, _dp), _p(pv, _dp),
                            _p(ii, _ip), _p(dout, _dp), _p(dq, _dp), _p(dk, _dp), _p(dv, _dp))
    return dq, dk, dv


def transpose(idx, cols: int):
    """Step 4.  idx [nb, rows, k] -> (ptr [nb, cols+1], col [nb, rows*k])."""
    idx = _i32(idx)
    nb, rows, k = idx.shape
    ptr = np.zeros((nb, cols + 1), dtype=np.int32)
    col = np.zeros((nb, rows * k), dtype=np.int32)
    rc = _load().oracle_transpose(nb, rows, k, cols, _p(idx, _ip), _p(ptr, _ip), _p(col, _ip))
    if rc != 0:
        raise ValueError("index outside [0, cols)")
    return ptr, col


def forward_all(q, k, v, B: int, L: int, K: int, Le: int, scale: float,
                drop_covered: bool = True):
    """Pool, select and attend from the inputs alone.  Returns a dict."""
    pq, pk, pv = pool(q, B, L), pool(k, B, L), pool(v, B, L)
    idx, gap = select(pq, pk, B, K)
    o, lse = attn_fwd(q, k, v, pk, pv, idx, B, K, Le, scale, drop_covered)
    return dict(pyr_q=pq, pyr_k=pk, pyr_v=pv, idx=idx, gap=gap, o=o, lse=lse)
