"""Thin ctypes binding of ``libllsa.so`` (C ABI declared in ``include/llsa.h``).

Argument marshalling only: every step of the operator runs in the library's
HIP kernels.  Tensors are torch CUDA (HIP) tensors, passed as raw device
pointers; the stream defaults to torch's current stream.  A missing library
raises at import time -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libllsa.so")
MAX_LEVELS = 6

(LLSA_OK, LLSA_ERR_INVALID, LLSA_ERR_UNSUPPORTED, LLSA_ERR_WORKSPACE, LLSA_ERR_HIP, LLSA_ERR_INDEX,
 LLSA_ERR_SCRATCH) = range(7)
NOALLOC_SCRATCH_BYTES = 32 << 20
LLSA_IDX_RANGE, LLSA_IDX_ORDER, LLSA_IDX_PARENT, LLSA_IDX_CSR_PTR, LLSA_IDX_CSR_COL = 1, 2, 4, 8, 16
LLSA_F32, LLSA_BF16 = 0, 1

_c_i32, _c_i64, _c_sz, _c_f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p


class Problem(ctypes.Structure):
    _fields_ = [("batch", _c_i32), ("heads", _c_i32), ("seq_len", _c_i32), ("head_dim", _c_i32),
                ("block", _c_i32), ("levels", _c_i32), ("topk", _c_i32), ("enrich", _c_i32),
                ("dtype", _c_i32), ("grad_dtype", _c_i32), ("scale", _c_f32),
                ("drop_covered", _c_i32), ("token_order", _c_i32), ("index_status", _vp)]


class Sizes(ctypes.Structure):
    _fields_ = [("levels", _c_i32), ("enrich", _c_i32),
                ("level_tokens", _c_i32 * (MAX_LEVELS + 1)), ("level_k", _c_i32 * (MAX_LEVELS + 1)),
                ("pyramid_elems", _c_i64), ("pyramid_offset", _c_i64 * (MAX_LEVELS + 2)),
                ("index_elems", _c_i64), ("index_offset", _c_i64 * (MAX_LEVELS + 2)),
                ("csr_ptr_elems", _c_i64), ("csr_ptr_offset", _c_i64 * (MAX_LEVELS + 2)),
                ("csr_col_elems", _c_i64), ("csr_col_offset", _c_i64 * (MAX_LEVELS + 2)),
                ("lse_elems", _c_i64), ("transpose_workspace_bytes", _c_sz),
                ("bwd_workspace_bytes", _c_sz)]


class LLSAError(RuntimeError):
    def __init__(self, name: str, status: int):
        super().__init__(f"{name}: {lib.llsa_strerror(status).decode()} (status {status})")
        self.status = status


def _load():
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is not built; run `python -m hierarchical_top_sparse_mean_amd.build`")
    L = ctypes.CDLL(_LIB_PATH)
    P = ctypes.POINTER(Problem)
    L.llsa_sizes_query.argtypes = [P, ctypes.POINTER(Sizes)]
    L.llsa_pool.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.llsa_select.argtypes = [P, _vp, _vp, _vp, _vp]
    L.llsa_select_transpose_workspace.argtypes = [P]
    L.llsa_select_transpose_workspace.restype = _c_sz
    L.llsa_select_transpose.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _c_sz, _vp]
    L.llsa_attn_fwd.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]
    L.llsa_index_transpose_workspace.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32]
    L.llsa_index_transpose_workspace.restype = _c_sz
    L.llsa_index_transpose.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _c_sz, _vp]
    L.llsa_index_transpose_levels_workspace.argtypes = [P]
    L.llsa_index_transpose_levels_workspace.restype = _c_sz
    L.llsa_index_transpose_levels.argtypes = [P, _vp, _vp, _vp, _vp, _c_sz, _vp]
    L.llsa_index_transpose_mask_workspace.argtypes = [_c_i32, _c_i32, _c_i32]
    L.llsa_index_transpose_mask_workspace.restype = _c_sz
    L.llsa_index_transpose_mask.argtypes = [_c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _c_sz,
                                            _vp]
    L.llsa_attn_bwd.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                _vp, _vp, _vp, _c_sz, _vp]
    L.llsa_attn_bwd_noalloc.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                        _vp, _vp, _vp, _vp]
    L.llsa_dense_attn_fwd.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp]
    L.llsa_dense_attn_bwd_workspace.argtypes = [P]
    L.llsa_dense_attn_bwd_workspace.restype = _c_sz
    L.llsa_dense_attn_bwd.argtypes = [P, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_sz,
                                      _vp]
    L.llsa_check_indices.argtypes = [P, _vp, _vp, _vp, _vp, _vp]
    L.llsa_check_indices_host.argtypes = [P, _vp, _vp, _vp, ctypes.POINTER(_c_i32)]
    L.llsa_strerror.argtypes = [ctypes.c_int]
    L.llsa_strerror.restype = ctypes.c_char_p
    for name in ("llsa_sizes_query", "llsa_pool", "llsa_select", "llsa_attn_fwd",
                 "llsa_index_transpose", "llsa_attn_bwd", "llsa_dense_attn_fwd",
                 "llsa_dense_attn_bwd", "llsa_index_transpose_mask", "llsa_select_transpose",
                 "llsa_index_transpose_levels", "llsa_check_indices", "llsa_check_indices_host",
                 "llsa_attn_bwd_noalloc"):
        getattr(L, name).restype = ctypes.c_int
    return L


lib = _load()


def problem(batch, heads, seq_len, head_dim=64, block=16, levels=2, topk=8, enrich=-1,
            dtype=torch.bfloat16, grad_dtype=torch.float32, scale=0.0, drop_covered=True,
            token_order=0, index_status=None) -> Problem:
    """index_status: a one-element int32 CUDA tensor (or a device address) to
    turn the debug index check on; None leaves it off."""
    code = {torch.float32: LLSA_F32, torch.bfloat16: LLSA_BF16}
    return Problem(batch, heads, seq_len, head_dim, block, levels, topk, enrich,
                   code.get(dtype, -1), code.get(grad_dtype, -1), float(scale), int(drop_covered),
                   int(token_order), _ptr(index_status))


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def _check(name, status):
    if status != LLSA_OK:
        raise LLSAError(name, status)


def llsa_sizes_query(p: Problem) -> Sizes:
    s = Sizes()
    _check("llsa_sizes_query", lib.llsa_sizes_query(ctypes.byref(p), ctypes.byref(s)))
    return s


def llsa_pool(p, q, k, v, pyr_q, pyr_k, pyr_v, stream=None):
    _check("llsa_pool", lib.llsa_pool(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(pyr_q),
                                      _ptr(pyr_k), _ptr(pyr_v), _stream(stream)))


def llsa_select(p, pyr_q, pyr_k, idx, stream=None):
    _check("llsa_select", lib.llsa_select(ctypes.byref(p), _ptr(pyr_q), _ptr(pyr_k), _ptr(idx),
                                          _stream(stream)))


def llsa_select_transpose_workspace(p) -> int:
    return int(lib.llsa_select_transpose_workspace(ctypes.byref(p)))


def llsa_select_transpose(p, pyr_q, pyr_k, idx, csr_ptr, csr_col, workspace, workspace_bytes,
                          stream=None):
    _check("llsa_select_transpose",
           lib.llsa_select_transpose(ctypes.byref(p), _ptr(pyr_q), _ptr(pyr_k), _ptr(idx),
                                     _ptr(csr_ptr), _ptr(csr_col), _ptr(workspace), workspace_bytes,
                                     _stream(stream)))


def llsa_attn_fwd(p, q, k, v, pyr_k, pyr_v, idx, o, lse, stream=None):
    _check("llsa_attn_fwd", lib.llsa_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                              _ptr(pyr_k), _ptr(pyr_v), _ptr(idx), _ptr(o),
                                              _ptr(lse), _stream(stream)))


def llsa_index_transpose_workspace(n_batch, n_rows, k, n_cols) -> int:
    return int(lib.llsa_index_transpose_workspace(n_batch, n_rows, k, n_cols))


def llsa_index_transpose(n_batch, n_rows, k, n_cols, idx, csr_ptr, csr_col, workspace=None,
                         workspace_bytes=0, stream=None):
    _check("llsa_index_transpose",
           lib.llsa_index_transpose(n_batch, n_rows, k, n_cols, _ptr(idx), _ptr(csr_ptr),
                                    _ptr(csr_col), _ptr(workspace), workspace_bytes,
                                    _stream(stream)))


def llsa_index_transpose_levels_workspace(p) -> int:
    return int(lib.llsa_index_transpose_levels_workspace(ctypes.byref(p)))


def llsa_index_transpose_levels(p, idx, csr_ptr, csr_col, workspace=None, workspace_bytes=0,
                                stream=None):
    _check("llsa_index_transpose_levels",
           lib.llsa_index_transpose_levels(ctypes.byref(p), _ptr(idx), _ptr(csr_ptr), _ptr(csr_col),
                                           _ptr(workspace), workspace_bytes, _stream(stream)))


def llsa_index_transpose_mask_workspace(n_batch, n_rows, n_cols) -> int:
    return int(lib.llsa_index_transpose_mask_workspace(n_batch, n_rows, n_cols))


def llsa_index_transpose_mask(n_batch, n_rows, k, n_cols, idx, csr_ptr, csr_col, workspace,
                              workspace_bytes, stream=None):
    _check("llsa_index_transpose_mask",
           lib.llsa_index_transpose_mask(n_batch, n_rows, k, n_cols, _ptr(idx), _ptr(csr_ptr),
                                         _ptr(csr_col), _ptr(workspace), workspace_bytes,
                                         _stream(stream)))


def llsa_attn_bwd(p, q, k, v, pyr_k, pyr_v, idx, csr_ptr, csr_col, o, lse, dout, dq, dk, dv,
                  workspace, workspace_bytes, stream=None):
    _check("llsa_attn_bwd",
           lib.llsa_attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(pyr_k), _ptr(pyr_v),
                             _ptr(idx), _ptr(csr_ptr), _ptr(csr_col), _ptr(o), _ptr(lse),
                             _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                             workspace_bytes, _stream(stream)))


def llsa_attn_bwd_noalloc(p, q, k, v, pyr_k, pyr_v, idx, csr_ptr, csr_col, o, lse, dout, dq, dk, dv,
                          stream=None):
    _check("llsa_attn_bwd_noalloc",
           lib.llsa_attn_bwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(pyr_k),
                                     _ptr(pyr_v), _ptr(idx), _ptr(csr_ptr), _ptr(csr_col), _ptr(o),
                                     _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                                     _stream(stream)))


def llsa_dense_attn_fwd(p, q, k, v, o, lse, stream=None):
    _check("llsa_dense_attn_fwd", lib.llsa_dense_attn_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                                          _ptr(o), _ptr(lse), _stream(stream)))


def llsa_dense_attn_bwd_workspace(p) -> int:
    return int(lib.llsa_dense_attn_bwd_workspace(ctypes.byref(p)))


def llsa_dense_attn_bwd(p, q, k, v, o, lse, dout, dq, dk, dv, workspace, workspace_bytes,
                        stream=None):
    _check("llsa_dense_attn_bwd",
           lib.llsa_dense_attn_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                   _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                   workspace_bytes, _stream(stream)))


def llsa_check_indices(p, idx, csr_ptr, csr_col, status, stream=None):
    _check("llsa_check_indices",
           lib.llsa_check_indices(ctypes.byref(p), _ptr(idx), _ptr(csr_ptr), _ptr(csr_col), _ptr(status),
                                  _stream(stream)))


def llsa_check_indices_host(p, idx, csr_ptr=None, csr_col=None) -> int:
    """The debug index check on host (CPU) int32 tensors laid out as on the
    device; returns the OR of LLSA_IDX_* flags (0: valid)."""
    def host(t):
        if t is None:
            return None
        assert t.device.type == "cpu" and t.dtype == torch.int32 and t.is_contiguous()
        return t.data_ptr()
    flags = _c_i32(0)
    _check("llsa_check_indices_host",
           lib.llsa_check_indices_host(ctypes.byref(p), host(idx), host(csr_ptr), host(csr_col),
                                       ctypes.byref(flags)))
    return int(flags.value)


# --------------------------------------------------------------- buffers --
class Buffers:
    """Device buffers of one problem (allocated with torch; the library never allocates)."""

    def __init__(self, p: Problem, device="cuda", backward=True):
        s = llsa_sizes_query(p)
        self.p, self.s = p, s
        dt = torch.float32 if p.dtype == LLSA_F32 else torch.bfloat16
        gdt = torch.float32 if p.grad_dtype == LLSA_F32 else torch.bfloat16
        shape = (p.batch, p.heads, p.seq_len, p.head_dim)
        f32 = dict(dtype=torch.float32, device=device)
        i32 = dict(dtype=torch.int32, device=device)
        self.pyr_q = torch.empty(s.pyramid_elems, **f32)
        self.pyr_k = torch.empty(s.pyramid_elems, **f32)
        self.pyr_v = torch.empty(s.pyramid_elems, **f32)
        self.idx = torch.empty(s.index_elems, **i32)
        self.o = torch.empty(shape, dtype=dt, device=device)
        self.lse = torch.empty(s.lse_elems, **f32)
        if backward:
            self.csr_ptr = torch.empty(s.csr_ptr_elems, **i32)
            self.csr_col = torch.empty(s.csr_col_elems, **i32)
            self.dq = torch.empty(shape, dtype=gdt, device=device)
            self.dk = torch.empty(shape, dtype=gdt, device=device)
            self.dv = torch.empty(shape, dtype=gdt, device=device)
            self.ws = torch.empty(max(int(s.bwd_workspace_bytes), 256), dtype=torch.uint8, device=device)
            # one workspace serves the per-level transposes, the transposes of all levels
            # and the fused selection + transposes
            self.tws_bytes = max(int(s.transpose_workspace_bytes), llsa_select_transpose_workspace(p),
                                 llsa_index_transpose_levels_workspace(p))
            self.tws = torch.empty(max(self.tws_bytes, 256), dtype=torch.uint8, device=device)

    def pyramid_level(self, buf, l):
        s, p = self.s, self.p
        bh, n = p.batch * p.heads, s.level_tokens[l]
        o = s.pyramid_offset[l]
        return buf[o:o + bh * n * p.head_dim].view(bh, n, p.head_dim)

    def index_level(self, l):
        s, p = self.s, self.p
        bh, n, k = p.batch * p.heads, s.level_tokens[l], s.level_k[l]
        o = s.index_offset[l]
        return self.idx[o:o + bh * n * k].view(bh, n, k)

    def csr_level(self, l):
        s, p = self.s, self.p
        bh, n, k = p.batch * p.heads, s.level_tokens[l], s.level_k[l]
        ptr = self.csr_ptr[s.csr_ptr_offset[l]:s.csr_ptr_offset[l] + bh * (n + 1)].view(bh, n + 1)
        col = self.csr_col[s.csr_col_offset[l]:s.csr_col_offset[l] + bh * n * k].view(bh, n * k)
        return ptr, col


def forward(B: Buffers, q, k, v, stream=None):
    """Pool, select and attend (three library calls)."""
    p = B.p
    llsa_pool(p, q, k, v, B.pyr_q, B.pyr_k, B.pyr_v, stream)
    llsa_select(p, B.pyr_q, B.pyr_k, B.idx, stream)
    llsa_attn_fwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.o, B.lse, stream)


def transpose_levels(B: Buffers, stream=None):
    """CSR of I^(l) for every level the backward pass reads (levels 1..Le+1), one call."""
    llsa_index_transpose_levels(B.p, B.idx, B.csr_ptr, B.csr_col, B.tws, B.tws_bytes, stream)


def backward(B: Buffers, q, k, v, dout, stream=None):
    p = B.p
    transpose_levels(B, stream)
    llsa_attn_bwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.csr_ptr, B.csr_col, B.o, B.lse, dout,
                  B.dq, B.dk, B.dv, B.ws, B.ws.numel(), stream)
