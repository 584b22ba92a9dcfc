// C ABI of the LLSA library: host-side validation, derived sizes and kernel
// launches.  Every check runs before any HIP call; nothing allocates device
// memory or synchronises (outside the debug index check).
#include <math.h>
#include <string.h>

#include <mutex>

#include "llsa.h"
#include "internal.hpp"

using llsa::Geometry;

// Scratch of llsa_attn_bwd_noalloc: the backward workspace for callers that
// cannot allocate.  Each GPU the library runs on holds its own copy until the
// process ends; in host code its device address comes from
// hipGetSymbolAddress (scratch_address below), never from the name.
static __device__ __align__(256) unsigned char scratch[LLSA_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned16(const void *p) { return p != nullptr && (((uintptr_t)p) & 15u) == 0; }
bool aligned4(const void *p);

int64_t ipow(int64_t b, int e) {
    int64_t r = 1;
    while (e-- > 0) r *= b;
    return r;
}

// Fills g from p; returns an llsa_status.
int make_geometry(const llsa_problem *p, Geometry *g, llsa_sizes *sz) {
    if (p == nullptr) return LLSA_ERR_INVALID;
    if (p->batch <= 0 || p->heads <= 0 || p->seq_len <= 0 || p->head_dim <= 0 || p->block <= 1 ||
        p->levels < 1 || p->topk < 1)
        return LLSA_ERR_INVALID;
    if (p->dtype != LLSA_F32 && p->dtype != LLSA_BF16) return LLSA_ERR_INVALID;
    if (p->grad_dtype != LLSA_F32 && p->grad_dtype != LLSA_BF16) return LLSA_ERR_INVALID;
    if (p->drop_covered != 0 && p->drop_covered != 1) return LLSA_ERR_INVALID;
    if (p->token_order != 0 && p->token_order != 1) return LLSA_ERR_INVALID;
    int log2S = 0;
    if (p->token_order == 1) {   // a square image with a power-of-two side
        while (log2S < 16 && ((int64_t)1 << (2 * log2S)) < p->seq_len) ++log2S;
        if (((int64_t)1 << (2 * log2S)) != p->seq_len) return LLSA_ERR_INVALID;
    }
    if (!(p->scale >= 0.0f) || isinf(p->scale)) return LLSA_ERR_INVALID;
    if (p->index_status != nullptr && !aligned4(p->index_status)) return LLSA_ERR_INVALID;
    if (p->levels > LLSA_MAX_LEVELS) return LLSA_ERR_UNSUPPORTED;
    // divisibility by block^levels (checked in 64 bits before anything else)
    int64_t span = 1;
    for (int l = 0; l < p->levels; ++l) {
        span *= p->block;
        if (span > p->seq_len) return LLSA_ERR_INVALID;
    }
    if (p->seq_len % span != 0) return LLSA_ERR_INVALID;
    const int L = p->levels;
    const int Le = p->enrich < 0 ? L - 1 : p->enrich;
    if (p->enrich < -1 || Le > L - 1) return LLSA_ERR_INVALID;
    if (p->head_dim != 64 || (p->block != 16 && p->block != 64)) return LLSA_ERR_UNSUPPORTED;
    if (p->topk > 32) return LLSA_ERR_UNSUPPORTED;
    // kernels address one head's rows with 32-bit byte offsets (seq_len * 128 B < 4 GiB)
    if (p->seq_len >= (1 << 25)) return LLSA_ERR_UNSUPPORTED;
    const int64_t bh = (int64_t)p->batch * p->heads;
    if (bh * p->seq_len * p->head_dim >= ((int64_t)1 << 40) || bh * p->seq_len >= ((int64_t)1 << 31) ||
        bh > (1 << 30))
        return LLSA_ERR_UNSUPPORTED;

    memset(g, 0, sizeof(*g));
    g->bh = (int)bh;
    g->N = p->seq_len;
    g->B = p->block;
    g->sub = p->block / 16;
    g->lgB = p->block == 16 ? 4 : 6;
    g->L = L;
    g->K = p->topk;
    g->Le = Le;
    g->n[0] = p->seq_len;
    for (int l = 1; l <= L; ++l) g->n[l] = (int)(p->seq_len / ipow(p->block, l));
    g->kl[L] = p->topk < g->n[L] ? p->topk : g->n[L];
    for (int l = L - 1; l >= 1; --l) {
        const int cand = g->kl[l + 1] * p->block;
        g->kl[l] = p->topk < cand ? p->topk : cand;
    }
    // every level's segment starts on a 64-byte boundary (16 floats / int32s)
    auto pad = [](int64_t x) { return (x + 15) / 16 * 16; };
    int64_t off = 0, ioff = 0, poff = 0, coff = 0;
    for (int l = 1; l <= L + 1; ++l) {
        g->pyr_off[l] = off;
        g->idx_off[l] = ioff;
        g->ptr_off[l] = poff;
        g->col_off[l] = coff;
        if (l <= L) {
            off += pad(bh * g->n[l] * 64);
            ioff += pad(bh * g->n[l] * g->kl[l]);
            if (l <= Le + 1) {
                poff += pad(bh * (g->n[l] + 1));
                coff += pad(bh * g->n[l] * g->kl[l]);
            }
        }
    }
    g->scale = p->scale > 0.0f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
    g->order = p->token_order;
    g->log2S = log2S;
    g->drop_covered = p->drop_covered;
    g->bf16 = p->dtype == LLSA_BF16;
    g->grad_bf16 = p->grad_dtype == LLSA_BF16;
    if (sz) {
        memset(sz, 0, sizeof(*sz));
        sz->levels = L;
        sz->enrich = Le;
        for (int l = 0; l <= L; ++l) {
            sz->level_tokens[l] = g->n[l];
            sz->level_k[l] = l == 0 ? 0 : g->kl[l];
        }
        for (int l = 1; l <= L + 1; ++l) {
            sz->pyramid_offset[l] = g->pyr_off[l];
            sz->index_offset[l] = g->idx_off[l];
            sz->csr_ptr_offset[l] = g->ptr_off[l];
            sz->csr_col_offset[l] = g->col_off[l];
        }
        sz->pyramid_elems = g->pyr_off[L + 1];
        sz->index_elems = g->idx_off[L + 1];
        sz->csr_ptr_elems = g->ptr_off[L + 1];
        sz->csr_col_elems = g->col_off[L + 1];
        sz->lse_elems = bh * p->seq_len;
        sz->transpose_workspace_bytes = llsa::transpose_workspace_bytes((int)bh, g->n[1], g->kl[1], g->n[1]);
        sz->bwd_workspace_bytes = llsa::bwd_workspace_bytes(*g);
    }
    return LLSA_OK;
}

int status_of(hipError_t e) { return e == hipSuccess ? LLSA_OK : LLSA_ERR_HIP; }

// Device address of the current device's scratch array, looked up once per
// device (the first llsa_attn_bwd_noalloc call with that device current).
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices];

hipError_t scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (scratch_ptr[dev] == nullptr) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || ptr == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
        scratch_ptr[dev] = ptr;
    }
    *out = scratch_ptr[dev];
    return hipSuccess;
}

bool aligned4(const void *p) { return p != nullptr && (((uintptr_t)p) & 3u) == 0; }

// Debug index check (p->index_status set): waits for the status word on the
// stream and maps it to a status.
int debug_status(const llsa_problem *p, hipStream_t s) {
    int32_t word = 0;
    if (hipMemcpyAsync(&word, p->index_status, sizeof(word), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return LLSA_ERR_HIP;
    return word == 0 ? LLSA_OK : LLSA_ERR_INDEX;
}

// Before a call that reads lists: with the debug check on, check idx (and the
// CSR when given) into the status word and return its verdict; LLSA_OK when
// the check is off.
int debug_check_inputs(const llsa_problem *p, const Geometry &g, const int32_t *idx,
                       const int32_t *csr_ptr, const int32_t *csr_col, hipStream_t s) {
    if (p->index_status == nullptr) return LLSA_OK;
    uint32_t *w = (uint32_t *)p->index_status;
    if (llsa::launch_status_clear(w, s) != hipSuccess ||
        llsa::launch_check_indices(g, idx, csr_ptr, csr_col, w, s) != hipSuccess)
        return LLSA_ERR_HIP;
    return debug_status(p, s);
}

// Workspace of llsa_select_transpose: the level transposes run one after
// another and share it; level 1 keeps the selection's counts when fused.
size_t select_transpose_ws(const Geometry &g) {
    const bool fused = llsa::select_count_fusable(g);
    size_t need = 0;
    for (int l = 1; l <= g.Le + 1; ++l) {
        const size_t b = (l == 1 && fused)
                             ? llsa::transpose_counted_workspace_bytes(g.bh, g.n[1], g.kl[1], g.n[1])
                             : llsa::transpose_workspace_bytes(g.bh, g.n[l], g.kl[l], g.n[l]);
        need = b > need ? b : need;
    }
    return need;
}

}  // namespace

extern "C" {

int llsa_sizes_query(const llsa_problem *p, llsa_sizes *out) {
    if (out == nullptr) return LLSA_ERR_INVALID;
    Geometry g;
    return make_geometry(p, &g, out);
}

int llsa_pool(const llsa_problem *p, const void *q, const void *k, const void *v, float *pyr_q,
              float *pyr_k, float *pyr_v, void *stream) {
    Geometry g;
    const int st = make_geometry(p, &g, nullptr);
    if (st != LLSA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(pyr_q) || !aligned16(pyr_k) ||
        !aligned16(pyr_v))
        return LLSA_ERR_INVALID;
    return status_of(llsa::launch_pool(g, q, k, v, pyr_q, pyr_k, pyr_v, (hipStream_t)stream));
}

int llsa_select(const llsa_problem *p, const float *pyr_q, const float *pyr_k, int32_t *idx,
                void *stream) {
    Geometry g;
    const int st = make_geometry(p, &g, nullptr);
    if (st != LLSA_OK) return st;
    if (!aligned16(pyr_q) || !aligned16(pyr_k) || !aligned16(idx)) return LLSA_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    uint32_t *dbg = (uint32_t *)p->index_status;
    if (dbg != nullptr && llsa::launch_status_clear(dbg, s) != hipSuccess) return LLSA_ERR_HIP;
    const int st2 = status_of(llsa::launch_select(g, pyr_q, pyr_k, idx, nullptr, dbg, s));
    if (st2 != LLSA_OK || dbg == nullptr) return st2;
    // debug check: the lists just written, on top of any out-of-range parent pick
    if (llsa::launch_check_indices(g, idx, nullptr, nullptr, dbg, s) != hipSuccess) return LLSA_ERR_HIP;
    return debug_status(p, s);
}

size_t llsa_select_transpose_workspace(const llsa_problem *p) {
    Geometry g;
    if (make_geometry(p, &g, nullptr) != LLSA_OK) return 0;
    return select_transpose_ws(g);
}

int llsa_select_transpose(const llsa_problem *p, const float *pyr_q, const float *pyr_k,
                          int32_t *idx, int32_t *csr_ptr, int32_t *csr_col, void *workspace,
                          size_t workspace_bytes, void *stream) {
    Geometry g;
    const int st = make_geometry(p, &g, nullptr);
    if (st != LLSA_OK) return st;
    if (g.bh > 65535 || g.n[1] > (1 << 24)) return LLSA_ERR_UNSUPPORTED;
    if (!aligned16(pyr_q) || !aligned16(pyr_k) || !aligned16(idx) || !aligned16(csr_ptr) ||
        !aligned16(csr_col))
        return LLSA_ERR_INVALID;
    const size_t need = select_transpose_ws(g);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return LLSA_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint32_t *dbg = (uint32_t *)p->index_status;
    if (dbg != nullptr && llsa::launch_status_clear(dbg, s) != hipSuccess) return LLSA_ERR_HIP;
    const bool fused = llsa::select_count_fusable(g);
    hipError_t e = llsa::launch_select(g, pyr_q, pyr_k, idx,
                                       fused ? llsa::transpose_counted_hist(workspace) : nullptr, dbg, s);
    for (int l = 1; l <= g.Le + 1 && e == hipSuccess; ++l) {
        const int32_t *il = idx + g.idx_off[l];
        int32_t *pl = csr_ptr + g.ptr_off[l], *cl = csr_col + g.col_off[l];
        e = (l == 1 && fused)
                ? llsa::launch_transpose_counted(g.bh, g.n[1], g.kl[1], g.n[1], il, pl, cl, workspace, s)
                : llsa::launch_transpose(g.bh, g.n[l], g.kl[l], g.n[l], il, pl, cl, workspace, s);
    }
    if (e != hipSuccess || dbg == nullptr) return status_of(e);
    if (llsa::launch_check_indices(g, idx, csr_ptr, csr_col, dbg, s) != hipSuccess) return LLSA_ERR_HIP;
    return debug_status(p, s);
}

size_t llsa_index_transpose_levels_workspace(const llsa_problem *p) {
    Geometry g;
    if (make_geometry(p, &g, nullptr) != LLSA_OK) return 0;
    size_t need = 0;
    for (int l = 1; l <= g.Le + 1; ++l) {
        const size_t b = llsa::transpose_workspace_bytes(g.bh, g.n[l], g.kl[l], g.n[l]);
        need = b > need ? b : need;
    }
    return need;
}

int llsa_index_transpose_levels(const llsa_problem *p, const int32_t *idx, int32_t *csr_ptr,
                                int32_t *csr_col, void *workspace, size_t workspace_bytes,
                                void *stream) {
    Geometry g;
    const int st = make_geometry(p, &g, nullptr);
    if (st != LLSA_OK) return st;
    if (g.bh > 65535 || g.n[1] > (1 << 24)) return LLSA_ERR_UNSUPPORTED;
    if (!aligned16(idx) || !aligned16(csr_ptr) || !aligned16(csr_col)) return LLSA_ERR_INVALID;
    const size_t need = llsa_index_transpose_levels_workspace(p);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)))
        return LLSA_ERR_WORKSPACE;
    const int dst = debug_check_inputs(p, g, idx, nullptr, nullptr, (hipStream_t)stream);
    if (dst != LLSA_OK) return dst;
    int rows[llsa::kMaxLevels + 1], ks[llsa::kMaxLevels + 1];
    const int32_t *il[llsa::kMaxLevels + 1];
    int32_t *pl[llsa::kMaxLevels + 1], *cl[llsa::kMaxLevels + 1];
    const int n = g.Le + 1;
    for (int i = 0; i < n; ++i) {
        const int l = i + 1;
        rows[i] = g.n[l];
        ks[i] = g.kl[l];
        il[i] = idx + g.idx_off[l];
        pl[i] = csr_ptr + g.ptr_off[l];
        cl[i] = csr_col + g.col_off[l];
    }
    return status_of(llsa::launch_transpose_many(g.bh, n, rows, ks, rows, il, pl, cl, workspace,
                                                 (hipStream_t)stream));
}

int llsa_attn_fwd(const llsa_problem *p, const void *q, const void *k, const void *v,
                  const float *pyr_k, const float *pyr_v, const int32_t *idx, void *o, float *lse,
                  void *stream) {
    Geometry g;
    const int st = make_geometry(p, &g, nullptr);
    if (st != LLSA_OK) return st;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(pyr_k) || !aligned16(pyr_v) ||
        !aligned16(idx) || !aligned16(o) || !aligned16(lse))
        return LLSA_ERR_INVALID;
    const int dst = debug_check_inputs(p, g, idx, nullptr, nullptr, (hipStream_t)stream);
    if (dst != LLSA_OK) return dst;
    return status_of(llsa::launch_attn_fwd(g, q, k, v, pyr_k, pyr_v, idx, o, lse, (hipStream_t)stream));
}

size_t llsa_index_transpose_workspace(int32_t n_batch, int32_t n_rows, int32_t k, int32_t n_cols) {
    return llsa::transpose_workspace_bytes(n_batch, n_rows, k, n_cols);
}

int llsa_index_transpose(int32_t n_batch, int32_t n_rows, int32_t k, int32_t n_cols,
                         const int32_t *idx, int32_t *csr_ptr, int32_t *csr_col, void *workspace,
                         size_t workspace_bytes, void *stream) {
    if (n_batch <= 0 || n_rows <= 0 || k <= 0 || n_cols <= 0) return LLSA_ERR_INVALID;
    if ((int64_t)n_rows * k >= ((int64_t)1 << 31) / n_batch) return LLSA_ERR_UNSUPPORTED;
    if (n_cols > (1 << 24) || n_batch > 65535) return LLSA_ERR_UNSUPPORTED;
    if (!aligned16(idx) || !aligned16(csr_ptr) || !aligned16(csr_col)) return LLSA_ERR_INVALID;
    const size_t need = llsa::transpose_workspace_bytes(n_batch, n_rows, k, n_cols);
    if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return LLSA_ERR_WORKSPACE;
    return status_of(llsa::launch_transpose(n_batch, n_rows, k, n_cols, idx, csr_ptr, csr_col,
                                            workspace, (hipStream_t)stream));
}

size_t llsa_index_transpose_mask_workspace(int32_t n_batch, int32_t n_rows, int32_t n_cols) {
    if (n_batch <= 0 || n_rows <= 0 || n_cols <= 0) return 0;
    return llsa::transpose_mask_workspace_bytes(n_batch, n_rows, n_cols);
}

int llsa_index_transpose_mask(int32_t n_batch, int32_t n_rows, int32_t k, int32_t n_cols,
                              const int32_t *idx, int32_t *csr_ptr, int32_t *csr_col,
                              void *workspace, size_t workspace_bytes, void *stream) {
    if (n_batch <= 0 || n_rows <= 0 || k <= 0 || n_cols <= 0) return LLSA_ERR_INVALID;
    if ((int64_t)n_rows * k >= ((int64_t)1 << 31) / n_batch) return LLSA_ERR_UNSUPPORTED;
    if ((int64_t)n_batch * n_cols >= ((int64_t)1 << 31) || n_cols > (1 << 24)) return LLSA_ERR_UNSUPPORTED;
    if (!aligned16(idx) || !aligned16(csr_ptr) || !aligned16(csr_col)) return LLSA_ERR_INVALID;
    const size_t need = llsa::transpose_mask_workspace_bytes(n_batch, n_rows, n_cols);
    if (workspace == nullptr || workspace_bytes < need) return LLSA_ERR_WORKSPACE;
    return status_of(llsa::launch_transpose_mask(n_batch, n_rows, k, n_cols, idx, csr_ptr, csr_col,
                                                 workspace, (hipStream_t)stream));
}

// Checks of llsa_attn_bwd and llsa_attn_bwd_noalloc that precede the
// workspace: shapes, the coarse-entry limit and pointer alignment.
int bwd_args_status(const llsa_problem *p, Geometry *g, const void *q, const void *k, const void *v,
                    const float *pyr_k, const float *pyr_v, const int32_t *idx,
                    const int32_t *csr_ptr, const int32_t *csr_col, const void *o, const float *lse,
                    const void *dout, void *dq, void *dk, void *dv) {
    const int st = make_geometry(p, g, nullptr);
    if (st != LLSA_OK) return st;
    int ncoarse = 0;
    for (int l = 2; l <= g->Le + 1; ++l) ncoarse += g->kl[l];
    if (ncoarse > 32) return LLSA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(pyr_k) || !aligned16(pyr_v) ||
        !aligned16(idx) || !aligned16(csr_ptr) || !aligned16(csr_col) || !aligned16(o) ||
        !aligned16(lse) || !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return LLSA_ERR_INVALID;
    return LLSA_OK;
}

int llsa_attn_bwd(const llsa_problem *p, const void *q, const void *k, const void *v,
                  const float *pyr_k, const float *pyr_v, const int32_t *idx,
                  const int32_t *csr_ptr, const int32_t *csr_col, const void *o, const float *lse,
                  const void *dout, void *dq, void *dk, void *dv, void *workspace,
                  size_t workspace_bytes, void *stream) {
    Geometry g;
    const int st = bwd_args_status(p, &g, q, k, v, pyr_k, pyr_v, idx, csr_ptr, csr_col, o, lse, dout,
                                   dq, dk, dv);
    if (st != LLSA_OK) return st;
    const size_t need = llsa::bwd_workspace_bytes(g);
    if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return LLSA_ERR_WORKSPACE;
    const int dst = debug_check_inputs(p, g, idx, csr_ptr, csr_col, (hipStream_t)stream);
    if (dst != LLSA_OK) return dst;
    return status_of(llsa::launch_attn_bwd(g, q, k, v, pyr_k, pyr_v, idx, csr_ptr, csr_col, o, lse,
                                           dout, dq, dk, dv, workspace, (hipStream_t)stream));
}

int llsa_attn_bwd_noalloc(const llsa_problem *p, const void *q, const void *k, const void *v,
                          const float *pyr_k, const float *pyr_v, const int32_t *idx,
                          const int32_t *csr_ptr, const int32_t *csr_col, const void *o,
                          const float *lse, const void *dout, void *dq, void *dk, void *dv,
                          void *stream) {
    Geometry g;
    const int st = bwd_args_status(p, &g, q, k, v, pyr_k, pyr_v, idx, csr_ptr, csr_col, o, lse, dout,
                                   dq, dk, dv);
    if (st != LLSA_OK) return st;
    if (llsa::bwd_workspace_bytes(g) > (size_t)LLSA_NOALLOC_SCRATCH_BYTES) return LLSA_ERR_SCRATCH;
    void *ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return LLSA_ERR_HIP;
    const int dst = debug_check_inputs(p, g, idx, csr_ptr, csr_col, (hipStream_t)stream);
    if (dst != LLSA_OK) return dst;
    return status_of(llsa::launch_attn_bwd(g, q, k, v, pyr_k, pyr_v, idx, csr_ptr, csr_col, o, lse,
                                           dout, dq, dk, dv, ws, (hipStream_t)stream));
}

int llsa_dense_attn_fwd(const llsa_problem *p, const void *q, const void *k, const void *v,
                        void *o, float *lse, void *stream) {
    if (p == nullptr) return LLSA_ERR_INVALID;
    if (p->batch <= 0 || p->heads <= 0 || p->seq_len <= 0 || p->head_dim <= 0) return LLSA_ERR_INVALID;
    if (!(p->scale >= 0.0f) || isinf(p->scale)) return LLSA_ERR_INVALID;
    if (p->head_dim != 64 || p->dtype != LLSA_BF16 || p->seq_len % 16 != 0) return LLSA_ERR_UNSUPPORTED;
    const int64_t bh = (int64_t)p->batch * p->heads;
    if (bh * p->seq_len >= ((int64_t)1 << 31)) return LLSA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return LLSA_ERR_INVALID;
    const float scale = p->scale > 0.0f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
    return status_of(llsa::launch_dense_fwd((int)bh, p->seq_len, scale, q, k, v, o, lse, (hipStream_t)stream));
}

int llsa_dense_attn_bwd(const llsa_problem *p, const void *q, const void *k, const void *v,
                        const void *o, const float *lse, const void *dout, float *dq, float *dk,
                        float *dv, void *workspace, size_t workspace_bytes, void *stream) {
    if (p == nullptr) return LLSA_ERR_INVALID;
    if (p->batch <= 0 || p->heads <= 0 || p->seq_len <= 0 || p->head_dim <= 0) return LLSA_ERR_INVALID;
    if (!(p->scale >= 0.0f) || isinf(p->scale)) return LLSA_ERR_INVALID;
    if (p->head_dim != 64 || p->dtype != LLSA_BF16 || p->seq_len % 16 != 0) return LLSA_ERR_UNSUPPORTED;
    const int64_t bh = (int64_t)p->batch * p->heads;
    if (bh * p->seq_len >= ((int64_t)1 << 31)) return LLSA_ERR_UNSUPPORTED;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
        !aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
        return LLSA_ERR_INVALID;
    if (workspace == nullptr || workspace_bytes < llsa_dense_attn_bwd_workspace(p))
        return LLSA_ERR_WORKSPACE;
    const float scale = p->scale > 0.0f ? p->scale : 1.0f / sqrtf((float)p->head_dim);
    return status_of(llsa::launch_dense_bwd((int)bh, p->seq_len, scale, q, k, v, o, lse, dout, dq,
                                            dk, dv, (float *)workspace, (hipStream_t)stream));
}

size_t llsa_dense_attn_bwd_workspace(const llsa_problem *p) {
    if (p == nullptr || p->batch <= 0 || p->heads <= 0 || p->seq_len <= 0) return 0;
    return sizeof(float) * (size_t)p->batch * p->heads * p->seq_len;
}

int llsa_check_indices(const llsa_problem *p, const int32_t *idx, const int32_t *csr_ptr,
                       const int32_t *csr_col, int32_t *status, void *stream) {
    Geometry g;
    const int st = make_geometry(p, &g, nullptr);
    if (st != LLSA_OK) return st;
    if (!aligned16(idx) || !aligned4(status)) return LLSA_ERR_INVALID;
    const bool csr = csr_ptr != nullptr && csr_col != nullptr;
    if (csr && (!aligned16(csr_ptr) || !aligned16(csr_col))) return LLSA_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    if (llsa::launch_status_clear((uint32_t *)status, s) != hipSuccess) return LLSA_ERR_HIP;
    return status_of(llsa::launch_check_indices(g, idx, csr ? csr_ptr : nullptr, csr ? csr_col : nullptr,
                                                (uint32_t *)status, s));
}

int llsa_check_indices_host(const llsa_problem *p, const int32_t *idx, const int32_t *csr_ptr,
                            const int32_t *csr_col, int32_t *flags) {
    Geometry g;
    const int st = make_geometry(p, &g, nullptr);
    if (st != LLSA_OK) return st;
    if (idx == nullptr || flags == nullptr) return LLSA_ERR_INVALID;
    const bool csr = csr_ptr != nullptr && csr_col != nullptr;
    *flags = (int32_t)llsa::check_indices_host(g, idx, csr ? csr_ptr : nullptr, csr ? csr_col : nullptr);
    return LLSA_OK;
}

const char *llsa_strerror(int status) {
    switch (status) {
    case LLSA_OK: return "ok";
    case LLSA_ERR_INVALID: return "invalid argument";
    case LLSA_ERR_UNSUPPORTED: return "unsupported problem";
    case LLSA_ERR_WORKSPACE: return "workspace missing or too small";
    case LLSA_ERR_HIP: return "kernel launch failed";
    case LLSA_ERR_INDEX: return "invalid index list or CSR (debug index check)";
    case LLSA_ERR_SCRATCH: return "problem needs more than the allocation-free call's static scratch";
    default: return "unknown status";
    }
}

}  // extern "C"
