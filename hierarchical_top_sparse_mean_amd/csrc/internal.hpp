// Host-side launchers of the gfx950 kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llsa {

constexpr int kMaxLevels = 6;

// Resolved problem geometry, computed once on the host by the C ABI layer.
struct Geometry {
    int bh;                          // batch * heads
    int N;                           // tokens
    int B;                           // block size (16 or 64)
    int sub;                         // 16-token tiles per block, B / 16
    int lgB;                         // log2(B)
    int L;                           // pooling steps
    int K;                           // requested picks
    int Le;                          // enrichment depth (coarse levels 2..Le+1)
    int n[kMaxLevels + 1];           // tokens per level, n[0] = N
    int kl[kMaxLevels + 1];          // picks per level
    int64_t pyr_off[kMaxLevels + 2]; // float offset of level l in a pyramid
    int64_t idx_off[kMaxLevels + 2]; // int32 offset of level l in the index buffer
    int64_t ptr_off[kMaxLevels + 2]; // int32 offset of level l CSR ptr
    int64_t col_off[kMaxLevels + 2]; // int32 offset of level l CSR col
    float scale;
    int drop_covered;
    bool bf16;                       // input dtype
    bool grad_bf16;                  // gradient dtype
    int order;                       // token order (0: as stored, 1: 2D patch order)
    int log2S;                       // image side for order 1
};

hipError_t launch_pool(const Geometry &g, const void *q, const void *k, const void *v,
                       float *pq, float *pk, float *pv, hipStream_t s);
// count_hist: when not null (and select_count_fusable), level 1 also counts
// its picks per key into it, one range per 128 rows (the first transpose step).
// status: when not null (debug index check), a parent pick outside its level
// sets LLSA_IDX_RANGE in it.
hipError_t launch_select(const Geometry &g, const float *pq, const float *pk, int32_t *idx,
                         int32_t *count_hist, uint32_t *status, hipStream_t s);
bool select_count_fusable(const Geometry &g);
constexpr int kSelectRowsPerRange = 128;
hipError_t launch_attn_fwd(const Geometry &g, const void *q, const void *k, const void *v,
                           const float *pk, const float *pv, const int32_t *idx, void *o,
                           float *lse, hipStream_t s);
size_t transpose_workspace_bytes(int nb, int rows, int k, int cols);
hipError_t launch_transpose(int nb, int rows, int k, int cols, const int32_t *idx,
                            int32_t *ptr, int32_t *col, void *ws, hipStream_t s);
hipError_t launch_transpose_many(int nb, int n, const int *rows, const int *k, const int *cols,
                                 const int32_t *const *idx, int32_t *const *ptr,
                                 int32_t *const *col, void *ws, hipStream_t s);
size_t transpose_counted_workspace_bytes(int nb, int rows, int k, int cols);
int32_t *transpose_counted_hist(void *ws);
hipError_t launch_transpose_counted(int nb, int rows, int k, int cols, const int32_t *idx,
                                    int32_t *ptr, int32_t *col, void *ws, hipStream_t s);
size_t transpose_mask_workspace_bytes(int nb, int rows, int cols);
hipError_t launch_transpose_mask(int nb, int rows, int k, int cols, const int32_t *idx,
                                 int32_t *ptr, int32_t *col, void *ws, hipStream_t s);
size_t bwd_workspace_bytes(const Geometry &g);
hipError_t launch_attn_bwd(const Geometry &g, const void *q, const void *k, const void *v,
                           const float *pk, const float *pv, const int32_t *idx,
                           const int32_t *csr_ptr, const int32_t *csr_col, const void *o,
                           const float *lse, const void *dout, void *dq, void *dk, void *dv,
                           void *ws, hipStream_t s);
// Debug index check: clear the status word; OR the flags of every failing pick
// row (all levels) and CSR key (levels 1..Le+1, when csr_ptr is not null) into it.
hipError_t launch_status_clear(uint32_t *status, hipStream_t s);
hipError_t launch_check_indices(const Geometry &g, const int32_t *idx, const int32_t *csr_ptr,
                                const int32_t *csr_col, uint32_t *status, hipStream_t s);
uint32_t check_indices_host(const Geometry &g, const int32_t *idx, const int32_t *csr_ptr,
                            const int32_t *csr_col);
hipError_t launch_dense_fwd(int bh, int N, float scale, const void *q, const void *k,
                            const void *v, void *o, float *lse, hipStream_t s);
hipError_t launch_dense_bwd(int bh, int N, float scale, const void *q, const void *k,
                            const void *v, const void *o, const float *lse, const void *dout,
                            float *dq, float *dk, float *dv, float *Dws, hipStream_t s);

}  // namespace llsa
