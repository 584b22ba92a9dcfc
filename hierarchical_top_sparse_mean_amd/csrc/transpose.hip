// Sparse index transpose ("Trainable Log-linear Sparse Attention for
// Efficient Diffusion Transformers", explainer "Step 4: Efficient Sparse
// Index Transpose"): query-major pick lists become key-major lists by a count
// per key, an exclusive prefix sum and a fill.
//
// One 1024-thread workgroup per matrix keeps the per-key counters in LDS (no
// global atomics): count with LDS atomics, exclusive scan built from
// wavefront prefix sums, then a fill of the row ids into a staging list with
// LDS fetch-add cursors.  The fill order inside a key's segment depends on
// atomic timing, so a final pass gives every entry its rank among the rows
// of its segment (rows are distinct there) and writes it to its final slot:
// the output is deterministic and rows ascend within each key.  The staging
// list lives in LDS when it fits next to the counters (the backward pass's
// matrices at 65536 tokens do), otherwise in the caller's workspace.
#include "common.hpp"
#include "internal.hpp"

namespace llsa {

constexpr int kTrThreads = 1024;
constexpr int kTrMaxCols = 32768;
constexpr int kTrLdsInts = 36864;   // 144 KB of counters + staging list

// inclusive prefix sum across a wave
__device__ __forceinline__ int wave_inclusive_scan(int v) {
    const int lane = lane_id();
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int t = __shfl_up(v, d, kWave);
        if (lane >= d) v += t;
    }
    return v;
}

// kLdsList: staging list in LDS (cols + rows*k <= kTrLdsInts), else in `stage`.
template <bool kLdsList>
__global__ __launch_bounds__(kTrThreads) void transpose_kernel(const int32_t *__restrict__ idx,
                                                              int32_t *__restrict__ ptr,
                                                              int32_t *__restrict__ col,
                                                              int32_t *__restrict__ stage, int rows,
                                                              int k, int cols) {
    __shared__ int32_t sm[kLdsList ? kTrLdsInts : kTrMaxCols];
    __shared__ int32_t wsum[kTrThreads / kWave];
    int32_t *cnt = sm;
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int64_t E = (int64_t)rows * k;
    const int32_t *I = idx + (int64_t)b * E;
    int32_t *P = ptr + (int64_t)b * (cols + 1);
    int32_t *C = col + (int64_t)b * E;
    int32_t *list = kLdsList ? sm + cols : stage + (int64_t)b * E;

    for (int c = tid; c < cols; c += kTrThreads) cnt[c] = 0;
    __syncthreads();
    // Entries are visited in chunks of kTrRegs per thread whose loads are all
    // issued before use (independent, so they overlap).
    constexpr int kTrRegs = 36;
    constexpr int64_t kChunk = (int64_t)kTrRegs * kTrThreads;
    int cv[kTrRegs];
    auto load_chunk = [&](int64_t base) {
#pragma unroll
        for (int j = 0; j < kTrRegs; ++j) {
            const int64_t e = base + tid + (int64_t)j * kTrThreads;
            cv[j] = e < E ? I[e] : -1;
        }
    };
    // count
    for (int64_t base = 0; base < E; base += kChunk) {
        load_chunk(base);
#pragma unroll
        for (int j = 0; j < kTrRegs; ++j)
            if (cv[j] >= 0) atomicAdd(&cnt[cv[j]], 1);
    }
    __syncthreads();
    // exclusive scan: each thread owns a contiguous run of counters
    const int per = (cols + kTrThreads - 1) / kTrThreads;
    const int c0 = min(cols, tid * per), c1 = min(cols, c0 + per);
    int local = 0;
    for (int c = c0; c < c1; ++c) local += cnt[c];
    const int incl = wave_inclusive_scan(local);
    if (lane_id() == kWave - 1) wsum[wave_id()] = incl;
    __syncthreads();
    int base_w = 0;
    for (int w = 0; w < wave_id(); ++w) base_w += wsum[w];
    int run = base_w + incl - local;
    for (int c = c0; c < c1; ++c) {
        const int n = cnt[c];
        cnt[c] = run;
        P[c] = run;
        run += n;
    }
    if (tid == 0) P[cols] = (int32_t)E;
    __syncthreads();
    // fill the staging list; afterwards cnt[c] is the end of key c's segment
    for (int64_t base = 0; base < E; base += kChunk) {
        load_chunk(base);
#pragma unroll
        for (int j = 0; j < kTrRegs; ++j)
            if (cv[j] >= 0) {
                const int64_t e = base + tid + (int64_t)j * kTrThreads;
                const int pos = atomicAdd(&cnt[cv[j]], 1);
                list[pos] = (int32_t)(e / k);
            }
    }
    __syncthreads();
    // rank every entry inside its segment and write it to its final slot
    for (int64_t base = 0; base < E; base += kChunk) {
        load_chunk(base);
#pragma unroll
        for (int j = 0; j < kTrRegs; ++j)
            if (cv[j] >= 0) {
                const int64_t e = base + tid + (int64_t)j * kTrThreads;
                const int c = cv[j];
                const int r = (int)(e / k);
                const int s = c == 0 ? 0 : cnt[c - 1];
                const int t = cnt[c];
                int rank = 0;
                for (int i = s; i < t; ++i) rank += (list[i] < r) ? 1 : 0;
                C[s + rank] = r;
            }
    }
}

static bool fits_lds(int rows, int k, int cols) { return (int64_t)rows * k + cols <= kTrLdsInts; }

size_t transpose_workspace_bytes(int nb, int rows, int k, int cols) {
    return fits_lds(rows, k, cols) ? 0 : sizeof(int32_t) * (size_t)nb * rows * k;
}

hipError_t launch_transpose(int nb, int rows, int k, int cols, const int32_t *idx, int32_t *ptr,
                            int32_t *col, void *ws, hipStream_t s) {
    if (fits_lds(rows, k, cols))
        hipLaunchKernelGGL(transpose_kernel<true>, dim3(nb), dim3(kTrThreads), 0, s, idx, ptr, col,
                           (int32_t *)nullptr, rows, k, cols);
    else
        hipLaunchKernelGGL(transpose_kernel<false>, dim3(nb), dim3(kTrThreads), 0, s, idx, ptr, col,
                           (int32_t *)ws, rows, k, cols);
    return hipGetLastError();
}

}  // namespace llsa
