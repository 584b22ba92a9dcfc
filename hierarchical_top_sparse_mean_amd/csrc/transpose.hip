// Sparse index transpose ("Trainable Log-linear Sparse Attention for
// Efficient Diffusion Transformers", explainer "Step 4: Efficient Sparse
// Index Transpose"): query-major pick lists become key-major lists by a count
// per key, an exclusive prefix sum and a fill.
//
// One 1024-thread workgroup per matrix keeps the per-key counters in LDS
// (no global atomics, no workspace): count with LDS atomics, exclusive scan
// built from wavefront prefix sums, fill with LDS fetch-add cursors, then sort
// every key's segment by row so the result does not depend on the order in
// which the fill atomics were served.
#include "common.hpp"
#include "internal.hpp"

namespace llsa {

constexpr int kTrThreads = 1024;
constexpr int kTrMaxCols = 32768;

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

__global__ __launch_bounds__(kTrThreads) void transpose_kernel(const int32_t *__restrict__ idx,
                                                              int32_t *__restrict__ ptr,
                                                              int32_t *__restrict__ col, int rows,
                                                              int k, int cols) {
    __shared__ int32_t cnt[kTrMaxCols];
    __shared__ int32_t wsum[kTrThreads / kWave];
    const int tid = threadIdx.x;
    const int b = blockIdx.x;
    const int64_t E = (int64_t)rows * k;
    const int32_t *I = idx + (int64_t)b * E;
    int32_t *P = ptr + (int64_t)b * (cols + 1);
    int32_t *C = col + (int64_t)b * E;

    for (int c = tid; c < cols; c += kTrThreads) cnt[c] = 0;
    __syncthreads();
    // count
    for (int64_t e = tid; e < E; e += kTrThreads) atomicAdd(&cnt[I[e]], 1);
    __syncthreads();
    // exclusive scan: each thread owns a contiguous run of counters
    const int per = (cols + kTrThreads - 1) / kTrThreads;
    const int c0 = min(cols, tid * per), c1 = min(cols, c0 + per);
    int local = 0;
    for (int c = c0; c < c1; ++c) local += cnt[c];
    const int incl = wave_inclusive_scan(local);
    if (lane_id() == kWave - 1) wsum[wave_id()] = incl;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave_id(); ++w) base += wsum[w];
    int run = base + incl - local;
    for (int c = c0; c < c1; ++c) {
        const int n = cnt[c];
        cnt[c] = run;
        P[c] = run;
        run += n;
    }
    if (tid == 0) P[cols] = (int32_t)E;
    __syncthreads();
    // fill: cnt[c] is the next free slot of key c
    for (int64_t e = tid; e < E; e += kTrThreads) {
        const int c = I[e];
        const int pos = atomicAdd(&cnt[c], 1);
        C[pos] = (int32_t)(e / k);
    }
    __syncthreads();
    // make every segment ascending (insertion sort; segments are short)
    for (int c = tid; c < cols; c += kTrThreads) {
        const int s = P[c], t = cnt[c];
        for (int i = s + 1; i < t; ++i) {
            const int x = C[i];
            int j = i - 1;
            while (j >= s && C[j] > x) {
                C[j + 1] = C[j];
                --j;
            }
            C[j + 1] = x;
        }
    }
}

size_t transpose_workspace_bytes(int, int, int, int) { return 0; }

hipError_t launch_transpose(int nb, int rows, int k, int cols, const int32_t *idx, int32_t *ptr,
                            int32_t *col, void *, hipStream_t s) {
    hipLaunchKernelGGL(transpose_kernel, dim3(nb), dim3(kTrThreads), 0, s, idx, ptr, col, rows, k,
                       cols);
    return hipGetLastError();
}

}  // namespace llsa
