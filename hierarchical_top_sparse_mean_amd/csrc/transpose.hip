// Sparse index transpose ("Trainable Log-linear Sparse Attention for
// Efficient Diffusion Transformers", explainer "Step 4: Efficient Sparse
// Index Transpose"): query-major pick lists become key-major lists by a count
// per key, an exclusive prefix sum and a fill.
//
// Four short kernels spread every matrix over many workgroups; none uses a
// global atomic and none needs memory cleared beforehand:
//  1 count  each workgroup counts the picks of a contiguous range of rows in
//           an LDS histogram and writes the whole histogram out;
//  2 prefix key by key (one thread per key), the histograms of the row ranges
//           become each range's offset inside the key's run, and the key's
//           total is kept;
//  3 scan   per matrix, the exclusive prefix of the key totals: csr_ptr;
//  4 fill   one wave per row range walks its picks in order, 64 at a time:
//           every pick sets its lane's bit in an LDS mask of its key, so its
//           rank among the chunk's picks of that key is a popcount, and the
//           rows land in ascending order at csr_ptr plus the range's offset.
// Keys are handled in windows of kTrWindow, each window by its own
// workgroups (the LDS holds one window's counters), so any number of keys
// takes the same path.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace llsa {

constexpr int kTrThreads = 256;
constexpr int kTrWindow = 4096;    // keys per LDS window of the count and fill
constexpr int kTrChunk = 1024;     // picks per row range (workgroup) of the count and fill
constexpr int kTrMaxRanges = 64;
struct TrPlan {
    int ranges;          // row ranges per matrix
    int rows_per;        // rows per range
    int windows;         // key windows per matrix
    size_t hist_ints;    // nb * ranges * cols
    size_t tot_ints;     // nb * cols
};

static TrPlan plan(int nb, int rows, int k, int cols) {
    TrPlan p;
    const int64_t picks = (int64_t)rows * k;
    const int64_t want = (picks + kTrChunk - 1) / kTrChunk;
    p.ranges = (int)(want < 1 ? 1 : (want > kTrMaxRanges ? kTrMaxRanges : want));
    p.rows_per = (rows + p.ranges - 1) / p.ranges;
    p.windows = (cols + kTrWindow - 1) / kTrWindow;
    p.hist_ints = (size_t)nb * p.ranges * cols;
    p.tot_ints = (size_t)nb * cols;
    return p;
}

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

size_t transpose_workspace_bytes(int nb, int rows, int k, int cols) {
    const TrPlan p = plan(nb, rows, k, cols);
    return align256(sizeof(int32_t) * p.hist_ints) + align256(sizeof(int32_t) * p.tot_ints);
}

// 1: histogram of the picks of rows [r0, r1) of matrix b, keys of window
// blockIdx.z.
__global__ __launch_bounds__(kTrThreads) void tr_count_kernel(const int32_t *__restrict__ idx,
                                                             int32_t *__restrict__ hist, int rows,
                                                             int k, int cols, int ranges,
                                                             int rows_per) {
    __shared__ int32_t h[kTrWindow];
    const int m = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int c0 = blockIdx.z * kTrWindow, wn = min(kTrWindow, cols - c0);
    const int r0 = min(rows, m * rows_per), r1 = min(rows, r0 + rows_per);
    const int32_t *I = idx + (int64_t)b * rows * k;
    for (int c = tid; c < wn; c += kTrThreads) h[c] = 0;
    __syncthreads();
    const int64_t e1 = (int64_t)r1 * k;
    for (int64_t e = (int64_t)r0 * k + tid; e < e1; e += kTrThreads) {
        const int c = I[e] - c0;
        if (c >= 0 && c < wn) atomicAdd(&h[c], 1);
    }
    __syncthreads();
    int32_t *H = hist + ((int64_t)b * ranges + m) * cols + c0;
    for (int c = tid; c < wn; c += kTrThreads) H[c] = h[c];
}

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

// 2: one thread per key c of matrix b: hist[b][m][c] becomes the number of
// picks of c in ranges before m, tot[b][c] the key's total.
__global__ __launch_bounds__(kTrThreads) void tr_prefix_kernel(int32_t *__restrict__ hist,
                                                              int32_t *__restrict__ tot, int cols,
                                                              int ranges) {
    const int b = blockIdx.y;
    const int c = blockIdx.x * kTrThreads + threadIdx.x;
    if (c >= cols) return;
    int32_t *H = hist + (int64_t)b * ranges * cols + c;
    int run = 0;
#pragma unroll 8
    for (int m = 0; m < ranges; ++m) {
        const int x = H[(int64_t)m * cols];
        H[(int64_t)m * cols] = run;
        run += x;
    }
    tot[(int64_t)b * cols + c] = run;
}

// 3: per matrix b, ptr[b][c] = number of picks of keys < c.
constexpr int kTrScanThreads = 1024;
__global__ __launch_bounds__(kTrScanThreads) void tr_scan_kernel(const int32_t *__restrict__ tot,
                                                                int32_t *__restrict__ ptr,
                                                                int cols) {
    __shared__ int32_t wsum[kTrScanThreads / kWave];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int32_t *T = tot + (int64_t)b * cols;
    // each thread owns a contiguous run of keys
    const int per = (cols + kTrScanThreads - 1) / kTrScanThreads;
    const int c0 = min(cols, tid * per), c1 = min(cols, c0 + per);
    int local = 0;
    for (int c = c0; c < c1; ++c) local += T[c];
    const int incl = wave_inclusive_scan(local);
    if (lane_id() == kWave - 1) wsum[wave_id()] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wave_id(); ++w) run += wsum[w];
    int32_t *P = ptr + (int64_t)b * (cols + 1);
    for (int c = c0; c < c1; ++c) {
        P[c] = run;
        run += T[c];
    }
    if (tid == kTrScanThreads - 1) P[cols] = run;   // the last thread owns the last keys
}

// 4: one wave per (row range, key window), picks in order, 64 at a time.
// The pick of lane l with key c sets bit l of mask[c]; its rank among the
// chunk's picks of c is the number of lower bits set, and the highest lane of
// each key advances the key's count seen so far (seen[c]) by the popcount.
// A pick lands at csr_ptr[c] + the range's offset for c + seen[c] + rank; the
// two global terms are read per pick, one chunk ahead.
__global__ __launch_bounds__(kWave) void tr_fill_ordered_kernel(const int32_t *__restrict__ idx,
                                                               const int32_t *__restrict__ hist,
                                                               const int32_t *__restrict__ ptr,
                                                               int32_t *__restrict__ col, int rows,
                                                               int k, int cols, int ranges,
                                                               int rows_per) {
    __shared__ int32_t seen[kTrWindow];
    __shared__ uint64_t mask[kTrWindow];
    const int m = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int c0 = blockIdx.z * kTrWindow, wn = min(kTrWindow, cols - c0);
    const int32_t *H = hist + ((int64_t)b * ranges + m) * cols;
    const int32_t *P = ptr + (int64_t)b * (cols + 1);
    for (int c = lane; c < wn; c += kWave) {
        seen[c] = 0;
        mask[c] = 0;
    }
    const int r0 = min(rows, m * rows_per), r1 = min(rows, r0 + rows_per);
    const int32_t *I = idx + (int64_t)b * rows * k;
    int32_t *C = col + (int64_t)b * rows * k;
    const int64_t e1 = (int64_t)r1 * k;
    int64_t e = (int64_t)r0 * k + lane;
    // key of pick x, or -1 outside the window (or out of range)
    auto key_at = [&](int64_t x) {
        const int c = x < e1 ? I[x] : -1;
        return (c >= c0 && c < c0 + wn) ? c : -1;
    };
    int cn = key_at(e);
    int bn = cn >= 0 ? P[cn] + H[cn] : 0;
    __syncthreads();
    for (; e - lane < e1; e += kWave) {
        const int c = cn, base = bn;
        cn = key_at(e + kWave);
        bn = cn >= 0 ? P[cn] + H[cn] : 0;
        const bool ok = c >= 0;
        const int cl = ok ? c - c0 : 0;
        if (ok) atomicOr((unsigned long long *)&mask[cl], 1ull << lane);
        __syncthreads();
        const uint64_t mk = ok ? mask[cl] : 0ull;
        const int rank = __popcll(mk & ((1ull << lane) - 1ull));
        if (ok) C[base + seen[cl] + rank] = (int32_t)(e / k);
        __syncthreads();
        if (ok && (mk >> lane) == 1ull) {   // highest lane of its key in the chunk
            seen[cl] += __popcll(mk);
            mask[cl] = 0ull;
        }
        __syncthreads();
    }
}

hipError_t launch_transpose(int nb, int rows, int k, int cols, const int32_t *idx, int32_t *ptr,
                            int32_t *col, void *ws, hipStream_t s) {
    const TrPlan p = plan(nb, rows, k, cols);
    int32_t *hist = (int32_t *)ws;
    int32_t *tot = (int32_t *)((char *)hist + align256(sizeof(int32_t) * p.hist_ints));
    const dim3 grid((unsigned)p.ranges, (unsigned)nb, (unsigned)p.windows);
    hipLaunchKernelGGL(tr_count_kernel, grid, dim3(kTrThreads), 0, s, idx, hist, rows, k, cols,
                       p.ranges, p.rows_per);
    const dim3 pgrid((unsigned)((cols + kTrThreads - 1) / kTrThreads), (unsigned)nb);
    hipLaunchKernelGGL(tr_prefix_kernel, pgrid, dim3(kTrThreads), 0, s, hist, tot, cols, p.ranges);
    hipLaunchKernelGGL(tr_scan_kernel, dim3((unsigned)nb), dim3(kTrScanThreads), 0, s, tot, ptr,
                       cols);
    hipLaunchKernelGGL(tr_fill_ordered_kernel, grid, dim3(kWave), 0, s, idx, hist, ptr, col, rows, k,
                       cols, p.ranges, p.rows_per);
    return hipGetLastError();
}

// ------------------------------------------------------------ mask baseline
// The same key-major lists built the way the pages contrast the transpose
// with: a dense bit mask of n_rows x n_cols per matrix, stored key-major
// (mask[b][c] holds the n_rows bits of key c), then read back column by
// column.  Its memory and time grow with n_rows * n_cols, quadratically in
// the sequence length; it exists to measure that against the transpose.
__global__ __launch_bounds__(256) void trm_clear_kernel(uint32_t *__restrict__ mask,
                                                       int64_t words) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < words; i += stride) mask[i] = 0u;
}

__global__ __launch_bounds__(256) void trm_set_kernel(const int32_t *__restrict__ idx,
                                                     uint32_t *__restrict__ mask, int nb, int rows,
                                                     int k, int cols, int wpc) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t E = (int64_t)rows * k;
    if (e >= (int64_t)nb * E) return;
    const int b = (int)(e / E);
    const int r = (int)((e % E) / k);
    const int c = idx[e];
    if (c < 0 || c >= cols) return;
    atomicOr(&mask[((int64_t)b * cols + c) * wpc + (r >> 5)], 1u << (r & 31));
}

// one wave per key: the popcount of its column -> tot
__global__ __launch_bounds__(256) void trm_count_kernel(const uint32_t *__restrict__ mask,
                                                       int32_t *__restrict__ tot, int64_t keys,
                                                       int wpc) {
    const int64_t key = (int64_t)blockIdx.x * 4 + wave_id();
    if (key >= keys) return;
    const uint32_t *m = mask + key * wpc;
    int n = 0;
    for (int w = lane_id(); w < wpc; w += kWave) n += __popc(m[w]);
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) n += __shfl_xor(n, d, kWave);
    if (lane_id() == 0) tot[key] = n;
}

// one wave per key: rows of its column in ascending order at ptr[c] onwards
__global__ __launch_bounds__(256) void trm_fill_kernel(const uint32_t *__restrict__ mask,
                                                      const int32_t *__restrict__ ptr,
                                                      int32_t *__restrict__ col, int nb, int rows,
                                                      int k, int cols, int wpc) {
    const int64_t key = (int64_t)blockIdx.x * 4 + wave_id();
    if (key >= (int64_t)nb * cols) return;
    const int b = (int)(key / cols), c = (int)(key % cols);
    const int lane = lane_id();
    const uint32_t *m = mask + key * wpc;
    int32_t *C = col + (int64_t)b * rows * k;
    int pos = __builtin_amdgcn_readfirstlane(ptr[(int64_t)b * (cols + 1) + c]);
    for (int w0 = 0; w0 < wpc; w0 += kWave) {
        const uint32_t bits = w0 + lane < wpc ? m[w0 + lane] : 0u;
        const int n = __popc(bits);
        // exclusive prefix of the popcounts across the wave
        int incl = n;
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const int t = __shfl_up(incl, d, kWave);
            if (lane >= d) incl += t;
        }
        int out = pos + incl - n;
        uint32_t rest = bits;
        while (rest) {
            const int bit = __builtin_ctz(rest);
            C[out++] = (w0 + lane) * 32 + bit;
            rest &= rest - 1u;
        }
        pos += __builtin_amdgcn_readlane(incl, kWave - 1);
    }
}

size_t transpose_mask_workspace_bytes(int nb, int rows, int cols) {
    const int wpc = (rows + 31) / 32;
    return align256(sizeof(uint32_t) * (size_t)nb * cols * wpc) +
           align256(sizeof(int32_t) * (size_t)nb * cols);
}

hipError_t launch_transpose_mask(int nb, int rows, int k, int cols, const int32_t *idx,
                                 int32_t *ptr, int32_t *col, void *ws, hipStream_t s) {
    const int wpc = (rows + 31) / 32;
    const int64_t words = (int64_t)nb * cols * wpc;
    uint32_t *mask = (uint32_t *)ws;
    int32_t *tot = (int32_t *)((char *)ws + align256(sizeof(uint32_t) * (size_t)words));
    const int64_t keys = (int64_t)nb * cols;
    const int64_t picks = (int64_t)nb * rows * k;
    const unsigned cgrid = (unsigned)std::min<int64_t>((words + 255) / 256, 65536);
    hipLaunchKernelGGL(trm_clear_kernel, dim3(cgrid), dim3(256), 0, s, mask, words);
    const dim3 kgrid((unsigned)((keys + 3) / 4));
    hipLaunchKernelGGL(trm_set_kernel, dim3((unsigned)((picks + 255) / 256)), dim3(256), 0, s, idx,
                       mask, nb, rows, k, cols, wpc);
    hipLaunchKernelGGL(trm_count_kernel, kgrid, dim3(256), 0, s, mask, tot, keys, wpc);
    hipLaunchKernelGGL(tr_scan_kernel, dim3((unsigned)nb), dim3(kTrScanThreads), 0, s, tot, ptr,
                       cols);
    hipLaunchKernelGGL(trm_fill_kernel, kgrid, dim3(256), 0, s, mask, ptr, col, nb, rows, k, cols,
                       wpc);
    return hipGetLastError();
}

}  // namespace llsa
