// Sparse index transpose ("Trainable Log-linear Sparse Attention for
// Efficient Diffusion Transformers", explainer "Step 4: Efficient Sparse
// Index Transpose"): query-major pick lists become key-major lists by a count
// per key, an exclusive prefix sum and a fill.
//
// Short kernels spread every matrix over many workgroups; none uses a global
// atomic and none needs memory cleared beforehand:
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
// With more than 4096 keys the masks do not fit in LDS; the fill then places
// rows with LDS fetch-add cursors into a staging copy, and a fifth kernel
// sorts every key's run by rank (an entry counts the entries that must
// precede it), one wave per key.  Both paths are deterministic.
#include "common.hpp"
#include "internal.hpp"

namespace llsa {

constexpr int kTrThreads = 256;
constexpr int kTrMaxCols = 32768;  // keys per matrix (LDS histogram of 128 KB)
constexpr int kTrChunk = 1024;     // picks per row range (workgroup) of the count and fill
constexpr int kTrMaxRanges = 64;
struct TrPlan {
    int ranges;          // row ranges per matrix
    int rows_per;        // rows per range
    size_t hist_ints;    // nb * ranges * cols
    size_t tot_ints;     // nb * cols
    size_t stage_ints;   // nb * rows * k
};

static TrPlan plan(int nb, int rows, int k, int cols) {
    TrPlan p;
    const int64_t picks = (int64_t)rows * k;
    const int64_t want = (picks + kTrChunk - 1) / kTrChunk;
    p.ranges = (int)(want < 1 ? 1 : (want > kTrMaxRanges ? kTrMaxRanges : want));
    p.rows_per = (rows + p.ranges - 1) / p.ranges;
    p.hist_ints = (size_t)nb * p.ranges * cols;
    p.tot_ints = (size_t)nb * cols;
    p.stage_ints = (size_t)nb * rows * k;
    return p;
}

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

size_t transpose_workspace_bytes(int nb, int rows, int k, int cols) {
    const TrPlan p = plan(nb, rows, k, cols);
    return align256(sizeof(int32_t) * p.hist_ints) + align256(sizeof(int32_t) * p.tot_ints) +
           align256(sizeof(int32_t) * p.stage_ints);
}

// 1: histogram of the picks of rows [r0, r1) of matrix b.
template <int CMAX>
__global__ __launch_bounds__(kTrThreads) void tr_count_kernel(const int32_t *__restrict__ idx,
                                                             int32_t *__restrict__ hist, int rows,
                                                             int k, int cols, int ranges,
                                                             int rows_per) {
    __shared__ int32_t h[CMAX];
    const int m = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int r0 = min(rows, m * rows_per), r1 = min(rows, r0 + rows_per);
    const int32_t *I = idx + (int64_t)b * rows * k;
    for (int c = tid; c < cols; c += kTrThreads) h[c] = 0;
    __syncthreads();
    const int64_t e1 = (int64_t)r1 * k;
    for (int64_t e = (int64_t)r0 * k + tid; e < e1; e += kTrThreads) {
        const int c = I[e];
        if (c >= 0 && c < cols) atomicAdd(&h[c], 1);
    }
    __syncthreads();
    int32_t *H = hist + ((int64_t)b * ranges + m) * cols;
    for (int c = tid; c < cols; c += kTrThreads) H[c] = h[c];
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
                                                                int32_t *__restrict__ ptr, int cols) {
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

// 4: rows [r0, r1) of matrix b go to their keys' runs, in arrival order.
template <int CMAX>
__global__ __launch_bounds__(kTrThreads) void tr_fill_kernel(const int32_t *__restrict__ idx,
                                                            const int32_t *__restrict__ hist,
                                                            const int32_t *__restrict__ ptr,
                                                            int32_t *__restrict__ stage, int rows,
                                                            int k, int cols, int ranges,
                                                            int rows_per) {
    __shared__ int32_t cur[CMAX];
    const int m = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int32_t *H = hist + ((int64_t)b * ranges + m) * cols;
    const int32_t *P = ptr + (int64_t)b * (cols + 1);
    for (int c = tid; c < cols; c += kTrThreads) cur[c] = P[c] + H[c];
    __syncthreads();
    const int r0 = min(rows, m * rows_per), r1 = min(rows, r0 + rows_per);
    const int32_t *I = idx + (int64_t)b * rows * k;
    int32_t *S = stage + (int64_t)b * rows * k;
    const int64_t e1 = (int64_t)r1 * k;
    for (int64_t e = (int64_t)r0 * k + tid; e < e1; e += kTrThreads) {
        const int c = I[e];
        if (c >= 0 && c < cols) S[atomicAdd(&cur[c], 1)] = (int32_t)(e / k);
    }
}

// 4, up to 4096 keys: one wave per row range, picks in order, 64 at a time.
// The pick of lane l with key c sets bit l of mask[c]; its rank among the
// chunk's picks of c is the number of lower bits set, and the highest lane of
// each key advances the key's count seen so far (seen[c]) by the popcount.
// A pick lands at csr_ptr[c] + the range's offset for c + seen[c] + rank; the
// two global terms are read per pick, one chunk ahead.
constexpr int kTrMaskCols = 4096;
__global__ __launch_bounds__(kWave) void tr_fill_ordered_kernel(const int32_t *__restrict__ idx,
                                                               const int32_t *__restrict__ hist,
                                                               const int32_t *__restrict__ ptr,
                                                               int32_t *__restrict__ col, int rows,
                                                               int k, int cols, int ranges,
                                                               int rows_per) {
    __shared__ int32_t seen[kTrMaskCols];
    __shared__ uint64_t mask[kTrMaskCols];
    const int m = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int32_t *H = hist + ((int64_t)b * ranges + m) * cols;
    const int32_t *P = ptr + (int64_t)b * (cols + 1);
    for (int c = lane; c < cols; c += kWave) {
        seen[c] = 0;
        mask[c] = 0;
    }
    const int r0 = min(rows, m * rows_per), r1 = min(rows, r0 + rows_per);
    const int32_t *I = idx + (int64_t)b * rows * k;
    int32_t *C = col + (int64_t)b * rows * k;
    const int64_t e1 = (int64_t)r1 * k;
    int64_t e = (int64_t)r0 * k + lane;
    auto key_at = [&](int64_t x) {
        const int c = x < e1 ? I[x] : -1;
        return (c >= 0 && c < cols) ? c : -1;
    };
    int cn = key_at(e);
    int bn = cn >= 0 ? P[cn] + H[cn] : 0;
    __syncthreads();
    for (; e - lane < e1; e += kWave) {
        const int c = cn, base = bn;
        cn = key_at(e + kWave);
        bn = cn >= 0 ? P[cn] + H[cn] : 0;
        const bool ok = c >= 0;
        if (ok) atomicOr((unsigned long long *)&mask[c], 1ull << lane);
        __syncthreads();
        const uint64_t mk = ok ? mask[c] : 0ull;
        const int rank = __popcll(mk & ((1ull << lane) - 1ull));
        if (ok) C[base + seen[c] + rank] = (int32_t)(e / k);
        __syncthreads();
        if (ok && (mk >> lane) == 1ull) {   // highest lane of its key in the chunk
            seen[c] += __popcll(mk);
            mask[c] = 0ull;
        }
        __syncthreads();
    }
}

// 5: one wave per key: entry j of the run goes to slot (number of entries
// smaller than it, or equal and earlier in the fill), 64 entries at a time.
__global__ __launch_bounds__(kTrThreads) void tr_order_kernel(const int32_t *__restrict__ stage,
                                                             const int32_t *__restrict__ ptr,
                                                             int32_t *__restrict__ col, int nb,
                                                             int rows, int k, int cols) {
    const int64_t key = (int64_t)blockIdx.x * (kTrThreads / kWave) + wave_id();
    if (key >= (int64_t)nb * cols) return;
    const int b = (int)(key / cols), c = (int)(key % cols);
    const int lane = lane_id();
    const int32_t *P = ptr + (int64_t)b * (cols + 1);
    const int s = __builtin_amdgcn_readfirstlane(P[c]);
    const int len = __builtin_amdgcn_readfirstlane(P[c + 1]) - s;
    if (len <= 0) return;
    const int32_t *S = stage + (int64_t)b * rows * k + s;
    int32_t *C = col + (int64_t)b * rows * k + s;
    for (int jb = 0; jb < len; jb += kWave) {
        const int j = jb + lane;
        const int vj = j < len ? S[j] : 0;
        int rank = 0;
        for (int ib = 0; ib < len; ib += kWave) {
            const int vi_l = ib + lane < len ? S[ib + lane] : 0;
            const int n = min(kWave, len - ib);
            for (int t = 0; t < n; ++t) {
                const int vi = __builtin_amdgcn_readlane(vi_l, t);
                rank += (vi < vj || (vi == vj && ib + t < j)) ? 1 : 0;
            }
        }
        if (j < len) C[rank] = vj;
    }
}

template <int CMAX>
static void launch_tr(int nb, int rows, int k, int cols, const TrPlan &p, const int32_t *idx,
                      int32_t *ptr, int32_t *col, int32_t *hist, int32_t *tot, int32_t *stage,
                      hipStream_t s) {
    const dim3 grid((unsigned)p.ranges, (unsigned)nb);
    hipLaunchKernelGGL(tr_count_kernel<CMAX>, grid, dim3(kTrThreads), 0, s, idx, hist, rows, k,
                       cols, p.ranges, p.rows_per);
    const dim3 pgrid((unsigned)((cols + kTrThreads - 1) / kTrThreads), (unsigned)nb);
    hipLaunchKernelGGL(tr_prefix_kernel, pgrid, dim3(kTrThreads), 0, s, hist, tot, cols, p.ranges);
    hipLaunchKernelGGL(tr_scan_kernel, dim3((unsigned)nb), dim3(kTrScanThreads), 0, s, tot, ptr,
                       cols);
    if (cols <= kTrMaskCols) {
        hipLaunchKernelGGL(tr_fill_ordered_kernel, grid, dim3(kWave), 0, s, idx, hist, ptr, col,
                           rows, k, cols, p.ranges, p.rows_per);
        return;
    }
    hipLaunchKernelGGL(tr_fill_kernel<CMAX>, grid, dim3(kTrThreads), 0, s, idx, hist, ptr, stage,
                       rows, k, cols, p.ranges, p.rows_per);
    const int64_t keys = (int64_t)nb * cols;
    const int wpg = kTrThreads / kWave;
    hipLaunchKernelGGL(tr_order_kernel, dim3((unsigned)((keys + wpg - 1) / wpg)), dim3(kTrThreads),
                       0, s, stage, ptr, col, nb, rows, k, cols);
}

hipError_t launch_transpose(int nb, int rows, int k, int cols, const int32_t *idx, int32_t *ptr,
                            int32_t *col, void *ws, hipStream_t s) {
    const TrPlan p = plan(nb, rows, k, cols);
    int32_t *hist = (int32_t *)ws;
    int32_t *tot = (int32_t *)((char *)hist + align256(sizeof(int32_t) * p.hist_ints));
    int32_t *stage = (int32_t *)((char *)tot + align256(sizeof(int32_t) * p.tot_ints));
    if (cols <= 4096)
        launch_tr<4096>(nb, rows, k, cols, p, idx, ptr, col, hist, tot, stage, s);
    else
        launch_tr<kTrMaxCols>(nb, rows, k, cols, p, idx, ptr, col, hist, tot, stage, s);
    return hipGetLastError();
}

}  // namespace llsa
