// Sparse index transpose ("Trainable Log-linear Sparse Attention for
// Efficient Diffusion Transformers", explainer "Step 4: Efficient Sparse
// Index Transpose"): query-major pick lists become key-major lists by a count
// per key, an exclusive prefix sum and a fill.
//
// The transpose is a stable counting sort of the picks by key (stable: the
// picks of one key keep their row order).  One pass sorts by up to 4096
// buckets; it has four short kernels that spread every matrix over many
// workgroups, use no global atomic and need no memory cleared beforehand:
//  1 count  each workgroup counts the picks of a contiguous range of elements
//           in an LDS histogram of the buckets and writes it out;
//  2 prefix bucket by bucket (one thread each), the histograms of the ranges
//           become each range's offset inside the bucket's run, and the
//           bucket's total is kept;
//  3 scan   per matrix, the exclusive prefix of the bucket totals;
//  4 fill   one wave per range walks its picks in order, 64 at a time: every
//           pick sets its lane's bit in an LDS mask of its bucket, so its rank
//           among the chunk's picks of that bucket is a popcount, and picks
//           land in element order at the scan plus the range's offset.
// Up to 4096 keys, the bucket is the key and one pass writes csr_ptr and
// csr_col.  Above, two passes (least significant digit first): the low 12
// bits of the key, into a staging list of (key, row) pairs, then the high
// bits, into csr_col; csr_ptr then comes from a binary search of every key in
// the sorted keys.  Every pick is read once per pass whatever the number of
// keys, and the histograms stay at 4096 buckets per range.
// Matrices of at most 131072 picks and 4096 keys take a single kernel
// instead (tr_one_kernel below), and several such matrices -- the levels of
// one problem -- share one launch.
#include <algorithm>

#include "common.hpp"
#include "internal.hpp"

namespace llsa {

constexpr int kTrThreads = 256;
constexpr int kTrBits = 12;
constexpr int kTrBuckets = 1 << kTrBits;   // buckets per pass (LDS counters and masks)
constexpr int kTrChunk = 1024;             // target picks per range (workgroup) of count and fill
constexpr int kTrMaxRanges = 64;
constexpr int kTrBatch = 8;                // global loads a thread issues before using them

// MODE 0: one pass, bucket = key, idx -> csr_col.
// MODE 1: first of two passes, bucket = low digit, idx -> (key, row) pairs.
// MODE 2: second pass, bucket = high digit, pairs -> csr_col and sorted keys.
struct TrPlan {
    int ranges;          // element ranges per matrix
    int per;             // elements per range
    int buckets;         // buckets of the pass (second pass: of the high digit)
    bool two_pass;
};

static TrPlan plan(int rows, int k, int cols) {
    TrPlan p;
    const int64_t picks = (int64_t)rows * k;
    const int64_t want = (picks + kTrChunk - 1) / kTrChunk;
    p.ranges = (int)(want < 1 ? 1 : (want > kTrMaxRanges ? kTrMaxRanges : want));
    p.per = (int)((picks + p.ranges - 1) / p.ranges);
    p.two_pass = cols > kTrBuckets;
    p.buckets = p.two_pass ? kTrBuckets : cols;
    return p;
}

static size_t align256(size_t b) { return (b + 255) / 256 * 256; }

// Workspace: histograms [nb, ranges, buckets], bucket totals [nb, buckets],
// and for two passes the first pass's scan [nb, buckets + 1], the second's
// [nb, buckets + 1], the staged pairs (keys, rows) and the sorted keys
// [nb, rows * k] each.
struct TrWs {
    int32_t *hist, *tot, *ptrA, *ptrB, *pkey, *prow, *skey;
};

static TrWs carve(void *ws, int nb, int rows, int k, const TrPlan &p, size_t *bytes) {
    TrWs w{};
    char *c = (char *)ws;
    size_t off = 0;
    auto take = [&](size_t n) {   // c == nullptr: sizes only
        int32_t *r = c ? (int32_t *)(c + off) : nullptr;
        off += align256(sizeof(int32_t) * n);
        return r;
    };
    const size_t E = (size_t)rows * k;
    w.hist = take((size_t)nb * p.ranges * p.buckets);
    w.tot = take((size_t)nb * p.buckets);
    if (p.two_pass) {
        w.ptrA = take((size_t)nb * (kTrBuckets + 1));
        w.ptrB = take((size_t)nb * (kTrBuckets + 1));
        w.pkey = take((size_t)nb * E);
        w.prow = take((size_t)nb * E);
        w.skey = take((size_t)nb * E);
    }
    if (bytes) *bytes = off;
    return w;
}

static bool tr_one_fits(int rows, int k, int cols);   // the one-launch kernel takes it

size_t transpose_workspace_bytes(int nb, int rows, int k, int cols) {
    if (tr_one_fits(rows, k, cols)) return 0;
    size_t bytes = 0;
    carve(nullptr, nb, rows, k, plan(rows, k, cols), &bytes);
    return bytes;
}

// The picks a pass reads: element e of matrix b has a key and a row, or is
// absent (key outside [0, cols), or past the staged count in the second pass).
struct TrSrc {
    const int32_t *idx;    // MODE 0 / 1: [nb, E]
    const int32_t *pkey;   // MODE 2: [nb, E]
    const int32_t *prow;
    const int32_t *ptrA;   // MODE 2: staged count of matrix b at ptrA[b][kTrBuckets]
    int64_t E;             // elements per matrix, rows * k
    int k, cols;
};

template <int MODE>
__device__ __forceinline__ int tr_count_of(const TrSrc &S, int b) {
    if constexpr (MODE == 2)
        return S.ptrA[(int64_t)b * (kTrBuckets + 1) + kTrBuckets];
    else
        return (int)S.E;
}

// bucket of element e (-1: absent); the pick's row goes to *row
template <int MODE>
__device__ __forceinline__ int tr_bucket(const TrSrc &S, int b, int64_t e, int n, int &key, int &row) {
    if (e >= n) return -1;
    const int64_t x = (int64_t)b * S.E + e;
    if constexpr (MODE == 2) {
        key = S.pkey[x];
        row = S.prow[x];
        return key >> kTrBits;
    } else {
        key = S.idx[x];
        row = (int)(e / S.k);
        if (key < 0 || key >= S.cols) return -1;
        return MODE == 0 ? key : (key & (kTrBuckets - 1));
    }
}

// 1: histogram of the buckets of elements [m * per, (m + 1) * per) of matrix b
template <int MODE>
__global__ __launch_bounds__(kTrThreads) void tr_count_kernel(TrSrc S, int32_t *__restrict__ hist,
                                                             int buckets, int ranges, int per) {
    __shared__ int32_t h[kTrBuckets];
    const int m = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    for (int c = tid; c < buckets; c += kTrThreads) h[c] = 0;
    __syncthreads();
    const int n = tr_count_of<MODE>(S, b);
    const int64_t e0 = (int64_t)m * per, e1 = min((int64_t)n, e0 + per);
    // kTrBatch loads in flight before their atomics (an LDS atomic between two
    // global loads would otherwise wait for the first)
    for (int64_t eb = e0 + tid; eb < e1; eb += kTrBatch * kTrThreads) {
        int c[kTrBatch];
#pragma unroll
        for (int j = 0; j < kTrBatch; ++j) {
            const int64_t e = eb + (int64_t)j * kTrThreads;
            int key, row;
            c[j] = tr_bucket<MODE>(S, b, e < e1 ? e : n, n, key, row);
        }
#pragma unroll
        for (int j = 0; j < kTrBatch; ++j)
            if (c[j] >= 0) atomicAdd(&h[c[j]], 1);
    }
    __syncthreads();
    int32_t *H = hist + ((int64_t)b * ranges + m) * buckets;
    for (int c = tid; c < buckets; c += kTrThreads) H[c] = h[c];
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

// 2: one thread per bucket c of matrix b: hist[b][m][c] becomes the number of
// picks of c in ranges before m, tot[b][c] the bucket's total.
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

// 3: per matrix b, ptr[b][c] = number of picks of buckets < c.
constexpr int kTrScanThreads = 1024;
__global__ __launch_bounds__(kTrScanThreads) void tr_scan_kernel(const int32_t *__restrict__ tot,
                                                                int32_t *__restrict__ ptr,
                                                                int cols) {
    __shared__ int32_t wsum[kTrScanThreads / kWave];
    const int b = blockIdx.x, tid = threadIdx.x;
    const int32_t *T = tot + (int64_t)b * cols;
    // each thread owns a contiguous run of buckets
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
    if (tid == kTrScanThreads - 1) P[cols] = run;   // the last thread owns the last buckets
}

// 4: one wave per element range, picks in order, 64 at a time.  The pick of
// lane l in bucket c sets bit l of mask[c]; its rank among the chunk's picks
// of c is the number of lower bits set, and the highest lane of each bucket
// advances the bucket's count seen so far (seen[c]) by the popcount.  A pick
// lands at ptr[c] + the range's offset for c + seen[c] + rank; the two global
// terms are read per pick, one chunk ahead.
template <int MODE>
__global__ __launch_bounds__(kWave) void tr_fill_kernel(TrSrc S, const int32_t *__restrict__ hist,
                                                       const int32_t *__restrict__ ptr,
                                                       int32_t *__restrict__ out_row,
                                                       int32_t *__restrict__ out_key, int buckets,
                                                       int ranges, int per) {
    __shared__ int32_t seen[kTrBuckets];
    __shared__ uint64_t mask[kTrBuckets];
    const int m = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
    const int32_t *H = hist + ((int64_t)b * ranges + m) * buckets;
    const int32_t *P = ptr + (int64_t)b * (buckets + 1);
    for (int c = lane; c < buckets; c += kWave) {
        seen[c] = 0;
        mask[c] = 0;
    }
    const int n = tr_count_of<MODE>(S, b);
    const int64_t e0 = (int64_t)m * per, e1 = min((int64_t)n, e0 + per);
    int32_t *OR = out_row + (int64_t)b * S.E;
    int32_t *OK = MODE == 0 ? nullptr : out_key + (int64_t)b * S.E;
    __syncthreads();
    for (int64_t eb = e0; eb < e1; eb += kTrBatch * kWave) {
        // kTrBatch chunks: their picks, then their buckets' global starts, all
        // in flight together
        int c[kTrBatch], key[kTrBatch], row[kTrBatch], base[kTrBatch];
#pragma unroll
        for (int j = 0; j < kTrBatch; ++j) {
            const int64_t e = eb + (int64_t)j * kWave + lane;
            c[j] = tr_bucket<MODE>(S, b, e < e1 ? e : n, n, key[j], row[j]);
        }
#pragma unroll
        for (int j = 0; j < kTrBatch; ++j) base[j] = c[j] >= 0 ? P[c[j]] + H[c[j]] : 0;
#pragma unroll
        for (int j = 0; j < kTrBatch; ++j) {
            if (eb + (int64_t)j * kWave >= e1) break;
            const bool ok = c[j] >= 0;
            const int cl = ok ? c[j] : 0;
            if (ok) atomicOr((unsigned long long *)&mask[cl], 1ull << lane);
            __syncthreads();
            const uint64_t mk = ok ? mask[cl] : 0ull;
            const int rank = __popcll(mk & ((1ull << lane) - 1ull));
            if (ok) {
                const int pos = base[j] + seen[cl] + rank;
                OR[pos] = row[j];
                if constexpr (MODE != 0) OK[pos] = key[j];
            }
            __syncthreads();
            if (ok && (mk >> lane) == 1ull) {   // highest lane of its bucket in the chunk
                seen[cl] += __popcll(mk);
                mask[cl] = 0ull;
            }
            __syncthreads();
        }
    }
}

// Two passes: ptr[b][c] = number of sorted keys below c (binary search).
__global__ __launch_bounds__(kTrThreads) void tr_bounds_kernel(const int32_t *__restrict__ skey,
                                                              const int32_t *__restrict__ ptrA,
                                                              int32_t *__restrict__ ptr, int64_t E,
                                                              int cols) {
    const int b = blockIdx.y;
    const int c = blockIdx.x * kTrThreads + threadIdx.x;
    if (c > cols) return;
    const int n = ptrA[(int64_t)b * (kTrBuckets + 1) + kTrBuckets];
    const int32_t *K = skey + (int64_t)b * E;
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (K[mid] < c)
            lo = mid + 1;
        else
            hi = mid;
    }
    ptr[(int64_t)b * (cols + 1) + c] = lo;
}

// Matrices of at most kTrOneMaxPicks picks and kTrOneMaxCols keys: the whole
// transpose in one launch.  Workgroup (part, b) owns keys [512 part, 512 part
// + 512) of matrix b and reads every pick of the matrix; the parts of one
// matrix run side by side on one XCD, so that all but the first read of a
// pick come from that XCD's L2.  Every workgroup scans all the picks of
// its matrix, so fewer, wider parts do less work in total; 512 keys keep the
// per-slice counters and masks at 96 KB of LDS (128 KB with the part's
// queue), one workgroup per CU, and the levels of a 65536-token problem in
// fewer workgroups than CUs:
//  - wave w holds elements [w per, (w + 1) per); the number of picks with a
//    smaller key gives where the part's lists start;
//  - the part's picks form a sequence in element order, cut into 16 slices:
//    either equal slices of an LDS queue that the waves fill in order, or
//    each wave's own elements.  Wave s counts the picks of slice s per key,
//    so an exclusive prefix over the slices, plus the scan over the keys, is
//    the first slot of each (slice, key);
//  - each wave places its slice's picks 64 at a time, ranking the picks of
//    one key inside a chunk by a popcount of an LDS lane mask as the fill
//    kernel does, with its own masks and cursors: the 16 waves place their
//    picks independently and every list keeps its row order.
// No workspace, no global atomic, nothing to clear beforehand.
constexpr int kTrOneThreads = 1024;
constexpr int kTrOneWaves = kTrOneThreads / kWave;
constexpr int kTrOneKeys = 512;                                    // keys per workgroup
constexpr int kTrOneChunks = 32;                                   // 64-pick chunks per round
constexpr int kTrOneRound = kTrOneChunks * kWave;                  // picks a wave holds at once
constexpr int kTrOneMaxPicks = 4 * kTrOneWaves * kTrOneRound;      // 131072 per matrix
constexpr int kTrOneMaxCols = 4096;
constexpr int kTrOneQueue = 8192;                                 // picks of a part queued in LDS
constexpr int kTrOneQueueMinPer = 1024;                           // elements per wave from which the queue pays
constexpr int kTrOneEBits = 17;                                    // a queued pick: key << 17 | element
static_assert(kTrOneMaxPicks <= (1 << kTrOneEBits), "element index must fit its field");
static_assert(((uint64_t)kTrOneKeys << kTrOneEBits) <= (1ull << 32), "key offset and element fit 32 bits");
static_assert(kTrOneKeys <= kTrOneThreads && kTrOneKeys % kWave == 0, "a thread per key of the part");
static_assert(kTrOneQueue >= kTrOneWaves * 2 * kWave, "the per-wave queues fit the part queue");

static bool tr_one_fits(int rows, int k, int cols) {
    return (int64_t)rows * k <= kTrOneMaxPicks && cols <= kTrOneMaxCols;
}

// Several matrices (the levels of one problem, all with nb batches) in one
// launch: x-blocks [first_i, first_i + parts_i) belong to matrix i.
constexpr int kTrOneMaxMats = 8;
struct TrOneMat {
    const int32_t *idx;
    int32_t *ptr, *col;
    int rows, k, cols, parts;
};
struct TrOneArgs {
    TrOneMat m[kTrOneMaxMats];
    int nmat;
};

__global__ __launch_bounds__(kTrOneThreads) void tr_one_kernel(TrOneArgs A) {
    // the parts of one matrix side by side on one XCD (workgroup L runs on XCD L % 8)
    const int lin = xcd_remap((int)(blockIdx.x + gridDim.x * blockIdx.y), (int)(gridDim.x * gridDim.y));
    const int b = lin / (int)gridDim.x;
    int mi = 0, part = lin % (int)gridDim.x;
    while (mi + 1 < A.nmat && part >= A.m[mi].parts) part -= A.m[mi++].parts;
    const int32_t *__restrict__ idx = A.m[mi].idx;
    int32_t *__restrict__ ptr = A.m[mi].ptr;
    int32_t *__restrict__ col = A.m[mi].col;
    const int rows = A.m[mi].rows, k = A.m[mi].k, cols = A.m[mi].cols;
    __shared__ int32_t cur[kTrOneWaves][kTrOneKeys];    // per-slice counts, then cursors
    __shared__ uint64_t mask[kTrOneWaves][kTrOneKeys];
    __shared__ uint32_t queue[kTrOneQueue];             // the part's picks, in element order
    __shared__ int32_t below_w[kTrOneWaves];
    __shared__ int32_t inr_w[kTrOneWaves];
    __shared__ int32_t scan_w[kTrOneKeys / kWave];
    const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
    const uint64_t lower = (1ull << lane) - 1ull;
    const int c0 = part * kTrOneKeys, nk = min(kTrOneKeys, cols - c0);
    const int E = rows * k;
    const int per = (E + kTrOneWaves - 1) / kTrOneWaves;
    const int ew0 = min(E, w * per), ew1 = min(E, ew0 + per);
    const int32_t *I = idx + (int64_t)b * E;
    for (int i = tid; i < kTrOneWaves * kTrOneKeys; i += kTrOneThreads) {
        (&cur[0][0])[i] = 0;
        (&mask[0][0])[i] = 0ull;
    }
    // the wave's picks, a round (32 chunks) at a time, all loads of a round in
    // flight together; one round holds every pick of a matrix of 32768 picks
    const int rounds = (ew1 - ew0 + kTrOneRound - 1) / kTrOneRound;
    int kv[kTrOneChunks];
    auto load = [&](int r) {
#pragma unroll
        for (int j = 0; j < kTrOneChunks; ++j) {
            const int e = ew0 + r * kTrOneRound + j * kWave + lane;
            kv[j] = e < ew1 ? I[e] : -1;
        }
    };
    auto in_part = [&](int c) { return c >= c0 && c < c0 + nk; };
    auto pack = [&](int c, int e) { return ((uint32_t)(c - c0) << kTrOneEBits) | (uint32_t)e; };
    load(0);
    // picks with a smaller key (where the part's lists start) and picks of the part, per wave
    int below = 0, inr = 0;
    for (int r = 0; r < rounds; ++r) {
#pragma unroll
        for (int j = 0; j < kTrOneChunks; ++j) {
            below += (kv[j] >= 0 && kv[j] < c0) ? 1 : 0;
            inr += in_part(kv[j]) ? 1 : 0;
        }
        if (r + 1 < rounds) load(r + 1);
    }
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        below += __shfl_xor(below, d, kWave);
        inr += __shfl_xor(inr, d, kWave);
    }
    if (lane == 0) {
        below_w[w] = below;
        inr_w[w] = inr;
    }
    __syncthreads();
    int qoff = 0, qtot = 0;
#pragma unroll
    for (int x = 0; x < kTrOneWaves; ++x) {
        const int v = inr_w[x];
        qoff += x < w ? v : 0;
        qtot += v;
    }
    // Picks are local: the rows of one wave's element range pick mostly the
    // keys of one part, so that a part's picks sit in a few waves.  When they
    // fit, and the waves hold enough elements for the balance to pay for the
    // second pass over them, they are queued in element order (ballot and
    // popcount keep the order inside a chunk) and every wave counts and places
    // an equal slice of the queue; otherwise every wave counts and places its
    // own elements' picks.
    const bool queued = qtot <= kTrOneQueue && per >= kTrOneQueueMinPer;   // uniform over the workgroup
    const int s0 = w * qtot / kTrOneWaves, s1 = (w + 1) * qtot / kTrOneWaves;
    if (queued) {
        for (int r = 0; r < rounds; ++r) {
            if (rounds > 1) load(r);
            const int er = ew0 + r * kTrOneRound;
#pragma unroll
            for (int j = 0; j < kTrOneChunks; ++j) {
                const bool in = in_part(kv[j]);
                const uint64_t bal = __ballot(in);
                if (in) queue[qoff + __popcll(bal & lower)] = pack(kv[j], er + j * kWave + lane);
                qoff += __popcll(bal);
            }
        }
        __syncthreads();
        for (int e = s0 + lane; e < s1; e += kWave) atomicAdd(&cur[w][queue[e] >> kTrOneEBits], 1);
    } else {
        for (int r = 0; r < rounds; ++r) {
            if (rounds > 1) load(r);
#pragma unroll
            for (int j = 0; j < kTrOneChunks; ++j)
                if (in_part(kv[j])) atomicAdd(&cur[w][kv[j] - c0], 1);
        }
    }
    __syncthreads();
    // thread t < kTrOneKeys: key c0 + t -- prefix over the waves, then the scan over keys
    int tot = 0;
    if (tid < kTrOneKeys) {
#pragma unroll
        for (int x = 0; x < kTrOneWaves; ++x) {
            const int v = cur[x][tid];
            cur[x][tid] = tot;
            tot += v;
        }
    }
    const int incl = wave_inclusive_scan(tot);
    if (tid < kTrOneKeys && lane == kWave - 1) scan_w[w] = incl;
    __syncthreads();
    if (tid < kTrOneKeys) {
        int start = incl - tot;
#pragma unroll
        for (int x = 0; x < kTrOneWaves; ++x) start += below_w[x];
        for (int x = 0; x < w; ++x) start += scan_w[x];
        int32_t *P = ptr + (int64_t)b * (cols + 1);
        if (tid < nk) P[c0 + tid] = start;
        if (c0 + nk == cols && tid == kTrOneKeys - 1) P[cols] = start + tot;   // all valid picks
#pragma unroll
        for (int x = 0; x < kTrOneWaves; ++x) cur[x][tid] += start;
    }
    __syncthreads();
    int32_t *C = col + (int64_t)b * E;
    // places the queued picks Q[0, n), n <= 64, in order: the picks of one key
    // are ranked by a popcount of an LDS lane mask, then the highest lane of
    // each key moves its cursor on
    auto place = [&](const uint32_t *Q, int n) {
        wave_lds_sync();
        const bool ok = lane < n;
        const uint32_t v = ok ? Q[lane] : 0u;
        const int cl = (int)(v >> kTrOneEBits);
        if (ok) atomicOr((unsigned long long *)&mask[w][cl], 1ull << lane);
        wave_lds_sync();
        const uint64_t mk = ok ? mask[w][cl] : 0ull;
        if (ok) C[cur[w][cl] + __popcll(mk & lower)] = (int)(v & ((1u << kTrOneEBits) - 1u)) / k;
        wave_lds_sync();
        if (ok && (mk >> lane) == 1ull) {   // highest lane of its key in the chunk
            cur[w][cl] += __popcll(mk);
            mask[w][cl] = 0ull;
        }
    };
    if (queued) {
        for (int h = s0; h < s1; h += kWave) place(queue + h, min(kWave, s1 - h));
        return;
    }
    // the wave's own elements, scanned again; their picks of the part go
    // through a queue of 128 of its own (below 64 between chunks)
    uint32_t *Q = queue + w * 2 * kWave;
    int fill = 0;
    for (int r = 0; r < rounds; ++r) {
        if (rounds > 1) load(r);
        const int er = ew0 + r * kTrOneRound;
#pragma unroll
        for (int j = 0; j < kTrOneChunks; ++j) {
            const bool in = in_part(kv[j]);
            const uint64_t bal = __ballot(in);
            if (in) Q[fill + __popcll(bal & lower)] = pack(kv[j], er + j * kWave + lane);
            fill += __popcll(bal);
            if (fill >= kWave) {
                place(Q, kWave);
                if (lane < fill - kWave) Q[lane] = Q[kWave + lane];   // reads [64, 128), writes [0, 64)
                fill -= kWave;
                wave_lds_sync();
            }
        }
    }
    if (fill > 0) place(Q, fill);
}

static void launch_tr_one(const TrOneMat *mats, int n, int nb, hipStream_t s) {
    for (int i0 = 0; i0 < n; i0 += kTrOneMaxMats) {
        TrOneArgs A{};
        A.nmat = std::min(n - i0, kTrOneMaxMats);
        int parts = 0;
        for (int i = 0; i < A.nmat; ++i) {
            A.m[i] = mats[i0 + i];
            A.m[i].parts = (A.m[i].cols + kTrOneKeys - 1) / kTrOneKeys;
            parts += A.m[i].parts;
        }
        hipLaunchKernelGGL(tr_one_kernel, dim3((unsigned)parts, (unsigned)nb), dim3(kTrOneThreads), 0, s, A);
    }
}

template <int MODE>
static void tr_pass(const TrSrc &S, const TrPlan &p, int nb, int buckets, const TrWs &w,
                    int32_t *scan_out, int32_t *out_row, int32_t *out_key, hipStream_t s) {
    const dim3 grid((unsigned)p.ranges, (unsigned)nb);
    hipLaunchKernelGGL(tr_count_kernel<MODE>, grid, dim3(kTrThreads), 0, s, S, w.hist, buckets,
                       p.ranges, p.per);
    const dim3 pgrid((unsigned)((buckets + kTrThreads - 1) / kTrThreads), (unsigned)nb);
    hipLaunchKernelGGL(tr_prefix_kernel, pgrid, dim3(kTrThreads), 0, s, w.hist, w.tot, buckets, p.ranges);
    hipLaunchKernelGGL(tr_scan_kernel, dim3((unsigned)nb), dim3(kTrScanThreads), 0, s, w.tot,
                       scan_out, buckets);
    hipLaunchKernelGGL(tr_fill_kernel<MODE>, grid, dim3(kWave), 0, s, S, w.hist, scan_out, out_row,
                       out_key, buckets, p.ranges, p.per);
}

hipError_t launch_transpose(int nb, int rows, int k, int cols, const int32_t *idx, int32_t *ptr,
                            int32_t *col, void *ws, hipStream_t s) {
    const TrPlan p = plan(rows, k, cols);
    const TrWs w = carve(ws, nb, rows, k, p, nullptr);
    TrSrc S{};
    S.idx = idx;
    S.E = (int64_t)rows * k;
    S.k = k;
    S.cols = cols;
    if (tr_one_fits(rows, k, cols)) {
        const TrOneMat m{idx, ptr, col, rows, k, cols, 0};
        launch_tr_one(&m, 1, nb, s);
        return hipGetLastError();
    }
    if (!p.two_pass) {
        tr_pass<0>(S, p, nb, cols, w, ptr, col, nullptr, s);
        return hipGetLastError();
    }
    // low digit: idx -> staged (key, row) pairs in (low digit, row) order
    tr_pass<1>(S, p, nb, kTrBuckets, w, w.ptrA, w.prow, w.pkey, s);
    // high digit: pairs -> csr_col and the sorted keys, in (key, row) order
    TrSrc S2 = S;
    S2.pkey = w.pkey;
    S2.prow = w.prow;
    S2.ptrA = w.ptrA;
    const int hi_buckets = (cols + kTrBuckets - 1) >> kTrBits;
    tr_pass<2>(S2, p, nb, hi_buckets, w, w.ptrB, col, w.skey, s);
    const dim3 bgrid((unsigned)((cols + 1 + kTrThreads - 1) / kTrThreads), (unsigned)nb);
    hipLaunchKernelGGL(tr_bounds_kernel, bgrid, dim3(kTrThreads), 0, s, w.skey, w.ptrA, ptr, S.E, cols);
    return hipGetLastError();
}

// Several matrices with nb batches each: those the one-launch kernel takes
// share one launch, the others run one after another (sharing the workspace).
hipError_t launch_transpose_many(int nb, int n, const int *rows, const int *k, const int *cols,
                                 const int32_t *const *idx, int32_t *const *ptr,
                                 int32_t *const *col, void *ws, hipStream_t s) {
    TrOneMat one[64];
    int n_one = 0;
    for (int i = 0; i < n; ++i) {
        if (n_one < 64 && tr_one_fits(rows[i], k[i], cols[i]))
            one[n_one++] = TrOneMat{idx[i], ptr[i], col[i], rows[i], k[i], cols[i], 0};
        else {
            const hipError_t e = launch_transpose(nb, rows[i], k[i], cols[i], idx[i], ptr[i], col[i], ws, s);
            if (e != hipSuccess) return e;
        }
    }
    if (n_one > 0) launch_tr_one(one, n_one, nb, s);
    return hipGetLastError();
}

// The same transpose when the selection already counted the picks (one range
// per 128 rows, see select_count_fusable): prefix, scan and fill only.
static TrPlan counted_plan(int rows, int k, int cols) {
    TrPlan p;
    p.ranges = rows / kSelectRowsPerRange;
    p.per = kSelectRowsPerRange * k;
    p.two_pass = false;
    p.buckets = cols;
    return p;
}

size_t transpose_counted_workspace_bytes(int nb, int rows, int k, int cols) {
    size_t bytes = 0;
    carve(nullptr, nb, rows, k, counted_plan(rows, k, cols), &bytes);
    return bytes;
}

int32_t *transpose_counted_hist(void *ws) { return (int32_t *)ws; }

hipError_t launch_transpose_counted(int nb, int rows, int k, int cols, const int32_t *idx,
                                    int32_t *ptr, int32_t *col, void *ws, hipStream_t s) {
    const TrPlan p = counted_plan(rows, k, cols);
    const TrWs w = carve(ws, nb, rows, k, p, nullptr);
    TrSrc S{};
    S.idx = idx;
    S.E = (int64_t)rows * k;
    S.k = k;
    S.cols = cols;
    const dim3 grid((unsigned)p.ranges, (unsigned)nb);
    const dim3 pgrid((unsigned)((cols + kTrThreads - 1) / kTrThreads), (unsigned)nb);
    hipLaunchKernelGGL(tr_prefix_kernel, pgrid, dim3(kTrThreads), 0, s, w.hist, w.tot, cols, p.ranges);
    hipLaunchKernelGGL(tr_scan_kernel, dim3((unsigned)nb), dim3(kTrScanThreads), 0, s, w.tot, ptr, cols);
    hipLaunchKernelGGL(tr_fill_kernel<0>, grid, dim3(kWave), 0, s, S, w.hist, ptr, col, nullptr, cols,
                       p.ranges, p.per);
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
