// Hierarchical Top-K selection ("Trainable Log-linear Sparse Attention for
// Efficient Diffusion Transformers", explainer "Step 2: Hierarchical Top-K
// Selection"): dense scores at the coarsest level, then at every finer level
// only the B children of the parent's picks are scored.
//
// One wave serves 16 query rows that share their candidates: at a finer level
// these are 16 of the B children of one parent, whose candidate list is the
// children of the parent's K picks (B / 16 tiles of 16 contiguous pooled keys
// per pick); at the coarsest level a 16-row slice against all keys.
// Scores are float32 on the matrix cores (v_mfma_f32_16x16x4_f32), computed
// transposed so that lane l owns query l%16 and 4 candidates of each
// 16-candidate tile.  Top-K runs in registers on 64-bit keys (order-preserving score bits, inverted index), so
// one unsigned compare orders by score and breaks ties toward the lower index:
// every lane sorts its candidates in groups of KM with bitonic networks and
// merges them into a running top-KM list, then the 4 lanes of a query merge
// their lists through two butterfly exchanges.
#include "common.hpp"
#include "internal.hpp"
#include "llsa.h"

namespace llsa {

__device__ __forceinline__ uint64_t score_key(float s, uint32_t idx) {
    uint32_t u = __builtin_bit_cast(uint32_t, s);
    if (s == 0.0f) u = 0u;  // -0 and +0 compare equal
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint64_t)(~idx);
}

template <int N>
__device__ __forceinline__ void sort_desc(uint64_t (&a)[N]) {
#pragma unroll
    for (int k = 2; k <= N; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int p = i ^ j;
                if (p > i) {
                    const bool desc = (i & k) == 0;
                    const uint64_t x = a[i], y = a[p];
                    const bool sw = desc ? (x < y) : (x > y);
                    a[i] = sw ? y : x;
                    a[p] = sw ? x : y;
                }
            }
}

// r, g sorted descending; r becomes the N largest of both, descending.
template <int N>
__device__ __forceinline__ void merge_top(uint64_t (&r)[N], const uint64_t (&g)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const uint64_t y = g[N - 1 - i];
        r[i] = r[i] > y ? r[i] : y;
    }
#pragma unroll
    for (int j = N >> 1; j > 0; j >>= 1)
#pragma unroll
        for (int i = 0; i < N; ++i) {
            const int p = i ^ j;
            if (p > i) {
                const uint64_t x = r[i], y = r[p];
                r[i] = x < y ? y : x;
                r[p] = x < y ? x : y;
            }
        }
}

template <int N>
__device__ __forceinline__ void sort_asc_u32(uint32_t (&a)[N]) {
#pragma unroll
    for (int k = 2; k <= N; k <<= 1)
#pragma unroll
        for (int j = k >> 1; j > 0; j >>= 1)
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int p = i ^ j;
                if (p > i) {
                    const bool asc = (i & k) == 0;
                    const uint32_t x = a[i], y = a[p];
                    const bool sw = asc ? (x > y) : (x < y);
                    a[i] = sw ? y : x;
                    a[p] = sw ? x : y;
                }
            }
}

constexpr int kSelCountKeys = 4096;   // keys a fused count can hold

// parent == nullptr: coarsest level, candidates 0..n-1, row groups are
// 16-row slices.  Otherwise: row group gi = 16 of the B children of parent
// gi / sub (sub = B / 16), candidates = children of that parent's picks
// [0..kp), tile t = sub-tile t % sub of pick t / sub.
// SPLIT = 4: the four waves of a workgroup share one row group and take a
// quarter of its candidate tiles each (the coarsest level has few groups);
// their lists are merged through LDS at the end.
// COUNT: the first step of the index transpose, fused.  The workgroup's 8
// waves hold 128 consecutive rows of one head; it counts their picks per key
// (n <= 4096 keys) in LDS and writes the histogram as range gi / 8 of
// hist [heads, groups_per_head / 8, n].
template <int KM, int SPLIT, bool COUNT>
__global__ __launch_bounds__(COUNT ? 512 : 256) void select_kernel(const float *__restrict__ ql,
                                                     const float *__restrict__ kl,
                                                     const int32_t *__restrict__ parent,
                                                     int32_t *__restrict__ out, int n, int kout,
                                                     int kp, int groups_per_head,
                                                     int64_t groups_total, int sub,
                                                     int32_t *__restrict__ hist,
                                                     uint32_t *__restrict__ status) {
    static_assert(SPLIT == 1 || SPLIT == 4, "a row group takes one wave or the whole workgroup");
    static_assert(!COUNT || SPLIT == 1, "the fused count takes four row groups per workgroup");
    __shared__ uint64_t part_best[SPLIT == 1 ? 1 : SPLIT][kBlock][KM];
    __shared__ int32_t hcount[COUNT ? kSelCountKeys : 1];
    if constexpr (COUNT) {
        for (int c = threadIdx.x; c < n; c += blockDim.x) hcount[c] = 0;
        __syncthreads();
    }
    const int part = SPLIT == 1 ? 0 : wave_id();
    constexpr int kWpg = COUNT ? 8 : 4;   // waves per workgroup
    const int64_t gid = SPLIT == 1 ? (int64_t)xcd_remap(blockIdx.x, gridDim.x) * kWpg + wave_id()
                                   : (int64_t)xcd_remap(blockIdx.x, gridDim.x);
    if (gid >= groups_total) return;
    const int h = (int)(gid / groups_per_head);
    const int gi = (int)(gid % groups_per_head);
    const int lane = lane_id();
    const int g = lane >> 4, col = lane & 15;

    const float *qh = ql + (int64_t)h * n * kHeadDim;
    const float *kh = kl + (int64_t)h * n * kHeadDim;
    const int row = gi * kBlock + col;
    const bool row_ok = row < n;
    const bool dense = parent == nullptr;
    const int ntiles = dense ? (n + kBlock - 1) / kBlock : kp * sub;
    const int32_t *prow = dense ? nullptr : parent + ((int64_t)h * (groups_per_head / sub) + gi / sub) * kp;
    // the parent's picks, one per lane (kp <= 32), requested first: every
    // candidate address needs them, and waiting for a load waits for every
    // load issued before it
    const int ppick = !dense && lane < kp ? prow[lane] : 0;

    float qf[16];
    {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(qh + (int64_t)(row_ok ? row : 0) * kHeadDim + 16 * g);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4 t = row_ok ? src[j] : f32x4{0.f, 0.f, 0.f, 0.f};
            qf[4 * j] = t[0];
            qf[4 * j + 1] = t[1];
            qf[4 * j + 2] = t[2];
            qf[4 * j + 3] = t[3];
        }
    }

    uint64_t best[KM];
#pragma unroll
    for (int i = 0; i < KM; ++i) best[i] = 0;

    const int tb = part * ntiles / SPLIT, te = (part + 1) * ntiles / SPLIT;
    // candidate tiles come CH at a time, CH = 4 tiles (16 keys per lane) for
    // K <= 16: the kernel then fits 4 waves per SIMD, so that a level-1 grid of
    // 4 row groups per SIMD runs in one round rather than a full one and a
    // third.  K = 32 needs 8 tiles per sorted group, read in two batches of 4.
    // All loads of a batch are in flight before its first tile is used.
    constexpr int CH = KM > 16 ? 8 : 4;
    constexpr int LB = 4;
    for (int t0 = tb; t0 < te; t0 += CH) {
        uint64_t keys[4 * CH];
#pragma unroll
        for (int hb = 0; hb < CH; hb += LB) {
            // tiles past the end re-read the last tile and are masked out
            float kf[LB][16];
            int base[LB];
#pragma unroll
            for (int t = 0; t < LB; ++t) {
                const int tile = min(t0 + hb + t, te - 1);
                base[t] = dense ? tile * kBlock
                                : (__builtin_amdgcn_readlane(ppick, tile / sub) * sub + tile % sub) * kBlock;
                const int cand = base[t] + col;
                // a parent pick outside its level (never one the selection wrote) reads row 0,
                // and the debug index check reports it
                const bool in_level = (unsigned)cand < (unsigned)n;
                const int64_t crow = in_level ? cand : 0;
                if (!dense && !in_level && status != nullptr) atomicOr(status, (uint32_t)LLSA_IDX_RANGE);
                const f32x4 *src = reinterpret_cast<const f32x4 *>(kh + crow * kHeadDim + 16 * g);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x4 tt = src[j];
                    kf[t][4 * j] = tt[0];
                    kf[t][4 * j + 1] = tt[1];
                    kf[t][4 * j + 2] = tt[2];
                    kf[t][4 * j + 3] = tt[3];
                }
            }
#pragma unroll
            for (int t = 0; t < LB; ++t) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int s = 0; s < 16; ++s) acc = mfma_f32_4(kf[t][s], qf[s], acc);
                const bool live = t0 + hb + t < te;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int c = base[t] + 4 * g + i;
                    keys[4 * (hb + t) + i] = (live && (unsigned)c < (unsigned)n) ? score_key(acc[i], (uint32_t)c) : 0ull;
                }
            }
        }
#pragma unroll
        for (int grp = 0; grp < 4 * CH / KM; ++grp) {
            if (t0 + grp * KM / 4 >= te) break;   // every tile of the group is past the end
            uint64_t part[KM];
#pragma unroll
            for (int i = 0; i < KM; ++i) part[i] = keys[grp * KM + i];
            sort_desc<KM>(part);
            if (t0 == tb && grp == 0) {   // the first group is the running list
#pragma unroll
                for (int i = 0; i < KM; ++i) best[i] = part[i];
            } else {
                merge_top<KM>(best, part);
            }
        }
    }
    // the 4 lanes holding one query merge their lists
    auto merge_lanes = [&]() {
#pragma unroll
        for (int m = 16; m <= 32; m <<= 1) {
            uint64_t other[KM];
#pragma unroll
            for (int i = 0; i < KM; ++i) {
                const uint32_t lo = shfl_xor_u((uint32_t)best[i], m);
                const uint32_t hi = shfl_xor_u((uint32_t)(best[i] >> 32), m);
                other[i] = ((uint64_t)hi << 32) | lo;
            }
            merge_top<KM>(best, other);
        }
    };
    merge_lanes();
    if constexpr (SPLIT > 1) {
        // part w's list of query c16 -> LDS; wave 0 merges lane group g = part g
        if (g == 0) {
#pragma unroll
            for (int i = 0; i < KM; ++i) part_best[part][col][i] = best[i];
        }
        __syncthreads();
        if (part != 0) return;
#pragma unroll
        for (int i = 0; i < KM; ++i) best[i] = part_best[g][col][i];
        merge_lanes();
    }
    uint32_t sel[KM];
#pragma unroll
    for (int i = 0; i < KM; ++i) sel[i] = (i < kout) ? ~(uint32_t)best[i] : 0xffffffffu;
    sort_asc_u32<KM>(sel);
    if (g == 0 && row_ok) {
        int32_t *dst = out + ((int64_t)h * n + row) * kout;
#pragma unroll
        for (int i = 0; i < KM; ++i)
            if (i < kout) dst[i] = (int32_t)sel[i];
    }
    if constexpr (COUNT) {
        if (g == 0 && row_ok) {
#pragma unroll
            for (int i = 0; i < KM; ++i)
                if (i < kout) atomicAdd(&hcount[sel[i]], 1);
        }
        __syncthreads();
        const int nr = groups_per_head / kWpg;
        int32_t *H = hist + ((int64_t)h * nr + gi / kWpg) * n;
        for (int c = threadIdx.x; c < n; c += blockDim.x) H[c] = hcount[c];
    }
}

template <int KM>
static void launch_level(const Geometry &g, int l, const float *pq, const float *pk, int32_t *idx,
                         int32_t *hist, uint32_t *status, hipStream_t s) {
    const bool dense = (l == g.L);
    const int n = g.n[l];
    const int gph = dense ? (n + kBlock - 1) / kBlock : n / kBlock;
    const int64_t total = (int64_t)g.bh * gph;
    const int32_t *parent = dense ? nullptr : idx + g.idx_off[l + 1];
    const int kp = dense ? 0 : g.kl[l + 1];
    const int ntiles = dense ? gph : kp * g.sub;
    // split a row group over the workgroup when groups are too few to fill
    // the chip and each has tiles enough for four waves
    if (hist != nullptr)   // fused count (select_count_fusable holds)
        hipLaunchKernelGGL((select_kernel<KM, 1, true>), dim3((unsigned)(total / 8)), dim3(512), 0,
                           s, pq + g.pyr_off[l], pk + g.pyr_off[l], parent, idx + g.idx_off[l], n,
                           g.kl[l], kp, gph, total, g.sub, hist, status);
    else if (total < 1024 && ntiles >= 4 * 2)
        hipLaunchKernelGGL((select_kernel<KM, 4, false>), dim3((unsigned)total), dim3(256), 0, s,
                           pq + g.pyr_off[l], pk + g.pyr_off[l], parent, idx + g.idx_off[l], n,
                           g.kl[l], kp, gph, total, g.sub, nullptr, status);
    else
        hipLaunchKernelGGL((select_kernel<KM, 1, false>), dim3((unsigned)((total + 3) / 4)), dim3(256),
                           0, s, pq + g.pyr_off[l], pk + g.pyr_off[l], parent, idx + g.idx_off[l], n,
                           g.kl[l], kp, gph, total, g.sub, nullptr, status);
}

// The level-1 selection can also count its picks for the transpose when the
// level has at most 4096 keys, its row groups come eight to a workgroup and a
// level-1 row group is not split over a workgroup.
bool select_count_fusable(const Geometry &g) {
    const int n = g.n[1];
    const bool dense = g.L == 1;
    const int gph = dense ? (n + kBlock - 1) / kBlock : n / kBlock;
    const int64_t total = (int64_t)g.bh * gph;
    const int ntiles = dense ? gph : g.kl[2] * g.sub;
    const bool split = total < 1024 && ntiles >= 4 * 2;
    return n <= kSelCountKeys && gph % 8 == 0 && !split;
}

hipError_t launch_select(const Geometry &g, const float *pq, const float *pk, int32_t *idx,
                         int32_t *count_hist, uint32_t *status, hipStream_t s) {
    for (int l = g.L; l >= 1; --l) {
        int32_t *hist = l == 1 ? count_hist : nullptr;
        if (g.K <= 8)
            launch_level<8>(g, l, pq, pk, idx, hist, status, s);
        else if (g.K <= 16)
            launch_level<16>(g, l, pq, pk, idx, hist, status, s);
        else
            launch_level<32>(g, l, pq, pk, idx, hist, status, s);
    }
    return hipGetLastError();
}

}  // namespace llsa
