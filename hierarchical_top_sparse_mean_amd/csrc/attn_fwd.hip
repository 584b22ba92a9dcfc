// Sparse attention with hierarchical KV enrichment and reweighting
// ("Trainable Log-linear Sparse Attention for Efficient Diffusion
// Transformers", explainer "Step 3: Hierarchical KV Enrichment + KV
// Reweighting"), driven only by the index lists.
//
// bf16 path: one wave per tile of 16 queries (a query block of B = 16 or one
// quarter of a block of B = 64; the tiles of a block share its picks, and a
// picked key block is B / 16 key tiles).  Scores are computed
// transposed, S^T = K Q^T, on v_mfma_f32_16x16x32_bf16 so that lane l owns
// query l%16 and keys 4(l/16)..+3 of every 16-key tile; that register layout
// is exactly the B operand of O^T += V^T P^T, so probabilities never leave
// registers.  Q, K and V tiles are loaded as whole 128-byte rows and pass
// through LDS: the Q and K operand rows are read back as they are, V with the
// gfx950 transposing LDS load.  The query block's own Q and O rows, which
// nothing else reads, go through non-temporal loads and stores, so the L2
// keeps the gathered K / V tiles that neighbouring query blocks share.
// Coarse tokens (float32 pyramid) are converted to bf16 on the fly and carry
// the logit bias log2(B^l).  Softmax runs in the exp2 domain over chunks of
// up to 8 tiles with one cross-lane max per chunk.
//
// f32 path: one thread per query, all arithmetic in float32 (used for f32
// inputs, where the output tolerance is tighter than bf16 products allow).
#include "common.hpp"
#include "internal.hpp"
#include "attn_tile.hpp"

namespace llsa {

constexpr int kMaxCoarseLevels = kMaxLevels - 1;

struct FwdArgs {
    int bh, N, n1, K1;
    int sub;                                   // 16-token tiles per block (B / 16)
    int nt1;                                   // query tiles per head, n1 * sub
    float lgB;                                 // log2(B): the bias of level l is l * lgB
    int ncl;                                   // coarse levels used (2..ncl+1)
    int ncoarse;                               // coarse entries per query block
    int cl_n[kMaxCoarseLevels];                // tokens at that level
    int cl_k[kMaxCoarseLevels];                // picks at that level
    int cl_span[kMaxCoarseLevels];             // level-1 blocks under one token
    int64_t cl_idx_off[kMaxCoarseLevels];      // index offset of the level
    int64_t cl_pyr_off[kMaxCoarseLevels];      // pyramid offset of the level
    float sl2;                                 // scale * log2(e)
    int drop;                                  // drop fully covered coarse picks
    TokMap tm;                                 // storage row of a sequence position
};

static FwdArgs make_fwd_args(const Geometry &g) {
    FwdArgs a{};
    a.bh = g.bh;
    a.N = g.N;
    a.n1 = g.n[1];
    a.K1 = g.kl[1];
    a.sub = g.sub;
    a.nt1 = g.n[1] * g.sub;
    a.lgB = (float)g.lgB;
    a.ncl = g.Le < g.L - 1 ? g.Le : g.L - 1;
    a.ncoarse = 0;
    int64_t span = 1;
    for (int j = 0; j < a.ncl; ++j) {
        const int l = j + 2;
        span *= g.B;
        a.cl_n[j] = g.n[l];
        a.cl_k[j] = g.kl[l];
        a.cl_span[j] = (int)span;
        a.cl_idx_off[j] = g.idx_off[l];
        a.cl_pyr_off[j] = g.pyr_off[l];
        a.ncoarse += g.kl[l];
    }
    a.sl2 = g.scale * kLog2e;
    a.drop = g.drop_covered;
    a.tm = TokMap{g.order, g.log2S};
    return a;
}

// Coarse entry e of query block ib (levels in order, picks in order): returns
// the pooled-token row offset (floats) and the log2 weight, or false if the
// entry does not exist or is dropped.
__device__ __forceinline__ bool coarse_entry(const FwdArgs &a, const int32_t *__restrict__ idx,
                                             const int32_t *__restrict__ fine, int h, int ib,
                                             int e, int64_t &row_off, float &bias) {
    if (e >= a.ncoarse) return false;
    int j = 0;
    int pick = e;
    while (j < a.ncl - 1 && pick >= a.cl_k[j]) {
        pick -= a.cl_k[j];
        ++j;
    }
    const int span = a.cl_span[j];
    const int anc = ib / span;
    const int c = idx[a.cl_idx_off[j] + ((int64_t)h * a.cl_n[j] + anc) * a.cl_k[j] + pick];
    if (a.drop && a.K1 >= span) {
        int cov = 0;
        for (int f = 0; f < a.K1; ++f) cov += (fine[f] / span == c) ? 1 : 0;
        if (cov == span) return false;
    }
    row_off = a.cl_pyr_off[j] + ((int64_t)h * a.cl_n[j] + c) * kHeadDim;
    bias = a.lgB * (float)(j + 2);  // log2(B^l)
    return true;
}

// Level slot j and pick number of coarse entry e (arithmetic only).
__device__ __forceinline__ bool coarse_locate(const FwdArgs &a, int e, int &j, int &pick) {
    j = 0;
    pick = e;
    while (j < a.ncl - 1 && pick >= a.cl_k[j]) {
        pick -= a.cl_k[j];
        ++j;
    }
    return e < a.ncoarse;
}

// A coarse pick can only be fully covered by the fine picks when K_1 reaches
// the B^(l-1) level-1 blocks under it (B for level 2, the smallest).
__host__ __device__ __forceinline__ bool drop_possible(const FwdArgs &a) {
    return a.drop && a.ncl > 0 && a.K1 >= a.cl_span[0];
}

// Coarse tile ct of query block ib, prefetched as raw float32 rows: the lane's
// operand row (entry ct*16 + c16) of pooled K and its 16 V columns 16g..16g+15,
// and the log2 weights of the score rows 4g+i (-inf where absent / dropped).
struct CoarseRows {
    f32x4 k0, k1, k2, k3;   // K row, dims 8g..8g+7 and 32+8g..32+8g+7
    f32x4 v0, v1, v2, v3;   // V row, dims 16g..16g+15
    float bias[4];
};

// Pick index of the lane's operand row of coarse tile ct (one read; issued
// early so the pooled-row reads that depend on it do not wait behind later
// loads).
__device__ __forceinline__ int coarse_pick(const FwdArgs &a, const int32_t *__restrict__ idx, int h,
                                           int ib, int ct, int c16) {
    int j, pick;
    const bool ok = coarse_locate(a, ct * kBlock + c16, j, pick);
    const int js = ok ? j : 0, ps = ok ? pick : 0;
    return idx[a.cl_idx_off[js] + ((int64_t)h * a.cl_n[js] + ib / a.cl_span[js]) * a.cl_k[js] + ps];
}

__device__ __forceinline__ void prefetch_coarse(const FwdArgs &a, const int32_t *__restrict__ idx,
                                                const int32_t *__restrict__ fine,
                                                const float *__restrict__ pk,
                                                const float *__restrict__ pv, int h, int ib, int ct,
                                                int c, int g, int c16, CoarseRows &R) {
    int j, pick;
    bool ok = coarse_locate(a, ct * kBlock + c16, j, pick);
    const int js = ok ? j : 0;
    // absent rows read a valid row of the same level and are zeroed below
    const int64_t src = a.cl_pyr_off[js] + ((int64_t)h * a.cl_n[js] + c) * kHeadDim;
    const f32x4 *ks = reinterpret_cast<const f32x4 *>(pk + src);
    const f32x4 *vsrc = reinterpret_cast<const f32x4 *>(pv + src + 16 * g);
    R.k0 = ks[2 * g];
    R.k1 = ks[2 * g + 1];
    R.k2 = ks[8 + 2 * g];
    R.k3 = ks[8 + 2 * g + 1];
    R.v0 = vsrc[0];
    R.v1 = vsrc[1];
    R.v2 = vsrc[2];
    R.v3 = vsrc[3];
    if (drop_possible(a)) {
        int64_t r2;
        float b2;
        ok = coarse_entry(a, idx, fine, h, ib, ct * kBlock + c16, r2, b2);
    }
    if (!ok) {
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        R.k0 = R.k1 = R.k2 = R.k3 = R.v0 = R.v1 = R.v2 = R.v3 = z;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int j2, p2;
        const bool ok2 = coarse_locate(a, ct * kBlock + 4 * g + i, j2, p2);
        R.bias[i] = ok2 ? a.lgB * (float)(j2 + 2) : -INFINITY;
    }
    if (drop_possible(a)) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int64_t r2;
            float b2;
            if (!coarse_entry(a, idx, fine, h, ib, ct * kBlock + 4 * g + i, r2, b2)) R.bias[i] = -INFINITY;
        }
    }
}

__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ pk, const float *__restrict__ pv, const int32_t *__restrict__ idx,
    __bf16 *__restrict__ o, float *__restrict__ lse, FwdArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 vs_all[4][kFwdTiles * kTileElems];
    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t blk = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * 4 + w;   // query tile
    if (blk >= (int64_t)a.bh * a.nt1) return;
    const int h = (int)(blk / a.nt1);
    const int qt = (int)(blk % a.nt1);
    const int ib = qt / a.sub;   // its query block
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    const __bf16 *kh = k + head_off;
    const __bf16 *vh = v + head_off;
    __bf16 *vw = vs_all[w];

    // element offset (within the head) of row r of 16-token tile b
    auto trow = [&](int b, int r) { return (int64_t)tok_row(a.tm, b * kBlock + r) * kHeadDim; };
    const __bf16 *qrow = q + head_off + trow(qt, c16);
    const bf16x8 qa0 = load_bf16x8(qrow + 8 * g);
    const bf16x8 qa1 = load_bf16x8(qrow + 32 + 8 * g);
    const int32_t *fine = idx + ((int64_t)h * a.n1 + ib) * a.K1;
    const int nft = a.K1 * a.sub;   // fine key tiles: sub-tile t % sub of pick t / sub
    const int nct = (a.ncoarse + kBlock - 1) / kBlock;

    float m = -INFINITY, lsum = 0.f;
    f32x4 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float bias[kFwdTiles][4];
    f32x4 st[kFwdTiles];
    CoarseRows cr;
    const int cpick0 = nct > 0 ? coarse_pick(a, idx, h, ib, 0, c16) : 0;

    // ---- fine key blocks, weight 1.  All loads of a chunk are issued before
    // any is consumed (tiles past the chunk's end re-read its last tile); the
    // first coarse tile is fetched right after the first chunk's loads so its
    // two dependent reads (pick index, then pooled rows) overlap them.
    for (int t0 = 0; t0 < nft; t0 += kFwdTiles) {
        const int nt = min(kFwdTiles, nft - t0);
        bf16x8 kr[kFwdTiles][2], vr[kFwdTiles][2];
#pragma unroll
        for (int t = 0; t < kFwdTiles; ++t) {
            const int tt = t0 + min(t, nt - 1);
            const int f = __builtin_amdgcn_readfirstlane(fine[tt / a.sub]) * a.sub + tt % a.sub;
            const __bf16 *kt = kh + trow(f, c16);
            kr[t][0] = load_bf16x8(kt + 8 * g);
            kr[t][1] = load_bf16x8(kt + 32 + 8 * g);
            // 16-byte chunks `lane` and `lane + 64` of the tile: rows lane/8 and lane/8 + 8
            vr[t][0] = load_bf16x8(vh + trow(f, lane >> 3) + (lane & 7) * 8);
            vr[t][1] = load_bf16x8(vh + trow(f, (lane >> 3) + 8) + (lane & 7) * 8);
        }
        if (t0 == 0 && nct > 0) prefetch_coarse(a, idx, fine, pk, pv, h, ib, 0, cpick0, g, c16, cr);
#pragma unroll
        for (int t = 0; t < kFwdTiles; ++t) {
            if (t < nt) {
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const int ci = lane + kWave * r;
                    store_bf16x8(vw + t * kTileElems + (ci >> 3) * kVStride + (ci & 7) * 8, vr[t][r]);
                }
                st[t] = mfma_bf16_32(kr[t][1], qa1, mfma_bf16_32(kr[t][0], qa0, f32x4{0.f, 0.f, 0.f, 0.f})) * a.sl2;
            }
        }
        softmax_pv_chunk<false>(st, bias, nt, vw, m, lsum, oacc, g, c16);
    }
    // ---- coarse tokens of levels 2..ncl+1, weight B^l, one tile at a time
    for (int ct = 0; ct < nct; ++ct) {
        if (ct > 0) prefetch_coarse(a, idx, fine, pk, pv, h, ib, ct, coarse_pick(a, idx, h, ib, ct, c16), g, c16, cr);
        __bf16 *vrow = vw + c16 * kVStride + 16 * g;
        store_bf16x8(vrow, f32_to_bf16x8(cr.v0, cr.v1));
        store_bf16x8(vrow + 8, f32_to_bf16x8(cr.v2, cr.v3));
        const bf16x8 ka0 = f32_to_bf16x8(cr.k0, cr.k1);
        const bf16x8 ka1 = f32_to_bf16x8(cr.k2, cr.k3);
        st[0] = mfma_bf16_32(ka1, qa1, mfma_bf16_32(ka0, qa0, f32x4{0.f, 0.f, 0.f, 0.f})) * a.sl2;
#pragma unroll
        for (int i = 0; i < 4; ++i) bias[0][i] = cr.bias[i];
        softmax_pv_chunk(st, bias, 1, vw, m, lsum, oacc, g, c16);
    }
    // ---- normalise and store
    lsum = sum4_groups(lsum);
    const float inv = 1.0f / lsum;
    __bf16 *orow = o + head_off + trow(qt, c16) + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        const f32x4 r = oacc[dt] * inv;
        const bf16x4 rb = to_bf16x4(f32x4{r[0], r[1], r[2], r[3]});
        *reinterpret_cast<u32x2 *>(orow + 16 * dt) = __builtin_bit_cast(u32x2, rb);
    }
    if (g == 0) lse[(int64_t)h * a.N + tok_row(a.tm, qt * kBlock + c16)] = (m + log2f(lsum)) * kLn2;
}

// ------------------------------------------------------------ fast path
// K_1 = KT fine tiles and at most 16 coarse entries (one tile) with no pick
// that can be dropped (K_1 < B): the shape of every bf16 workload here.  The 4
// query blocks of a workgroup lie under one level-2 node and share their
// coarse picks, so the workgroup stages that coarse tile once in LDS as bf16
// (pooled K rows for the MFMA operand, V rows for the transposing read).
// Fine and coarse tiles form one softmax chunk: one max, no rescaling, and
// every loop is unrolled.
template <int KT, int ORD>
__global__ __launch_bounds__(256, 3) void attn_fwd_fast_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ pk, const float *__restrict__ pv, const int32_t *__restrict__ idx,
    __bf16 *__restrict__ o, float *__restrict__ lse, FwdArgs a) {
    static_assert(KT % 4 == 0 && KT <= kFwdTiles, "fine tiles are paired within halves");
    constexpr int kHalf = KT / 2;   // V tiles staged at a time (LDS per wave)
    __shared__ __attribute__((aligned(16))) __bf16 vs_all[4][kHalf * kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 qs_all[4][kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 ck[kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 cv[kTileElems];
    __shared__ float cbias[kBlock];
    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t blk0 = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * 4;   // all 4 blocks valid
    const int64_t blk = blk0 + w;
    const int h = (int)(blk0 / a.n1);
    const int ib0 = (int)(blk0 % a.n1);
    const int ib = ib0 + w;
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    const __bf16 *kh = k + head_off;
    const __bf16 *vh = v + head_off;
    __bf16 *vw = vs_all[w];

    // ---- this wave's loads, in the order they are used (the memory counter
    // is waited on in order): the coarse tile's pyramid rows, Q, every fine K
    // tile, then every V tile, each tile as whole 128-byte rows per
    // instruction (lane l: rows l / 8 and l / 8 + 8, 16-byte chunk l % 8);
    // rows reach the MFMA operand layout through LDS
    // element offset (within the head) of row r of sequence block b
    auto trow = [&](int b, int r) { return (int64_t)tok_tile_row<ORD>(a.tm, b, r) * kHeadDim; };
    const int lr = lane >> 3, lc = (lane & 7) * 8;
    // ---- coarse tile, staged by the whole workgroup: thread (entry e, quarter p);
    // its pick and pyramid rows are requested here, written to LDS after the
    // fine scores
    const int ce = threadIdx.x >> 4, cpart = threadIdx.x & 15;   // 16 entries x 16 x 4 columns
    int cj, cpick;
    const bool cok = coarse_locate(a, ce, cj, cpick);
    const int cjs = cok ? cj : 0, cps = cok ? cpick : 0;
    f32x4 ckk, cvv;
    {
        const int anc = ib0 >> (4 * (cjs + 1));                       // ancestor at level js+2
        const int c = idx[a.cl_idx_off[cjs] + ((int64_t)h * a.cl_n[cjs] + anc) * a.cl_k[cjs] + cps];
        const int64_t row = a.cl_pyr_off[cjs] + ((int64_t)h * a.cl_n[cjs] + c) * kHeadDim + 4 * cpart;
        ckk = *reinterpret_cast<const f32x4 *>(pk + row);
        cvv = *reinterpret_cast<const f32x4 *>(pv + row);
    }
    const bf16x8 qr0 = load_bf16x8_nt(q + head_off + trow(ib, lr) + lc);
    const bf16x8 qr1 = load_bf16x8_nt(q + head_off + trow(ib, lr + 8) + lc);
    const int32_t *fine = idx + blk * KT;
    bf16x8 kr[KT][2], vr[KT][2];
    int fp[KT];
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        fp[t] = __builtin_amdgcn_readfirstlane(fine[t]);
        kr[t][0] = load_bf16x8(kh + trow(fp[t], lr) + lc);
        kr[t][1] = load_bf16x8(kh + trow(fp[t], lr + 8) + lc);
    }
#pragma unroll
    for (int t = 0; t < KT; ++t) {
        vr[t][0] = load_bf16x8(vh + trow(fp[t], lr) + lc);
        vr[t][1] = load_bf16x8(vh + trow(fp[t], lr + 8) + lc);
    }
    auto stage_rows = [&](__bf16 *dst, bf16x8 r0, bf16x8 r1) {
        store_bf16x8(dst + (lane >> 3) * kVStride + (lane & 7) * 8, r0);
        store_bf16x8(dst + ((lane >> 3) + 8) * kVStride + (lane & 7) * 8, r1);
    };
    // ---- fine scores: K tiles pass through the V staging slots, kHalf at a
    // time (V stays in registers until its half is staged)
    __bf16 *qw = qs_all[w];
    auto stage_k_half = [&](int half) {
#pragma unroll
        for (int t = 0; t < kHalf; ++t)
            stage_rows(vw + t * kTileElems, kr[half * kHalf + t][0], kr[half * kHalf + t][1]);
    };
    stage_rows(qw, qr0, qr1);
    stage_k_half(0);
    wave_lds_sync();
    const bf16x8 qa0 = load_bf16x8(qw + c16 * kVStride + 8 * g);
    const bf16x8 qa1 = load_bf16x8(qw + c16 * kVStride + 32 + 8 * g);
    f32x4 st[KT];
    auto score_half = [&](int half) {
#pragma unroll
        for (int t = 0; t < kHalf; ++t) {
            const __bf16 *kro = vw + t * kTileElems + c16 * kVStride + 8 * g;
            st[half * kHalf + t] =
                mfma_bf16_32(load_bf16x8(kro + 32), qa1,
                             mfma_bf16_32(load_bf16x8(kro), qa0, f32x4{0.f, 0.f, 0.f, 0.f})) * a.sl2;
        }
    };
    score_half(0);
    wave_lds_sync();
    stage_k_half(1);
    wave_lds_sync();
    score_half(1);
    // the coarse tile goes to LDS only now: its pyramid rows were requested
    // after the fine K rows (their address waits for the pick), and writing
    // it earlier would hold the fine scores until every K row had arrived
    {
        if (!cok) ckk = cvv = f32x4{0.f, 0.f, 0.f, 0.f};
        const bf16x4 kb = to_bf16x4(f32x4{ckk[0], ckk[1], ckk[2], ckk[3]});
        const bf16x4 vb = to_bf16x4(f32x4{cvv[0], cvv[1], cvv[2], cvv[3]});
        *reinterpret_cast<u32x2 *>(&ck[ce * kVStride + 4 * cpart]) = __builtin_bit_cast(u32x2, kb);
        *reinterpret_cast<u32x2 *>(&cv[ce * kVStride + 4 * cpart]) = __builtin_bit_cast(u32x2, vb);
        if (cpart == 0) cbias[ce] = cok ? 4.0f * (float)(cjs + 2) : -INFINITY;
    }
    __syncthreads();   // coarse tile staged
    const __bf16 *ckr = ck + c16 * kVStride;
    f32x4 sc = mfma_bf16_32(load_bf16x8(ckr + 32 + 8 * g), qa1,
                            mfma_bf16_32(load_bf16x8(ckr + 8 * g), qa0, f32x4{0.f, 0.f, 0.f, 0.f})) * a.sl2;
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[i] += cbias[4 * g + i];
    // ---- one softmax over all KT + 1 tiles
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[t][i]);
#pragma unroll
    for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[i]);
    mx = max4_groups(mx);
    float lsum = 0.f;
    f32x4 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int rofs = (4 * g + (c16 >> 2)) * kVStride + 4 * (c16 & 3);
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        wave_lds_sync();
#pragma unroll
        for (int t = 0; t < kHalf; ++t)
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const int ci = lane + kWave * r;
                store_bf16x8(vw + t * kTileElems + (ci >> 3) * kVStride + (ci & 7) * 8, vr[half * kHalf + t][r]);
            }
        wave_lds_sync();
#pragma unroll
        for (int tp = 0; tp < kHalf / 2; ++tp) {
            const int t0 = half * kHalf + 2 * tp;
            float p0[4], p1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p0[i] = fast_exp2(st[t0][i] - mx);
                p1[i] = fast_exp2(st[t0 + 1][i] - mx);
                lsum += p0[i] + p1[i];
            }
            const bf16x8 pb = cat8(to_bf16x4(f32x4{p0[0], p0[1], p0[2], p0[3]}),
                                   to_bf16x4(f32x4{p1[0], p1[1], p1[2], p1[3]}));
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x4 v0 = lds_read_tr4(vw + (2 * tp) * kTileElems + rofs + 16 * dt);
                const bf16x4 v1 = lds_read_tr4(vw + (2 * tp + 1) * kTileElems + rofs + 16 * dt);
                oacc[dt] = mfma_bf16_32(cat8(v0, v1), pb, oacc[dt]);
            }
        }
    }
    {
        float pc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pc[i] = fast_exp2(sc[i] - mx);
            lsum += pc[i];
        }
        const bf16x4 pcb = to_bf16x4(f32x4{pc[0], pc[1], pc[2], pc[3]});
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            oacc[dt] = mfma_bf16_16(lds_read_tr4(cv + rofs + 16 * dt), pcb, oacc[dt]);
    }
    // ---- normalise and store: O (lane: query c16, dims 16 dt + 4 g ..)
    // passes through the free V slot so that the stores write whole rows
    lsum = sum4_groups(lsum);
    const float inv = 1.0f / lsum;
    wave_lds_sync();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        const f32x4 r = oacc[dt] * inv;
        const bf16x4 rb = to_bf16x4(f32x4{r[0], r[1], r[2], r[3]});
        *reinterpret_cast<u32x2 *>(vw + c16 * kVStride + 16 * dt + 4 * g) = __builtin_bit_cast(u32x2, rb);
    }
    wave_lds_sync();
    store_bf16x8_nt(o + head_off + trow(ib, lr) + lc, load_bf16x8(vw + lr * kVStride + lc));
    store_bf16x8_nt(o + head_off + trow(ib, lr + 8) + lc, load_bf16x8(vw + (lr + 8) * kVStride + lc));
    if (g == 0) lse[(int64_t)h * a.N + tok_tile_row<ORD>(a.tm, ib, c16)] = (mx + log2f(lsum)) * kLn2;
}

// ---------------------------------------------------------- chunked path
// The fast path's loads and layout for other shapes (B = 16): any K_1 (fine
// tiles in chunks of 8, the last chunk masked), with a shared coarse tile of at
// most 16 entries (CO) or none (no enrichment).  Every chunk updates the
// running max and rescales (online softmax); the coarse tile comes last.  The
// next chunk's K rows go out half by half as the chunk's V halves are staged,
// and its V rows once the chunk's P V is done, so the loads overlap the work.
// Several chunks need the registers of two waves per SIMD.
template <int NCH, bool CO, int ORD>
__global__ __launch_bounds__(256, NCH == 1 ? 3 : 2) void attn_fwd_chunk_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ pk, const float *__restrict__ pv, const int32_t *__restrict__ idx,
    __bf16 *__restrict__ o, float *__restrict__ lse, FwdArgs a) {
    constexpr int KT = kFwdTiles;
    constexpr int kHalf = KT / 2;   // V tiles staged at a time (LDS per wave)
    __shared__ __attribute__((aligned(16))) __bf16 vs_all[4][kHalf * kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 qs_all[4][kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 ck[CO ? kTileElems : 8];
    __shared__ __attribute__((aligned(16))) __bf16 cv[CO ? kTileElems : 8];
    __shared__ float cbias[kBlock];
    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t blk0 = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * 4;   // all 4 blocks valid
    const int64_t blk = blk0 + w;
    const int h = (int)(blk0 / a.n1);
    const int ib0 = (int)(blk0 % a.n1);
    const int ib = ib0 + w;
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    const __bf16 *kh = k + head_off;
    const __bf16 *vh = v + head_off;
    __bf16 *vw = vs_all[w];
    __bf16 *qw = qs_all[w];
    auto trow = [&](int b, int r) { return (int64_t)tok_tile_row<ORD>(a.tm, b, r) * kHeadDim; };
    const int lr = lane >> 3, lc = (lane & 7) * 8;
    auto stage_rows = [&](__bf16 *dst, bf16x8 r0, bf16x8 r1) {
        store_bf16x8(dst + lr * kVStride + lc, r0);
        store_bf16x8(dst + (lr + 8) * kVStride + lc, r1);
    };
    // Loads go out in the order they are used (the memory counter is waited
    // on in order): Q, the coarse entry's pick, the first chunk's K then V
    // tiles, the coarse pyramid rows.
    const int32_t *fine = idx + blk * a.K1;
    bf16x8 kr[KT][2], vr[KT][2];
    auto chunk_tile = [&](int c0, int t) {   // tiles past the chunk's end re-read its last tile
        return __builtin_amdgcn_readfirstlane(fine[c0 + min(t, min(KT, a.K1 - c0) - 1)]);
    };
    auto load_k = [&](int c0, int t0, int t1) {   // tiles t0 .. t1 - 1
#pragma unroll
        for (int t = t0; t < t1; ++t) {
            const int f = chunk_tile(c0, t);
            kr[t][0] = load_bf16x8(kh + trow(f, lr) + lc);
            kr[t][1] = load_bf16x8(kh + trow(f, lr + 8) + lc);
        }
    };
    auto load_v = [&](int c0) {
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            const int f = chunk_tile(c0, t);
            vr[t][0] = load_bf16x8(vh + trow(f, lr) + lc);
            vr[t][1] = load_bf16x8(vh + trow(f, lr + 8) + lc);
        }
    };
    const bf16x8 qr0 = load_bf16x8_nt(q + head_off + trow(ib, lr) + lc);
    const bf16x8 qr1 = load_bf16x8_nt(q + head_off + trow(ib, lr + 8) + lc);
    const int ce = threadIdx.x >> 4, cpart = threadIdx.x & 15;   // coarse entry, quarter
    int cj = 0, cpick = 0, cc = 0;
    bool cok = false;
    if constexpr (CO) {
        cok = coarse_locate(a, ce, cj, cpick);
        cj = cok ? cj : 0;
        cpick = cok ? cpick : 0;
        const int anc = ib0 >> (4 * (cj + 1));   // ancestor at level cj+2
        cc = idx[a.cl_idx_off[cj] + ((int64_t)h * a.cl_n[cj] + anc) * a.cl_k[cj] + cpick];
    }
    load_k(0, 0, KT);
    load_v(0);
    f32x4 ckk = {0.f, 0.f, 0.f, 0.f}, cvv = ckk;
    if constexpr (CO) {
        const int64_t row = a.cl_pyr_off[cj] + ((int64_t)h * a.cl_n[cj] + cc) * kHeadDim + 4 * cpart;
        ckk = *reinterpret_cast<const f32x4 *>(pk + row);
        cvv = *reinterpret_cast<const f32x4 *>(pv + row);
    }
    stage_rows(qw, qr0, qr1);
    float m = -INFINITY, lsum = 0.f;
    f32x4 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int rofs = (4 * g + (c16 >> 2)) * kVStride + 4 * (c16 & 3);
    wave_lds_sync();
    const bf16x8 qa0 = load_bf16x8(qw + c16 * kVStride + 8 * g);
    const bf16x8 qa1 = load_bf16x8(qw + c16 * kVStride + 32 + 8 * g);
#pragma unroll 1
    for (int c0 = 0; c0 < NCH * KT; c0 += KT) {
        const int nt = min(KT, a.K1 - c0);   // live tiles of this chunk (>= 1)
        const bool more = c0 + KT < a.K1;    // another chunk follows
        f32x4 st[KT];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            wave_lds_sync();
#pragma unroll
            for (int t = 0; t < kHalf; ++t)
                stage_rows(vw + t * kTileElems, kr[half * kHalf + t][0], kr[half * kHalf + t][1]);
            wave_lds_sync();
#pragma unroll
            for (int t = 0; t < kHalf; ++t) {
                const __bf16 *kro = vw + t * kTileElems + c16 * kVStride + 8 * g;
                st[half * kHalf + t] =
                    mfma_bf16_32(load_bf16x8(kro + 32), qa1,
                                 mfma_bf16_32(load_bf16x8(kro), qa0, f32x4{0.f, 0.f, 0.f, 0.f})) * a.sl2;
            }
        }
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < KT; ++t) {
            if (t >= nt) st[t] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[t][i]);
        }
        const float mnew = fmaxf(m, max4_groups(mx));   // finite: tile 0 of a chunk is live
        const float alpha = fast_exp2(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            wave_lds_sync();
#pragma unroll
            for (int t = 0; t < kHalf; ++t)
                stage_rows(vw + t * kTileElems, vr[half * kHalf + t][0], vr[half * kHalf + t][1]);
            // this half of the V rows is staged: the next chunk's K rows of the same half go out
            if (more) load_k(c0 + KT, half * kHalf, (half + 1) * kHalf);
            wave_lds_sync();
#pragma unroll
            for (int tp = 0; tp < kHalf / 2; ++tp) {
                const int t0 = half * kHalf + 2 * tp;
                float p0[4], p1[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p0[i] = fast_exp2(st[t0][i] - m);
                    p1[i] = fast_exp2(st[t0 + 1][i] - m);
                    lsum += p0[i] + p1[i];
                }
                const bf16x8 pb = cat8(to_bf16x4(f32x4{p0[0], p0[1], p0[2], p0[3]}),
                                       to_bf16x4(f32x4{p1[0], p1[1], p1[2], p1[3]}));
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x4 v0 = lds_read_tr4(vw + (2 * tp) * kTileElems + rofs + 16 * dt);
                    const bf16x4 v1 = lds_read_tr4(vw + (2 * tp + 1) * kTileElems + rofs + 16 * dt);
                    oacc[dt] = mfma_bf16_32(cat8(v0, v1), pb, oacc[dt]);
                }
            }
        }
        if (more) load_v(c0 + KT);
    }
    if constexpr (CO) {
        // coarse tile, staged by the whole workgroup: thread (entry e, quarter p)
        if (!cok) ckk = cvv = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<u32x2 *>(&ck[ce * kVStride + 4 * cpart]) = __builtin_bit_cast(u32x2, to_bf16x4(ckk));
        *reinterpret_cast<u32x2 *>(&cv[ce * kVStride + 4 * cpart]) = __builtin_bit_cast(u32x2, to_bf16x4(cvv));
        if (cpart == 0) cbias[ce] = cok ? 4.0f * (float)(cj + 2) : -INFINITY;
        __syncthreads();
        const __bf16 *ckr = ck + c16 * kVStride;
        f32x4 sc = mfma_bf16_32(load_bf16x8(ckr + 32 + 8 * g), qa1,
                                mfma_bf16_32(load_bf16x8(ckr + 8 * g), qa0, f32x4{0.f, 0.f, 0.f, 0.f})) * a.sl2;
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] += cbias[4 * g + i];
            if (drop_possible(a)) {
                // a level-2 pick whose 16 children are all fine picks of this
                // block is dropped for it (only level 2 can be covered: K_1 <= 32)
                int j2, p2;
                if (coarse_locate(a, 4 * g + i, j2, p2) && j2 == 0) {
                    const int c = idx[a.cl_idx_off[0] + ((int64_t)h * a.cl_n[0] + (ib >> 4)) * a.cl_k[0] + p2];
                    int cov = 0;
                    for (int f = 0; f < a.K1; ++f) cov += (fine[f] >> 4) == c ? 1 : 0;
                    if (cov == kBlock) sc[i] = -INFINITY;
                }
            }
            mx = fmaxf(mx, sc[i]);
        }
        const float mnew = fmaxf(m, max4_groups(mx));   // finite: the fine tiles came first
        const float alpha = fast_exp2(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
        float pc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pc[i] = fast_exp2(sc[i] - m);
            lsum += pc[i];
        }
        const bf16x4 pcb = to_bf16x4(f32x4{pc[0], pc[1], pc[2], pc[3]});
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            oacc[dt] = mfma_bf16_16(lds_read_tr4(cv + rofs + 16 * dt), pcb, oacc[dt]);
    }
    // ---- normalise and store (whole rows through the free V slot)
    lsum = sum4_groups(lsum);
    const float inv = 1.0f / lsum;
    wave_lds_sync();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        const f32x4 r = oacc[dt] * inv;
        *reinterpret_cast<u32x2 *>(vw + c16 * kVStride + 16 * dt + 4 * g) = __builtin_bit_cast(u32x2, to_bf16x4(r));
    }
    wave_lds_sync();
    store_bf16x8_nt(o + head_off + trow(ib, lr) + lc, load_bf16x8(vw + lr * kVStride + lc));
    store_bf16x8_nt(o + head_off + trow(ib, lr + 8) + lc, load_bf16x8(vw + (lr + 8) * kVStride + lc));
    if (g == 0) lse[(int64_t)h * a.N + tok_tile_row<ORD>(a.tm, ib, c16)] = (m + log2f(lsum)) * kLn2;
}

// ------------------------------------------------------ blocks of 64 tokens
// One workgroup per query block of B = 64, one wave per 16-query tile of it.
// The 4 tiles share the block's picks, so the workgroup loads each picked key
// block (4 key tiles, K and V) once into LDS -- each wave one tile, as whole
// rows -- and all four waves attend to it: a quarter of the gathers of one
// wave per tile.  Picked blocks alternate between two LDS buffers (the next
// block's rows are in flight while one is used) under an online softmax; a
// coarse tile of at most 16 entries, shared by the block, goes first.  K_1 <
// B, so no coarse pick can be covered.
template <int ORD>
__global__ __launch_bounds__(256, 2) void attn_fwd_b64_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ pk, const float *__restrict__ pv, const int32_t *__restrict__ idx,
    __bf16 *__restrict__ o, float *__restrict__ lse, FwdArgs a) {
    constexpr int kSub = 4;   // tiles per block
    __shared__ __attribute__((aligned(16))) __bf16 kbuf[2][kSub][kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 vbuf[2][kSub][kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 qs_all[kSub][kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 ck[kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 cv[kTileElems];
    __shared__ float cbias[kBlock];
    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t blk = xcd_remap(blockIdx.x, gridDim.x);   // query block
    const int h = (int)(blk / a.n1);
    const int ib = (int)(blk % a.n1);
    const int qt = ib * kSub + w;   // this wave's query tile
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    const __bf16 *kh = k + head_off;
    const __bf16 *vh = v + head_off;
    auto trow = [&](int b, int r) { return (int64_t)tok_tile_row<ORD>(a.tm, b, r) * kHeadDim; };
    const int lr = lane >> 3, lc = (lane & 7) * 8;
    auto stage_rows = [&](__bf16 *dst, bf16x8 r0, bf16x8 r1) {
        store_bf16x8(dst + lr * kVStride + lc, r0);
        store_bf16x8(dst + (lr + 8) * kVStride + lc, r1);
    };
    __bf16 *qw = qs_all[w];
    stage_rows(qw, load_bf16x8_nt(q + head_off + trow(qt, lr) + lc),
               load_bf16x8_nt(q + head_off + trow(qt, lr + 8) + lc));
    const int32_t *fine = idx + blk * a.K1;
    // wave w's tile of picked block j, as whole rows
    bf16x8 kr[2], vr[2];
    auto load_tile = [&](int j) {
        const int f = __builtin_amdgcn_readfirstlane(fine[j]) * kSub + w;
        const int64_t o0 = trow(f, lr) + lc, o1 = trow(f, lr + 8) + lc;
        kr[0] = load_bf16x8(kh + o0);
        kr[1] = load_bf16x8(kh + o1);
        vr[0] = load_bf16x8(vh + o0);
        vr[1] = load_bf16x8(vh + o1);
    };
    load_tile(0);
    if (a.ncoarse > 0) {   // coarse tile, staged by the whole workgroup: thread (entry e, quarter p)
        const int e = threadIdx.x >> 4, part = threadIdx.x & 15;
        int j, pick;
        const bool ok = coarse_locate(a, e, j, pick);
        const int js = ok ? j : 0, ps = ok ? pick : 0;
        const int c = idx[a.cl_idx_off[js] + ((int64_t)h * a.cl_n[js] + ib / a.cl_span[js]) * a.cl_k[js] + ps];
        const int64_t row = a.cl_pyr_off[js] + ((int64_t)h * a.cl_n[js] + c) * kHeadDim + 4 * part;
        f32x4 kk = *reinterpret_cast<const f32x4 *>(pk + row);
        f32x4 vv = *reinterpret_cast<const f32x4 *>(pv + row);
        if (!ok) kk = vv = f32x4{0.f, 0.f, 0.f, 0.f};
        *reinterpret_cast<u32x2 *>(&ck[e * kVStride + 4 * part]) = __builtin_bit_cast(u32x2, to_bf16x4(kk));
        *reinterpret_cast<u32x2 *>(&cv[e * kVStride + 4 * part]) = __builtin_bit_cast(u32x2, to_bf16x4(vv));
        if (part == 0) cbias[e] = ok ? a.lgB * (float)(js + 2) : -INFINITY;
    }
    wave_lds_sync();
    const bf16x8 qa0 = load_bf16x8(qw + c16 * kVStride + 8 * g);
    const bf16x8 qa1 = load_bf16x8(qw + c16 * kVStride + 32 + 8 * g);
    const int rofs = (4 * g + (c16 >> 2)) * kVStride + 4 * (c16 & 3);
    float m = -INFINITY, lsum = 0.f;
    f32x4 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (a.ncoarse > 0) {
        __syncthreads();   // coarse tile staged
        const __bf16 *ckr = ck + c16 * kVStride;
        f32x4 sc = mfma_bf16_32(load_bf16x8(ckr + 32 + 8 * g), qa1,
                                mfma_bf16_32(load_bf16x8(ckr + 8 * g), qa0, f32x4{0.f, 0.f, 0.f, 0.f})) * a.sl2;
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] += cbias[4 * g + i];
            mx = fmaxf(mx, sc[i]);
        }
        m = max4_groups(mx);   // entry 0 exists
        float pc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pc[i] = fast_exp2(sc[i] - m);
            lsum += pc[i];
        }
        const bf16x4 pcb = to_bf16x4(f32x4{pc[0], pc[1], pc[2], pc[3]});
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            oacc[dt] = mfma_bf16_16(lds_read_tr4(cv + rofs + 16 * dt), pcb, oacc[dt]);
    }
    for (int j = 0; j < a.K1; ++j) {
        const int buf = j & 1;
        stage_rows(kbuf[buf][w], kr[0], kr[1]);
        stage_rows(vbuf[buf][w], vr[0], vr[1]);
        // all four tiles of block j staged; every wave is done with block j - 2
        __syncthreads();
        if (j + 1 < a.K1) load_tile(j + 1);   // the next block in flight
        f32x4 st[kSub];
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < kSub; ++t) {
            const __bf16 *kro = kbuf[buf][t] + c16 * kVStride + 8 * g;
            st[t] = mfma_bf16_32(load_bf16x8(kro + 32), qa1,
                                 mfma_bf16_32(load_bf16x8(kro), qa0, f32x4{0.f, 0.f, 0.f, 0.f})) * a.sl2;
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[t][i]);
        }
        const float mnew = fmaxf(m, max4_groups(mx));
        const float alpha = fast_exp2(m - mnew);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
#pragma unroll
        for (int tp = 0; tp < kSub / 2; ++tp) {
            float p0[4], p1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p0[i] = fast_exp2(st[2 * tp][i] - m);
                p1[i] = fast_exp2(st[2 * tp + 1][i] - m);
                lsum += p0[i] + p1[i];
            }
            const bf16x8 pb = cat8(to_bf16x4(f32x4{p0[0], p0[1], p0[2], p0[3]}),
                                   to_bf16x4(f32x4{p1[0], p1[1], p1[2], p1[3]}));
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x4 v0 = lds_read_tr4(vbuf[buf][2 * tp] + rofs + 16 * dt);
                const bf16x4 v1 = lds_read_tr4(vbuf[buf][2 * tp + 1] + rofs + 16 * dt);
                oacc[dt] = mfma_bf16_32(cat8(v0, v1), pb, oacc[dt]);
            }
        }
    }
    // ---- normalise and store (whole rows through the wave's Q slot)
    lsum = sum4_groups(lsum);
    const float inv = 1.0f / lsum;
    wave_lds_sync();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        const f32x4 r = oacc[dt] * inv;
        *reinterpret_cast<u32x2 *>(qw + c16 * kVStride + 16 * dt + 4 * g) = __builtin_bit_cast(u32x2, to_bf16x4(r));
    }
    wave_lds_sync();
    store_bf16x8_nt(o + head_off + trow(qt, lr) + lc, load_bf16x8(qw + lr * kVStride + lc));
    store_bf16x8_nt(o + head_off + trow(qt, lr + 8) + lc, load_bf16x8(qw + (lr + 8) * kVStride + lc));
    if (g == 0) lse[(int64_t)h * a.N + tok_tile_row<ORD>(a.tm, qt, c16)] = (m + log2f(lsum)) * kLn2;
}

// ---------------------------------------------------------------- f32 path
// Float32 inputs on the matrix cores (v_mfma_f32_16x16x4_f32): one wave per
// 16-query tile, any block size, fine-tile count and number of coarse tiles,
// and no LDS.  Scores are computed transposed, S^T = K Q^T, so lane (g, c)
// holds query c against keys 4g .. 4g + 3 of a key tile; Q and K come in the
// row layout (load_row16).  O^T += V^T P^T takes P straight from the score
// registers: step i of a key tile pairs key 4g + i of lane group g with the
// V rows in the column layout (lane (g, c): dims 4c .. 4c + 3 of row 4g + i,
// four whole rows per load instruction), and output row r of dim chunk dt
// stands for dim 4r + dt, so that lane (g, c) ends with dims 16g .. 16g + 15
// of query c.  The softmax runs online, key tile by key tile.
__global__ __launch_bounds__(256) void attn_fwd_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ pk, const float *__restrict__ pv, const int32_t *__restrict__ idx,
    float *__restrict__ o, float *__restrict__ lse, FwdArgs a) {
    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t blk = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * 4 + w;   // query tile
    if (blk >= (int64_t)a.bh * a.nt1) return;
    const int h = (int)(blk / a.nt1);
    const int qt = (int)(blk % a.nt1);
    const int ib = qt / a.sub;   // its query block
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    const float *kh = k + head_off;
    const float *vh = v + head_off;
    // element offset (within the head) of row r of 16-token tile b
    auto trow = [&](int b, int r) { return (int64_t)tok_row(a.tm, b * kBlock + r) * kHeadDim; };
    float qf[16];
    load_row16(q + head_off + trow(qt, c16) + 16 * g, qf);
    const int32_t *fine = idx + ((int64_t)h * a.n1 + ib) * a.K1;
    const int nft = a.K1 * a.sub;   // fine key tiles: sub-tile t % sub of pick t / sub
    const int nct = (a.ncoarse + kBlock - 1) / kBlock;

    float m = -INFINITY, lsum = 0.f;
    f32x4 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    struct KV {
        float kr[16];   // K row c (row layout)
        f32x4 vc[4];    // V rows 4g + i, dims 4c .. 4c + 3 (column layout)
    };
    auto load_fine = [&](int tt, KV &T) {
        const int f = __builtin_amdgcn_readfirstlane(fine[tt / a.sub]) * a.sub + tt % a.sub;
        load_row16(kh + trow(f, c16) + 16 * g, T.kr);
#pragma unroll
        for (int i = 0; i < 4; ++i) T.vc[i] = *reinterpret_cast<const f32x4 *>(vh + trow(f, 4 * g + i) + 4 * c16);
    };
    // one key tile; bias: log2 weight of keys 4g + i (-inf masks a key)
    auto attend = [&](const KV &T, const float (&bias)[4]) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int d = 0; d < 16; ++d) s = mfma_f32_4(T.kr[d], qf[d], s);
        float z[4], mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            z[i] = s[i] * a.sl2 + bias[i];
            mx = fmaxf(mx, z[i]);
        }
        mx = max4_groups(mx);
        const float mnew = fmaxf(m, mx);
        const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
        const float alpha = fast_exp2(m - msafe);
        m = mnew;
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(z[i] - msafe);
            lsum += p;
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) oacc[dt] = mfma_f32_4(T.vc[i][dt], p, oacc[dt]);
        }
    };
    // ---- fine key tiles, weight 1: two register sets, the next tile's loads
    // in flight while a tile is computed
    const float nobias[4] = {0.f, 0.f, 0.f, 0.f};
    KV T0, T1;
    if (nft > 0) load_fine(0, T0);
    for (int tt = 0; tt < nft; tt += 2) {
        if (tt + 1 < nft) load_fine(tt + 1, T1);
        attend(T0, nobias);
        if (tt + 2 < nft) load_fine(tt + 2, T0);
        if (tt + 1 < nft) attend(T1, nobias);
    }
    // ---- coarse tokens of levels 2..ncl+1, weight B^l, 16 entries a tile;
    // absent or dropped entries read row 0 of the pyramid and are masked
    for (int ct = 0; ct < nct; ++ct) {
        KV T;
        float bias[4];
        int64_t roff = 0;
        float bb;
        const bool okk = coarse_entry(a, idx, fine, h, ib, ct * kBlock + c16, roff, bb);
        load_row16(pk + (okk ? roff : 0) + 16 * g, T.kr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int64_t ri = 0;
            float bi = 0.f;
            const bool ok = coarse_entry(a, idx, fine, h, ib, ct * kBlock + 4 * g + i, ri, bi);
            T.vc[i] = *reinterpret_cast<const f32x4 *>(pv + (ok ? ri : 0) + 4 * c16);
            if (!ok) T.vc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
            bias[i] = ok ? bi : -INFINITY;
        }
        attend(T, bias);
    }
    // ---- normalise and store: lane (g, c) writes dims 16g .. 16g + 15 of query c
    lsum = sum4_groups(lsum);
    const float inv = 1.0f / lsum;
    float *orow = o + head_off + trow(qt, c16) + 16 * g;
#pragma unroll
    for (int j = 0; j < 4; ++j)
        *reinterpret_cast<f32x4 *>(orow + 4 * j) = f32x4{oacc[0][j], oacc[1][j], oacc[2][j], oacc[3][j]} * inv;
    if (g == 0) lse[(int64_t)h * a.N + tok_row(a.tm, qt * kBlock + c16)] = (m + log2f(lsum)) * kLn2;
}

hipError_t launch_attn_fwd(const Geometry &g, const void *q, const void *k, const void *v,
                           const float *pk, const float *pv, const int32_t *idx, void *o,
                           float *lse, hipStream_t s) {
    const FwdArgs a = make_fwd_args(g);
    if (g.bf16) {
        const int64_t blocks = (int64_t)g.bh * g.n[1];
        const int64_t tiles = (int64_t)g.bh * a.nt1;
        const bool fast = g.B == kBlock && g.L >= 2 && a.K1 == 8 && a.ncoarse > 0 &&
                          a.ncoarse <= kBlock && !drop_possible(a) && a.n1 % 4 == 0;
        // any K_1 and at most one coarse tile, in chunks of 8 fine tiles
        const bool chunked = g.B == kBlock && a.n1 % 4 == 0 && a.ncoarse <= kBlock && a.K1 <= 4 * kFwdTiles;
        const int nch = (a.K1 + kFwdTiles - 1) / kFwdTiles;
        const bool co = a.ncoarse > 0;
        using Kern = void (*)(const __bf16 *, const __bf16 *, const __bf16 *, const float *, const float *,
                              const int32_t *, __bf16 *, float *, FwdArgs);
        Kern kern = nullptr;
        if (fast)
            kern = g.order == 0 ? attn_fwd_fast_kernel<8, 0> : attn_fwd_fast_kernel<8, 1>;
        else if (g.B == 4 * kBlock && a.ncoarse <= kBlock) {   // one workgroup per query block
            hipLaunchKernelGGL(g.order == 0 ? attn_fwd_b64_kernel<0> : attn_fwd_b64_kernel<1>,
                               dim3((unsigned)blocks), dim3(256), 0, s, (const __bf16 *)q,
                               (const __bf16 *)k, (const __bf16 *)v, pk, pv, idx, (__bf16 *)o, lse, a);
            return hipGetLastError();
        } else if (chunked) {
            static const Kern table[2][2][4] = {
                {{attn_fwd_chunk_kernel<1, false, 0>, attn_fwd_chunk_kernel<2, false, 0>,
                  attn_fwd_chunk_kernel<3, false, 0>, attn_fwd_chunk_kernel<4, false, 0>},
                 {attn_fwd_chunk_kernel<1, true, 0>, attn_fwd_chunk_kernel<2, true, 0>,
                  attn_fwd_chunk_kernel<3, true, 0>, attn_fwd_chunk_kernel<4, true, 0>}},
                {{attn_fwd_chunk_kernel<1, false, 1>, attn_fwd_chunk_kernel<2, false, 1>,
                  attn_fwd_chunk_kernel<3, false, 1>, attn_fwd_chunk_kernel<4, false, 1>},
                 {attn_fwd_chunk_kernel<1, true, 1>, attn_fwd_chunk_kernel<2, true, 1>,
                  attn_fwd_chunk_kernel<3, true, 1>, attn_fwd_chunk_kernel<4, true, 1>}}};
            kern = table[g.order][co ? 1 : 0][nch - 1];
        }
        if (kern != nullptr)
            hipLaunchKernelGGL(kern, dim3((unsigned)(blocks / 4)), dim3(256), 0, s, (const __bf16 *)q,
                               (const __bf16 *)k, (const __bf16 *)v, pk, pv, idx, (__bf16 *)o, lse, a);
        else
            hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0,
                               s, (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, pk, pv, idx,
                               (__bf16 *)o, lse, a);
    } else {
        const int64_t tiles = (int64_t)g.bh * a.nt1;
        hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0,
                           s, (const float *)q, (const float *)k, (const float *)v, pk, pv, idx,
                           (float *)o, lse, a);
    }
    return hipGetLastError();
}

}  // namespace llsa
