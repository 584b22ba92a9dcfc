// Backward pass of the enriched sparse attention for the loss <O, dO> with
// the picks held fixed ("Trainable Log-linear Sparse Attention for Efficient
// Diffusion Transformers", explainer "Step 4: Efficient Sparse Index
// Transpose": the key-major index lists drive the key-side gradients, no
// dense mask is ever formed).
//
// Work is organised by 16-token tiles; a block of B = 64 tokens is 4 tiles
// that share its picks.  Three passes:
//  A  query-major (one wave per query tile, a workgroup per 16 tiles, which
//     lie under one level-2 node):
//     D = rowsum(dO * O) -- formed in float32 as sum_j P_j dP_j over the
//     attended set, which is the same value without the rounding of the
//     stored bf16 O (float32 inputs read O) --, dQ over fine and coarse keys,
//     and the coarse-token
//     gradient partials summed over the workgroup's query tiles (every tile
//     under one level-2 node shares its coarse picks).
//  B  coarse reduce: for every pooled token c of level l, sum the partials of
//     the level-l rows that picked c, read from the CSR of I^(l).
//  C  key-major (one wave per key tile): dK, dV of the tile's 16 tokens
//     from the query blocks in its block's CSR(I^(1)) segment, plus the pooled-token
//     gradients of every coarse level spread back through the mean (each of
//     the B^l tokens under a pooled token receives 1/B^l of its gradient).
// Accumulation order is fixed everywhere (no float atomics), so results are
// bitwise reproducible.  Rows a pass reads or writes once (its own Q and dO
// or K and V, and the gradients) use non-temporal loads and stores, leaving
// the L2 to the gathered tiles.
#include "common.hpp"
#include "internal.hpp"

namespace llsa {

constexpr int kMaxCoarseLv = kMaxLevels - 1;
constexpr int kTS = 72;              // bf16 LDS row stride (144 B)
constexpr int kTE = kBlock * kTS;    // elements of one staged 16 x 64 tile

struct BwdArgs {
    int bh, N, n1, K1;
    int sub;      // 16-token tiles per block (B / 16)
    int nt1;      // tiles per head, n1 * sub
    int npg;      // partial groups (16 consecutive query tiles) per head
    float lgB;    // log2(B)
    float invB;   // 1 / B
    int ncl, ncoarse;
    int cl_n[kMaxCoarseLv], cl_k[kMaxCoarseLv], cl_span[kMaxCoarseLv], cl_entry0[kMaxCoarseLv];
    int cl_groups[kMaxCoarseLv];          // partial groups under one token of the level
    int64_t cl_idx_off[kMaxCoarseLv], cl_pyr_off[kMaxCoarseLv];
    int64_t cl_ptr_off[kMaxCoarseLv], cl_col_off[kMaxCoarseLv];
    int64_t cl_grad_off[kMaxCoarseLv];   // float offset of level in dpk / dpv
    float scale, sl2;
    int drop;
    int grad_bf16;
    TokMap tm;   // storage row of a sequence position (D stays in sequence order)
};

struct BwdWs {
    float *D;        // [bh, N]
    float *partial;  // [bh * npg, ncoarse, 2, 64]
    float *dpk;      // coarse-level gradients, per level [bh, n_l, 64]
    float *dpv;
};

static BwdArgs make_bwd_args(const Geometry &g) {
    BwdArgs a{};
    a.bh = g.bh;
    a.N = g.N;
    a.n1 = g.n[1];
    a.K1 = g.kl[1];
    a.sub = g.sub;
    a.nt1 = g.n[1] * g.sub;
    a.npg = g.L >= 2 ? a.nt1 / kBlock : 0;   // B^2 / 16 is a multiple of 16
    a.lgB = (float)g.lgB;
    a.invB = 1.0f / (float)g.B;
    a.ncl = g.Le < g.L - 1 ? g.Le : g.L - 1;
    a.ncoarse = 0;
    int64_t span = 1, goff = 0;
    for (int j = 0; j < a.ncl; ++j) {
        const int l = j + 2;
        span *= g.B;
        a.cl_n[j] = g.n[l];
        a.cl_k[j] = g.kl[l];
        a.cl_span[j] = (int)span;
        a.cl_groups[j] = (int)(span * g.sub / kBlock);
        a.cl_entry0[j] = a.ncoarse;
        a.cl_idx_off[j] = g.idx_off[l];
        a.cl_pyr_off[j] = g.pyr_off[l];
        a.cl_ptr_off[j] = g.ptr_off[l];
        a.cl_col_off[j] = g.col_off[l];
        a.cl_grad_off[j] = goff;
        goff += (int64_t)g.bh * g.n[l] * kHeadDim;
        a.ncoarse += g.kl[l];
    }
    a.scale = g.scale;
    a.sl2 = g.scale * kLog2e;
    a.drop = g.drop_covered;
    a.grad_bf16 = g.grad_bf16 ? 1 : 0;
    a.tm = TokMap{g.order, g.log2S};
    return a;
}

static BwdWs carve_ws(const Geometry &g, const BwdArgs &a, void *ws) {
    BwdWs w{};
    char *p = (char *)ws;
    auto take = [&](size_t bytes) {
        char *r = p;
        p += (bytes + 255) / 256 * 256;
        return (float *)r;
    };
    w.D = take(sizeof(float) * (size_t)g.bh * g.N);
    w.partial = take(sizeof(float) * (size_t)g.bh * (size_t)a.npg * a.ncoarse * 2 * kHeadDim);
    size_t coarse = 0;
    for (int j = 0; j < a.ncl; ++j) coarse += (size_t)g.bh * a.cl_n[j] * kHeadDim;
    w.dpk = take(sizeof(float) * coarse);
    w.dpv = take(sizeof(float) * coarse);
    return w;
}

size_t bwd_workspace_bytes(const Geometry &g) {
    const BwdArgs a = make_bwd_args(g);
    size_t total = 0;
    auto add = [&](size_t bytes) { total += (bytes + 255) / 256 * 256; };
    add(sizeof(float) * (size_t)g.bh * g.N);
    add(sizeof(float) * (size_t)g.bh * (size_t)a.npg * a.ncoarse * 2 * kHeadDim);
    size_t coarse = 0;
    for (int j = 0; j < a.ncl; ++j) coarse += (size_t)g.bh * a.cl_n[j] * kHeadDim;
    add(sizeof(float) * coarse);
    add(sizeof(float) * coarse);
    return total;
}

// Coarse entry e of query block ib: level slot j, pooled token c, log2 weight;
// false when the entry does not exist or is dropped for this block.
__device__ __forceinline__ bool bwd_coarse_entry(const BwdArgs &a, const int32_t *__restrict__ idx,
                                                 const int32_t *__restrict__ fine, int h, int ib,
                                                 int e, int &j, int &c, float &bias) {
    if (e >= a.ncoarse) return false;
    j = 0;
    int pick = e;
    while (j < a.ncl - 1 && pick >= a.cl_k[j]) {
        pick -= a.cl_k[j];
        ++j;
    }
    const int span = a.cl_span[j];
    c = idx[a.cl_idx_off[j] + ((int64_t)h * a.cl_n[j] + ib / span) * a.cl_k[j] + pick];
    bias = a.lgB * (float)(j + 2);
    if (a.drop && a.K1 >= span) {
        int cov = 0;
        for (int f = 0; f < a.K1; ++f) cov += (fine[f] / span == c) ? 1 : 0;
        if (cov == span) return false;
    }
    return true;
}

__device__ __forceinline__ void store_grad4(void *base, int64_t off, f32x4 v, int bf) {
    if (bf) {
        const bf16x4 b = to_bf16x4(f32x4{v[0], v[1], v[2], v[3]});
        __builtin_nontemporal_store(__builtin_bit_cast(u32x2, b), reinterpret_cast<u32x2 *>((__bf16 *)base + off));
    } else {
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>((float *)base + off));
    }
}
__device__ __forceinline__ void store_grad1(void *base, int64_t off, float v, int bf) {
    if (bf)
        ((__bf16 *)base)[off] = (__bf16)v;
    else
        ((float *)base)[off] = v;
}

__device__ __forceinline__ float bf_lo(uint32_t x) { return __builtin_bit_cast(float, x << 16); }
__device__ __forceinline__ float bf_hi(uint32_t x) { return __builtin_bit_cast(float, x & 0xffff0000u); }

__device__ __forceinline__ float dot8(bf16x8 a, bf16x8 b) {
    const u32x4 x = __builtin_bit_cast(u32x4, a), y = __builtin_bit_cast(u32x4, b);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) s += bf_lo(x[j]) * bf_lo(y[j]) + bf_hi(x[j]) * bf_hi(y[j]);
    return s;
}

// ================================================================ pass A
// x ~= hi + lo with both parts in bf16 (relative error about 2^-17): the
// gradient contractions run as two bf16 MFMAs so that rounding dS or P to
// bf16 does not limit the accuracy of sums over hundreds of queries.
// The empty asm statements pin each packed pair in its register: without
// them the compiler re-converts element by element and re-packs with
// v_perm_b32 wherever the value feeds a 16x16x16 MFMA operand.
__device__ __forceinline__ void split4(const float (&x)[4], bf16x4 &hi, bf16x4 &lo) {
    const f32x4 xv = {x[0], x[1], x[2], x[3]};
    u32x2 hb = __builtin_bit_cast(u32x2, to_bf16x4(xv));
    asm("" : "+v"(hb));
    const f32x4 back = {__builtin_bit_cast(float, hb[0] << 16),   // hi widened back by shifts
                        __builtin_bit_cast(float, hb[0] & 0xffff0000u),
                        __builtin_bit_cast(float, hb[1] << 16),
                        __builtin_bit_cast(float, hb[1] & 0xffff0000u)};
    u32x2 lb = __builtin_bit_cast(u32x2, to_bf16x4(xv - back));
    asm("" : "+v"(lb));
    hi = __builtin_bit_cast(bf16x4, hb);
    lo = __builtin_bit_cast(bf16x4, lb);
}

// Operand rows of coarse tile ct for query block ib: lane row = entry ct*16+c16.
struct CoarseTile {
    bf16x8 ka0, ka1, va0, va1;  // pooled K / V rows (bf16) as MFMA operands
    float bias_row;             // log2 weight of entry c16, -inf if absent / dropped
    float bias4[4];             // same for entries 4g+i
};

__device__ __forceinline__ void load_coarse_tile(const BwdArgs &a, const float *__restrict__ pk,
                                                 const float *__restrict__ pv,
                                                 const int32_t *__restrict__ idx,
                                                 const int32_t *__restrict__ fine, int h, int ib,
                                                 int ct, int g, int c16, CoarseTile &T) {
    int jl, cc;
    float bias;
    const bool ok = bwd_coarse_entry(a, idx, fine, h, ib, ct * kBlock + c16, jl, cc, bias);
    f32x4 k0 = {0.f, 0.f, 0.f, 0.f}, k1 = k0, k2 = k0, k3 = k0, v0 = k0, v1 = k0, v2 = k0, v3 = k0;
    if (ok) {
        const int64_t roff = a.cl_pyr_off[jl] + ((int64_t)h * a.cl_n[jl] + cc) * kHeadDim;
        const f32x4 *ks = reinterpret_cast<const f32x4 *>(pk + roff);
        const f32x4 *vsrc = reinterpret_cast<const f32x4 *>(pv + roff);
        k0 = ks[2 * g];
        k1 = ks[2 * g + 1];
        k2 = ks[8 + 2 * g];
        k3 = ks[8 + 2 * g + 1];
        v0 = vsrc[2 * g];
        v1 = vsrc[2 * g + 1];
        v2 = vsrc[8 + 2 * g];
        v3 = vsrc[8 + 2 * g + 1];
    }
    T.bias_row = ok ? bias : -INFINITY;
    T.ka0 = f32_to_bf16x8(k0, k1);
    T.ka1 = f32_to_bf16x8(k2, k3);
    T.va0 = f32_to_bf16x8(v0, v1);
    T.va1 = f32_to_bf16x8(v2, v3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int j2, c2;
        float b2;
        T.bias4[i] = bwd_coarse_entry(a, idx, fine, h, ib, ct * kBlock + 4 * g + i, j2, c2, b2) ? b2 : -INFINITY;
    }
}

// One workgroup (4 waves) per 16 consecutive query tiles (a level-2 node for
// B = 16), wave w taking tiles w, w + 4, w + 8, w + 12 in turn, so that the
// four waves work on neighbouring tiles at any time; the fine key tiles of a query tile
// stream through two register sets (the next tile's K / V are in flight while
// the current one is computed).
template <int NCT>
__global__ __launch_bounds__(256, 2) void bwd_dq_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ pk, const float *__restrict__ pv, const int32_t *__restrict__ idx,
    const float *__restrict__ lse, const __bf16 *__restrict__ dout, void *__restrict__ dq, BwdWs ws,
    BwdArgs a) {
    constexpr int NT = NCT > 0 ? NCT : 1;
    constexpr int kTileBytes = 4 * (3 + NT) * kTE * 2;
    constexpr int kRedBytes = 4 * 2 * kBlock * kHeadDim * 4;   // one coarse tile at a time
    __shared__ __attribute__((aligned(16))) char smem[kTileBytes > kRedBytes ? kTileBytes : kRedBytes];
    __shared__ float lds_row[4][2][kBlock];  // per query: lse2, D
    typedef __bf16 Tile[kTE];
    Tile *lds_k = reinterpret_cast<Tile *>(smem);
    Tile *lds_q = lds_k + 4;
    Tile *lds_do = lds_q + 4;
    Tile(*lds_ck)[NT] = reinterpret_cast<Tile(*)[NT]>(lds_do + 4);
    typedef float RedTile[2][kBlock * kHeadDim];
    RedTile *lds_red = reinterpret_cast<RedTile *>(smem);

    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int groups_per_head = (a.nt1 + kBlock - 1) / kBlock;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = bid / groups_per_head;
    const int G = bid % groups_per_head;
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const int nft = a.K1 * a.sub;   // fine key tiles: sub-tile t % sub of pick t / sub

    f32x4 dkc[NT][4], dvc[NT][4];
#pragma unroll
    for (int ct = 0; ct < NT; ++ct)
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            dkc[ct][dt] = zero4;
            dvc[ct][dt] = zero4;
        }

    const int rofs = (4 * g + (c16 >> 2)) * kTS + 4 * (c16 & 3);  // transposed-read address
    struct TileRegs {
        bf16x8 ka0, ka1, va0, va1;
    };
    for (int jb = 0; jb < 4; ++jb) {
        const int qt = G * kBlock + jb * 4 + w;   // query tile: the waves take neighbours at a time
        if (qt >= a.nt1) break;
        const int ib = qt / a.sub;                // its query block
        const int64_t row = (int64_t)qt * kBlock + c16;          // sequence position
        const int64_t srow = tok_row(a.tm, qt * kBlock + c16);   // its storage row
        const __bf16 *qrow = q + head_off + srow * kHeadDim;
        const __bf16 *drow = dout + head_off + srow * kHeadDim;
        const int32_t *fine = idx + ((int64_t)h * a.n1 + ib) * a.K1;
        auto load_tile = [&](int t, TileRegs &R) {
            const int tt = min(t, nft - 1);
            const int f = __builtin_amdgcn_readfirstlane(fine[tt / a.sub]) * a.sub + tt % a.sub;
            const int64_t kr = (int64_t)tok_row(a.tm, f * kBlock + c16) * kHeadDim;
            const __bf16 *kt = k + head_off + kr;
            const __bf16 *vt = v + head_off + kr;
            R.ka0 = load_bf16x8(kt + 8 * g);
            R.ka1 = load_bf16x8(kt + 32 + 8 * g);
            R.va0 = load_bf16x8(vt + 8 * g);
            R.va1 = load_bf16x8(vt + 32 + 8 * g);
        };
        const bf16x8 qa0 = load_bf16x8(qrow + 8 * g), qa1 = load_bf16x8(qrow + 32 + 8 * g);
        const bf16x8 da0 = load_bf16x8(drow + 8 * g), da1 = load_bf16x8(drow + 32 + 8 * g);
        const float lse2 = lse[(int64_t)h * a.N + srow] * kLog2e;
        TileRegs RA, RB;
        load_tile(0, RA);
        load_tile(1, RB);
        CoarseTile T[NT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) load_coarse_tile(a, pk, pv, idx, fine, h, ib, ct, g, c16, T[ct]);
        store_bf16x8(&lds_q[w][c16 * kTS + 8 * g], qa0);
        store_bf16x8(&lds_q[w][c16 * kTS + 32 + 8 * g], qa1);
        store_bf16x8(&lds_do[w][c16 * kTS + 8 * g], da0);
        store_bf16x8(&lds_do[w][c16 * kTS + 32 + 8 * g], da1);

        // dQ = scale * (A - D B) with A = sum_j P_j dP_j k_j, B = sum_j P_j k_j and
        // D = sum_j P_j dP_j (= dO . O): one streaming pass over the fine tiles,
        // no D needed up front.  Coarse tiles come last, when D is complete.
        f32x4 accA[4], accB[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            accA[dt] = zero4;
            accB[dt] = zero4;
        }
        float dsum = 0.f;
        auto fine_tile = [&](const TileRegs &R) {
            wave_lds_sync();
            store_bf16x8(&lds_k[w][c16 * kTS + 8 * g], R.ka0);
            store_bf16x8(&lds_k[w][c16 * kTS + 32 + 8 * g], R.ka1);
            const f32x4 s = mfma_bf16_32(R.ka1, qa1, mfma_bf16_32(R.ka0, qa0, zero4));
            const f32x4 dp = mfma_bf16_32(R.va1, da1, mfma_bf16_32(R.va0, da0, zero4));
            float p[4], x[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = fast_exp2(s[i] * a.sl2 - lse2);
                x[i] = p[i] * dp[i];
                dsum += x[i];
            }
            bf16x4 phi, plo, xhi, xlo;
            split4(p, phi, plo);
            split4(x, xhi, xlo);
            const bf16x8 pcat = cat8(phi, plo), xcat = cat8(xhi, xlo);
            wave_lds_sync();
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x4 kT = lds_read_tr4(&lds_k[w][rofs + 16 * dt]);
                const bf16x8 kk = cat8(kT, kT);
                accA[dt] = mfma_bf16_32(kk, xcat, accA[dt]);
                accB[dt] = mfma_bf16_32(kk, pcat, accB[dt]);
            }
        };
        for (int t = 0; t < nft; t += 2) {
            fine_tile(RA);
            load_tile(t + 2, RA);
            if (t + 1 < nft) fine_tile(RB);
            load_tile(t + 3, RB);
        }
        // ---- coarse tiles: scores in both orientations, then D is complete
        f32x4 cs[NT], cdp[NT], cs2[NT], cdp2[NT];
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            // transposed orientation: lane (query c16, entries 4g+i) -> dQ
            cs[ct] = mfma_bf16_32(T[ct].ka1, qa1, mfma_bf16_32(T[ct].ka0, qa0, zero4));
            cdp[ct] = mfma_bf16_32(T[ct].va1, da1, mfma_bf16_32(T[ct].va0, da0, zero4));
            // plain orientation: lane (entry c16, queries 4g+i) -> coarse partials
            cs2[ct] = mfma_bf16_32(qa1, T[ct].ka1, mfma_bf16_32(qa0, T[ct].ka0, zero4));
            cdp2[ct] = mfma_bf16_32(da1, T[ct].va1, mfma_bf16_32(da0, T[ct].va0, zero4));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cs[ct][i] = fast_exp2(cs[ct][i] * a.sl2 + T[ct].bias4[i] - lse2);
                dsum += cs[ct][i] * cdp[ct][i];
            }
        }
        const float Dq = sum4_groups(dsum);
        if (g == 0) {
            ws.D[(int64_t)h * a.N + row] = Dq;
            lds_row[w][0][c16] = lse2;
            lds_row[w][1][c16] = Dq;
        }
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) {
            wave_lds_sync();
            store_bf16x8(&lds_ck[w][ct][c16 * kTS + 8 * g], T[ct].ka0);
            store_bf16x8(&lds_ck[w][ct][c16 * kTS + 32 + 8 * g], T[ct].ka1);
            wave_lds_sync();
            float ds[4], ds2[4], p2[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ds[i] = cs[ct][i] * (cdp[ct][i] - Dq);
                const float l2q = lds_row[w][0][4 * g + i];
                const float Dqi = lds_row[w][1][4 * g + i];
                p2[i] = fast_exp2(cs2[ct][i] * a.sl2 + T[ct].bias_row - l2q);
                ds2[i] = p2[i] * (cdp2[ct][i] - Dqi);
            }
            bf16x4 dhi, dlo, d2hi, d2lo, p2hi, p2lo;
            split4(ds, dhi, dlo);
            split4(ds2, d2hi, d2lo);
            split4(p2, p2hi, p2lo);
            const bf16x8 dcat = cat8(dhi, dlo), d2cat = cat8(d2hi, d2lo), p2cat = cat8(p2hi, p2lo);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x4 kT = lds_read_tr4(&lds_ck[w][ct][rofs + 16 * dt]);
                accA[dt] = mfma_bf16_32(cat8(kT, kT), dcat, accA[dt]);   // + Kc^T dS_c
                const bf16x4 qT = lds_read_tr4(&lds_q[w][rofs + 16 * dt]);
                const bf16x4 dT = lds_read_tr4(&lds_do[w][rofs + 16 * dt]);
                dkc[ct][dt] = mfma_bf16_32(d2cat, cat8(qT, qT), dkc[ct][dt]);
                dvc[ct][dt] = mfma_bf16_32(p2cat, cat8(dT, dT), dvc[ct][dt]);
            }
        }
        f32x4 dqacc[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) dqacc[dt] = accA[dt] - Dq * accB[dt];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            store_grad4(dq, head_off + srow * kHeadDim + 16 * dt + 4 * g, dqacc[dt] * a.scale, a.grad_bf16);
        wave_lds_sync();
    }
    // ---- reduce the coarse partials over the 4 waves, one coarse tile at a time
    float *part = ws.partial + ((int64_t)h * a.npg + G) * a.ncoarse * 2 * kHeadDim;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
        __syncthreads();
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ent = 4 * g + i, dim = 16 * dt + c16;
                lds_red[w][0][ent * kHeadDim + dim] = dkc[ct][dt][i] * a.scale;
                lds_red[w][1][ent * kHeadDim + dim] = dvc[ct][dt][i];
            }
        __syncthreads();
        const int n_ent = min(kBlock, a.ncoarse - ct * kBlock);
        for (int x = threadIdx.x; x < n_ent * 2 * kHeadDim; x += 256) {
            const int er = x / (2 * kHeadDim), kv = (x / kHeadDim) & 1, dim = x % kHeadDim;
            const int oo = er * kHeadDim + dim;
            part[(ct * kBlock) * 2 * kHeadDim + x] =
                lds_red[0][kv][oo] + lds_red[1][kv][oo] + lds_red[2][kv][oo] + lds_red[3][kv][oo];
        }
    }
}

// Pass A for B = 16 with K_1 = K1T (even) fine picks per query block and one
// coarse tile of at most 16 entries (CO) or none.  The 16 query blocks under
// a level-2 node share their coarse picks, so the workgroup stages that tile
// once in LDS as bf16 together with its log2 weights.  Wave w takes blocks
// w, w + 4, w + 8, w + 12 of the node, so the four waves work on neighbouring
// blocks at any time (neighbours pick many of the same key blocks, which the
// L1 then serves once).  Every wave streams the
// 4 K1T fine tiles of its 4 query blocks through two register sets without a
// break at block boundaries (the next block's first tiles and its Q / dO are
// in flight while a block's coarse part is computed); the wave's fine picks
// are read once, one per lane.  From K1T = 16 on a level-2 pick can be fully
// covered by a block's fine picks; it is then dropped for that block.
constexpr int kPtS = 20;                  // float row stride of the P / dS exchange
constexpr int kOutS = 68;                 // float row stride of a staged 16 x 64 output tile

template <int K1T, bool CO, int ORD>
__global__ __launch_bounds__(256, 2) void bwd_dq_fast_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ pk, const float *__restrict__ pv, const int32_t *__restrict__ idx,
    const float *__restrict__ lse, const __bf16 *__restrict__ dout, void *__restrict__ dq, BwdWs ws,
    BwdArgs a) {
    // per wave two K / V slot pairs (K0, V0, K1, V1: the two tiles of a pair),
    // Q and dO; then the coarse K, V tiles
    constexpr int kTileBytes = (4 * 6 + 2) * kTE * 2;
    constexpr int kRedBytes = 4 * 2 * kBlock * kHeadDim * 4;   // coarse partials of 4 waves
    __shared__ __attribute__((aligned(16))) char smem[kTileBytes > kRedBytes ? kTileBytes : kRedBytes];
    static_assert(K1T % 2 == 0 && K1T <= 32, "fine tiles stream in pairs, two pick registers");
    static_assert(kBlock * kOutS * 4 <= 2 * kTE * 2, "dQ rows fit the second slot pair");
    constexpr int NT = 4 * K1T;   // fine tiles per wave
    __shared__ float cbias[kBlock];
    __shared__ int ccol[kBlock];   // level-2 pooled token of each coarse entry (-1: other level)
    __shared__ __attribute__((aligned(16))) float lds_pt[4][2][kBlock * kPtS];  // coarse P, dS entry-major
    typedef __bf16 Tile[kTE];
    Tile *lds_kv = reinterpret_cast<Tile *>(smem);
    Tile *lds_q = lds_kv + 16;
    Tile *lds_do = lds_q + 4;
    __bf16 *ck = reinterpret_cast<__bf16 *>(lds_do + 4);
    __bf16 *cv = ck + kTE;
    typedef float RedTile[2][kBlock * kHeadDim];
    RedTile *lds_red = reinterpret_cast<RedTile *>(smem);

    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int gph = a.n1 / kBlock;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = bid / gph;
    const int G = bid % gph;
    const int ib0 = G * kBlock;
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    __bf16 *const k0s = lds_kv[4 * w], *const v0s = lds_kv[4 * w + 1];
    __bf16 *const k1s = lds_kv[4 * w + 2], *const v1s = lds_kv[4 * w + 3];
    float *const out_w = reinterpret_cast<float *>(k1s);   // dQ rows, over the second slot pair

    // ---- coarse tile, staged by the whole workgroup: thread (entry e, quarter
    // p).  Its pyramid rows are requested first and written to LDS once the
    // wave's first fine loads are out (the memory counter is waited on in
    // order, so the fine loads do not wait for the LDS writes).
    const int ce = threadIdx.x >> 4, cpart = threadIdx.x & 15;
    bool cok = false;
    int cjs = 0, ccol_v = -1;
    f32x4 ckk = zero4, cvv = zero4;
    if constexpr (CO) {
        int j = 0, pick = ce;
        while (j < a.ncl - 1 && pick >= a.cl_k[j]) {
            pick -= a.cl_k[j];
            ++j;
        }
        cok = ce < a.ncoarse;
        cjs = cok ? j : 0;
        const int ps = cok ? pick : 0;
        const int anc = ib0 >> (4 * (cjs + 1));   // ancestor at level js + 2
        const int c = idx[a.cl_idx_off[cjs] + ((int64_t)h * a.cl_n[cjs] + anc) * a.cl_k[cjs] + ps];
        const int64_t roff = a.cl_pyr_off[cjs] + ((int64_t)h * a.cl_n[cjs] + c) * kHeadDim + 4 * cpart;
        ckk = *reinterpret_cast<const f32x4 *>(pk + roff);
        cvv = *reinterpret_cast<const f32x4 *>(pv + roff);
        ccol_v = cok && cjs == 0 ? c : -1;
    }

    // ---- this wave's fine picks: pick u (block u / K1T, pick u % K1T) sits in
    // lane u of fidx0 (u < 64) or lane u - 64 of fidx1
    // block jb of this wave is ib0 + 4 jb + w: the four waves work on four
    // neighbouring blocks at a time, whose picks overlap in the L1
    const int32_t *hpicks = idx + ((int64_t)h * a.n1 + ib0) * K1T;
    auto wpick = [&](int u) { return hpicks[((u / K1T) * 4 + w) * K1T + u % K1T]; };
    const int fidx0 = lane < NT ? wpick(lane) : 0;
    const int fidx1 = NT > kWave && lane < NT - kWave ? wpick(kWave + lane) : 0;
    auto pick = [&](int u) {
        if constexpr (NT <= kWave)
            return __builtin_amdgcn_readlane(fidx0, u);
        else
            return u < kWave ? __builtin_amdgcn_readlane(fidx0, u) : __builtin_amdgcn_readlane(fidx1, u - kWave);
    };
    struct TileRegs {
        bf16x8 ka0, ka1, va0, va1;
    };
    // Global loads read whole 128-byte rows (lane l: row l / 8 and l / 8 + 8,
    // 16-byte chunk l % 8); the rows pass through LDS, from where the MFMA
    // operands (lane: row c16, dims 8g.. and 32+8g..) are read back.
    const int lrow = lane >> 3, lcol = (lane & 7) * 8;
    auto stage_rows = [&](__bf16 *dst, bf16x8 r0, bf16x8 r1) {
        store_bf16x8(dst + lrow * kTS + lcol, r0);
        store_bf16x8(dst + (lrow + 8) * kTS + lcol, r1);
    };
    // element offset (within the head) of row r of sequence block b
    auto trow = [&](int b, int r) { return (int64_t)tok_tile_row<ORD>(a.tm, b, r) * kHeadDim; };
    // K / V rows through buffer loads with 32-bit byte offsets within the head
    const uint32_t head_bytes = (uint32_t)a.N * kHeadDim * 2;
    const Rsrc rk = make_rsrc(k + head_off, head_bytes), rv = make_rsrc(v + head_off, head_bytes);
    auto load_tile = [&](int u, TileRegs &R) {
        const int f = pick(u);
        const uint32_t o0 = ((uint32_t)tok_tile_row<ORD>(a.tm, f, lrow) * kHeadDim + lcol) * 2u;
        const uint32_t o1 = ((uint32_t)tok_tile_row<ORD>(a.tm, f, lrow + 8) * kHeadDim + lcol) * 2u;
        R.ka0 = buf_load_bf16x8(rk, o0);
        R.ka1 = buf_load_bf16x8(rk, o1);
        R.va0 = buf_load_bf16x8(rv, o0);
        R.va1 = buf_load_bf16x8(rv, o1);
    };
    struct QRegs {
        bf16x8 qa0, qa1, da0, da1;
        float lse2;
    };
    auto load_q = [&](int jb, QRegs &X) {
        const int b = ib0 + jb * 4 + w;
        const int64_t o0 = head_off + trow(b, lrow) + lcol, o1 = head_off + trow(b, lrow + 8) + lcol;
        X.qa0 = load_bf16x8_nt(q + o0);
        X.qa1 = load_bf16x8_nt(q + o1);
        X.da0 = load_bf16x8_nt(dout + o0);
        X.da1 = load_bf16x8_nt(dout + o1);
        X.lse2 = lse[(int64_t)h * a.N + tok_tile_row<ORD>(a.tm, b, c16)] * kLog2e;
    };
    QRegs X;
    load_q(0, X);
    constexpr int PD = 2;   // tiles in flight
    TileRegs R[PD];
#pragma unroll
    for (int r = 0; r < PD; ++r) load_tile(r, R[r]);
    if constexpr (CO) {
        if (!cok) ckk = cvv = zero4;
        const bf16x4 kb = to_bf16x4(f32x4{ckk[0], ckk[1], ckk[2], ckk[3]});
        const bf16x4 vb = to_bf16x4(f32x4{cvv[0], cvv[1], cvv[2], cvv[3]});
        *reinterpret_cast<u32x2 *>(&ck[ce * kTS + 4 * cpart]) = __builtin_bit_cast(u32x2, kb);
        *reinterpret_cast<u32x2 *>(&cv[ce * kTS + 4 * cpart]) = __builtin_bit_cast(u32x2, vb);
        if (cpart == 0) {
            cbias[ce] = cok ? 4.0f * (float)(cjs + 2) : -INFINITY;
            ccol[ce] = ccol_v;
        }
    }

    f32x4 dkc[4], dvc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        dkc[dt] = zero4;
        dvc[dt] = zero4;
    }
    const int rofs = (4 * g + (c16 >> 2)) * kTS + 4 * (c16 & 3);  // transposed-read address
    __syncthreads();   // coarse tile staged

    for (int jb = 0; jb < 4; ++jb) {
        const int64_t row = (int64_t)(ib0 + jb * 4 + w) * kBlock + c16;
        const float lse2 = X.lse2;
        wave_lds_sync();
        stage_rows(lds_q[w], X.qa0, X.qa1);
        stage_rows(lds_do[w], X.da0, X.da1);
        wave_lds_sync();
        const bf16x8 qa0 = load_bf16x8(&lds_q[w][c16 * kTS + 8 * g]);
        const bf16x8 qa1 = load_bf16x8(&lds_q[w][c16 * kTS + 32 + 8 * g]);
        const bf16x8 da0 = load_bf16x8(&lds_do[w][c16 * kTS + 8 * g]);
        const bf16x8 da1 = load_bf16x8(&lds_do[w][c16 * kTS + 32 + 8 * g]);

        // dQ = scale * (A - D B), A = sum_j P_j dP_j k_j, B = sum_j P_j k_j,
        // D = sum_j P_j dP_j; the coarse entries come last, when D is complete.
        f32x4 accA[4], accB[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            accA[dt] = zero4;
            accB[dt] = zero4;
        }
        float dsum = 0.f;
        // Two fine tiles at a time, each in a slot pair of its own: their
        // score chains are independent, and the key-side contractions take
        // the 16 keys of both tiles as the 32 k-slots of one MFMA (the hi and
        // lo parts of P and P dP in two MFMAs).  The next pair's loads go out
        // as soon as this pair's rows are staged.
        auto score = [&](const __bf16 *ks, const __bf16 *vs, float (&p)[4], float (&x)[4]) {
            const __bf16 *kr = ks + c16 * kTS + 8 * g;
            const __bf16 *vr = vs + c16 * kTS + 8 * g;
            const f32x4 s = mfma_bf16_32(load_bf16x8(kr + 32), qa1, mfma_bf16_32(load_bf16x8(kr), qa0, zero4));
            const f32x4 dp = mfma_bf16_32(load_bf16x8(vr + 32), da1, mfma_bf16_32(load_bf16x8(vr), da0, zero4));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[i] = fast_exp2(s[i] * a.sl2 - lse2);
                x[i] = p[i] * dp[i];
            }
        };
        auto tile_pair = [&](int t) {
            const int u = jb * K1T + t;   // first tile of the pair
            wave_lds_sync();
            stage_rows(k0s, R[0].ka0, R[0].ka1);
            stage_rows(v0s, R[0].va0, R[0].va1);
            stage_rows(k1s, R[1].ka0, R[1].ka1);
            stage_rows(v1s, R[1].va0, R[1].va1);
#pragma unroll
            for (int r = 0; r < PD; ++r)
                if (u + PD + r < NT) load_tile(u + PD + r, R[r]);
            wave_lds_sync();
            float p0[4], x0[4], p1[4], x1[4];
            score(k0s, v0s, p0, x0);
            score(k1s, v1s, p1, x1);
#pragma unroll
            for (int i = 0; i < 4; ++i) dsum += x0[i] + x1[i];
            bf16x4 phi0, plo0, xhi0, xlo0, phi1, plo1, xhi1, xlo1;
            split4(p0, phi0, plo0);
            split4(x0, xhi0, xlo0);
            split4(p1, phi1, plo1);
            split4(x1, xhi1, xlo1);
            const bf16x8 ph = cat8(phi0, phi1), pl = cat8(plo0, plo1);
            const bf16x8 xh = cat8(xhi0, xhi1), xl = cat8(xlo0, xlo1);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x8 kk = cat8(lds_read_tr4(k0s + rofs + 16 * dt), lds_read_tr4(k1s + rofs + 16 * dt));
                accA[dt] = mfma_bf16_32(kk, xl, mfma_bf16_32(kk, xh, accA[dt]));
                accB[dt] = mfma_bf16_32(kk, pl, mfma_bf16_32(kk, ph, accB[dt]));
            }
        };
        if constexpr (K1T <= 8) {
#pragma unroll
            for (int t = 0; t < K1T; t += PD) tile_pair(t);
        } else {   // unrolled fully, longer lists hoist too much into registers
#pragma unroll 2
            for (int t = 0; t < K1T; t += PD) tile_pair(t);
        }
        if constexpr (!CO) {
            if (jb + 1 < 4) load_q(jb + 1, X);
            const float Dq = sum4_groups(dsum);
            if (g == 0) ws.D[(int64_t)h * a.N + row] = Dq;
            wave_lds_sync();
#pragma unroll
            for (int dt = 0; dt < 4; ++dt)
                *reinterpret_cast<f32x4 *>(&out_w[c16 * kOutS + 16 * dt + 4 * g]) =
                    (accA[dt] - Dq * accB[dt]) * a.scale;
            wave_lds_sync();
#pragma unroll
            for (int it = 0; it < 4; ++it) {
                const int r = g + 4 * it;
                store_grad4(dq, head_off + trow(ib0 + jb * 4 + w, r) + 4 * c16,
                            *reinterpret_cast<const f32x4 *>(&out_w[r * kOutS + 4 * c16]), a.grad_bf16);
            }
            continue;
        } else {
        // ---- coarse entries: lane (query c16, entries 4g+i)
        const __bf16 *ckr = ck + c16 * kTS;
        const __bf16 *cvr = cv + c16 * kTS;
        f32x4 cs = mfma_bf16_32(load_bf16x8(ckr + 32 + 8 * g), qa1,
                                mfma_bf16_32(load_bf16x8(ckr + 8 * g), qa0, zero4));
        const f32x4 cdp = mfma_bf16_32(load_bf16x8(cvr + 32 + 8 * g), da1,
                                       mfma_bf16_32(load_bf16x8(cvr + 8 * g), da0, zero4));
        if (jb + 1 < 4) load_q(jb + 1, X);   // next block's Q / dO in flight from here
#pragma unroll
        for (int i = 0; i < 4; ++i) cs[i] = fast_exp2(cs[i] * a.sl2 + cbias[4 * g + i] - lse2);
        if constexpr (K1T >= kBlock) {
            if (a.drop) {   // entries whose 16 children are all fine picks of this block
                int cov[4] = {0, 0, 0, 0}, cc[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) cc[i] = ccol[4 * g + i];
                for (int t = 0; t < K1T; ++t) {
                    const int f = pick(jb * K1T + t) >> 4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) cov[i] += f == cc[i] ? 1 : 0;
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (cov[i] == kBlock) cs[i] = 0.f;
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) dsum += cs[i] * cdp[i];
        const float Dq = sum4_groups(dsum);
        if (g == 0) ws.D[(int64_t)h * a.N + row] = Dq;
        float ds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) ds[i] = cs[i] * (cdp[i] - Dq);
        // P and dS go through LDS entry-major: read back, lane (entry c16,
        // queries 4g+i) holds the operand of the coarse-partial contractions
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lds_pt[w][0][(4 * g + i) * kPtS + c16] = cs[i];
            lds_pt[w][1][(4 * g + i) * kPtS + c16] = ds[i];
        }
        wave_lds_sync();
        const f32x4 p2v = *reinterpret_cast<const f32x4 *>(&lds_pt[w][0][c16 * kPtS + 4 * g]);
        const f32x4 d2v = *reinterpret_cast<const f32x4 *>(&lds_pt[w][1][c16 * kPtS + 4 * g]);
        float ds2[4], p2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p2[i] = p2v[i];
            ds2[i] = d2v[i];
        }
        bf16x4 dhi, dlo, d2hi, d2lo, p2hi, p2lo;
        split4(ds, dhi, dlo);
        split4(ds2, d2hi, d2lo);
        split4(p2, p2hi, p2lo);
        const bf16x8 dcat = cat8(dhi, dlo), d2cat = cat8(d2hi, d2lo), p2cat = cat8(p2hi, p2lo);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const bf16x4 kT = lds_read_tr4(&ck[rofs + 16 * dt]);
            accA[dt] = mfma_bf16_32(cat8(kT, kT), dcat, accA[dt]);   // + Kc^T dS_c
            const bf16x4 qT = lds_read_tr4(&lds_q[w][rofs + 16 * dt]);
            const bf16x4 dT = lds_read_tr4(&lds_do[w][rofs + 16 * dt]);
            dkc[dt] = mfma_bf16_32(d2cat, cat8(qT, qT), dkc[dt]);
            dvc[dt] = mfma_bf16_32(p2cat, cat8(dT, dT), dvc[dt]);
        }
        // dQ (lane: query c16, dims 16 dt + 4 g ..) passes through LDS so
        // that every store writes whole rows (lane l: row l / 16 + 4 it)
        wave_lds_sync();
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            *reinterpret_cast<f32x4 *>(&out_w[c16 * kOutS + 16 * dt + 4 * g]) =
                (accA[dt] - Dq * accB[dt]) * a.scale;
        wave_lds_sync();
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = g + 4 * it;
            store_grad4(dq, head_off + trow(ib0 + jb * 4 + w, r) + 4 * c16,
                        *reinterpret_cast<const f32x4 *>(&out_w[r * kOutS + 4 * c16]), a.grad_bf16);
        }
        }
    }
    if constexpr (!CO) return;
    // ---- reduce the coarse partials over the 4 waves
    __syncthreads();
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ent = 4 * g + i, dim = 16 * dt + c16;
            lds_red[w][0][ent * kHeadDim + dim] = dkc[dt][i] * a.scale;
            lds_red[w][1][ent * kHeadDim + dim] = dvc[dt][i];
        }
    __syncthreads();
    float *part = ws.partial + ((int64_t)h * a.npg + G) * a.ncoarse * 2 * kHeadDim;
    for (int x = threadIdx.x; x < a.ncoarse * 2 * kHeadDim; x += 256) {
        const int er = x / (2 * kHeadDim), kv = (x / kHeadDim) & 1, dim = x % kHeadDim;
        const int oo = er * kHeadDim + dim;
        part[x] = lds_red[0][kv][oo] + lds_red[1][kv][oo] + lds_red[2][kv][oo] + lds_red[3][kv][oo];
    }
}

// Pass A for blocks of 64 tokens: one workgroup per 4 consecutive query blocks
// (16 query tiles: a group of the coarse partials), one wave per tile of the
// block in hand.  A block's 4 tiles share its picks, so the workgroup loads
// each picked key block (4 key tiles, K and V) once into LDS -- each wave one
// tile, as whole rows -- and every wave uses all four: a quarter of the
// gathers of one wave per tile.  Picked blocks alternate between two LDS
// buffers (the next block's rows are in flight while one is used).  The
// coarse tile (at most 16 entries, shared by the 4 blocks) and the partial
// reduction are as in the B = 16 kernel; K_1 < B, so nothing is dropped.
template <int ORD>
__global__ __launch_bounds__(256, 2) void bwd_dq_b64_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ pk, const float *__restrict__ pv, const int32_t *__restrict__ idx,
    const float *__restrict__ lse, const __bf16 *__restrict__ dout, void *__restrict__ dq, BwdWs ws,
    BwdArgs a) {
    constexpr int kSub = 4;
    typedef __bf16 Tile[kTE];
    __shared__ __attribute__((aligned(16))) Tile kvbuf[2][2][kSub];   // [K, V][buffer][tile]
    Tile(*kbuf)[kSub] = kvbuf[0];
    Tile(*vbuf)[kSub] = kvbuf[1];
    __shared__ __attribute__((aligned(16))) Tile lds_q[kSub];
    __shared__ __attribute__((aligned(16))) Tile lds_do[kSub];
    __shared__ __attribute__((aligned(16))) __bf16 ck[kTE];
    __shared__ __attribute__((aligned(16))) __bf16 cv[kTE];
    __shared__ float cbias[kBlock];
    __shared__ __attribute__((aligned(16))) float lds_pt[kSub][2][kBlock * kPtS];
    static_assert(sizeof(kvbuf) >= 4 * 2 * kBlock * kHeadDim * 4, "partials fit the buffers");
    typedef float RedTile[2][kBlock * kHeadDim];
    RedTile *lds_red = reinterpret_cast<RedTile *>(&kvbuf[0][0][0][0]);   // after the last block

    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int gph = a.n1 / kSub;   // workgroups per head
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = bid / gph;
    const int G = bid % gph;       // partial group: query blocks 4G .. 4G + 3
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
    const bool co = a.ncoarse > 0;
    auto trow = [&](int b, int r) { return (int64_t)tok_tile_row<ORD>(a.tm, b, r) * kHeadDim; };
    const int lrow = lane >> 3, lcol = (lane & 7) * 8;
    auto stage_rows = [&](__bf16 *dst, bf16x8 r0, bf16x8 r1) {
        store_bf16x8(dst + lrow * kTS + lcol, r0);
        store_bf16x8(dst + (lrow + 8) * kTS + lcol, r1);
    };
    if (co) {   // coarse tile, staged by the whole workgroup: thread (entry e, quarter p)
        const int e = threadIdx.x >> 4, part = threadIdx.x & 15;
        int j = 0, pick = e;
        while (j < a.ncl - 1 && pick >= a.cl_k[j]) {
            pick -= a.cl_k[j];
            ++j;
        }
        const bool ok = e < a.ncoarse;
        const int js = ok ? j : 0, ps = ok ? pick : 0;
        const int c = idx[a.cl_idx_off[js] + ((int64_t)h * a.cl_n[js] + 4 * G / a.cl_span[js]) * a.cl_k[js] + ps];
        const int64_t roff = a.cl_pyr_off[js] + ((int64_t)h * a.cl_n[js] + c) * kHeadDim + 4 * part;
        f32x4 kk = *reinterpret_cast<const f32x4 *>(pk + roff);
        f32x4 vv = *reinterpret_cast<const f32x4 *>(pv + roff);
        if (!ok) kk = vv = zero4;
        *reinterpret_cast<u32x2 *>(&ck[e * kTS + 4 * part]) = __builtin_bit_cast(u32x2, to_bf16x4(kk));
        *reinterpret_cast<u32x2 *>(&cv[e * kTS + 4 * part]) = __builtin_bit_cast(u32x2, to_bf16x4(vv));
        if (part == 0) cbias[e] = ok ? a.lgB * (float)(js + 2) : -INFINITY;
    }
    f32x4 dkc[4], dvc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        dkc[dt] = zero4;
        dvc[dt] = zero4;
    }
    const int rofs = (4 * g + (c16 >> 2)) * kTS + 4 * (c16 & 3);  // transposed-read address
    bf16x8 kr[2], vr[2];
    for (int jb = 0; jb < kSub; ++jb) {
        const int ib = 4 * G + jb;          // query block in hand
        const int qt = ib * kSub + w;       // this wave's tile of it
        const int32_t *fine = idx + ((int64_t)h * a.n1 + ib) * a.K1;
        auto load_tile = [&](int j) {       // wave w's tile of picked block j
            const int f = __builtin_amdgcn_readfirstlane(fine[j]) * kSub + w;
            const int64_t o0 = head_off + trow(f, lrow) + lcol, o1 = head_off + trow(f, lrow + 8) + lcol;
            kr[0] = load_bf16x8(k + o0);
            kr[1] = load_bf16x8(k + o1);
            vr[0] = load_bf16x8(v + o0);
            vr[1] = load_bf16x8(v + o1);
        };
        load_tile(0);
        const float lse2 = lse[(int64_t)h * a.N + tok_tile_row<ORD>(a.tm, qt, c16)] * kLog2e;
        wave_lds_sync();
        stage_rows(lds_q[w], load_bf16x8_nt(q + head_off + trow(qt, lrow) + lcol),
                   load_bf16x8_nt(q + head_off + trow(qt, lrow + 8) + lcol));
        stage_rows(lds_do[w], load_bf16x8_nt(dout + head_off + trow(qt, lrow) + lcol),
                   load_bf16x8_nt(dout + head_off + trow(qt, lrow + 8) + lcol));
        wave_lds_sync();
        const bf16x8 qa0 = load_bf16x8(&lds_q[w][c16 * kTS + 8 * g]);
        const bf16x8 qa1 = load_bf16x8(&lds_q[w][c16 * kTS + 32 + 8 * g]);
        const bf16x8 da0 = load_bf16x8(&lds_do[w][c16 * kTS + 8 * g]);
        const bf16x8 da1 = load_bf16x8(&lds_do[w][c16 * kTS + 32 + 8 * g]);
        f32x4 accA[4], accB[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            accA[dt] = zero4;
            accB[dt] = zero4;
        }
        float dsum = 0.f;
        for (int j = 0; j < a.K1; ++j) {
            const int buf = j & 1;
            stage_rows(kbuf[buf][w], kr[0], kr[1]);
            stage_rows(vbuf[buf][w], vr[0], vr[1]);
            // the block's four key tiles staged; every wave is done with block j - 2
            __syncthreads();
            if (j + 1 < a.K1) load_tile(j + 1);
#pragma unroll 1
            for (int t = 0; t < kSub; ++t) {
                const __bf16 *kt = kbuf[buf][t], *vt = vbuf[buf][t];
                const f32x4 s = mfma_bf16_32(load_bf16x8(&kt[c16 * kTS + 32 + 8 * g]), qa1,
                                             mfma_bf16_32(load_bf16x8(&kt[c16 * kTS + 8 * g]), qa0, zero4));
                const f32x4 dp = mfma_bf16_32(load_bf16x8(&vt[c16 * kTS + 32 + 8 * g]), da1,
                                              mfma_bf16_32(load_bf16x8(&vt[c16 * kTS + 8 * g]), da0, zero4));
                float p[4], x[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[i] = fast_exp2(s[i] * a.sl2 - lse2);
                    x[i] = p[i] * dp[i];
                    dsum += x[i];
                }
                bf16x4 phi, plo, xhi, xlo;
                split4(p, phi, plo);
                split4(x, xhi, xlo);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x4 kT = lds_read_tr4(&kt[rofs + 16 * dt]);
                    accA[dt] = mfma_bf16_16(kT, xhi, accA[dt]);
                    accB[dt] = mfma_bf16_16(kT, phi, accB[dt]);
                }
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    const bf16x4 kT = lds_read_tr4(&kt[rofs + 16 * dt]);
                    accA[dt] = mfma_bf16_16(kT, xlo, accA[dt]);
                    accB[dt] = mfma_bf16_16(kT, plo, accB[dt]);
                }
            }
        }
        float Dq;
        if (co) {
            // ---- coarse entries: lane (query c16, entries 4g+i)
            const __bf16 *ckr = ck + c16 * kTS;
            const __bf16 *cvr = cv + c16 * kTS;
            f32x4 cs = mfma_bf16_32(load_bf16x8(ckr + 32 + 8 * g), qa1,
                                    mfma_bf16_32(load_bf16x8(ckr + 8 * g), qa0, zero4));
            const f32x4 cdp = mfma_bf16_32(load_bf16x8(cvr + 32 + 8 * g), da1,
                                           mfma_bf16_32(load_bf16x8(cvr + 8 * g), da0, zero4));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                cs[i] = fast_exp2(cs[i] * a.sl2 + cbias[4 * g + i] - lse2);
                dsum += cs[i] * cdp[i];
            }
            Dq = sum4_groups(dsum);
            float ds[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ds[i] = cs[i] * (cdp[i] - Dq);
            // P and dS entry-major through LDS: lane (entry c16, queries 4g+i)
            wave_lds_sync();
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                lds_pt[w][0][(4 * g + i) * kPtS + c16] = cs[i];
                lds_pt[w][1][(4 * g + i) * kPtS + c16] = ds[i];
            }
            wave_lds_sync();
            const f32x4 p2v = *reinterpret_cast<const f32x4 *>(&lds_pt[w][0][c16 * kPtS + 4 * g]);
            const f32x4 d2v = *reinterpret_cast<const f32x4 *>(&lds_pt[w][1][c16 * kPtS + 4 * g]);
            float ds2[4], p2[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p2[i] = p2v[i];
                ds2[i] = d2v[i];
            }
            bf16x4 dhi, dlo, d2hi, d2lo, p2hi, p2lo;
            split4(ds, dhi, dlo);
            split4(ds2, d2hi, d2lo);
            split4(p2, p2hi, p2lo);
            const bf16x8 dcat = cat8(dhi, dlo), d2cat = cat8(d2hi, d2lo), p2cat = cat8(p2hi, p2lo);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x4 kT = lds_read_tr4(&ck[rofs + 16 * dt]);
                accA[dt] = mfma_bf16_32(cat8(kT, kT), dcat, accA[dt]);   // + Kc^T dS_c
                const bf16x4 qT = lds_read_tr4(&lds_q[w][rofs + 16 * dt]);
                const bf16x4 dT = lds_read_tr4(&lds_do[w][rofs + 16 * dt]);
                dkc[dt] = mfma_bf16_32(d2cat, cat8(qT, qT), dkc[dt]);
                dvc[dt] = mfma_bf16_32(p2cat, cat8(dT, dT), dvc[dt]);
            }
        } else {
            Dq = sum4_groups(dsum);
        }
        if (g == 0) ws.D[(int64_t)h * a.N + (int64_t)qt * kBlock + c16] = Dq;
        // dQ (lane: query c16, dims 16 dt + 4 g ..) through a quarter of the
        // key buffers once every wave is done with them, then whole rows
        // (lane l: row l / 16 + 4 it)
        static_assert(sizeof(kvbuf) / 2 >= 4 * kBlock * kOutS * sizeof(float), "dQ staging fits");
        float *stage = reinterpret_cast<float *>(&kvbuf[0][0][0][0]) + w * kBlock * kOutS;
        __syncthreads();
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
            *reinterpret_cast<f32x4 *>(&stage[c16 * kOutS + 16 * dt + 4 * g]) = (accA[dt] - Dq * accB[dt]) * a.scale;
        wave_lds_sync();
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = g + 4 * it;
            store_grad4(dq, head_off + trow(qt, r) + 4 * c16,
                        *reinterpret_cast<const f32x4 *>(&stage[r * kOutS + 4 * c16]), a.grad_bf16);
        }
        __syncthreads();   // all waves done with this block's key buffers
    }
    if (!co) return;
    // ---- reduce the coarse partials over the 4 waves (the key buffers are free)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ent = 4 * g + i, dim = 16 * dt + c16;
            lds_red[w][0][ent * kHeadDim + dim] = dkc[dt][i] * a.scale;
            lds_red[w][1][ent * kHeadDim + dim] = dvc[dt][i];
        }
    __syncthreads();
    float *part = ws.partial + ((int64_t)h * a.npg + G) * a.ncoarse * 2 * kHeadDim;
    for (int x = threadIdx.x; x < a.ncoarse * 2 * kHeadDim; x += 256) {
        const int er = x / (2 * kHeadDim), kv = (x / kHeadDim) & 1, dim = x % kHeadDim;
        const int oo = er * kHeadDim + dim;
        part[x] = lds_red[0][kv][oo] + lds_red[1][kv][oo] + lds_red[2][kv][oo] + lds_red[3][kv][oo];
    }
}

// ================================================================ pass B
// One wave per pooled token c of level l (lanes = columns): the level-l rows
// that picked c come from the CSR of I^(l); each lane looks up one row's slot
// of c, then the wave sums the partials of every group of 16 query tiles under
// each row.
__global__ __launch_bounds__(256) void bwd_coarse_reduce_kernel(const int32_t *__restrict__ idx,
                                                                const int32_t *__restrict__ csr_ptr,
                                                                const int32_t *__restrict__ csr_col,
                                                                BwdWs ws, BwdArgs a, int j) {
    const int nl = a.cl_n[j], kl = a.cl_k[j];
    const int64_t tok = (int64_t)blockIdx.x * 4 + wave_id();
    if (tok >= (int64_t)a.bh * nl) return;
    const int lane = lane_id();
    const int h = (int)(tok / nl);
    const int c = (int)(tok % nl);
    const int32_t *P = csr_ptr + a.cl_ptr_off[j] + (int64_t)h * (nl + 1);
    const int32_t *C = csr_col + a.cl_col_off[j] + (int64_t)h * nl * kl;
    const int32_t *I = idx + a.cl_idx_off[j] + (int64_t)h * nl * kl;
    const int nodes = a.cl_groups[j];   // partial groups under one level-l token
    const int e0 = P[c], e1 = P[c + 1];
    float sk = 0.f, sv = 0.f;
    for (int base = e0; base < e1; base += kWave) {
        const int cnt = min(kWave, e1 - base);
        int ent = -1, g0 = 0;
        if (lane < cnt) {
            const int r = C[base + lane];
            const int32_t *row = I + (int64_t)r * kl;
            int slot = kl;
            if (kl == 8) {   // the whole row in two loads (rows are 32-byte aligned)
                const i32x4 lo = *reinterpret_cast<const i32x4 *>(row);
                const i32x4 hi = *reinterpret_cast<const i32x4 *>(row + 4);
#pragma unroll
                for (int i = 3; i >= 0; --i) {
                    slot = hi[i] == c ? 4 + i : slot;
                }
#pragma unroll
                for (int i = 3; i >= 0; --i) {
                    slot = lo[i] == c ? i : slot;
                }
            } else {
                for (int i = kl - 1; i >= 0; --i) slot = row[i] == c ? i : slot;
            }
            if (slot < kl) {
                ent = a.cl_entry0[j] + slot;
                g0 = r * nodes;
            }
        }
        // eight rows at a time: all their partial rows are requested before
        // any is added (an entry that is not a pick of its row, which only
        // inconsistent lists produce, contributes nothing)
        for (int j0 = 0; j0 < cnt; j0 += 8) {
            for (int s = 0; s < nodes; ++s) {
                float pk8[8], pv8[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int jj = min(j0 + u, cnt - 1);
                    const int e = __builtin_amdgcn_readlane(ent, jj);
                    const int64_t G0 = (int64_t)h * a.npg + __builtin_amdgcn_readlane(g0, jj);
                    const float *pp = ws.partial + ((G0 + s) * a.ncoarse + max(e, 0)) * 2 * kHeadDim;
                    const bool use = j0 + u < cnt && e >= 0;
                    pk8[u] = use ? pp[lane] : 0.f;
                    pv8[u] = use ? pp[kHeadDim + lane] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    sk += pk8[u];
                    sv += pv8[u];
                }
            }
        }
    }
    ws.dpk[a.cl_grad_off[j] + ((int64_t)h * nl + c) * kHeadDim + lane] = sk;
    ws.dpv[a.cl_grad_off[j] + ((int64_t)h * nl + c) * kHeadDim + lane] = sv;
}

// ================================================================ pass C
// One wave per key tile, in a workgroup of its own: key blocks differ widely
// in how many query blocks picked them, and no wave waits for a slower
// sibling before its slot is reused.  The query tiles of the blocks in the
// key block's CSR segment (SUB = B / 16 per block) go two at a time: a pair
// is staged in LDS, the next pair's Q / dO loads go out into the freed
// registers, and the pair is computed while they are in flight.
constexpr int kDkvDepth = 2;
template <int ORD, int SUB>
__global__ __launch_bounds__(64, 3) void bwd_dkv_bf16_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ lse, const __bf16 *__restrict__ dout, const int32_t *__restrict__ csr_ptr,
    const int32_t *__restrict__ csr_col, void *__restrict__ dk, void *__restrict__ dv, BwdWs ws,
    BwdArgs a) {
    // two slots (Q, dO, lse / D) for the two query tiles of a pair; the
    // output rows reuse the second slot's Q and dO
    __shared__ __attribute__((aligned(16))) __bf16 lds_qd[2][2][kTE];
    __shared__ __attribute__((aligned(16))) float lds_ld[2][2 * kBlock];   // lse, D of the tile's queries
    static_assert(kBlock * kOutS * 4 <= 2 * kTE * 2, "output rows fit the second slot");
    float *const lds_out = reinterpret_cast<float *>(&lds_qd[1][0][0]);
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t kb = xcd_remap(blockIdx.x, gridDim.x);
    if (kb >= (int64_t)a.bh * a.nt1) return;
    const int h = (int)(kb / a.nt1);
    const int f = (int)(kb % a.nt1);   // key tile
    const int fb = f / SUB;            // its key block
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    // element offset (within the head) of row r of 16-token tile b
    auto trow = [&](int b, int r) { return (int64_t)tok_tile_row<ORD>(a.tm, b, r) * kHeadDim; };
    const int32_t *P = csr_ptr + (int64_t)h * (a.n1 + 1);
    const int32_t *C = csr_col + (int64_t)h * a.n1 * a.K1;
    const int e0 = __builtin_amdgcn_readfirstlane(P[fb]), e1 = __builtin_amdgcn_readfirstlane(P[fb + 1]);
    f32x4 dka[4], dva[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        dka[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dva[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // about half of the key blocks are picked by no query block: their tiles
    // only receive the pooled-level gradients below and never read K or V
    if (e1 > e0) {
    const __bf16 *krow = k + head_off + trow(f, c16);
    const __bf16 *vrow = v + head_off + trow(f, c16);
    const bf16x8 kb0 = load_bf16x8_nt(krow + 8 * g), kb1 = load_bf16x8_nt(krow + 32 + 8 * g);
    const bf16x8 vb0 = load_bf16x8_nt(vrow + 8 * g), vb1 = load_bf16x8_nt(vrow + 32 + 8 * g);
    const int rofs = (4 * g + (c16 >> 2)) * kTS + 4 * (c16 & 3);
    // Per query block: its Q / dO tiles loaded as whole 128-byte rows per
    // instruction (lane l: rows l / 8 and l / 8 + 8, 16-byte chunk l % 8),
    // which pass through LDS before the MFMA operand rows are read back; and
    // one float per lane (lanes 0-15 the queries' lse, 16-31 their D).
    struct Pair {
        bf16x8 qa0, qa1, da0, da1;
        float ld;
    };
    const float *ld_src = lane < kBlock ? lse : ws.D;
    const int lrow = lane >> 3, lcol = (lane & 7) * 8;
    const uint32_t head_bytes = (uint32_t)a.N * kHeadDim * 2;
    const Rsrc rq = make_rsrc(q + head_off, head_bytes), rdo = make_rsrc(dout + head_off, head_bytes);
    // byte offset (within the head) of column lcol of row r of tile b
    auto brow = [&](int b, int r) {
        return ((uint32_t)tok_tile_row<ORD>(a.tm, b, r) * kHeadDim + lcol) * 2u;
    };
    auto load_pair = [&](int ib, Pair &X) {
        const uint32_t o0 = brow(ib, lrow), o1 = brow(ib, lrow + 8);
        X.qa0 = buf_load_bf16x8(rq, o0);
        X.qa1 = buf_load_bf16x8(rq, o1);
        X.da0 = buf_load_bf16x8(rdo, o0);
        X.da1 = buf_load_bf16x8(rdo, o1);
        // lse is stored by token row, D by sequence position
        X.ld = ld_src[(int64_t)h * a.N + (lane < kBlock ? tok_tile_row<ORD>(a.tm, ib, c16) : ib * kBlock + c16)];
    };
    // tile jt of the current batch of the segment (clamped to its last tile)
    int colv = 0, ntl = 0;
    auto qtile_of = [&](int jt) {
        const int jc = min(jt, ntl - 1);
        return __builtin_amdgcn_readlane(colv, jc / SUB) * SUB + jc % SUB;
    };
    // S, dP and the softmax gradient of the query tile in slot t; lane (key
    // c16, queries 4g + i)
    auto scores = [&](int t, bf16x4 &phi, bf16x4 &plo, bf16x4 &dhi, bf16x4 &dlo) {
        const __bf16 *lq = lds_qd[t][0], *ldo = lds_qd[t][1];
        const bf16x8 qa0 = load_bf16x8(&lq[c16 * kTS + 8 * g]);
        const bf16x8 qa1 = load_bf16x8(&lq[c16 * kTS + 32 + 8 * g]);
        const bf16x8 da0 = load_bf16x8(&ldo[c16 * kTS + 8 * g]);
        const bf16x8 da1 = load_bf16x8(&ldo[c16 * kTS + 32 + 8 * g]);
        f32x4 s = mfma_bf16_32(qa0, kb0, f32x4{0.f, 0.f, 0.f, 0.f});
        s = mfma_bf16_32(qa1, kb1, s);
        f32x4 dp = mfma_bf16_32(da0, vb0, f32x4{0.f, 0.f, 0.f, 0.f});
        dp = mfma_bf16_32(da1, vb1, dp);
        const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&lds_ld[t][4 * g]);
        const f32x4 D4 = *reinterpret_cast<const f32x4 *>(&lds_ld[t][kBlock + 4 * g]);
        float pp[4], ds[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pp[i] = fast_exp2(s[i] * a.sl2 - l4[i] * kLog2e);
            ds[i] = pp[i] * (dp[i] - D4[i]);
        }
        split4(pp, phi, plo);
        split4(ds, dhi, dlo);
    };
    auto stage = [&](int t, const Pair &X) {
        store_bf16x8(&lds_qd[t][0][lrow * kTS + lcol], X.qa0);
        store_bf16x8(&lds_qd[t][0][(lrow + 8) * kTS + lcol], X.qa1);
        store_bf16x8(&lds_qd[t][1][lrow * kTS + lcol], X.da0);
        store_bf16x8(&lds_qd[t][1][(lrow + 8) * kTS + lcol], X.da1);
        if (lane < 2 * kBlock) lds_ld[t][lane] = X.ld;
    };
    // one query tile: hi and lo parts as two 16x16x16 products each
    auto compute_one = [&](const Pair &X) {
        wave_lds_sync();
        stage(0, X);
        wave_lds_sync();
        bf16x4 phi, plo, dhi, dlo;
        scores(0, phi, plo, dhi, dlo);
        bf16x4 dT[4], qT[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            dT[dt] = lds_read_tr4(&lds_qd[0][1][rofs + 16 * dt]);
            qT[dt] = lds_read_tr4(&lds_qd[0][0][rofs + 16 * dt]);
            dva[dt] = mfma_bf16_16(phi, dT[dt], dva[dt]);
            dka[dt] = mfma_bf16_16(dhi, qT[dt], dka[dt]);
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            dva[dt] = mfma_bf16_16(plo, dT[dt], dva[dt]);
            dka[dt] = mfma_bf16_16(dlo, qT[dt], dka[dt]);
        }
    };
    // two query tiles: their score chains are independent, and the
    // contractions over queries take the 16 queries of both tiles as the 32
    // k-slots of one MFMA (hi and lo parts in two).  Once both are staged the
    // registers are refilled (reload) while the pair is computed.
    auto compute_pair = [&](Pair &X0, Pair &X1, int n0, bool reload) {
        wave_lds_sync();
        stage(0, X0);
        stage(1, X1);
        if (reload) {
            load_pair(qtile_of(n0), X0);
            load_pair(qtile_of(n0 + 1), X1);
        }
        wave_lds_sync();
        bf16x4 phi0, plo0, dhi0, dlo0, phi1, plo1, dhi1, dlo1;
        scores(0, phi0, plo0, dhi0, dlo0);
        scores(1, phi1, plo1, dhi1, dlo1);
        const bf16x8 ph = cat8(phi0, phi1), pl = cat8(plo0, plo1);
        const bf16x8 dh = cat8(dhi0, dhi1), dl = cat8(dlo0, dlo1);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
            const bf16x8 dT = cat8(lds_read_tr4(&lds_qd[0][1][rofs + 16 * dt]),
                                   lds_read_tr4(&lds_qd[1][1][rofs + 16 * dt]));
            const bf16x8 qT = cat8(lds_read_tr4(&lds_qd[0][0][rofs + 16 * dt]),
                                   lds_read_tr4(&lds_qd[1][0][rofs + 16 * dt]));
            dva[dt] = mfma_bf16_32(pl, dT, mfma_bf16_32(ph, dT, dva[dt]));
            dka[dt] = mfma_bf16_32(dl, qT, mfma_bf16_32(dh, qT, dka[dt]));
        }
    };
    // The segment's query blocks are read 64 at a time into one register
    // (lane j holds entry j); tile j of a batch is sub-tile j % SUB of entry
    // j / SUB.  Ring of kDkvDepth register sets taken two at a time: sets
    // (r, r + 1) hold tiles j + r, j + r + 1 and are refilled with the tiles
    // kDkvDepth further on.
    static_assert(kDkvDepth % 2 == 0, "register sets go in pairs");
    for (int base = e0; base < e1; base += kWave) {
        const int cnt = min(kWave, e1 - base);
        colv = lane < cnt ? C[base + lane] : 0;
        ntl = cnt * SUB;
        Pair R[kDkvDepth];
#pragma unroll
        for (int r = 0; r < kDkvDepth; ++r) load_pair(qtile_of(r), R[r]);
        int j = 0;
        for (; j + kDkvDepth <= ntl; j += kDkvDepth)
#pragma unroll
            for (int r = 0; r < kDkvDepth; r += 2) compute_pair(R[r], R[r + 1], j + kDkvDepth + r, true);
        // the last ntl - j < kDkvDepth tiles sit in sets 0 .. ntl - j - 1
#pragma unroll
        for (int r = 0; r + 1 < kDkvDepth; r += 2) {
            if (j + r + 1 < ntl)
                compute_pair(R[r], R[r + 1], 0, false);
            else if (j + r < ntl)
                compute_one(R[r]);
        }
    }
    }
    // Pooled-level gradients, spread back with weight 1/B^l: every key row of
    // the block gets the same 64 values.  Lane l covers dims 4 (l % 16) .. +3.
    const int oc = 4 * c16;
    f32x4 ck = f32x4{0.f, 0.f, 0.f, 0.f}, cv = ck;
    {
        float inv = a.invB;
        for (int j = 0; j < a.ncl; ++j) {
            inv *= a.invB;
            const int64_t off = a.cl_grad_off[j] + ((int64_t)h * a.cl_n[j] + fb / a.cl_span[j]) * kHeadDim + oc;
            ck += *reinterpret_cast<const f32x4 *>(ws.dpk + off) * inv;
            cv += *reinterpret_cast<const f32x4 *>(ws.dpv + off) * inv;
        }
    }
    // The accumulators hold lane (dim 16dt + c16, keys 4g + i); they pass
    // through LDS so that every store writes whole rows (lane l: row
    // l / 16 + 4 it, dims 4 (l % 16) .. +3).
    auto store_tile = [&](const f32x4 *acc, float mul, f32x4 add, void *dst) {
        wave_lds_sync();
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_out[(4 * g + i) * kOutS + 16 * dt + c16] = acc[dt][i];
        wave_lds_sync();
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = g + 4 * it;
            const f32x4 x = *reinterpret_cast<const f32x4 *>(&lds_out[r * kOutS + oc]) * mul + add;
            const int64_t off = head_off + trow(f, r) + oc;
            if (a.grad_bf16)
                __builtin_nontemporal_store(__builtin_bit_cast(u32x2, to_bf16x4(x)),
                                            reinterpret_cast<u32x2 *>((__bf16 *)dst + off));
            else
                __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>((float *)dst + off));
        }
    };
    store_tile(dka, a.scale, ck, dk);
    store_tile(dva, 1.0f, cv, dv);
}

// Pass C for blocks of 64 tokens: one workgroup per key block, one wave per
// 16-key tile of it.  The 4 key tiles share the block's CSR segment, so the
// workgroup loads each query block's 4 tiles (Q, dO rows and their lse, D)
// once into LDS -- each wave one tile -- and every wave works through all
// four: a quarter of the gathers of one wave per key tile.  Query blocks
// alternate between two LDS buffers; the next one's rows are in flight while
// one is used.
template <int ORD>
__global__ __launch_bounds__(256, 2) void bwd_dkv_b64_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ lse, const __bf16 *__restrict__ dout, const int32_t *__restrict__ csr_ptr,
    const int32_t *__restrict__ csr_col, void *__restrict__ dk, void *__restrict__ dv, BwdWs ws,
    BwdArgs a) {
    constexpr int kSub = 4;
    __shared__ __attribute__((aligned(16))) __bf16 qbuf[2][kSub][kTE];
    __shared__ __attribute__((aligned(16))) __bf16 dbuf[2][kSub][kTE];
    __shared__ __attribute__((aligned(16))) float ldbuf[2][kSub][2 * kBlock];   // lse, D per query tile
    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t kb = xcd_remap(blockIdx.x, gridDim.x);   // key block
    const int h = (int)(kb / a.n1);
    const int fb = (int)(kb % a.n1);
    const int f = fb * kSub + w;   // this wave's key tile
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    auto trow = [&](int b, int r) { return (int64_t)tok_tile_row<ORD>(a.tm, b, r) * kHeadDim; };
    const int32_t *P = csr_ptr + (int64_t)h * (a.n1 + 1);
    const int32_t *C = csr_col + (int64_t)h * a.n1 * a.K1;
    const int e0 = __builtin_amdgcn_readfirstlane(P[fb]), e1 = __builtin_amdgcn_readfirstlane(P[fb + 1]);
    f32x4 dka[4], dva[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        dka[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dva[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int lrow = lane >> 3, lcol = (lane & 7) * 8;
    const int rofs = (4 * g + (c16 >> 2)) * kTS + 4 * (c16 & 3);
    if (e1 > e0) {
        const __bf16 *krow = k + head_off + trow(f, c16);
        const __bf16 *vrow = v + head_off + trow(f, c16);
        const bf16x8 kb0 = load_bf16x8(krow + 8 * g), kb1 = load_bf16x8(krow + 32 + 8 * g);
        const bf16x8 vb0 = load_bf16x8(vrow + 8 * g), vb1 = load_bf16x8(vrow + 32 + 8 * g);
        const uint32_t head_bytes = (uint32_t)a.N * kHeadDim * 2;
        const Rsrc rq = make_rsrc(q + head_off, head_bytes), rdo = make_rsrc(dout + head_off, head_bytes);
        auto brow = [&](int b, int r) {
            return ((uint32_t)tok_tile_row<ORD>(a.tm, b, r) * kHeadDim + lcol) * 2u;
        };
        // wave w's query tile of CSR entry e, as whole rows, and one float per
        // lane (lanes 0-15 the tile's lse, 16-31 its D)
        bf16x8 xq0, xq1, xd0, xd1;
        float xld;
        const float *ld_src = lane < kBlock ? lse : ws.D;
        auto load_entry = [&](int e) {
            const int qt = __builtin_amdgcn_readfirstlane(C[e]) * kSub + w;
            const uint32_t o0 = brow(qt, lrow), o1 = brow(qt, lrow + 8);
            xq0 = buf_load_bf16x8(rq, o0);
            xq1 = buf_load_bf16x8(rq, o1);
            xd0 = buf_load_bf16x8(rdo, o0);
            xd1 = buf_load_bf16x8(rdo, o1);
            xld = ld_src[(int64_t)h * a.N +
                         (lane < kBlock ? tok_tile_row<ORD>(a.tm, qt, c16) : qt * kBlock + c16)];
        };
        load_entry(e0);
        for (int e = e0; e < e1; ++e) {
            const int buf = (e - e0) & 1;
            store_bf16x8(&qbuf[buf][w][lrow * kTS + lcol], xq0);
            store_bf16x8(&qbuf[buf][w][(lrow + 8) * kTS + lcol], xq1);
            store_bf16x8(&dbuf[buf][w][lrow * kTS + lcol], xd0);
            store_bf16x8(&dbuf[buf][w][(lrow + 8) * kTS + lcol], xd1);
            if (lane < 2 * kBlock) ldbuf[buf][w][lane] = xld;
            // the entry's four tiles staged; every wave is done with entry e - 2
            __syncthreads();
            if (e + 1 < e1) load_entry(e + 1);
#pragma unroll 1
            for (int t = 0; t < kSub; ++t) {
                const __bf16 *qs = qbuf[buf][t], *ds_ = dbuf[buf][t];
                const f32x4 s = mfma_bf16_32(load_bf16x8(&qs[c16 * kTS + 32 + 8 * g]), kb1,
                                             mfma_bf16_32(load_bf16x8(&qs[c16 * kTS + 8 * g]), kb0,
                                                          f32x4{0.f, 0.f, 0.f, 0.f}));
                const f32x4 dp = mfma_bf16_32(load_bf16x8(&ds_[c16 * kTS + 32 + 8 * g]), vb1,
                                              mfma_bf16_32(load_bf16x8(&ds_[c16 * kTS + 8 * g]), vb0,
                                                           f32x4{0.f, 0.f, 0.f, 0.f}));
                const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&ldbuf[buf][t][4 * g]);
                const f32x4 D4 = *reinterpret_cast<const f32x4 *>(&ldbuf[buf][t][kBlock + 4 * g]);
                float pp[4], dsv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pp[i] = fast_exp2(s[i] * a.sl2 - l4[i] * kLog2e);
                    dsv[i] = pp[i] * (dp[i] - D4[i]);
                }
                bf16x4 phi, plo, dhi, dlo;
                split4(pp, phi, plo);
                split4(dsv, dhi, dlo);
                bf16x4 dT[4], qT[4];
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    dT[dt] = lds_read_tr4(&ds_[rofs + 16 * dt]);
                    qT[dt] = lds_read_tr4(&qs[rofs + 16 * dt]);
                    dva[dt] = mfma_bf16_16(phi, dT[dt], dva[dt]);
                    dka[dt] = mfma_bf16_16(dhi, qT[dt], dka[dt]);
                }
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    dva[dt] = mfma_bf16_16(plo, dT[dt], dva[dt]);
                    dka[dt] = mfma_bf16_16(dlo, qT[dt], dka[dt]);
                }
            }
        }
        __syncthreads();   // the buffers become the output staging below
    }
    // pooled-level gradients, spread back with weight 1/B^l (lane: dims 4 (l % 16) ..)
    const int oc = 4 * c16;
    f32x4 ck = f32x4{0.f, 0.f, 0.f, 0.f}, cv = ck;
    {
        float inv = a.invB;
        for (int j = 0; j < a.ncl; ++j) {
            inv *= a.invB;
            const int64_t off = a.cl_grad_off[j] + ((int64_t)h * a.cl_n[j] + fb / a.cl_span[j]) * kHeadDim + oc;
            ck += *reinterpret_cast<const f32x4 *>(ws.dpk + off) * inv;
            cv += *reinterpret_cast<const f32x4 *>(ws.dpv + off) * inv;
        }
    }
    float *lds_out = reinterpret_cast<float *>(qbuf[0][0]) + w * kBlock * kOutS;   // 4 x 4352 B fit
    auto store_tile = [&](const f32x4 *acc, float mul, f32x4 add, void *dst) {
        wave_lds_sync();
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) lds_out[(4 * g + i) * kOutS + 16 * dt + c16] = acc[dt][i];
        wave_lds_sync();
#pragma unroll
        for (int it = 0; it < 4; ++it) {
            const int r = g + 4 * it;
            const f32x4 x = *reinterpret_cast<const f32x4 *>(&lds_out[r * kOutS + oc]) * mul + add;
            const int64_t off = head_off + trow(f, r) + oc;
            if (a.grad_bf16)
                __builtin_nontemporal_store(__builtin_bit_cast(u32x2, to_bf16x4(x)),
                                            reinterpret_cast<u32x2 *>((__bf16 *)dst + off));
            else
                __builtin_nontemporal_store(x, reinterpret_cast<f32x4 *>((float *)dst + off));
        }
    };
    store_tile(dka, a.scale, ck, dk);
    store_tile(dva, 1.0f, cv, dv);
}

// ================================================================ f32 path
// Float32 inputs run on the float32 matrix cores (16 x 16 x 4).  Keys and
// queries are visited in a fixed order throughout and every sum is taken in a
// fixed order, so the results are reproducible.

// Pass A (f32): one workgroup per group of 16 consecutive query tiles (all
// under one level-2 node, so they share their coarse entries), wave w taking
// tiles w, w + 4, w + 8, w + 12 (neighbours at a time, which share key tiles
// in the L1), on the float32 matrix cores and laid out as the float32 forward
// (scores transposed, lane (g, c): query c against keys 4g .. 4g + 3; row
// layout for Q, dO, K and V in the score products, column layout for K in
// dQ^T += K^T dS^T).  D = rowsum(dO * O) comes from O first, so dS = P (dP -
// D) is formed tile by tile.  The pooled-token gradients of each coarse tile
// are then summed over the group: the coarse scores are recomputed query-major
// (lane (g, c): entry c against queries 4g .. 4g + 3), so P and dS feed
// dK_c^T += Q^T dS and dV_c^T += dO^T P with Q and dO in the column layout;
// the 4 waves' sums meet in LDS, in wave order, and are written as the group's
// partial rows, which the coarse reduction adds per pooled token.
__global__ __launch_bounds__(256, 2) void bwd_dq_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ pk, const float *__restrict__ pv, const int32_t *__restrict__ idx,
    const float *__restrict__ o, const float *__restrict__ lse, const float *__restrict__ dout,
    void *__restrict__ dq, BwdWs ws, BwdArgs a) {
    __shared__ __attribute__((aligned(16))) float red[4][2][kBlock * kHeadDim];   // waves' coarse sums
    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int gph = (a.nt1 + kBlock - 1) / kBlock;   // groups per head
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    if (bid >= a.bh * gph) return;   // the whole workgroup
    const int h = bid / gph;
    const int G = bid % gph;
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    auto trow = [&](int b, int r) { return (int64_t)tok_row(a.tm, b * kBlock + r) * kHeadDim; };
    const int nft = a.K1 * a.sub;
    const int nct = (a.ncoarse + kBlock - 1) / kBlock;
    struct KVT {
        float kr[16], vr[16];   // K and V row c (row layout)
        f32x4 kc[4];            // K rows 4g + i, dims 4c .. 4c + 3 (column layout)
    };
    // pooled row of coarse entry e (-1: no such entry) and its log2 weight for
    // query block ib (-inf where the entry is dropped for the block)
    auto coarse_row = [&](int ib, const int32_t *fine, int e, float &bias) -> int64_t {
        int jl = 0, c = -1;
        float b = 0.f;
        const bool ok = bwd_coarse_entry(a, idx, fine, h, ib, e, jl, c, b);
        bias = ok ? b : -INFINITY;
        return c >= 0 ? a.cl_pyr_off[jl] + ((int64_t)h * a.cl_n[jl] + c) * kHeadDim : -1;
    };
    float Dv[4], L2v[4];   // D and lse * log2(e) of query c16 of the wave's tiles
    // ---- dQ of the wave's 4 tiles
    for (int jt = 0; jt < 4; ++jt) {
        const int qt = G * kBlock + 4 * jt + w;
        Dv[jt] = L2v[jt] = 0.f;
        if (qt >= a.nt1) break;   // ragged last group (single level only)
        const int ib = qt / a.sub;
        const int64_t qoff = head_off + trow(qt, c16) + 16 * g;
        float qf[16], gf[16];
        load_row16(q + qoff, qf);
        load_row16(dout + qoff, gf);
        float D;
        {
            float of[16];
            load_row16(o + qoff, of);
            float part = 0.f;
#pragma unroll
            for (int d = 0; d < 16; ++d) part = fmaf(gf[d], of[d], part);
            D = sum4_groups(part);
        }
        if (g == 0) ws.D[(int64_t)h * a.N + (int64_t)qt * kBlock + c16] = D;   // by sequence position
        const float lse2 = lse[(int64_t)h * a.N + tok_row(a.tm, qt * kBlock + c16)] * kLog2e;
        Dv[jt] = D;
        L2v[jt] = lse2;
        const int32_t *fine = idx + ((int64_t)h * a.n1 + ib) * a.K1;
        f32x4 acc[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        auto load_fine = [&](int tt, KVT &T) {
            const int f = __builtin_amdgcn_readfirstlane(fine[tt / a.sub]) * a.sub + tt % a.sub;
            const int64_t rc = head_off + trow(f, c16) + 16 * g;
            load_row16(k + rc, T.kr);
            load_row16(v + rc, T.vr);
#pragma unroll
            for (int i = 0; i < 4; ++i) T.kc[i] = *reinterpret_cast<const f32x4 *>(k + head_off + trow(f, 4 * g + i) + 4 * c16);
        };
        auto visit = [&](const KVT &T, const float (&bias)[4]) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = s;
#pragma unroll
            for (int d = 0; d < 16; ++d) {
                s = mfma_f32_4(T.kr[d], qf[d], s);
                dp = mfma_f32_4(T.vr[d], gf[d], dp);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(s[i] * a.sl2 + bias[i] - lse2);
                const float ds = p * (dp[i] - D);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) acc[dt] = mfma_f32_4(T.kc[i][dt], ds, acc[dt]);
            }
        };
        const float nobias[4] = {0.f, 0.f, 0.f, 0.f};
        KVT T0, T1;
        if (nft > 0) load_fine(0, T0);
        for (int tt = 0; tt < nft; tt += 2) {
            if (tt + 1 < nft) load_fine(tt + 1, T1);
            visit(T0, nobias);
            if (tt + 2 < nft) load_fine(tt + 2, T0);
            if (tt + 1 < nft) visit(T1, nobias);
        }
        // coarse entries, 16 a tile; absent or dropped ones read row 0 and are masked
        for (int ct = 0; ct < nct; ++ct) {
            KVT T;
            float bias[4], bk;
            const int64_t rk = coarse_row(ib, fine, ct * kBlock + c16, bk);
            const int64_t rks = rk < 0 ? 0 : rk;
            load_row16(pk + rks + 16 * g, T.kr);
            load_row16(pv + rks + 16 * g, T.vr);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t ri = coarse_row(ib, fine, ct * kBlock + 4 * g + i, bias[i]);
                T.kc[i] = *reinterpret_cast<const f32x4 *>(pk + (ri < 0 ? 0 : ri) + 4 * c16);
            }
            visit(T, bias);
        }
        // lane (g, c) holds dims 16g + 4j + dt of query c
#pragma unroll
        for (int j = 0; j < 4; ++j)
            store_grad4(dq, qoff + 4 * j, f32x4{acc[0][j], acc[1][j], acc[2][j], acc[3][j]} * a.scale, a.grad_bf16);
    }
    // ---- pooled-token gradients of the group, one coarse tile at a time
    for (int ct = 0; ct < nct; ++ct) {
        f32x4 gk[4], gv[4];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) gk[dt] = gv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        float er[16], ev[16];   // entry c16's pooled K and V rows (the same for the whole group)
        bool loaded = false;
        for (int jt = 0; jt < 4; ++jt) {
            const int qt = G * kBlock + 4 * jt + w;
            if (qt >= a.nt1) break;
            const int ib = qt / a.sub;
            const int32_t *fine = idx + ((int64_t)h * a.n1 + ib) * a.K1;
            float bias;
            const int64_t rk = coarse_row(ib, fine, ct * kBlock + c16, bias);
            if (!loaded) {
                const int64_t rks = rk < 0 ? 0 : rk;
                load_row16(pk + rks + 16 * g, er);
                load_row16(pv + rks + 16 * g, ev);
                loaded = true;
            }
            const int64_t qoff = head_off + trow(qt, c16) + 16 * g;
            float qf[16], gf[16];
            load_row16(q + qoff, qf);
            load_row16(dout + qoff, gf);
            f32x4 qc[4], dc[4];
            float l2[4], Dq[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t r = head_off + trow(qt, 4 * g + i) + 4 * c16;
                qc[i] = *reinterpret_cast<const f32x4 *>(q + r);
                dc[i] = *reinterpret_cast<const f32x4 *>(dout + r);
                l2[i] = __shfl(L2v[jt], 4 * g + i, kWave);   // lane 4g + i holds query 4g + i
                Dq[i] = __shfl(Dv[jt], 4 * g + i, kWave);
            }
            f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = s;
#pragma unroll
            for (int d = 0; d < 16; ++d) {
                s = mfma_f32_4(qf[d], er[d], s);
                dp = mfma_f32_4(gf[d], ev[d], dp);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float p = fast_exp2(s[i] * a.sl2 + bias - l2[i]);
                const float ds = p * (dp[i] - Dq[i]);
#pragma unroll
                for (int dt = 0; dt < 4; ++dt) {
                    gk[dt] = mfma_f32_4(qc[i][dt], ds, gk[dt]);
                    gv[dt] = mfma_f32_4(dc[i][dt], p, gv[dt]);
                }
            }
        }
        // lane (g, c): dims 16g + 4j + dt of entry c
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            *reinterpret_cast<f32x4 *>(&red[w][0][c16 * kHeadDim + 16 * g + 4 * j]) =
                f32x4{gk[0][j], gk[1][j], gk[2][j], gk[3][j]} * a.scale;
            *reinterpret_cast<f32x4 *>(&red[w][1][c16 * kHeadDim + 16 * g + 4 * j]) =
                f32x4{gv[0][j], gv[1][j], gv[2][j], gv[3][j]};
        }
        __syncthreads();
        const int ne = min(kBlock, a.ncoarse - ct * kBlock);
        float *part = ws.partial + (((int64_t)h * a.npg + G) * a.ncoarse + ct * kBlock) * 2 * kHeadDim;
        for (int x = threadIdx.x; x < ne * 2 * kHeadDim; x += 256) {
            const int e = x / (2 * kHeadDim), kv = (x / kHeadDim) & 1, dim = x % kHeadDim;
            const int oo = e * kHeadDim + dim;
            part[x] = red[0][kv][oo] + red[1][kv][oo] + red[2][kv][oo] + red[3][kv][oo];
        }
        __syncthreads();
    }
}

// Pass C (f32): one wave per 16-key tile on the matrix cores, walking the
// query tiles of its key block's CSR segment.  Scores are computed query-major
// here, S = Q K^T: lane (g, c) holds key c against queries 4g .. 4g + 3 of a
// query tile, so P and dS feed dV^T += dO^T P and dK^T += Q^T dS straight from
// the score registers, with dO and Q in the column layout; lane (g, c) ends
// with dims 16g .. 16g + 15 of key c.
__global__ __launch_bounds__(256) void bwd_dkv_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ lse, const float *__restrict__ dout, const int32_t *__restrict__ csr_ptr,
    const int32_t *__restrict__ csr_col, void *__restrict__ dk, void *__restrict__ dv, BwdWs ws,
    BwdArgs a) {
    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int64_t kb = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * 4 + w;   // key tile
    if (kb >= (int64_t)a.bh * a.nt1) return;
    const int h = (int)(kb / a.nt1);
    const int f = (int)(kb % a.nt1);
    const int fb = f / a.sub;   // its key block
    const int64_t head_off = (int64_t)h * a.N * kHeadDim;
    auto trow = [&](int b, int r) { return (int64_t)tok_row(a.tm, b * kBlock + r) * kHeadDim; };
    const int64_t koff = head_off + trow(f, c16) + 16 * g;
    float kf[16], vf[16];
    load_row16(k + koff, kf);
    load_row16(v + koff, vf);
    const int32_t *P = csr_ptr + (int64_t)h * (a.n1 + 1);
    const int32_t *C = csr_col + (int64_t)h * a.n1 * a.K1;
    const int e0 = __builtin_amdgcn_readfirstlane(P[fb]), e1 = __builtin_amdgcn_readfirstlane(P[fb + 1]);
    f32x4 gk[4], gv[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) gk[dt] = gv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    struct QT {
        float qr[16], dr[16];   // Q and dO row c (row layout)
        f32x4 qc[4], dc[4];     // Q and dO rows 4g + i, dims 4c .. 4c + 3 (column layout)
        float l2[4], Dv[4];     // lse * log2(e) and D of queries 4g + i
    };
    auto load_q = [&](int et, QT &X) {
        const int qt = __builtin_amdgcn_readfirstlane(C[et / a.sub]) * a.sub + et % a.sub;
        const int64_t rc = head_off + trow(qt, c16) + 16 * g;
        load_row16(q + rc, X.qr);
        load_row16(dout + rc, X.dr);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int pos = qt * kBlock + 4 * g + i;
            const int64_t srow = tok_row(a.tm, pos);
            X.qc[i] = *reinterpret_cast<const f32x4 *>(q + head_off + srow * kHeadDim + 4 * c16);
            X.dc[i] = *reinterpret_cast<const f32x4 *>(dout + head_off + srow * kHeadDim + 4 * c16);
            X.l2[i] = lse[(int64_t)h * a.N + srow] * kLog2e;
            X.Dv[i] = ws.D[(int64_t)h * a.N + pos];
        }
    };
    auto visit = [&](const QT &X) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = s;
#pragma unroll
        for (int d = 0; d < 16; ++d) {
            s = mfma_f32_4(X.qr[d], kf[d], s);
            dp = mfma_f32_4(X.dr[d], vf[d], dp);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float p = fast_exp2(s[i] * a.sl2 - X.l2[i]);
            const float ds = p * (dp[i] - X.Dv[i]);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                gv[dt] = mfma_f32_4(X.dc[i][dt], p, gv[dt]);
                gk[dt] = mfma_f32_4(X.qc[i][dt], ds, gk[dt]);
            }
        }
    };
    QT X;
    for (int et = e0 * a.sub; et < e1 * a.sub; ++et) {   // query tiles of the segment's blocks
        load_q(et, X);
        visit(X);
    }
    // pooled-level gradients, spread back with weight 1/B^l (dims 16g + 4j .. + 3)
    f32x4 ck[4], cv[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) ck[j] = cv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    float inv = 1.f;
    for (int jl = 0; jl < a.ncl; ++jl) {
        inv *= a.invB;
        const int64_t off = a.cl_grad_off[jl] + ((int64_t)h * a.cl_n[jl] + fb / a.cl_span[jl]) * kHeadDim + 16 * g;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ck[j] += *reinterpret_cast<const f32x4 *>(ws.dpk + off + 4 * j) * (inv * a.invB);
            cv[j] += *reinterpret_cast<const f32x4 *>(ws.dpv + off + 4 * j) * (inv * a.invB);
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        store_grad4(dk, koff + 4 * j, f32x4{gk[0][j], gk[1][j], gk[2][j], gk[3][j]} * a.scale + ck[j], a.grad_bf16);
        store_grad4(dv, koff + 4 * j, f32x4{gv[0][j], gv[1][j], gv[2][j], gv[3][j]} + cv[j], a.grad_bf16);
    }
}

hipError_t launch_attn_bwd(const Geometry &g, const void *q, const void *k, const void *v,
                           const float *pk, const float *pv, const int32_t *idx,
                           const int32_t *csr_ptr, const int32_t *csr_col, const void *o,
                           const float *lse, const void *dout, void *dq, void *dk, void *dv,
                           void *wsp, hipStream_t s) {
    const BwdArgs a = make_bwd_args(g);
    const BwdWs ws = carve_ws(g, a, wsp);
    if (g.bf16) {
        const int gph = (a.nt1 + kBlock - 1) / kBlock;
        const int nct = (a.ncoarse + kBlock - 1) / kBlock;
        const dim3 grid((unsigned)(g.bh * gph));
        // the streaming kernel for B = 16, at most one coarse tile and K_1 in {8, 16, 20, 32}
        using Kern = void (*)(const __bf16 *, const __bf16 *, const __bf16 *, const float *,
                              const float *, const int32_t *, const float *, const __bf16 *, void *,
                              BwdWs, BwdArgs);
        static const Kern table[2][2][4] = {
            {{bwd_dq_fast_kernel<8, false, 0>, bwd_dq_fast_kernel<16, false, 0>,
              bwd_dq_fast_kernel<20, false, 0>, bwd_dq_fast_kernel<32, false, 0>},
             {bwd_dq_fast_kernel<8, true, 0>, bwd_dq_fast_kernel<16, true, 0>,
              bwd_dq_fast_kernel<20, true, 0>, bwd_dq_fast_kernel<32, true, 0>}},
            {{bwd_dq_fast_kernel<8, false, 1>, bwd_dq_fast_kernel<16, false, 1>,
              bwd_dq_fast_kernel<20, false, 1>, bwd_dq_fast_kernel<32, false, 1>},
             {bwd_dq_fast_kernel<8, true, 1>, bwd_dq_fast_kernel<16, true, 1>,
              bwd_dq_fast_kernel<20, true, 1>, bwd_dq_fast_kernel<32, true, 1>}}};
        const int kslot = a.K1 == 8 ? 0 : a.K1 == 16 ? 1 : a.K1 == 20 ? 2 : a.K1 == 32 ? 3 : -1;
        const bool fast = g.B == kBlock && a.n1 % kBlock == 0 && nct <= 1 && kslot >= 0;
        if (fast)
            hipLaunchKernelGGL(table[g.order][nct][kslot], grid, dim3(256), 0, s, (const __bf16 *)q,
                               (const __bf16 *)k, (const __bf16 *)v, pk, pv, idx, lse,
                               (const __bf16 *)dout, dq, ws, a);
        else if (g.B == 4 * kBlock && nct <= 1 && a.n1 % 4 == 0)   // blocks of 64: shared key tiles
            hipLaunchKernelGGL((g.order == 0 ? bwd_dq_b64_kernel<0> : bwd_dq_b64_kernel<1>),
                               dim3((unsigned)(g.bh * (a.n1 / 4))), dim3(256), 0, s, (const __bf16 *)q,
                               (const __bf16 *)k, (const __bf16 *)v, pk, pv, idx, lse,
                               (const __bf16 *)dout, dq, ws, a);
        else if (nct == 0)
            hipLaunchKernelGGL(bwd_dq_bf16_kernel<0>, grid, dim3(256), 0, s, (const __bf16 *)q,
                               (const __bf16 *)k, (const __bf16 *)v, pk, pv, idx, lse,
                               (const __bf16 *)dout, dq, ws, a);
        else if (nct == 1)
            hipLaunchKernelGGL(bwd_dq_bf16_kernel<1>, grid, dim3(256), 0, s, (const __bf16 *)q,
                               (const __bf16 *)k, (const __bf16 *)v, pk, pv, idx, lse,
                               (const __bf16 *)dout, dq, ws, a);
        else
            hipLaunchKernelGGL(bwd_dq_bf16_kernel<2>, grid, dim3(256), 0, s, (const __bf16 *)q,
                               (const __bf16 *)k, (const __bf16 *)v, pk, pv, idx, lse,
                               (const __bf16 *)dout, dq, ws, a);
        for (int j = 0; j < a.ncl; ++j) {
            const int64_t toks = (int64_t)g.bh * a.cl_n[j];
            hipLaunchKernelGGL(bwd_coarse_reduce_kernel, dim3((unsigned)((toks + 3) / 4)),
                               dim3(256), 0, s, idx, csr_ptr, csr_col, ws, a, j);
        }
        const int64_t kts = (int64_t)g.bh * a.nt1;   // key tiles
        if (g.sub == 1) {
            hipLaunchKernelGGL((g.order == 0 ? bwd_dkv_bf16_kernel<0, 1> : bwd_dkv_bf16_kernel<1, 1>),
                               dim3((unsigned)kts), dim3(kWave), 0, s, (const __bf16 *)q,
                               (const __bf16 *)k, (const __bf16 *)v, lse, (const __bf16 *)dout,
                               csr_ptr + g.ptr_off[1], csr_col + g.col_off[1], dk, dv, ws, a);
        } else {   // blocks of 64 tokens: a workgroup per key block
            hipLaunchKernelGGL((g.order == 0 ? bwd_dkv_b64_kernel<0> : bwd_dkv_b64_kernel<1>),
                               dim3((unsigned)((int64_t)g.bh * a.n1)), dim3(256), 0, s, (const __bf16 *)q,
                               (const __bf16 *)k, (const __bf16 *)v, lse, (const __bf16 *)dout,
                               csr_ptr + g.ptr_off[1], csr_col + g.col_off[1], dk, dv, ws, a);
        }
    } else {
        const int64_t tiles = (int64_t)g.bh * a.nt1;   // query tiles = key tiles
        const int64_t groups = (int64_t)g.bh * ((a.nt1 + kBlock - 1) / kBlock);
        hipLaunchKernelGGL(bwd_dq_f32_kernel, dim3((unsigned)groups), dim3(256), 0, s,
                           (const float *)q, (const float *)k, (const float *)v, pk, pv, idx,
                           (const float *)o, lse, (const float *)dout, dq, ws, a);
        for (int j = 0; j < a.ncl; ++j) {
            const int64_t toks = (int64_t)g.bh * a.cl_n[j];
            hipLaunchKernelGGL(bwd_coarse_reduce_kernel, dim3((unsigned)((toks + 3) / 4)),
                               dim3(256), 0, s, idx, csr_ptr, csr_col, ws, a, j);
        }
        hipLaunchKernelGGL(bwd_dkv_f32_kernel, dim3((unsigned)((tiles + 3) / 4)), dim3(256), 0,
                           s, (const float *)q, (const float *)k, (const float *)v, lse,
                           (const float *)dout, csr_ptr + g.ptr_off[1], csr_col + g.col_off[1], dk,
                           dv, ws, a);
    }
    return hipGetLastError();
}

}  // namespace llsa
