// Dense (full, non-causal) softmax attention forward in the same tile style
// as the sparse kernel: the comparator for the speed-up of the enriched
// sparse attention over full attention ("Trainable Log-linear Sparse
// Attention for Efficient Diffusion Transformers", explainer "The
// Scoreboard").
//
// One 512-thread workgroup owns 128 queries (8 waves x 16).  For every step of
// 128 keys the workgroup stages the K and V tiles in LDS once (K as row-major
// rows for the MFMA A operand, V for the transposing read), and each wave runs
// the same S^T = K Q^T / online softmax / O^T += V^T P^T chunk as the sparse
// forward.
#include "common.hpp"
#include "internal.hpp"
#include "attn_tile.hpp"

namespace llsa {

constexpr int kDenseWaves = 8;
constexpr int kDenseKeys = kFwdTiles * kBlock;  // keys per step

__global__ __launch_bounds__(512) void dense_fwd_bf16_kernel(const __bf16 *__restrict__ q,
                                                            const __bf16 *__restrict__ k,
                                                            const __bf16 *__restrict__ v,
                                                            __bf16 *__restrict__ o,
                                                            float *__restrict__ lse, int N,
                                                            int qtiles_per_head, float sl2) {
    __shared__ __attribute__((aligned(16))) __bf16 ks[kFwdTiles * kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 vs[kFwdTiles * kTileElems];
    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = bid / qtiles_per_head;
    const int qt = bid % qtiles_per_head;
    const int64_t head_off = (int64_t)h * N * kHeadDim;
    const int q0 = qt * (kDenseWaves * kBlock) + w * kBlock;
    const bool active = q0 < N;
    const __bf16 *qrow = q + head_off + (int64_t)((active ? q0 : 0) + c16) * kHeadDim;
    const bf16x8 qa0 = load_bf16x8(qrow + 8 * g);
    const bf16x8 qa1 = load_bf16x8(qrow + 32 + 8 * g);

    float m = -INFINITY, lsum = 0.f;
    f32x4 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float bias[kFwdTiles][4];   // unused: every weight is 1
    f32x4 st[kFwdTiles];

    for (int k0 = 0; k0 < N; k0 += kDenseKeys) {
        const int nt = min(kFwdTiles, (N - k0) / kBlock);
        __syncthreads();
        // stage: 128 keys x 64 dims of K and of V = 1024 chunks of 16 B each
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int ci = threadIdx.x + 512 * r;      // chunk id in [0, 1024)
            const int key = ci >> 3, col = (ci & 7) * 8;
            if (key < nt * kBlock) {
                const int64_t src = head_off + (int64_t)(k0 + key) * kHeadDim + col;
                const int dst = (key >> 4) * kTileElems + (key & 15) * kVStride + col;
                store_bf16x8(ks + dst, load_bf16x8(k + src));
                store_bf16x8(vs + dst, load_bf16x8(v + src));
            }
        }
        __syncthreads();
        if (active) {
#pragma unroll
            for (int t = 0; t < kFwdTiles; ++t) {
                if (t < nt) {
                    const __bf16 *kr = ks + t * kTileElems + c16 * kVStride;
                    const bf16x8 ka0 = load_bf16x8(kr + 8 * g);
                    const bf16x8 ka1 = load_bf16x8(kr + 32 + 8 * g);
                    f32x4 s = mfma_bf16_32(ka0, qa0, f32x4{0.f, 0.f, 0.f, 0.f});
                    s = mfma_bf16_32(ka1, qa1, s);
                    st[t] = s * sl2;
                }
            }
            softmax_pv_chunk<false>(st, bias, nt, vs, m, lsum, oacc, g, c16);
        }
    }
    if (!active) return;
    lsum = sum4_groups(lsum);
    const float inv = 1.0f / lsum;
    __bf16 *orow = o + head_off + (int64_t)(q0 + c16) * kHeadDim + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        const f32x4 r = oacc[dt] * inv;
        const bf16x4 rb = to_bf16x4(f32x4{r[0], r[1], r[2], r[3]});
        *reinterpret_cast<u32x2 *>(orow + 16 * dt) = __builtin_bit_cast(u32x2, rb);
    }
    if (g == 0) lse[(int64_t)h * N + q0 + c16] = (m + log2f(lsum)) * kLn2;
}

// ------------------------------------------------------------ backward
// Dense backward for the loss <O, dO> in two passes of the same style, the
// comparator for the sparse backward: a query-major pass for dQ (which also
// forms D = rowsum(dO * O) for its queries) and a key-major pass for dK, dV.
// Gradients are float32; P and dS enter the MFMAs in bf16, as in common
// flash-attention backward kernels.

// dQ: one 512-thread workgroup per 128 queries (8 waves x 16); K and V tiles
// of 128 keys are staged in LDS per step.  Per wave and key tile:
// S^T = K Q^T and dP^T = V dO^T (lane: query c16, keys 4g+i), P = exp(S - lse),
// dS = P (dP - D), and dQ^T += K^T dS^T over tile pairs.
__global__ __launch_bounds__(512) void dense_bwd_dq_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const __bf16 *__restrict__ o, const float *__restrict__ lse, const __bf16 *__restrict__ dout,
    float *__restrict__ dq, float *__restrict__ Dws, int N, int qtiles_per_head, float sl2,
    float scale) {
    __shared__ __attribute__((aligned(16))) __bf16 ks[kFwdTiles * kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 vs[kFwdTiles * kTileElems];
    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = bid / qtiles_per_head;
    const int qt = bid % qtiles_per_head;
    const int64_t head_off = (int64_t)h * N * kHeadDim;
    const int q0 = qt * (kDenseWaves * kBlock) + w * kBlock;
    const bool active = q0 < N;
    const int64_t row = (int64_t)(active ? q0 : 0) + c16;
    const __bf16 *qrow = q + head_off + row * kHeadDim;
    const __bf16 *drow = dout + head_off + row * kHeadDim;
    const __bf16 *orow = o + head_off + row * kHeadDim;
    const bf16x8 qa0 = load_bf16x8(qrow + 8 * g), qa1 = load_bf16x8(qrow + 32 + 8 * g);
    const bf16x8 da0 = load_bf16x8(drow + 8 * g), da1 = load_bf16x8(drow + 32 + 8 * g);
    // D of query c16: the lane's 16 dims, then the 4 lanes of the query
    float dpart = 0.f;
    {
        const bf16x8 oa0 = load_bf16x8(orow + 8 * g), oa1 = load_bf16x8(orow + 32 + 8 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i)
            dpart += (float)da0[i] * (float)oa0[i] + (float)da1[i] * (float)oa1[i];
    }
    const float Dq = sum4_groups(dpart);
    const float lse2 = lse[(int64_t)h * N + row] * kLog2e;
    if (active && g == 0) Dws[(int64_t)h * N + row] = Dq;
    f32x4 acc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int rofs = (4 * g + (c16 >> 2)) * kVStride + 4 * (c16 & 3);
    for (int k0 = 0; k0 < N; k0 += kDenseKeys) {
        const int nt = min(kFwdTiles, (N - k0) / kBlock);
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int ci = threadIdx.x + 512 * r;
            const int key = ci >> 3, col = (ci & 7) * 8;
            const int dst = (key >> 4) * kTileElems + (key & 15) * kVStride + col;
            bf16x8 kk = {}, vv = {};   // rows past the end stay zero
            if (key < nt * kBlock) {
                const int64_t src = head_off + (int64_t)(k0 + key) * kHeadDim + col;
                kk = load_bf16x8(k + src);
                vv = load_bf16x8(v + src);
            }
            store_bf16x8(ks + dst, kk);
            store_bf16x8(vs + dst, vv);
        }
        __syncthreads();
        if (!active) continue;
#pragma unroll
        for (int tp = 0; tp < kFwdTiles / 2; ++tp) {
            bf16x4 dsb[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int t = 2 * tp + u;
                const __bf16 *kr = ks + t * kTileElems + c16 * kVStride;
                const __bf16 *vr = vs + t * kTileElems + c16 * kVStride;
                const f32x4 st = mfma_bf16_32(load_bf16x8(kr + 32 + 8 * g), qa1,
                                              mfma_bf16_32(load_bf16x8(kr + 8 * g), qa0, f32x4{0.f, 0.f, 0.f, 0.f}));
                const f32x4 dp = mfma_bf16_32(load_bf16x8(vr + 32 + 8 * g), da1,
                                              mfma_bf16_32(load_bf16x8(vr + 8 * g), da0, f32x4{0.f, 0.f, 0.f, 0.f}));
                f32x4 ds;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    ds[i] = t < nt ? fast_exp2(st[i] * sl2 - lse2) * (dp[i] - Dq) : 0.f;
                dsb[u] = to_bf16x4(ds);
            }
            const bf16x8 dsc = cat8(dsb[0], dsb[1]);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x4 k0t = lds_read_tr4(ks + (2 * tp) * kTileElems + rofs + 16 * dt);
                const bf16x4 k1t = lds_read_tr4(ks + (2 * tp + 1) * kTileElems + rofs + 16 * dt);
                acc[dt] = mfma_bf16_32(cat8(k0t, k1t), dsc, acc[dt]);
            }
        }
    }
    if (!active) return;
    float *dqrow = dq + head_off + row * kHeadDim + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
        *reinterpret_cast<f32x4 *>(dqrow + 16 * dt) = acc[dt] * scale;
}

// dK, dV: one 512-thread workgroup per 128 keys (8 waves x 16); Q and dO
// tiles of 128 queries are staged in LDS per step with their lse and D.  Per
// wave and query tile: S = Q K^T and dP = dO V^T (lane: key c16, queries
// 4g+i), and over tile pairs dV += P^T dO, dK += dS^T Q.
__global__ __launch_bounds__(512) void dense_bwd_dkv_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const float *__restrict__ lse, const float *__restrict__ Dws, const __bf16 *__restrict__ dout,
    float *__restrict__ dk, float *__restrict__ dv, int N, int ktiles_per_head, float sl2,
    float scale) {
    __shared__ __attribute__((aligned(16))) __bf16 qs[kFwdTiles * kTileElems];
    __shared__ __attribute__((aligned(16))) __bf16 ds_[kFwdTiles * kTileElems];
    __shared__ __attribute__((aligned(16))) float ls[kDenseKeys], Ds[kDenseKeys];
    const int w = wave_id();
    const int lane = lane_id();
    const int g = lane >> 4, c16 = lane & 15;
    const int bid = xcd_remap(blockIdx.x, gridDim.x);
    const int h = bid / ktiles_per_head;
    const int kt = bid % ktiles_per_head;
    const int64_t head_off = (int64_t)h * N * kHeadDim;
    const int f0 = kt * (kDenseWaves * kBlock) + w * kBlock;
    const bool active = f0 < N;
    const int64_t krow_i = (int64_t)(active ? f0 : 0) + c16;
    const __bf16 *krow = k + head_off + krow_i * kHeadDim;
    const __bf16 *vrow = v + head_off + krow_i * kHeadDim;
    const bf16x8 kb0 = load_bf16x8(krow + 8 * g), kb1 = load_bf16x8(krow + 32 + 8 * g);
    const bf16x8 vb0 = load_bf16x8(vrow + 8 * g), vb1 = load_bf16x8(vrow + 32 + 8 * g);
    f32x4 dka[4], dva[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
        dka[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dva[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const int rofs = (4 * g + (c16 >> 2)) * kVStride + 4 * (c16 & 3);
    for (int q0 = 0; q0 < N; q0 += kDenseKeys) {
        const int nt = min(kFwdTiles, (N - q0) / kBlock);
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int ci = threadIdx.x + 512 * r;
            const int qq = ci >> 3, col = (ci & 7) * 8;
            const int dst = (qq >> 4) * kTileElems + (qq & 15) * kVStride + col;
            bf16x8 qv = {}, dv8 = {};   // rows past the end stay zero
            if (qq < nt * kBlock) {
                const int64_t src = head_off + (int64_t)(q0 + qq) * kHeadDim + col;
                qv = load_bf16x8(q + src);
                dv8 = load_bf16x8(dout + src);
            }
            store_bf16x8(qs + dst, qv);
            store_bf16x8(ds_ + dst, dv8);
        }
        if (threadIdx.x < kDenseKeys) {
            const int qq = threadIdx.x;
            const bool ok = qq < nt * kBlock;
            ls[qq] = ok ? lse[(int64_t)h * N + q0 + qq] * kLog2e : INFINITY;
            Ds[qq] = ok ? Dws[(int64_t)h * N + q0 + qq] : 0.f;
        }
        __syncthreads();
        if (!active) continue;
#pragma unroll
        for (int tp = 0; tp < kFwdTiles / 2; ++tp) {
            bf16x4 pb[2], db[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int t = 2 * tp + u;
                const __bf16 *qr = qs + t * kTileElems + c16 * kVStride;
                const __bf16 *dr = ds_ + t * kTileElems + c16 * kVStride;
                const f32x4 s = mfma_bf16_32(load_bf16x8(qr + 32 + 8 * g), kb1,
                                             mfma_bf16_32(load_bf16x8(qr + 8 * g), kb0, f32x4{0.f, 0.f, 0.f, 0.f}));
                const f32x4 dp = mfma_bf16_32(load_bf16x8(dr + 32 + 8 * g), vb1,
                                              mfma_bf16_32(load_bf16x8(dr + 8 * g), vb0, f32x4{0.f, 0.f, 0.f, 0.f}));
                const f32x4 l4 = *reinterpret_cast<const f32x4 *>(&ls[t * kBlock + 4 * g]);
                const f32x4 D4 = *reinterpret_cast<const f32x4 *>(&Ds[t * kBlock + 4 * g]);
                f32x4 pp, dsv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    pp[i] = fast_exp2(s[i] * sl2 - l4[i]);   // lse of absent queries is +inf
                    dsv[i] = pp[i] * (dp[i] - D4[i]);
                }
                pb[u] = to_bf16x4(pp);
                db[u] = to_bf16x4(dsv);
            }
            const bf16x8 pc = cat8(pb[0], pb[1]), dc = cat8(db[0], db[1]);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x4 d0 = lds_read_tr4(ds_ + (2 * tp) * kTileElems + rofs + 16 * dt);
                const bf16x4 d1 = lds_read_tr4(ds_ + (2 * tp + 1) * kTileElems + rofs + 16 * dt);
                const bf16x4 q0t = lds_read_tr4(qs + (2 * tp) * kTileElems + rofs + 16 * dt);
                const bf16x4 q1t = lds_read_tr4(qs + (2 * tp + 1) * kTileElems + rofs + 16 * dt);
                dva[dt] = mfma_bf16_32(pc, cat8(d0, d1), dva[dt]);
                dka[dt] = mfma_bf16_32(dc, cat8(q0t, q1t), dka[dt]);
            }
        }
    }
    if (!active) return;
    // C layout: lane (dim 16dt + c16, keys 4g+i)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t off = head_off + ((int64_t)f0 + 4 * g + i) * kHeadDim + 16 * dt + c16;
            dk[off] = dka[dt][i] * scale;
            dv[off] = dva[dt][i];
        }
}

hipError_t launch_dense_bwd(int bh, int N, float scale, const void *q, const void *k,
                            const void *v, const void *o, const float *lse, const void *dout,
                            float *dq, float *dk, float *dv, float *Dws, hipStream_t s) {
    const int tiles = (N + kDenseWaves * kBlock - 1) / (kDenseWaves * kBlock);
    const float sl2 = scale * kLog2e;
    hipLaunchKernelGGL(dense_bwd_dq_kernel, dim3((unsigned)(bh * tiles)), dim3(512), 0, s,
                       (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (const __bf16 *)o,
                       lse, (const __bf16 *)dout, dq, Dws, N, tiles, sl2, scale);
    hipLaunchKernelGGL(dense_bwd_dkv_kernel, dim3((unsigned)(bh * tiles)), dim3(512), 0, s,
                       (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, lse, Dws,
                       (const __bf16 *)dout, dk, dv, N, tiles, sl2, scale);
    return hipGetLastError();
}

hipError_t launch_dense_fwd(int bh, int N, float scale, const void *q, const void *k,
                            const void *v, void *o, float *lse, hipStream_t s) {
    const int qtiles = (N + kDenseWaves * kBlock - 1) / (kDenseWaves * kBlock);
    hipLaunchKernelGGL(dense_fwd_bf16_kernel, dim3((unsigned)(bh * qtiles)), dim3(512), 0, s,
                       (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (__bf16 *)o, lse, N,
                       qtiles, scale * kLog2e);
    return hipGetLastError();
}

}  // namespace llsa
