// Hierarchical compression: mean pooling of Q, K and V into a float32 pyramid
// ("Trainable Log-linear Sparse Attention for Efficient Diffusion
// Transformers", explainer "Step 1: Hierarchical Compression").
//
// A streaming, HBM-bound pass.  One 256-thread workgroup pools 16 consecutive
// level-1 blocks (16 tokens each) of one tensor, 4 per wave; lane (b, hh, c)
// of a wave reads rows of block b at 16-byte column chunk c, bf16 rows 8 hh ..
// 8 hh + 7 (two lanes per chunk, added with one exchange) and float32 rows all
// 16, so every load instruction reads whole row segments.  Small waves keep
// the last round of the grid nearly full.  Level 2 is formed from the level-1 means in
// LDS; deeper levels (rare, small) are pooled from the level below by a
// second kernel.  Blocks of 64 tokens take a kernel of their own (one wave per
// block) and every level above 1 comes from the level below.
#include "common.hpp"
#include "internal.hpp"

namespace llsa {

template <typename T> struct ElemTraits;
template <> struct ElemTraits<__bf16> { static constexpr int kPerChunk = 8; };
template <> struct ElemTraits<float> { static constexpr int kPerChunk = 4; };

__device__ __forceinline__ void chunk_to_f32(u32x4 r, float *o, __bf16 *) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        o[2 * j] = __builtin_bit_cast(float, r[j] << 16);
        o[2 * j + 1] = __builtin_bit_cast(float, r[j] & 0xffff0000u);
    }
}
__device__ __forceinline__ void chunk_to_f32(u32x4 r, float *o, float *) {
    const f32x4 v = __builtin_bit_cast(f32x4, r);
    o[0] = v[0];
    o[1] = v[1];
    o[2] = v[2];
    o[3] = v[3];
}

template <typename T, int ORD>
__global__ __launch_bounds__(256) void pool_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                   const T *__restrict__ v, float *__restrict__ pq,
                                                   float *__restrict__ pk, float *__restrict__ pv,
                                                   int64_t total_blocks, int wg_per_tensor,
                                                   int do_level2, int64_t level2_off, int n1,
                                                   TokMap tm) {
    constexpr int EPC = ElemTraits<T>::kPerChunk;  // elements per 16-byte chunk
    constexpr int CPR = kHeadDim / EPC;            // chunks per row
    constexpr int BPW = 4;                         // level-1 blocks per wave
    constexpr int RS = kWave / (BPW * CPR);        // lanes that share a block's chunk, a row range each
    constexpr int RPL = kBlock / RS;               // rows per lane
    constexpr int BPG = 4 * BPW;                   // level-1 blocks per workgroup
    __shared__ float lvl1[BPG][kHeadDim];

    const int tensor = blockIdx.x / wg_per_tensor;
    const int wg = blockIdx.x % wg_per_tensor;
    const T *x = tensor == 0 ? q : (tensor == 1 ? k : v);
    float *out = tensor == 0 ? pq : (tensor == 1 ? pk : pv);

    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int c = lane % CPR, hh = (lane / CPR) % RS, b = lane / (CPR * RS);
    const int64_t blk0 = (int64_t)wg * BPG;
    const int64_t blk = blk0 + w * BPW + b;

    float acc[EPC];
#pragma unroll
    for (int j = 0; j < EPC; ++j) acc[j] = 0.f;
    if (blk < total_blocks) {
        // block blk of head h: sequence positions lb*16 .. lb*16+15
        const int64_t h = blk / n1;
        const int lb = (int)(blk % n1);
        const T *src = x + h * (int64_t)n1 * kBlock * kHeadDim + c * EPC;
        u32x4 r[RPL];
#pragma unroll
        for (int t = 0; t < RPL; ++t)
            r[t] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
                src + (int64_t)tok_tile_row<ORD>(tm, lb, hh * RPL + t) * kHeadDim));
#pragma unroll
        for (int t = 0; t < RPL; ++t) {
            float f[EPC];
            chunk_to_f32(r[t], f, (T *)nullptr);
#pragma unroll
            for (int j = 0; j < EPC; ++j) acc[j] += f[j];
        }
        if constexpr (RS == 2) {   // the two row halves of the block's chunk (lanes CPR apart)
#pragma unroll
            for (int j = 0; j < EPC; ++j) acc[j] += shfl_xor_f(acc[j], CPR);
        }
        static_assert(RS == 1 || RS == 2, "one or two lanes per chunk");
#pragma unroll
        for (int j = 0; j < EPC; ++j) acc[j] *= (1.0f / kBlock);
        float *dst = out + blk * kHeadDim + c * EPC;
        if (hh != 0) {
        } else if constexpr (EPC == 8) {
            *reinterpret_cast<f32x4 *>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]};
            *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
        } else {
            *reinterpret_cast<f32x4 *>(dst) = f32x4{acc[0], acc[1], acc[2], acc[3]};
        }
    }
    if (!do_level2) return;
#pragma unroll
    for (int j = 0; j < EPC; ++j) lvl1[w * BPW + b][c * EPC + j] = acc[j];
    __syncthreads();
    // level 2: BPG / 16 tokens per workgroup, one thread per (token, column)
    constexpr int T2 = BPG / kBlock;
    if (threadIdx.x < T2 * kHeadDim) {
        const int j = threadIdx.x / kHeadDim, e = threadIdx.x % kHeadDim;
        const int64_t tok2 = blk0 / kBlock + j;
        if (tok2 * kBlock < total_blocks) {
            float s = 0.f;
#pragma unroll
            for (int t = 0; t < kBlock; ++t) s += lvl1[j * kBlock + t][e];
            out[level2_off + tok2 * kHeadDim + e] = s * (1.0f / kBlock);
        }
    }
}

// Level 1 for blocks of 64 tokens: one wave per block of one tensor.  Lane
// (r, c) reads rows r, r + RPI, r + 2 RPI, ... at 16-byte chunk c, so every
// load instruction reads whole rows; the partial sums of one chunk meet
// through butterfly shuffles.
template <typename T, int ORD>
__global__ __launch_bounds__(256) void pool64_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                     const T *__restrict__ v, float *__restrict__ pq,
                                                     float *__restrict__ pk, float *__restrict__ pv,
                                                     int64_t total_blocks, int wg_per_tensor, int n1,
                                                     TokMap tm) {
    constexpr int kB = 64;
    constexpr int EPC = ElemTraits<T>::kPerChunk;  // elements per 16-byte chunk
    constexpr int CPR = kHeadDim / EPC;            // chunks per row
    constexpr int RPI = kWave / CPR;               // rows per load instruction
    constexpr int NLD = kB / RPI;                  // loads per lane
    const int tensor = blockIdx.x / wg_per_tensor;
    const int wg = blockIdx.x % wg_per_tensor;
    const T *x = tensor == 0 ? q : (tensor == 1 ? k : v);
    float *out = tensor == 0 ? pq : (tensor == 1 ? pk : pv);
    const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int r = lane / CPR, c = lane % CPR;
    const int64_t blk = (int64_t)wg * 4 + w;
    if (blk >= total_blocks) return;
    const int64_t h = blk / n1;
    const int lb = (int)(blk % n1);
    const T *src = x + h * (int64_t)n1 * kB * kHeadDim + c * EPC;
    u32x4 rr[NLD];
#pragma unroll
    for (int i = 0; i < NLD; ++i)
        rr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(
            src + (int64_t)tok_tile_row<ORD>(tm, lb * (kB / kBlock) + (r + RPI * i) / kBlock,
                                             (r + RPI * i) % kBlock) * kHeadDim));
    float acc[EPC];
#pragma unroll
    for (int j = 0; j < EPC; ++j) acc[j] = 0.f;
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
        float f[EPC];
        chunk_to_f32(rr[i], f, (T *)nullptr);
#pragma unroll
        for (int j = 0; j < EPC; ++j) acc[j] += f[j];
    }
#pragma unroll
    for (int m = CPR; m < kWave; m <<= 1)
#pragma unroll
        for (int j = 0; j < EPC; ++j) acc[j] += shfl_xor_f(acc[j], m);
    if (r == 0) {
        float *dst = out + blk * kHeadDim + c * EPC;
#pragma unroll
        for (int j = 0; j < EPC; j += 4)
            *reinterpret_cast<f32x4 *>(dst + j) =
                f32x4{acc[j], acc[j + 1], acc[j + 2], acc[j + 3]} * (1.0f / kB);
    }
}

// Level l from level l-1 (float32), one thread per output element.
__global__ __launch_bounds__(256) void pool_up_kernel(float *__restrict__ pq, float *__restrict__ pk,
                                                      float *__restrict__ pv, int64_t src_off,
                                                      int64_t dst_off, int64_t total_out, int B) {
    const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int tensor = blockIdx.y;
    if (t >= total_out) return;
    float *p = tensor == 0 ? pq : (tensor == 1 ? pk : pv);
    const int64_t tok = t / kHeadDim, e = t % kHeadDim;
    const float *src = p + src_off + tok * B * kHeadDim + e;
    float s = 0.f;
    for (int j = 0; j < B; ++j) s += src[j * kHeadDim];
    p[dst_off + t] = s * (1.0f / (float)B);
}

template <typename T>
static void launch_pool_t(const Geometry &g, const T *q, const T *k, const T *v, float *pq,
                          float *pk, float *pv, hipStream_t s) {
    if (g.B == 64) {
        const int64_t total_blocks = (int64_t)g.bh * g.n[1];
        const int wg_per_tensor = (int)((total_blocks + 3) / 4);
        const TokMap tm{g.order, g.log2S};
        if (g.order == 0)
            hipLaunchKernelGGL((pool64_kernel<T, 0>), dim3(3 * wg_per_tensor), dim3(256), 0, s, q, k, v,
                               pq, pk, pv, total_blocks, wg_per_tensor, g.n[1], tm);
        else
            hipLaunchKernelGGL((pool64_kernel<T, 1>), dim3(3 * wg_per_tensor), dim3(256), 0, s, q, k, v,
                               pq, pk, pv, total_blocks, wg_per_tensor, g.n[1], tm);
        return;
    }
    constexpr int BPG = 16;   // 4 waves x 4 level-1 blocks
    const int64_t total_blocks = (int64_t)g.bh * g.n[1];
    const int wg_per_tensor = (int)((total_blocks + BPG - 1) / BPG);
    const int do2 = g.L >= 2 ? 1 : 0;
    const TokMap tm{g.order, g.log2S};
    if (g.order == 0)
        hipLaunchKernelGGL((pool_kernel<T, 0>), dim3(3 * wg_per_tensor), dim3(256), 0, s, q, k, v,
                           pq, pk, pv, total_blocks, wg_per_tensor, do2, g.pyr_off[2], g.n[1], tm);
    else
        hipLaunchKernelGGL((pool_kernel<T, 1>), dim3(3 * wg_per_tensor), dim3(256), 0, s, q, k, v,
                           pq, pk, pv, total_blocks, wg_per_tensor, do2, g.pyr_off[2], g.n[1], tm);
}

hipError_t launch_pool(const Geometry &g, const void *q, const void *k, const void *v, float *pq,
                       float *pk, float *pv, hipStream_t s) {
    if (g.bf16)
        launch_pool_t<__bf16>(g, (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, pq, pk,
                              pv, s);
    else
        launch_pool_t<float>(g, (const float *)q, (const float *)k, (const float *)v, pq, pk, pv,
                             s);
    // levels the first kernel did not form (above 2 for B = 16, above 1 for B = 64)
    for (int l = g.B == 16 ? 3 : 2; l <= g.L; ++l) {
        const int64_t total = (int64_t)g.bh * g.n[l] * kHeadDim;
        hipLaunchKernelGGL(pool_up_kernel, dim3((unsigned)((total + 255) / 256), 3), dim3(256), 0,
                           s, pq, pk, pv, g.pyr_off[l - 1], g.pyr_off[l], total, g.B);
    }
    return hipGetLastError();
}

}  // namespace llsa
