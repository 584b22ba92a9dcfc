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

hipError_t launch_dense_fwd(int bh, int N, float scale, const void *q, const void *k,
                            const void *v, void *o, float *lse, hipStream_t s) {
    const int qtiles = (N + kDenseWaves * kBlock - 1) / (kDenseWaves * kBlock);
    hipLaunchKernelGGL(dense_fwd_bf16_kernel, dim3((unsigned)(bh * qtiles)), dim3(512), 0, s,
                       (const __bf16 *)q, (const __bf16 *)k, (const __bf16 *)v, (__bf16 *)o, lse, N,
                       qtiles, scale * kLog2e);
    return hipGetLastError();
}

}  // namespace llsa
