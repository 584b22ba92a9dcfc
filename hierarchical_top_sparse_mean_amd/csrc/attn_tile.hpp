// Score-tile softmax and P.V step shared by the sparse and the dense
// attention forward kernels (bf16 inputs, float32 accumulation).
#pragma once
#include "common.hpp"

namespace llsa {

constexpr int kFwdTiles = 8;     // key tiles per softmax chunk
constexpr int kVStride = 72;     // bf16 per LDS row of a staged tile (144 B, 16-B aligned)
constexpr int kTileElems = kBlock * kVStride;

// st[t] holds scale*log2(e)*score of key tile t in the transposed layout:
// lane l owns query l%16 and keys 4(l/16)..+3 of the tile; bias[t] is the
// log2 weight of those keys (-inf masks a key).  vw holds the nt V tiles
// (row-major, kVStride) in LDS.  m / lsum / oacc are the running max, the
// lane-partial denominator and O^T (lane: query l%16, dims 16dt+4(l/16)+i).
// kBias = false ignores `bias` (all weights 1).
template <bool kBias = true>
__device__ __forceinline__ void softmax_pv_chunk(f32x4 (&st)[kFwdTiles], const float (&bias)[kFwdTiles][4],
                                                 int nt, const __bf16 *vw, float &m, float &lsum,
                                                 f32x4 (&oacc)[4], int g, int c16) {
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < kFwdTiles; ++t)
        if (t < nt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, st[t][i] + (kBias ? bias[t][i] : 0.f));
    mx = max4_groups(mx);
    const float mnew = fmaxf(m, mx);
    const float msafe = (mnew == -INFINITY) ? 0.f : mnew;
    const float alpha = fast_exp2(m - msafe);
    m = mnew;
    lsum *= alpha;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
    wave_lds_sync();
#pragma unroll
    for (int tp = 0; tp < kFwdTiles / 2; ++tp) {
        const int t = 2 * tp;
        if (t < nt) {
            const bool two = (t + 1) < nt;
            float p0[4], p1[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p0[i] = fast_exp2(st[t][i] + (kBias ? bias[t][i] : 0.f) - msafe);
                p1[i] = two ? fast_exp2(st[t + 1][i] + (kBias ? bias[t + 1][i] : 0.f) - msafe) : 0.f;
                lsum += p0[i] + p1[i];
            }
            const bf16x8 pb = cat8(to_bf16x4(f32x4{p0[0], p0[1], p0[2], p0[3]}),
                                   to_bf16x4(f32x4{p1[0], p1[1], p1[2], p1[3]}));
            const int rofs = (4 * g + (c16 >> 2)) * kVStride + 4 * (c16 & 3);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
                const bf16x4 v0 = lds_read_tr4(vw + t * kTileElems + rofs + 16 * dt);
                const bf16x4 v1 = two ? lds_read_tr4(vw + (t + 1) * kTileElems + rofs + 16 * dt)
                                      : bf16x4{(__bf16)0.f, (__bf16)0.f, (__bf16)0.f, (__bf16)0.f};
                oacc[dt] = mfma_bf16_32(cat8(v0, v1), pb, oacc[dt]);
            }
        }
    }
    wave_lds_sync();
}


}  // namespace llsa
