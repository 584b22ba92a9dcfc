// Device-side helpers shared by the gfx950 kernels of the LLSA library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace llsa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 lds_bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));

constexpr int kHeadDim = 64;   // supported head dimension
constexpr int kBlock = 16;     // supported block size B (= one MFMA tile edge)
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

#define LLSA_LDS __attribute__((address_space(3)))

// 16x16 output += A(16 x 32) * B(32 x 16), bf16 in, f32 accumulate.
// Lane l holds A[l%16][k-slots of group l/16] and B[k-slots][l%16];
// result C[m][n] sits in lane n + 16*(m/4), register m%4.
__device__ __forceinline__ f32x4 mfma_bf16_32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// Same with 4 k-slots per lane (16 x 16 x 16).
__device__ __forceinline__ f32x4 mfma_bf16_16(bf16x4 a, bf16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                      __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
}
// f32: one k-slot per lane (16 x 16 x 4).
__device__ __forceinline__ f32x4 mfma_f32_4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
// Float32 operands of the 16 x 16 x 4 product straight from memory.  Row
// layout: lane (g = l / 16, c = l % 16) takes dims 16g .. 16g + 15 of its own
// row (64 contiguous bytes), so step d of a 16-step product over the head
// dimension covers dims d, 16 + d, 32 + d and 48 + d in the four lane groups.
// (The column layout, lane (g, c) holding dims 4c .. 4c + 3 of rows 4g + i,
// is one 16-byte load per row and needs no helper.)
__device__ __forceinline__ void load_row16(const float *p, float (&x)[16]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const f32x4 t = reinterpret_cast<const f32x4 *>(p)[j];
#pragma unroll
        for (int e = 0; e < 4; ++e) x[4 * j + e] = t[e];
    }
}

// Transposing LDS read of 4 bf16: within each 16-lane group, lane i receives
// element i%4 of the 8-byte chunks addressed by lanes i/4, i/4+4, i/4+8, i/4+12.
// Pointing lane s of group g at M[r0 + s/4][c0 + 4*(s%4)] of a row-major bf16
// matrix M therefore hands lane i the column M[r0 .. r0+3][c0 + i].
__device__ __forceinline__ bf16x4 lds_read_tr4(const __bf16 *p) {
    lds_bf16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((LLSA_LDS lds_bf16x4 *)(p));
    return __builtin_bit_cast(bf16x4, r);
}

__device__ __forceinline__ bf16x8 cat8(bf16x4 a, bf16x4 b) {
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 2^x on the transcendental unit (v_exp_f32) without the library's range
// scaling: results below 2^-126 may flush to zero, which only ever concerns
// softmax weights that are negligible next to the row's largest.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round-to-nearest bf16 of four floats, two per v_cvt_pk_bf16_f32.
__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) { return __builtin_convertvector(x, bf16x4); }

__device__ __forceinline__ bf16x8 load_bf16x8(const __bf16 *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void store_bf16x8(__bf16 *p, bf16x8 v) {
    *reinterpret_cast<u32x4 *>(p) = __builtin_bit_cast(u32x4, v);
}
// Non-temporal (streaming) forms for rows a kernel reads or writes once: they
// do not displace the gathered tiles that neighbouring workgroups re-read
// from L2.
__device__ __forceinline__ bf16x8 load_bf16x8_nt(const __bf16 *p) {
    return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p)));
}
__device__ __forceinline__ void store_bf16x8_nt(__bf16 *p, bf16x8 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4, v), reinterpret_cast<u32x4 *>(p));
}

// Buffer resource over the n_bytes at p (p the same for the whole wave):
// loads through it take a 32-bit byte offset, which saves the 64-bit address
// arithmetic of a global load, and read zero at offsets past n_bytes.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void *p, uint32_t n_bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)n_bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8 buf_load_bf16x8(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ float buf_load_f32(Rsrc r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}

__device__ __forceinline__ bf16x8 f32_to_bf16x8(f32x4 a, f32x4 b) {
    return cat8(to_bf16x4(a), to_bf16x4(b));
}

__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
}
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }
__device__ __forceinline__ uint32_t shfl_xor_u(uint32_t v, int m) {
    return (uint32_t)__shfl_xor((int)v, m, kWave);
}

// Orders the 4 lanes {l, l^16, l^32, l^48} that share one query in the
// transposed score layout.
__device__ __forceinline__ float max4_groups(float v) {
    v = fmaxf(v, shfl_xor_f(v, 16));
    v = fmaxf(v, shfl_xor_f(v, 32));
    return v;
}
__device__ __forceinline__ float sum4_groups(float v) {
    v += shfl_xor_f(v, 16);
    v += shfl_xor_f(v, 32);
    return v;
}

// The dispatcher hands workgroup i to XCD i % 8, and every XCD has its own
// L2.  Renumbering so that each XCD walks one contiguous range of the logical
// grid keeps neighbouring work -- which gathers the same key/value tiles --
// inside one L2.  Bijective for any grid size.
constexpr int kNumXcd = 8;
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    const int per = nblocks / kNumXcd, rem = nblocks % kNumXcd;
    const int x = bid % kNumXcd, i = bid / kNumXcd;
    return x * per + (x < rem ? x : rem) + i;
}

// Token order of the [.., seq_len, ..] tensors (Q, K, V, O, dO, dQ, dK, dV,
// lse).  order 0: the sequence as stored.  order 1: the tensors hold an
// S x S image in raster order, and the method runs on the sequence of nested
// 2^i x 2^i patches (Z order: position t has x in the even and y in the odd
// bits of t), so 16 consecutive positions are a 4 x 4 patch and a level-l
// token pools a 4^l x 4^l patch ("Trainable Log-linear Sparse Attention for
// Efficient Diffusion Transformers", explainer "Step 5: Index Reordering for
// Images").  Pyramids, index lists and CSR are in sequence order either way.
struct TokMap {
    int order;   // 0 or 1
    int log2S;   // image side, order 1 only
};

__device__ __forceinline__ uint32_t compact_even_bits(uint32_t v) {
    v &= 0x55555555u;
    v = (v | (v >> 1)) & 0x33333333u;
    v = (v | (v >> 2)) & 0x0f0f0f0fu;
    v = (v | (v >> 4)) & 0x00ff00ffu;
    v = (v | (v >> 8)) & 0x0000ffffu;
    return v;
}

// Storage row (within one head) of sequence position t; ORD fixes the order
// at compile time for the hot kernels, tok_row() reads it from m.
template <int ORD>
__device__ __forceinline__ int tok_row_o(const TokMap &m, int t) {
    if constexpr (ORD == 0) {
        return t;
    } else {
        const uint32_t x = compact_even_bits((uint32_t)t), y = compact_even_bits((uint32_t)t >> 1);
        return (int)((y << m.log2S) | x);
    }
}
__device__ __forceinline__ int tok_row(const TokMap &m, int t) {
    return m.order == 0 ? t : tok_row_o<1>(m, t);
}
// Storage row of row r (< 16) of 16-token tile b.  In order 1 a tile is a
// 4 x 4 patch: the row is the patch corner's row (a function of b alone, so
// scalar when b is) plus the fixed offset of r inside the patch.
template <int ORD>
__device__ __forceinline__ int tok_tile_row(const TokMap &m, int b, int r) {
    if constexpr (ORD == 0) {
        return b * 16 + r;
    } else {
        const uint32_t t0 = (uint32_t)b << 4;
        const int corner = (int)((compact_even_bits(t0 >> 1) << m.log2S) | compact_even_bits(t0));
        const int x = (r & 1) | ((r >> 1) & 2), y = ((r >> 1) & 1) | ((r >> 2) & 2);
        return corner + (y << m.log2S) + x;
    }
}

// Wave-scope ordering for data exchanged through LDS by lanes of one wave.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace llsa
