// la_mfma.hpp -- 16x16 matrix-core tiles for the chunked kernels (gfx950).
//
// A 16x16 float32 accumulator tile is held by one wave in the MFMA result
// layout: lane l holds rows 4*(l/16)+i (i = 0..3) of column l%16.
//
// Operands are supplied per lane in "groups" of four consecutive contraction
// indices: lane l gives row l%16 of A at k = k0 + 4*(l/16) .. +3 and column
// l%16 of B at the same k.  That is exactly the result layout, so a result
// tile can be fed back as the B operand of the next product with no data
// movement (its rows are the contraction index).  The matrix cores sum over
// k, so any assignment of k values to register slots is correct as long as
// A and B use the same one; these helpers use one assignment everywhere:
//   * k16 step: one group per lane (four f32 16x16x4 MFMAs, or one bf16
//     16x16x32 MFMA whose second group is zero);
//   * k32 step (bf16 only): two groups, k0 + 4*(l/16) and k0 + 16 + 4*(l/16),
//     packed into one 16x16x32 MFMA.
#pragma once

#include "la_common.hpp"

namespace la {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Element type of MFMA operands for each I/O type: float32 inputs keep
// float32 matrix-core arithmetic, bfloat16 inputs use bf16 matrix cores.
template <class DT> struct OpOf;
template <> struct OpOf<F32> { typedef float type; typedef float4 group; };
template <> struct OpOf<BF16> { typedef bf16_t type; typedef uint2 group; };

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---- groups: four consecutive operand elements of one lane

__device__ __forceinline__ float4 ld_group(const float *p) { return *reinterpret_cast<const float4 *>(p); }
__device__ __forceinline__ uint2 ld_group(const bf16_t *p) { return *reinterpret_cast<const uint2 *>(p); }

__device__ __forceinline__ void st_group(float *p, float4 g) { *reinterpret_cast<float4 *>(p) = g; }
__device__ __forceinline__ void st_group(bf16_t *p, uint2 g) { *reinterpret_cast<uint2 *>(p) = g; }

template <class Op> struct Group;
template <> struct Group<float> {
    typedef float4 type;
    static __device__ __forceinline__ float4 make(float a, float b, float c, float d) { return make_float4(a, b, c, d); }
    static __device__ __forceinline__ float4 make(const f32x4 &v) { return make_float4(v[0], v[1], v[2], v[3]); }
    static __device__ __forceinline__ void unpack(const float4 &g, float (&x)[4]) { x[0] = g.x; x[1] = g.y; x[2] = g.z; x[3] = g.w; }
};
template <> struct Group<bf16_t> {
    typedef uint2 type;
    static __device__ __forceinline__ uint2 make(float a, float b, float c, float d) {
        return make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
    }
    static __device__ __forceinline__ uint2 make(const f32x4 &v) { return make(v[0], v[1], v[2], v[3]); }
    static __device__ __forceinline__ void unpack(const uint2 &g, float (&x)[4]) {
        x[0] = lo_bf16(g.x); x[1] = hi_bf16(g.x); x[2] = lo_bf16(g.y); x[3] = hi_bf16(g.y);
    }
};

// ---- matrix-core steps

typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 32x32 tile step in the natural operand layouts: lane l supplies
// A[l%32][8*(l/32) .. +7] and B[8*(l/32) .. +7][l%32] (eight consecutive k,
// one 16-byte register quad each); acc[r] is C[8*(r/4) + 4*(l/32) + r%4][l%32].
// Its accumulators are never mixed with the 16x16 steps.
__device__ __forceinline__ void mma32x32(f32x16 &acc, const uint4 &a, const uint4 &b) {
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  acc, 0, 0, 0);
}

// acc += A(16 x 16) B(16 x 16), one group per lane.
__device__ __forceinline__ void mma16(f32x4 &acc, const float4 &a, const float4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, b.x, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, b.y, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, b.z, acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, b.w, acc, 0, 0, 0);
}
// bf16: issued as the 16x16x32 opcode with the second group zero, so that every
// bf16 accumulation chain uses one MFMA shape.  (A 16x16x32 result consumed as
// srcC by a 16x16x16 MFMA was emitted back to back by the compiler and read
// partly stale accumulators: rows 4*(l/16)+{0,1} of the tile came out wrong.)
__device__ __forceinline__ void mma16(f32x4 &acc, const uint2 &a, const uint2 &b) {
    const uint4 a8 = make_uint4(a.x, a.y, 0u, 0u);
    const uint4 b8 = make_uint4(b.x, b.y, 0u, 0u);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a8), __builtin_bit_cast(bf16x8, b8),
                                                  acc, 0, 0, 0);
}

// acc += A(16 x 32) B(32 x 16): groups (a0, b0) at k0 and (a1, b1) at k0 + 16.
__device__ __forceinline__ void mma32(f32x4 &acc, const float4 &a0, const float4 &a1, const float4 &b0,
                                      const float4 &b1) {
    mma16(acc, a0, b0);
    mma16(acc, a1, b1);
}
__device__ __forceinline__ void mma32(f32x4 &acc, const uint2 &a0, const uint2 &a1, const uint2 &b0,
                                      const uint2 &b1) {
    const uint4 a = make_uint4(a0.x, a0.y, a1.x, a1.y);
    const uint4 b = make_uint4(b0.x, b0.y, b1.x, b1.y);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  acc, 0, 0, 0);
}

// acc += A[0:16, 0:K] * B'[0:16, 0:K]^T with both operands in LDS, row-major
// with the contraction index contiguous (A rows: lda apart; B' rows: ldb
// apart).  `a` and `b` point at row 0, column 0 of the tiles.  K % 16 == 0.
template <int K, class Op>
__device__ __forceinline__ void tile_mma_ll(f32x4 &acc, const Op *a, int lda, const Op *b, int ldb, int lane) {
    const Op *ar = a + (lane & 15) * lda + 4 * (lane >> 4);
    const Op *br = b + (lane & 15) * ldb + 4 * (lane >> 4);
#pragma unroll
    for (int k = 0; k + 32 <= K; k += 32)
        mma32(acc, ld_group(ar + k), ld_group(ar + k + 16), ld_group(br + k), ld_group(br + k + 16));
    if constexpr (K % 32 == 16) mma16(acc, ld_group(ar + K - 16), ld_group(br + K - 16));
}

// acc += A[0:16, k-blocks kb0..kb0+NK-1] * Breg where the B operand is held in
// registers as groups, one per 16-row block of B (result-layout tiles
// converted with Group<Op>::make).  A in LDS row-major (k contiguous).
template <int NK, class Op, class G>
__device__ __forceinline__ void tile_mma_lr(f32x4 &acc, const Op *a, int lda, const G *bg, int lane) {
    const Op *ar = a + (lane & 15) * lda + 4 * (lane >> 4);
#pragma unroll
    for (int s = 0; s + 2 <= NK; s += 2) mma32(acc, ld_group(ar + 16 * s), ld_group(ar + 16 * s + 16), bg[s], bg[s + 1]);
    if constexpr (NK % 2 == 1) mma16(acc, ld_group(ar + 16 * (NK - 1)), bg[NK - 1]);
}

// As tile_mma_lr, for the first `nk` (<= NKMAX) k-blocks only: the
// block-lower-triangular products.  `nk` folds to a constant when the caller's
// loop is unrolled.
template <int NKMAX, class Op, class G>
__device__ __forceinline__ void tile_mma_lr_n(f32x4 &acc, const Op *a, int lda, const G *bg, int nk, int lane) {
    const Op *ar = a + (lane & 15) * lda + 4 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < NKMAX; s += 2) {
        if (s + 2 <= nk) mma32(acc, ld_group(ar + 16 * s), ld_group(ar + 16 * s + 16), bg[s], bg[s + 1]);
        else if (s + 1 == nk) mma16(acc, ld_group(ar + 16 * s), bg[s]);
    }
}

// acc += Areg * B over the first `nk` (<= NKMAX) k-blocks, with the A operand
// in registers as groups (result-layout tiles of A^T, one per k-block) and B
// supplied transposed from LDS: row n of `b` (rows ldb apart) holds column n
// of B with k contiguous.  The result is the transpose of what tile_mma_lr_n
// gives for the swapped product, so each lane ends up with four consecutive
// columns of one row of that product.
template <int NKMAX, class Op, class G>
__device__ __forceinline__ void tile_mma_rl_n(f32x4 &acc, const G *ag, const Op *b, int ldb, int nk, int lane) {
    const Op *br = b + (lane & 15) * ldb + 4 * (lane >> 4);
#pragma unroll
    for (int s = 0; s < NKMAX; s += 2) {
        if (s + 2 <= nk) mma32(acc, ag[s], ag[s + 1], ld_group(br + 16 * s), ld_group(br + 16 * s + 16));
        else if (s + 1 == nk) mma16(acc, ag[s], ld_group(br + 16 * s));
    }
}

}  // namespace la
