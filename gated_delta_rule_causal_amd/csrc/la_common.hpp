// la_common.hpp -- device helpers shared by the gfx950 kernels.
//
// bfloat16 is carried as raw 16-bit patterns (uint16_t); conversion to float
// is exact (shift into the high half), conversion from float rounds to
// nearest-even.  Everything here is gfx950-only code: wave64, MFMA, LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

typedef uint16_t bf16_t;

constexpr int kWave = 64;

// ----------------------------------------------------------------- bfloat16

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// float -> bfloat16, round to nearest even: gfx950's v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// two floats -> packed pair of bf16 (low half = a), one conversion instruction
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const bf16x2_t h = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element type tags of q, k, v, out.
struct F32 { typedef float storage; static constexpr int bytes = 4; };
struct BF16 { typedef bf16_t storage; static constexpr int bytes = 2; };

// Load 8 consecutive elements starting at p (16- or 32-byte aligned) as float.
__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    float4 a = reinterpret_cast<const float4 *>(p)[0];
    float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void load8(const bf16_t *p, float (&x)[8]) {
    uint4 w = *reinterpret_cast<const uint4 *>(p);
    x[0] = lo_bf16(w.x); x[1] = hi_bf16(w.x);
    x[2] = lo_bf16(w.y); x[3] = hi_bf16(w.y);
    x[4] = lo_bf16(w.z); x[5] = hi_bf16(w.z);
    x[6] = lo_bf16(w.w); x[7] = hi_bf16(w.w);
}

__device__ __forceinline__ float load1(const float *p) { return *p; }
__device__ __forceinline__ float load1(const bf16_t *p) { return bf16_to_f32(*p); }
__device__ __forceinline__ void store1(float *p, float x) { *p = x; }
__device__ __forceinline__ void store1(bf16_t *p, float x) { *p = f32_to_bf16(x); }

// s_waitcnt immediate (gfx9 encoding) that waits for every outstanding vector
// memory load and leaves the LDS and export counters free.
constexpr int kWaitVmcnt0 = 0x0F70;
// the same, leaving the n most recently issued vector memory loads in flight
// (loads complete in the order they were issued)
constexpr int wait_vmcnt(int n) { return kWaitVmcnt0 | (n & 15) | ((n >> 4) << 14); }

// ------------------------------------------------------------- feature map

// elu(x) + 1: x + 1 above zero, exp(x) at or below zero (always > 0).
__device__ __forceinline__ float phi_elu1(float x) { return x > 0.f ? x + 1.f : __expf(x); }

template <int PHI>
__device__ __forceinline__ float apply_phi(float x) {
    if constexpr (PHI == 1) return phi_elu1(x);
    else return x;
}

// ------------------------------------------------------- lane reductions

// Sum over aligned groups of G lanes (G a power of two <= 64); every lane of
// the group receives the total.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
    for (int m = G / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, G);
    return x;
}

}  // namespace la
