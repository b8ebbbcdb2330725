// la_probe.hip -- peak probes for the roofline denominators (gfx950).
//
// Two kernels measure what the GPU actually sustains, so that roofline
// fractions can be quoted against measured peaks as well as AMD's published
// ones:
//   * a streaming copy: every lane moves 16-byte vectors from one buffer to
//     another in a grid-stride loop (each byte read once and written once);
//   * a matrix-core loop: every wave issues independent chains of
//     v_mfma_f32_32x32x16_bf16 on register operands, with no memory traffic
//     inside the loop.
// They are measurement tools; the operator's entry points live in la.h.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_probe.h"

namespace {

__global__ void __launch_bounds__(256) probe_copy_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                          size_t n) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride)
        dst[i] = src[i];
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// NACC independent accumulator chains per wave, `iters` steps each; every
// chain feeds its own result back, so the matrix cores see NACC products in
// flight.  The operands are small integers held in registers (exact in bf16).
constexpr int kNacc = 4;

__global__ void __launch_bounds__(256) probe_mfma_kernel(float *out, int iters) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
    for (int i = 0; i < 8; ++i) {
        a[i] = static_cast<__bf16>(static_cast<float>((lane + i) & 3));
        b[i] = static_cast<__bf16>(static_cast<float>((lane * 3 + i) & 1));
    }
    f32x16 acc[kNacc];
    for (int j = 0; j < kNacc; ++j)
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kNacc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
    for (int j = 0; j < kNacc; ++j)
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    out[static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int la_probe_copy(const void *src, void *dst, size_t bytes, void *stream) {
    if (!src || !dst || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) % 16)
        return 1;
    const size_t n = bytes / 16;
    // 2048 workgroups of 256 lanes: eight per compute unit, each lane moving
    // many vectors in a grid-stride loop
    hipLaunchKernelGGL(probe_copy_kernel, dim3(2048), dim3(256), 0, static_cast<hipStream_t>(stream),
                       static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

double la_probe_mfma_flops(int blocks, int iters) {
    // 4 waves per workgroup, kNacc products of 32 x 32 x 16 (2 flops each) per step
    return static_cast<double>(blocks) * 4 * kNacc * static_cast<double>(iters) * 2.0 * 32 * 32 * 16;
}

int la_probe_mfma(float *out, int blocks, int iters, void *stream) {
    if (!out || blocks <= 0 || iters <= 0) return 1;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream), out, iters);
    return hipGetLastError() == hipSuccess ? 0 : 3;
}

}  // extern "C"
