// la_chunk_common.hpp -- pieces shared by the chunked-forward kernels.
#pragma once

#include "la_internal.hpp"
#include "la_mfma.hpp"

namespace la {

// Kernel arguments of the chunked forward (device pointers, raw element types).
struct ChunkParams {
    const void *q, *k, *v;
    const float *gate, *beta;
    const float *S0, *z0;
    void *out;
    float *S_T, *z_T;
    int T, d_v, n_vblk, n_heads;
    // normalized linear attention over sequence segments (n_seg > 1): the
    // workgroups of segment s start from slot 0 + ... + slot s of seg_state,
    // [head][n_seg][d_v * d_k + d_k] float32 (slot 0: the initial state,
    // slot s >= 1: the state increment of segment s - 1)
    int seg_len = 0, n_seg = 1;
    const float *seg_state = nullptr;
    // normalized / retention: heads per batch entry (the per-head decay of
    // head bh is gate[bh % H]; gate NULL = no decay) and whether the
    // normalizer is carried (normalized) or not (retention)
    int H = 1;
    int normalize = 1;
};

// Copy rows [0, n) of a D-wide row-major global tile (row stride `lds`
// elements) into LDS rows of stride `ldd`, and zero rows [n, R).  16-byte
// vector copies; every row start must be 16-byte aligned on both sides.
template <int R, int D, class E>
__device__ __forceinline__ void stage_rows(E *dst, int ldd, const E *src, size_t lds, int n, int tid, int nthr) {
    constexpr int VE = 16 / sizeof(E);        // elements per 16-byte vector
    constexpr int VPR = D / VE;               // vectors per row
    static_assert(D % VE == 0, "row width");
    for (int e = tid; e < R * VPR; e += nthr) {
        const int r = e / VPR, c = (e % VPR) * VE;
        uint4 x = make_uint4(0u, 0u, 0u, 0u);
        if (r < n) x = *reinterpret_cast<const uint4 *>(src + r * lds + c);
        *reinterpret_cast<uint4 *>(dst + r * ldd + c) = x;
    }
}

// Register staging of an R x D row-major tile: load() issues every 16-byte
// global read of the tile at once, store() writes the registers to LDS with
// rows >= n as zeros.  Issued one chunk ahead, the reads complete while the
// current chunk computes; the workgroup barriers only wait for LDS.  Rows
// beyond n read row 0 instead (always valid) and the zeroing happens at
// store time: no register of a load in flight is written by another
// instruction, which would make the compiler wait for every outstanding load.
template <int R, int D, int NTHR, class E>
struct TilePrefetch {
    static constexpr int VE = 16 / sizeof(E);
    static constexpr int VPR = D / VE;
    static constexpr int TOTAL = R * VPR;
    static constexpr int PER = (TOTAL + NTHR - 1) / NTHR;
    static_assert(D % VE == 0, "row width");
    static_assert(PER <= 32, "row-valid mask");
    uint4 r[PER];
    uint32_t valid;   // bit i: r[i] holds a row < n

    // Every lane issues every load (lanes past the tile re-read its last
    // element, rows past n re-read row 0): no load sits behind a branch, so the
    // compiler's count of loads in flight is the same on every path and its
    // waits for one tile never extend to loads issued after it.
    __device__ __forceinline__ void load(const E *src, size_t lds, int n, int tid) {
        valid = 0;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + i * NTHR;
            const int ec = (TOTAL % NTHR == 0 || e < TOTAL) ? e : TOTAL - 1;
            const int row = ec / VPR, col = (ec % VPR) * VE;
            r[i] = *reinterpret_cast<const uint4 *>(src + (row < n ? row : 0) * lds + col);
            valid |= (row < n && ec == e ? 1u : 0u) << i;
        }
    }
    // SW != 0: on rows with bit 3 set, element column c goes to c ^ SW
    template <int SW = 0>
    __device__ __forceinline__ void store(E *dst, int ldd, int tid) const {
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = tid + i * NTHR;
            const int row = e / VPR, col = (e % VPR) * VE;
            if (TOTAL % NTHR == 0 || e < TOTAL)
                *reinterpret_cast<uint4 *>(dst + row * ldd + (col ^ (SW * ((row >> 3) & 1)))) =
                    (valid >> i) & 1u ? r[i] : make_uint4(0u, 0u, 0u, 0u);
        }
    }
};

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4):
// lane l's 16 bytes land at LDS byte address lds_base + 16 l, whatever global
// address each lane gives; lds_base must be wave-uniform.  It is issued from
// inline assembly, so the compiler neither waits for it nor counts it: the
// issuing wave waits for it (s_waitcnt on the vector-memory counter) before
// the barrier that hands the tile to its readers.  The load reads M0, which the
// compiler sets with a scalar move right before the statement; gfx9 needs one
// wait state between the two, and the compiler does not insert it for inline
// assembly, so the statement starts with one.
__device__ __forceinline__ void lds_dma16(const void *src, unsigned lds_base) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_base) : "memory");
}
// The same with a wave-uniform 64-bit base and a 32-bit per-lane byte offset
// (global address = base + offset), so that a caller whose lane offsets do
// not change between calls keeps them in registers and moves only the base.
__device__ __forceinline__ void lds_dma16(const void *base, unsigned offset, unsigned lds_base) {
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(offset), "s"(base), "{m0}"(lds_base) : "memory");
}
// LDS byte address of a __shared__ object (the low half of its generic address)
template <class T>
__device__ __forceinline__ unsigned lds_addr(const T *p) {
    return static_cast<unsigned>(reinterpret_cast<uintptr_t>(p));
}

// Workgroup -> (head, value block).  The dispatcher deals workgroups to the
// 8 XCDs round robin (workgroup i runs on XCD i % 8); when the head count is
// a multiple of 8 the value blocks of one head are given ids that differ by
// multiples of 8, so they run on one XCD and share its L2 for the re-read
// queries and keys.
__device__ __forceinline__ void block_to_head(int bid, int n_heads, int n_vblk, int &bh, int &vb) {
    if ((n_heads & 7) == 0) {
        const int xcd = bid & 7, r = bid >> 3;
        vb = r % n_vblk;
        bh = (r / n_vblk) * 8 + xcd;
    } else {
        bh = bid / n_vblk;
        vb = bid % n_vblk;
    }
}

// A-operand group of K^T for key channel c = c0 + lane%16 and tokens
// t0 + 4*(lane/16) .. +3, read from a natural-layout K tile (rows = tokens,
// ldk elements apart; t0 and c0 multiples of 16).  SW != 0: rows with bit 3
// set store element column c at c ^ SW.
// bf16: one transposing LDS read (ds_read_b64_tr_b16): within each 16-lane
// group, lane a supplies row t0 + 4*(lane/16) + a/4, columns c0 + 4*(a%4)..+3,
// and lane j receives column c0 + j of the group's four rows.
template <int SW>
__device__ __forceinline__ uint2 kt_group(const bf16_t *sK, int ldk, int t0, int c0, int lane) {
    typedef short v4i16 __attribute__((ext_vector_type(4)));
    const int a = lane & 15, g = lane >> 4;
    const int row = t0 + 4 * g + (a >> 2);
    const bf16_t *src = sK + row * ldk + c0 + ((4 * (a & 3)) ^ (SW * ((row >> 3) & 1)));
    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)((__attribute__((address_space(3))) bf16_t *)src));
    return __builtin_bit_cast(uint2, r);
}
// float32: four scalar reads of the column (no swizzle)
template <int SW>
__device__ __forceinline__ float4 kt_group(const float *sK, int ldk, int t0, int c0, int lane) {
    static_assert(SW == 0, "float32 tiles are not swizzled");
    const float *src = sK + (t0 + 4 * (lane >> 4)) * ldk + c0 + (lane & 15);
    return make_float4(src[0], src[ldk], src[2 * ldk], src[3 * ldk]);
}

// DPP move with control CTRL; lanes whose source is invalid read 0
template <int CTRL>
__device__ __forceinline__ float dpp_or_zero(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// value of x in lane l (l uniform), as a scalar
__device__ __forceinline__ float read_lane(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ float wave_inclusive_sum(float x, int lane) {
    // within each 16-lane row: DPP row shifts by 1, 2, 4, 8 (sources outside
    // the row read as 0); then the totals of the rows below, read as scalars.
    // No LDS access, so the scan does not queue behind other waves' LDS work.
    x += dpp_or_zero<0x111>(x);
    x += dpp_or_zero<0x112>(x);
    x += dpp_or_zero<0x114>(x);
    x += dpp_or_zero<0x118>(x);
    const float t0 = read_lane(x, 15), t1 = read_lane(x, 31), t2 = read_lane(x, 47);
    const int row = lane >> 4;
    return x + (row >= 1 ? t0 : 0.f) + (row >= 2 ? t1 : 0.f) + (row >= 3 ? t2 : 0.f);
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }
__device__ __forceinline__ void from_f32(float &d, float x) { d = x; }
__device__ __forceinline__ void from_f32(bf16_t &d, float x) { d = f32_to_bf16(x); }

}  // namespace la
