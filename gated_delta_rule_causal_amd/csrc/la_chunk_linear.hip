// la_chunk_linear.hip -- chunked forward of normalized and gated linear
// attention (gfx950).
//
// Normalized (page "Beyond -- Linear attention and recurrent memory",
// section "The big idea"; page "Ch. 11 Linear attention and Hyena", 11.2):
// with phi = elu+1 and a chunk of C tokens entering with (S0, z0),
//   P   = M o (phiQ phiK^T)                       (M: j <= t, a token sees itself)
//   O   = (phiQ S0^T + P V) / (phiQ z0 + P 1)
//   S_C = S0 + V^T phiK,   z_C = z0 + phiK^T 1.
// The denominator uses the same rounded P as the numerator.  With a fixed
// per-head decay gamma (same page, section "Fixed decay versus an
// input-dependent gate": S and z both decay before each write) every term
// carries the power of gamma that unrolling the recurrence gives, for tokens
// t, j = 0 .. n-1 of the chunk:
//   P_tj *= gamma^(t-j),  the S0 / z0 terms of token t *= gamma^(t+1),
//   S_C = gamma^n S0 + sum_j gamma^(n-1-j) v_j phi(k_j)^T  (z_C likewise);
// every power is at most 1 and comes from a per-chunk table gamma^0..gamma^C.
// Retention (page "Ch. 11 Linear attention and Hyena", 11.3, RetNet bullet)
// is the same path without the normalizer.
//
// Gated (page "Ch. 11 Linear attention and Hyena", 11.3 and the solution to
// Exercise 11.5): per-channel gates gamma_t, decay between tokens j <= t of
// channel c is prod_{i=j+1}^t gamma_ic.  The chunk applies the page's
// cumulative-gate rescaling locally, with a reference point per 16-token
// block so that no factor exceeds the float32 range:
//   * key block J < query block I: reference e_J = last token of J,
//       q~_t = phi(q_t) prod_{e_J < i <= t} gamma_i   (<= 1 per channel)
//       k~_j = phi(k_j) prod_{j < i <= e_J} gamma_i   (<= 1)
//     formed as Qhat_t * rho_IJ with Qhat_t = phi(q_t) prod_{16I <= i <= t}
//     gamma_i and rho_IJ = product of the whole blocks strictly between.
//   * diagonal block I: reference r_I = 16I - 1,
//       Qhat_t (<= 1) and kd_j = phi(k_j) / prod_{16I <= i <= j} gamma_i.
//     kd is bounded only when a channel's gates over 16 tokens do not
//     multiply below ~1e-30 (documented precondition).
//   * inter-chunk: O += (Qhat_t * E_I) S0^T, E_I = prod_{i < 16I} gamma_i;
//     S_C = S0 diag(prod_all gamma) + V^T (phi(K) o prod_{j < i < C} gamma_i).
// All gate factors are running products of the gates themselves (within a
// block by a 16-lane scan), so no exponential or logarithm is evaluated; kd
// multiplies by the hardware reciprocal of the running product (about one
// ulp), and k~ is kd times the block's whole product.
//
// Work decomposition as in the delta-rule kernel: one workgroup per (b, h,
// block of DVB value channels); wave w keeps the transposed state slice of
// its 16 value channels in matrix-core accumulators across the sequence.
#include <algorithm>
#include <type_traits>

#include "la_chunk_common.hpp"

namespace la {

// Scaled variants of the LDS x LDS / LDS x register tile products: the A
// operand's contraction index k is multiplied by scale[k] (float32, in LDS)
// before it enters the matrix cores.
template <class Op>
__device__ __forceinline__ typename Group<Op>::type scaled_group(const Op *a, const float *s) {
    float x[4];
    Group<Op>::unpack(ld_group(a), x);
    const float4 f = *reinterpret_cast<const float4 *>(s);
    return Group<Op>::make(x[0] * f.x, x[1] * f.y, x[2] * f.z, x[3] * f.w);
}

template <int K, class Op>
__device__ __forceinline__ void tile_mma_ll_scaled(f32x4 &acc, const Op *a, int lda, const float *scale, const Op *b,
                                                   int ldb, int lane) {
    const int ko = 4 * (lane >> 4);
    const Op *ar = a + (lane & 15) * lda + ko;
    const Op *br = b + (lane & 15) * ldb + ko;
    const float *sr = scale + ko;
#pragma unroll
    for (int k = 0; k + 32 <= K; k += 32)
        mma32(acc, scaled_group(ar + k, sr + k), scaled_group(ar + k + 16, sr + k + 16), ld_group(br + k),
              ld_group(br + k + 16));
    if constexpr (K % 32 == 16) mma16(acc, scaled_group(ar + K - 16, sr + K - 16), ld_group(br + K - 16));
}

template <int NK, class Op, class G>
__device__ __forceinline__ void tile_mma_lr_scaled(f32x4 &acc, const Op *a, int lda, const float *scale, const G *bg,
                                                   int lane) {
    const int ko = 4 * (lane >> 4);
    const Op *ar = a + (lane & 15) * lda + ko;
    const float *sr = scale + ko;
#pragma unroll
    for (int s = 0; s + 2 <= NK; s += 2)
        mma32(acc, scaled_group(ar + 16 * s, sr + 16 * s), scaled_group(ar + 16 * s + 16, sr + 16 * s + 16), bg[s],
              bg[s + 1]);
    if constexpr (NK % 2 == 1) mma16(acc, scaled_group(ar + 16 * (NK - 1), sr + 16 * (NK - 1)), bg[NK - 1]);
}

// acc += Areg * B over NK k-blocks, B supplied transposed from LDS (row n of
// `b` holds column n of B, k contiguous) with its contraction index k
// multiplied by scale[k]; see tile_mma_rl_n.
template <int NK, class Op, class G>
__device__ __forceinline__ void tile_mma_rl_scaled(f32x4 &acc, const G *ag, const Op *b, int ldb, const float *scale,
                                                   int lane) {
    const int ko = 4 * (lane >> 4);
    const Op *br = b + (lane & 15) * ldb + ko;
    const float *sr = scale + ko;
#pragma unroll
    for (int s = 0; s + 2 <= NK; s += 2)
        mma32(acc, ag[s], ag[s + 1], scaled_group(br + 16 * s, sr + 16 * s), scaled_group(br + 16 * s + 16, sr + 16 * s + 16));
    if constexpr (NK % 2 == 1) mma16(acc, ag[NK - 1], scaled_group(br + 16 * (NK - 1), sr + 16 * (NK - 1)));
}

// DPP move with control CTRL on the rows in ROWMASK; lanes of the other rows
// (and lanes whose source is invalid) read 1
template <int CTRL, int ROWMASK>
__device__ __forceinline__ float dpp_or_one(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), CTRL, ROWMASK, 0xF, false));
}

// Inclusive product over each 16-lane row of a wave: lane i of a row gets
// x_0 * ... * x_i within each 16-lane row (lane i of the row): four DPP row
// shifts, each one v_mul_f32_dpp x, x[lane - k], x.  With the DPP bound
// control clear, a lane whose source lies outside its row is not written and
// keeps x, i.e. multiplies by 1.  (The s_nop covers the two wait states a DPP
// read needs after a vector write of its source.)
__device__ __forceinline__ float row_scan_mul(float x) {
    asm("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:1 row_mask:0xf bank_mask:0xf" : "+v"(x));
    asm("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf" : "+v"(x));
    asm("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf" : "+v"(x));
    asm("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf" : "+v"(x));
    return x;
}

// Four independent channels at once, one DPP step of all four before the next
// step of any: each DPP read then follows the write of its source by three
// other instructions, which covers the two wait states, so only the first
// instruction of the group needs the s_nop.
#define LA_DPP4(CTRL)                                                                                                   \
    "s_nop 1\n\t"                                                                                                   \
    "v_mul_f32_dpp %0, %4, %0 " CTRL "\n\tv_mul_f32_dpp %1, %5, %1 " CTRL "\n\t"                                     \
    "v_mul_f32_dpp %2, %6, %2 " CTRL "\n\tv_mul_f32_dpp %3, %7, %3 " CTRL
// x[i] <- y[i] (moved by the DPP control) times x[i]
#define LA_DPP4_OPS(x, y) "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]) : "v"(y[0]), "v"(y[1]), "v"(y[2]), "v"(y[3])
// the same with y = x, in place (the DPP source is read before the write), so
// that no copy of x is made for each step
#define LA_DPP4_SELF(CTRL)                                                                                              \
    "s_nop 1\n\t"                                                                                                   \
    "v_mul_f32_dpp %0, %0, %0 " CTRL "\n\tv_mul_f32_dpp %1, %1, %1 " CTRL "\n\t"                                     \
    "v_mul_f32_dpp %2, %2, %2 " CTRL "\n\tv_mul_f32_dpp %3, %3, %3 " CTRL
#define LA_DPP4_SELF_OPS(x) "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3])
__device__ __forceinline__ void row_scan_mul4(float (&x)[4]) {
    asm(LA_DPP4_SELF("row_shr:1 row_mask:0xf bank_mask:0xf") : LA_DPP4_SELF_OPS(x));
    asm(LA_DPP4_SELF("row_shr:2 row_mask:0xf bank_mask:0xf") : LA_DPP4_SELF_OPS(x));
    asm(LA_DPP4_SELF("row_shr:4 row_mask:0xf bank_mask:0xf") : LA_DPP4_SELF_OPS(x));
    asm(LA_DPP4_SELF("row_shr:8 row_mask:0xf bank_mask:0xf") : LA_DPP4_SELF_OPS(x));
}
// x <- y[last lane of the row before] * x on rows 1 and 3, then
// x <- x[lane 31] * x on rows 2 and 3 (with x = y on entry: the inclusive
// prefix over the whole wave, from the row-wise one)
__device__ __forceinline__ void wave_prefix_from_rows4(const float (&y)[4], float (&x)[4]) {
    asm(LA_DPP4("row_bcast:15 row_mask:0xa bank_mask:0xf") : LA_DPP4_OPS(x, y));
    asm(LA_DPP4_SELF("row_bcast:31 row_mask:0xc bank_mask:0xf") : LA_DPP4_SELF_OPS(x));
}
// x <- y[lane 31] * x on row 2
__device__ __forceinline__ void mul_bcast15_row2_4(const float (&y)[4], float (&x)[4]) {
    asm(LA_DPP4("row_bcast:15 row_mask:0x4 bank_mask:0xf") : LA_DPP4_OPS(x, y));
}

// Suffix products along each 16-lane row: lane i of a row gets x_i * ... *
// x_15 (four DPP row shifts to the left; a lane whose source lies past the
// row end keeps x), for one channel or four at once.
__device__ __forceinline__ float row_suffix_mul(float x) {
    asm("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shl:1 row_mask:0xf bank_mask:0xf" : "+v"(x));
    asm("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shl:2 row_mask:0xf bank_mask:0xf" : "+v"(x));
    asm("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shl:4 row_mask:0xf bank_mask:0xf" : "+v"(x));
    asm("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shl:8 row_mask:0xf bank_mask:0xf" : "+v"(x));
    return x;
}
__device__ __forceinline__ void row_suffix_mul4(float (&x)[4]) {
    asm(LA_DPP4_SELF("row_shl:1 row_mask:0xf bank_mask:0xf") : LA_DPP4_SELF_OPS(x));
    asm(LA_DPP4_SELF("row_shl:2 row_mask:0xf bank_mask:0xf") : LA_DPP4_SELF_OPS(x));
    asm(LA_DPP4_SELF("row_shl:4 row_mask:0xf bank_mask:0xf") : LA_DPP4_SELF_OPS(x));
    asm(LA_DPP4_SELF("row_shl:8 row_mask:0xf bank_mask:0xf") : LA_DPP4_SELF_OPS(x));
}
// the next lane's value within its 16-lane row, 1 at the row end: with
// x = row_suffix_mul(g), the exclusive suffix product g_{i+1} * ... * g_15
__device__ __forceinline__ float row_next_or_one(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(1.f), __float_as_int(x), 0x101, 0xF, 0xF, false));
}

// Below this product of one channel's gates over a 16-token block the fast
// diagonal factorization (key operand phi(k_j) / R_j) would leave the float32
// range; such a chunk takes gla_diag_exact for its diagonal score tiles and
// forms its key operands from suffix products instead.
constexpr float kGlaWeakBlock = 0x1p-64f;

// Exact diagonal 16x16 score tile of gated linear attention, for token block
// I of a chunk (n valid tokens, rows of q, k and the gates DK elements apart
// from the chunk's first token):
//   P_tj = sum_c phi(q_tc) phi(k_jc) prod_{j < i <= t} gamma_ic   (j <= t),
// zero above the diagonal and for tokens past n.  Every decay factor is a
// running product of the gates themselves and never exceeds 1, so the tile
// is exact (to float32 rounding) for any gates in (0, 1] (page "Ch. 11 Linear
// attention and Hyena", 11.3 and the solution to Exercise 11.5, which state
// the gate range).  Lane (j, cq): key token j of the block and one group of
// channels; its running key factors kd_c = phi(k_jc) prod_{j < i <= t}
// gamma_ic advance one query token t per step, and the row sum over the
// channel groups comes from two lane exchanges.  The inputs are re-read from
// global memory (they are in the cache: the chunk was just staged).
template <int PHI, class IO, int DK, class Op>
__device__ __forceinline__ void gla_diag_exact(const IO *q0, const IO *k0, const float *g0, int n, int I, Op *P,
                                               int ldc, int lane) {
    constexpr int NQ = DK / 8 < 4 ? DK / 8 : 4;   // channel groups over the lanes of a token
    constexpr int CPL = DK / NQ;                   // channels per lane, a multiple of 8
    const int j = lane & 15, cq = lane >> 4;
    const bool act = cq < NQ;
    const int c0 = (act ? cq : 0) * CPL;
    const int rj = 16 * I + j;
    const bool jon = act && rj < n;
    float kd[CPL];
#pragma unroll
    for (int cg = 0; cg < CPL; cg += 8) {
        float x[8];
        load8(k0 + static_cast<size_t>(min(rj, n - 1)) * DK + c0 + cg, x);
#pragma unroll
        for (int i = 0; i < 8; ++i) kd[cg + i] = jon ? apply_phi<PHI>(x[i]) : 0.f;
    }
#pragma unroll 1
    for (int t = 0; t < 16; ++t) {
        const int rt = 16 * I + t;
        const size_t row = static_cast<size_t>(min(rt, n - 1)) * DK + c0;
        const bool ton = rt < n, adv = t > j;
        float s = 0.f;
#pragma unroll
        for (int cg = 0; cg < CPL; cg += 8) {
            // one channel group's loads at a time: the routine shares the
            // register budget of the kernel it is inlined into
            asm volatile("" ::: "memory");
            float qv[8], gv[8];
            load8(q0 + row + cg, qv);
            load8(g0 + row + cg, gv);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                kd[cg + i] *= adv ? gv[i] : 1.f;
                s += (ton ? apply_phi<PHI>(qv[i]) : 0.f) * kd[cg + i];
            }
        }
        s += __shfl_xor(s, 16);
        s += __shfl_xor(s, 32);
        if (cq == 0) from_f32(P[t * ldc + j], t >= j ? s : 0.f);
    }
}

// pair index of an off-diagonal key block J <= I - 2 (blocks strictly between exist)
__host__ __device__ constexpr int rho_index(int I, int J) { return (I - 2) * (I - 1) / 2 + J; }

template <bool GATED, class DT, int DK, int DVB, int C>
struct LinearLds {
    typedef typename OpOf<DT>::type Op;
    static constexpr int NB = C / 16;
    static constexpr int NRHO = NB >= 3 ? (NB - 1) * (NB - 2) / 2 : 0;
    static constexpr int PAD = 16 / sizeof(Op);
    static constexpr int LDK = DK + PAD;
    static constexpr int LDC = C + PAD;
    static constexpr int LDG = DK + 4;
    static constexpr int LDV = DVB + PAD;   // value tile, rows = tokens
    static constexpr int P_BYTES = C * LDC * (int)sizeof(Op);
    static constexpr int G_BYTES = GATED ? C * LDG * 4 : 0;
    static constexpr int PG_BYTES = P_BYTES > G_BYTES ? P_BYTES : G_BYTES;
    static constexpr int F_FLOATS = GATED ? (NB + 1 + NRHO) * DK : DK + C + C + 4;   // normalized: z, den, gamma^0..C
    static constexpr int KT_ELEMS = GATED ? C * LDK : 8;   // gated: state-update key operand
    static constexpr int BYTES = (GATED ? 3 : 2) * C * LDK * (int)sizeof(Op) + KT_ELEMS * (int)sizeof(Op) +
                                 C * LDV * (int)sizeof(Op) + PG_BYTES + F_FLOATS * 4;
};

template <bool GATED, int PHI, class DT, int DK, int DVB, int C, int NW>
__global__ void __launch_bounds__(NW * 64) linear_chunk_kernel(const ChunkParams p) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef Group<Op> Gp;
    typedef typename Gp::type G4;
    typedef LinearLds<GATED, DT, DK, DVB, C> L;
    constexpr int WS = DVB / 16;                          // state waves
    constexpr int NTHR = NW * 64;
    constexpr int NB = C / 16;
    constexpr int NCB = DK / 16;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDG = L::LDG, LDV = L::LDV;
    constexpr int VE = 16 / sizeof(IO);                   // elements per 16-byte vector
    static_assert(C <= 64 && C % 16 == 0 && DK % 16 == 0 && DVB % 16 == 0 && WS <= NW, "tiling");
    static_assert(L::BYTES <= 160 * 1024, "LDS budget");

    __shared__ __align__(16) Op sQ[C * LDK];                 // phi(Q) | Qhat
    __shared__ __align__(16) Op sK[C * LDK];                 // phi(K) | k~ (off-diagonal reference)
    __shared__ __align__(16) Op sKd[GATED ? C * LDK : 8];    // kd (diagonal reference)
    __shared__ __align__(16) Op sKt[L::KT_ELEMS];            // gated: key operand of the state update, [t][c]
    __shared__ __align__(16) Op sV[C * LDV];                 // this block's values, [t][v]
    __shared__ __align__(16) unsigned char sPG[L::PG_BYTES]; // gates (f32), then P
    __shared__ __align__(16) float sF[L::F_FLOATS];
    __shared__ int sWeak;   // gated: this chunk takes the exact diagonal tiles
    Op *sP = reinterpret_cast<Op *>(sPG);
    float *sG = reinterpret_cast<float *>(sPG);
    float *sE = sF;                       // gated: prod of the chunk's gates before block I, [NB][DK]
    float *sD = sF + NB * DK;             // gated: prod of all the chunk's gates, [DK]
    float *sRho = sF + (NB + 1) * DK;     // gated: prod of the blocks strictly between J and I, [NRHO][DK]
    float *sZ = sF;                       // normalized: running z, [DK]
    float *sDen = sF + DK;                // normalized: denominators, [C]
    float *sPow = sF + DK + C;            // not gated: gamma^k of the per-head decay, k = 0 .. C

    // the wave index is uniform: role branches compile to scalar branches
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    // the workgroup's segment of the sequence: the whole of it unless the
    // normalized variant is split (n_seg > 1; see ChunkParams::seg_state)
    const int nhb = p.n_heads * p.n_vblk;
    const int seg = blockIdx.x / nhb;
    int bh, vb;
    block_to_head(blockIdx.x - seg * nhb, p.n_heads, p.n_vblk, bh, vb);
    const int tb = seg * p.seg_len;
    const int Tn = p.n_seg > 1 ? min(p.seg_len, p.T - tb) : p.T;   // tokens of this workgroup
    const int vloc = 16 * wave + lr;
    const int vch = vb * DVB + vloc;
    const size_t tok0 = static_cast<size_t>(bh) * p.T + tb;
    const IO *qh = static_cast<const IO *>(p.q) + tok0 * DK;
    const IO *kh = static_cast<const IO *>(p.k) + tok0 * DK;
    const IO *vh = static_cast<const IO *>(p.v) + tok0 * p.d_v + vb * DVB;
    IO *oh = static_cast<IO *>(p.out) + tok0 * p.d_v;
    const float *gh = GATED ? p.gate + tok0 * DK : nullptr;

    // not gated: log2 of the head's fixed decay (0 without one: every power is
    // 1, and `decay` is false so that the undecayed path skips the factors)
    const float l2g = __builtin_bit_cast(
        float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(
                   int, !GATED && p.gate ? __builtin_amdgcn_logf(p.gate[bh % p.H]) : 0.f)));
    const bool decay = !GATED && l2g != 0.f;
    if constexpr (!GATED) {
        for (int e = tid; e <= C; e += NTHR) sPow[e] = __builtin_amdgcn_exp2f(static_cast<float>(e) * l2g);
    }
    f32x4 st[NCB];
    const size_t srow = (static_cast<size_t>(bh) * p.d_v + (wave < WS ? vch : 0)) * DK;
    const size_t slot = static_cast<size_t>(p.d_v) * DK + DK;   // floats per seg_state slot
    const float *segs = p.n_seg > 1 ? p.seg_state + static_cast<size_t>(bh) * p.n_seg * slot : nullptr;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        st[cb] = zero4();
        if (p.n_seg == 1 && p.S0 && wave < WS) {
            const float4 s = *reinterpret_cast<const float4 *>(p.S0 + srow + 16 * cb + 4 * lg);
            st[cb] = f32x4{s.x, s.y, s.z, s.w};
        }
    }
    if (p.n_seg > 1 && wave < WS) {
        // entering state of segment seg: the initial state plus the increments
        // of the segments before it, added in order; the slots are read SB at
        // a time, so that their loads are in flight together
        constexpr int SB = NCB >= 8 ? 2 : 16 / NCB;
        const float *col = segs + static_cast<size_t>(vch) * DK + 4 * lg;
        for (int s0 = 0; s0 <= seg; s0 += SB) {
            float4 v[SB][NCB];
#pragma unroll
            for (int j = 0; j < SB; ++j)
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    v[j][cb] = *reinterpret_cast<const float4 *>(col + min(s0 + j, seg) * slot + 16 * cb);
#pragma unroll
            for (int j = 0; j < SB; ++j)
                if (s0 + j <= seg) {
                    // slot s0 + j reaches this segment's start after (seg - s0 - j)
                    // whole segments of decay
                    const float w = decay ? __builtin_amdgcn_exp2f(static_cast<float>((seg - s0 - j) * p.seg_len) * l2g)
                                          : 1.f;
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        st[cb] += w * f32x4{v[j][cb].x, v[j][cb].y, v[j][cb].z, v[j][cb].w};
                }
        }
    }
    if constexpr (!GATED) {
        for (int c = tid; c < DK && p.normalize; c += NTHR) {
            float z = 0.f;
            if (p.n_seg > 1) {
                const float *zc = segs + static_cast<size_t>(p.d_v) * DK + c;
                for (int s0 = 0; s0 <= seg; s0 += 8) {
                    float v[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) v[j] = zc[min(s0 + j, seg) * slot];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (s0 + j <= seg)
                            z += (decay ? __builtin_amdgcn_exp2f(static_cast<float>((seg - s0 - j) * p.seg_len) * l2g) : 1.f) *
                                 v[j];
                }
            } else if (p.z0) {
                z = p.z0[static_cast<size_t>(bh) * DK + c];
            }
            sZ[c] = z;
        }
    }
    // the entering state is in registers before any tile load is issued, so
    // the loop never waits on the global-memory counter for it
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // chunk inputs staged one chunk ahead in registers
    TilePrefetch<C, DK, NTHR, IO> pq, pk;
    TilePrefetch<C, DVB, NTHR, IO> pv;
    TilePrefetch<C, GATED ? DK : 4, NTHR, float> pgt;
    auto prefetch = [&](int c0) {
        const int n = min(C, Tn - c0);
        pq.load(qh + static_cast<size_t>(c0) * DK, DK, n, tid);
        pk.load(kh + static_cast<size_t>(c0) * DK, DK, n, tid);
        pv.load(vh + static_cast<size_t>(c0) * p.d_v, p.d_v, n, tid);
        if constexpr (GATED) pgt.load(gh + static_cast<size_t>(c0) * DK, DK, n, tid);
    };
    if (Tn > 0) prefetch(0);

    // The state waves keep a chunk's outputs in registers and store them after
    // the next chunk's commit and prefetch: the commit's wait on the
    // global-memory counter (for the staged loads) then never waits for
    // just-issued output stores.
    f32x4 ob[NB];
    auto store_outputs = [&](int oc0) {
        const int on = min(C, Tn - oc0);
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            const int t = 16 * I + lr;
            if (t < on) st_group(oh + static_cast<size_t>(oc0 + t) * p.d_v + vb * DVB + 16 * wave + 4 * lg, Gp::make(ob[I]));
        }
    };

    for (int c0 = 0; c0 < Tn; c0 += C) {
        const int n = min(C, Tn - c0);

        // ---- commit the staged chunk.  Values as they are (the products that
        // contract over tokens read them transposed); queries/keys raw (gated)
        // or with phi applied (normalized); gates as float32 with padded tokens
        // set to 1 (no decay).
        pv.store(sV, LDV, tid);
        if (GATED && tid == 0) sWeak = 0;
        if constexpr (!GATED) {
#pragma unroll
            for (int i = 0; i < pq.PER; ++i) {
                const int e = tid + i * NTHR;
                if (pq.TOTAL % NTHR != 0 && e >= pq.TOTAL) continue;
                const int t = e / pq.VPR, c = (e % pq.VPR) * VE;
                float xq[8], xk[8];
                if constexpr (VE == 8) {
                    const uint4 a = pq.r[i], b = pk.r[i];
                    xq[0] = lo_bf16(a.x); xq[1] = hi_bf16(a.x); xq[2] = lo_bf16(a.y); xq[3] = hi_bf16(a.y);
                    xq[4] = lo_bf16(a.z); xq[5] = hi_bf16(a.z); xq[6] = lo_bf16(a.w); xq[7] = hi_bf16(a.w);
                    xk[0] = lo_bf16(b.x); xk[1] = hi_bf16(b.x); xk[2] = lo_bf16(b.y); xk[3] = hi_bf16(b.y);
                    xk[4] = lo_bf16(b.z); xk[5] = hi_bf16(b.z); xk[6] = lo_bf16(b.w); xk[7] = hi_bf16(b.w);
                } else {
                    const uint4 a = pq.r[i], b = pk.r[i];
                    xq[0] = __uint_as_float(a.x); xq[1] = __uint_as_float(a.y);
                    xq[2] = __uint_as_float(a.z); xq[3] = __uint_as_float(a.w);
                    xk[0] = __uint_as_float(b.x); xk[1] = __uint_as_float(b.y);
                    xk[2] = __uint_as_float(b.z); xk[3] = __uint_as_float(b.w);
                }
                const bool on = t < n;   // padded tokens carry no feature (phi(0) would be 1)
                float fq[8], fk[8];
#pragma unroll
                for (int j = 0; j < VE; ++j) {
                    fq[j] = on ? apply_phi<PHI>(xq[j]) : 0.f;
                    fk[j] = on ? apply_phi<PHI>(xk[j]) : 0.f;
                }
#pragma unroll
                for (int j = 0; j < VE; j += 4) {
                    st_group(sQ + t * LDK + c + j, Gp::make(fq[j], fq[j + 1], fq[j + 2], fq[j + 3]));
                    st_group(sK + t * LDK + c + j, Gp::make(fk[j], fk[j + 1], fk[j + 2], fk[j + 3]));
                }
            }
        } else {
            pq.store(sQ, LDK, tid);
            pk.store(sK, LDK, tid);
#pragma unroll
            for (int i = 0; i < pgt.PER; ++i) {
                const int e = tid + i * NTHR;
                if (pgt.TOTAL % NTHR != 0 && e >= pgt.TOTAL) continue;
                const int t = e / pgt.VPR, c = (e % pgt.VPR) * 4;
                float4 g = make_float4(1.f, 1.f, 1.f, 1.f);
                if (t < n) g = *reinterpret_cast<const float4 *>(&pgt.r[i]);
                *reinterpret_cast<float4 *>(sG + t * LDG + c) = g;
            }
        }
        __syncthreads();
        // the next chunk's loads first (a chunk past the end re-reads the last
        // one, never used), then the stores: every path issues the same loads,
        // so the compiler's waits for them stay exact and never cover stores
        prefetch(min(c0 + C, ((Tn - 1) / C) * C));
        if (wave < WS && c0 > 0) store_outputs(c0 - C);

        if constexpr (GATED) {
            // ---- gate factors.  A wave takes four key channels of every token of
            // the chunk (lane = token): the products along the tokens of a 16-token
            // block are scans over a 16-lane DPP row, so every token's factors come
            // out at once and are written four channels at a time.
            const int t = lane, I = t >> 4;
            const bool in_tile = t < C, on = t < n;
            for (int c = 4 * wave; c < DK; c += 4 * NW) {
                float g[4] = {1.f, 1.f, 1.f, 1.f}, q[4] = {0.f, 0.f, 0.f, 0.f}, k[4] = {0.f, 0.f, 0.f, 0.f};
                if (in_tile) {
                    const float4 g4 = *reinterpret_cast<const float4 *>(sG + t * LDG + c);
                    g[0] = g4.x; g[1] = g4.y; g[2] = g4.z; g[3] = g4.w;   // 1 past the sequence end
                    Gp::unpack(ld_group(sQ + t * LDK + c), q);
                    Gp::unpack(ld_group(sK + t * LDK + c), k);
                }
                float run[4], rinv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    run[i] = row_scan_mul(g[i]);   // R_t = prod_{16I <= s <= t} g_s
                    rinv[i] = __builtin_amdgcn_rcpf(run[i]);
                }
                // strong decay somewhere in these channels (a block product below
                // kGlaWeakBlock; R_t only falls along a block): k~ from the
                // exclusive suffix products of the gates, which never exceed 1,
                // and the chunk's diagonal tiles by gla_diag_exact
                const bool weak = __builtin_amdgcn_ballot_w64(run[0] < kGlaWeakBlock || run[1] < kGlaWeakBlock ||
                                                              run[2] < kGlaWeakBlock || run[3] < kGlaWeakBlock) != 0;
                float sx[4] = {0.f, 0.f, 0.f, 0.f};
                if (weak) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) sx[i] = row_next_or_one(row_suffix_mul(g[i]));
                    if (lane == 0) sWeak = 1;
                }
                float tot[NB][4];   // whole-block products (uniform)
#pragma unroll
                for (int J = 0; J < NB; ++J)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        tot[J][i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(run[i]), 16 * J + 15));
                {
                    // per-chunk factors E_J, D and rho_{J1 J0}: products of the block
                    // totals, the same in every lane (no per-lane selection), written
                    // by lane 0 as one float4 (four channels) per factor
                    constexpr int NF = NB + 1 + L::NRHO;
                    float fe[NF][4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float acc = 1.f;
#pragma unroll
                        for (int J = 0; J < NB; ++J) {
                            fe[J][i] = acc;        // E_J: the blocks before J
                            acc *= tot[J][i];
                        }
                        fe[NB][i] = acc;           // D: all blocks
#pragma unroll
                        for (int J1 = 2; J1 < NB; ++J1)
#pragma unroll
                            for (int J0 = 0; J0 + 2 <= J1; ++J0) {
                                float r = 1.f;     // rho_{J1 J0}: the blocks strictly between
#pragma unroll
                                for (int J = J0 + 1; J < J1; ++J) r *= tot[J][i];
                                fe[NB + 1 + rho_index(J1, J0)][i] = r;
                            }
                    }
                    if (lane == 0) {
#pragma unroll
                        for (int f = 0; f < NF; ++f)
                            *reinterpret_cast<float4 *>(sE + f * DK + c) = make_float4(fe[f][0], fe[f][1], fe[f][2], fe[f][3]);
                    }
                }
                // Qhat = phi(q) R_t, kd = phi(k) / R_t, k~ = phi(k) prod_{t<s<=e_I} g_s
                // = kd * (block product), and the state-update operand k~ times the
                // product of the later blocks (natural layout)
                float fq[4], fd[4], fk[4], fa[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float tb = tot[0][i], after = 1.f;   // this token's block, the blocks after it
#pragma unroll
                    for (int J = 1; J < NB; ++J) {
                        if (J == I) tb = tot[J][i];
                        if (J > I) after *= tot[J][i];
                    }
                    fq[i] = on ? apply_phi<PHI>(q[i]) * run[i] : 0.f;
                    fd[i] = on && !weak ? apply_phi<PHI>(k[i]) * rinv[i] : 0.f;
                    fk[i] = weak ? (on ? apply_phi<PHI>(k[i]) * sx[i] : 0.f) : fd[i] * tb;
                    fa[i] = fk[i] * after;
                }
                if (in_tile) {
                    st_group(sQ + t * LDK + c, Gp::make(fq[0], fq[1], fq[2], fq[3]));
                    st_group(sKd + t * LDK + c, Gp::make(fd[0], fd[1], fd[2], fd[3]));
                    st_group(sK + t * LDK + c, Gp::make(fk[0], fk[1], fk[2], fk[3]));
                    st_group(sKt + t * LDK + c, Gp::make(fa[0], fa[1], fa[2], fa[3]));
                }
            }
            __syncthreads();   // the gate tile is dead from here on; its space holds P
        }

        // ---- intra-chunk scores P (16x16 tiles, block-lower-triangular)
        // Each tile is taken transposed (keys x queries), so that a lane holds
        // four consecutive columns j of one row t and writes them at once.
        const bool weak_chunk = GATED && __builtin_amdgcn_readfirstlane(sWeak) != 0;
        for (int tt = wave; tt < NB * NB; tt += NW) {
            const int I = tt / NB, J = tt % NB;
            const int t = 16 * I + lr, j0 = 16 * J + 4 * lg;
            if (J > I) {
                st_group(sP + t * LDC + j0, Gp::make(0.f, 0.f, 0.f, 0.f));
                continue;
            }
            if (GATED && J == I && weak_chunk) {
                gla_diag_exact<PHI, IO, DK>(qh + static_cast<size_t>(c0) * DK, kh + static_cast<size_t>(c0) * DK,
                                            gh + static_cast<size_t>(c0) * DK, n, I, sP + 16 * I * LDC + 16 * I, LDC, lane);
                continue;
            }
            f32x4 acc = zero4();
            if constexpr (GATED) {
                if (J == I)
                    tile_mma_ll<DK>(acc, sKd + 16 * J * LDK, LDK, sQ + 16 * I * LDK, LDK, lane);
                else if (J == I - 1)
                    tile_mma_ll<DK>(acc, sK + 16 * J * LDK, LDK, sQ + 16 * I * LDK, LDK, lane);
                else
                    tile_mma_ll_scaled<DK>(acc, sK + 16 * J * LDK, LDK, sRho + rho_index(I, J) * DK,
                                           sQ + 16 * I * LDK, LDK, lane);
            } else {
                tile_mma_ll<DK>(acc, sK + 16 * J * LDK, LDK, sQ + 16 * I * LDK, LDK, lane);
                // fixed decay: P_tj *= gamma^(t - j)
                if (decay) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[i] *= sPow[max(t - j0 - i, 0)];
                }
            }
            st_group(sP + t * LDC + j0, Gp::make(j0 <= t ? acc[0] : 0.f, j0 + 1 <= t ? acc[1] : 0.f,
                                                 j0 + 2 <= t ? acc[2] : 0.f, j0 + 3 <= t ? acc[3] : 0.f));
        }
        __syncthreads();

        if (!GATED && p.normalize) {
            // ---- denominators gamma^(t+1) phi(q_t).z0 + sum_j P_tj (the rounded
            // P of the numerator); 8 lanes per token
            for (int e = tid; e < 8 * C; e += NTHR) {
                const int t = e >> 3, part = e & 7;
                float dz = 0.f, dp = 0.f;
                for (int c = part; c < DK; c += 8) dz += to_f32(sQ[t * LDK + c]) * sZ[c];
                for (int j = part; j <= t; j += 8) dp += to_f32(sP[t * LDC + j]);
                const float d = group_sum<8>((decay ? sPow[t + 1] * dz : dz) + dp);
                if (part == 0) sDen[t] = d;
            }
            __syncthreads();
            // z_C = gamma^n z0 + sum_t gamma^(n-1-t) phi(k_t) (after every
            // denominator has read z0)
            for (int c = tid; c < DK; c += NTHR) {
                float s = 0.f;
                if (decay) {
#pragma unroll 8
                    for (int t = 0; t < n; ++t) s += sPow[n - 1 - t] * to_f32(sK[t * LDK + c]);
                    sZ[c] = sPow[n] * sZ[c] + s;
                } else {
#pragma unroll 8
                    for (int t = 0; t < C; ++t) s += to_f32(sK[t * LDK + c]);   // rows past n are zero
                    sZ[c] += s;
                }
            }
        }

        // ---- state-dependent part: this wave's 16 value channels
        if (wave < WS) {
            G4 sb[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) sb[cb] = Gp::make(st[cb]);
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                // O^T = S0 Q^T + V^T P^T: lane holds values 16*wave + 4*lg..+3 of
                // token 16 I + lr, stored at once
                f32x4 o = zero4();
                if constexpr (GATED) {
                    if (I == 0) tile_mma_rl_n<NCB>(o, sb, sQ, LDK, NCB, lane);
                    else tile_mma_rl_scaled<NCB>(o, sb, sQ + 16 * I * LDK, LDK, sE + I * DK, lane);
                } else {
                    tile_mma_rl_n<NCB>(o, sb, sQ + 16 * I * LDK, LDK, NCB, lane);
                    // fixed decay: the entering state reaches token t after t + 1 steps
                    if (decay) {
                        const float lead = sPow[16 * I + lr + 1];
#pragma unroll
                        for (int i = 0; i < 4; ++i) o[i] *= lead;
                    }
                }
                // + V^T P^T: V^T by transposing reads of the value tile
                const Op *prow = sP + (16 * I + lr) * LDC + 4 * lg;
#pragma unroll
                for (int t0 = 0; t0 + 32 <= C; t0 += 32)
                    mma32(o, kt_group<0>(sV, LDV, t0, 16 * wave, lane), kt_group<0>(sV, LDV, t0 + 16, 16 * wave, lane),
                          ld_group(prow + t0), ld_group(prow + t0 + 16));
                if constexpr (C % 32 == 16) mma16(o, kt_group<0>(sV, LDV, C - 16, 16 * wave, lane), ld_group(prow + C - 16));
                if (!GATED && p.normalize) {
                    const float inv = 1.f / sDen[16 * I + lr];
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] *= inv;
                }
                ob[I] = o;
            }
            // V^T operand groups of the state update (the same for every key
            // block); not gated: token t's value scaled by gamma^(n-1-t)
            G4 vg[NB];
#pragma unroll
            for (int s2 = 0; s2 < NB; ++s2) {
                vg[s2] = kt_group<0>(sV, LDV, 16 * s2, 16 * wave, lane);
                if (decay) {
                    float x[4];
                    Gp::unpack(vg[s2], x);
                    const int t0 = 16 * s2 + 4 * lg;
#pragma unroll
                    for (int i = 0; i < 4; ++i) x[i] *= sPow[max(n - 1 - t0 - i, 0)];
                    vg[s2] = Gp::make(x[0], x[1], x[2], x[3]);
                }
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if constexpr (GATED) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) st[cb][i] *= sD[16 * cb + 4 * lg + i];
                } else if (decay) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) st[cb][i] *= sPow[n];
                }
                // S^T += K^T V (gated: the scaled key operand): both from the
                // token-major tiles by transposing reads
                const Op *kt = GATED ? sKt : sK;
#pragma unroll
                for (int s2 = 0; s2 + 2 <= NB; s2 += 2)
                    mma32(st[cb], kt_group<0>(kt, LDK, 16 * s2, 16 * cb, lane),
                          kt_group<0>(kt, LDK, 16 * s2 + 16, 16 * cb, lane), vg[s2], vg[s2 + 1]);
                if constexpr (NB % 2 == 1)
                    mma16(st[cb], kt_group<0>(kt, LDK, 16 * (NB - 1), 16 * cb, lane), vg[NB - 1]);
            }
        }
        __syncthreads();
    }

    if (wave < WS && Tn > 0) store_outputs(((Tn - 1) / C) * C);
    const bool last_seg = seg == p.n_seg - 1;
    if (p.S_T && wave < WS && last_seg) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            *reinterpret_cast<float4 *>(p.S_T + srow + 16 * cb + 4 * lg) =
                make_float4(st[cb][0], st[cb][1], st[cb][2], st[cb][3]);
    }
    if constexpr (!GATED) {
        if (p.normalize && p.z_T && vb == 0 && last_seg)
            for (int c = tid; c < DK; c += NTHR) p.z_T[static_cast<size_t>(bh) * DK + c] = sZ[c];
    }
}

// ------------------------------------------------------------------ gated, pipelined
// Gated linear attention with the commit of chunk c+1 overlapping the
// state-dependent part of chunk c:
//   step A  state waves (DVB/16, each owning the state slice of 16 value
//           channels): the outputs of chunk c (kept in registers) and its
//           state update; the other waves: commit chunk c+1's staged q, k, v,
//           load chunk c+1's gate tile and chunk c+2's q, k, v;
//   step B  all waves: the gate factors of chunk c+1; then the state waves
//           store chunk c's outputs;
//   step C  all waves: the scores of chunk c+1.
// The raw q and V tiles are double-buffered (chunk c+1's are written while
// chunk c's are read).  The gate tile goes straight from global memory to LDS
// (direct loads, whole rows per instruction, in rows padded by 16 bytes so
// that the gate pass's reads of one channel group over 16 tokens touch every
// bank once); where that tile does not fit, each lane loads the gates of its
// token for exactly the channels its gate-factor passes handle instead.  The
// arithmetic is the gated path of linear_chunk_kernel, term for term.
template <class DT, int DK, int DVB, int C, int NW>
struct GlaLds {
    typedef typename OpOf<DT>::type Op;
    static constexpr int NB = C / 16;
    static constexpr int NRHO = NB >= 3 ? (NB - 1) * (NB - 2) / 2 : 0;
    static constexpr int PAD = 16 / sizeof(Op);
    static constexpr int LDK = DK + PAD, LDC = C + PAD, LDV = DVB + PAD;
    static constexpr int NTOT = NB + 3;   // block-total slots: NB totals, then three of ones
    static constexpr int F_FLOATS = (NB + 1 + NRHO + NTOT) * DK;
    static constexpr int BYTES = (5 * C * LDK + 2 * C * LDV + C * LDC) * (int)sizeof(Op) + F_FLOATS * 4;
    static constexpr int WS = DVB / 16, NH = NW - WS;
    static constexpr bool FITS = BYTES <= 160 * 1024 && NH >= 2;
    static constexpr int GLD = DK + 4;   // gate tile row stride (floats)
    static constexpr bool GDMA = BYTES + C * GLD * 4 <= 160 * 1024;
};

template <int PHI, class DT, int DK, int DVB, int C, int NW>
__global__ void __launch_bounds__(NW * 64) gla_pipelined_kernel(const ChunkParams p) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef Group<Op> Gp;
    typedef typename Gp::type G4;
    typedef GlaLds<DT, DK, DVB, C, NW> L;
    constexpr int WS = L::WS, NH = L::NH;
    constexpr int NB = C / 16, NCB = DK / 16;
    constexpr int LDK = L::LDK, LDC = L::LDC, LDV = L::LDV;
    constexpr int GI = (DK + 4 * NW - 1) / (4 * NW);   // gate-factor passes per wave and chunk
    static_assert(L::FITS, "pipelined layout does not fit");

    __shared__ __align__(16) Op sQ[2][C * LDK];    // raw q of the chunk being prepared, then Qhat
    __shared__ __align__(16) Op sK[C * LDK];       // raw k, then k~
    __shared__ __align__(16) Op sKd[C * LDK];      // kd (diagonal blocks)
    __shared__ __align__(16) Op sKt[C * LDK];      // state-update key operand
    __shared__ __align__(16) Op sV[2][C * LDV];    // values, [t][v]
    __shared__ __align__(16) Op sP[C * LDC];       // scores
    __shared__ __align__(16) float sF[L::F_FLOATS];   // E_J, D, rho, block totals
    constexpr bool GDMA = L::GDMA;
    constexpr int GLD = L::GLD;
    __shared__ __align__(16) float sG[GDMA ? C * GLD : 4];   // gates of the chunk being prepared
    __shared__ int sWeak;   // chunk c+1 takes the exact diagonal tiles
    float *sE = sF, *sD = sF + NB * DK, *sRho = sF + (NB + 1) * DK, *sTot = sRho + L::NRHO * DK;

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const bool state_wave = wave < WS;
    const int htid = tid - WS * 64;   // helper thread index (waves >= WS)
    int bh, vb;
    block_to_head(blockIdx.x, p.n_heads, p.n_vblk, bh, vb);
    const int vloc = 16 * wave + lr;
    const int vch = vb * DVB + vloc;
    const size_t tok0 = static_cast<size_t>(bh) * p.T;
    const IO *qh = static_cast<const IO *>(p.q) + tok0 * DK;
    const IO *kh = static_cast<const IO *>(p.k) + tok0 * DK;
    const IO *vh = static_cast<const IO *>(p.v) + tok0 * p.d_v + vb * DVB;
    IO *oh = static_cast<IO *>(p.out) + tok0 * p.d_v;
    const float *gh = p.gate + tok0 * DK;
    const int nchunks = (p.T + C - 1) / C;
    const int clast = nchunks - 1;
    auto rows = [&](int c) { return min(C, p.T - c * C); };

    f32x4 st[NCB];
    const size_t srow = (static_cast<size_t>(bh) * p.d_v + (state_wave ? vch : 0)) * DK;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        st[cb] = zero4();
        if (p.S0 && state_wave) {
            const float4 s = *reinterpret_cast<const float4 *>(p.S0 + srow + 16 * cb + 4 * lg);
            st[cb] = f32x4{s.x, s.y, s.z, s.w};
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    // block-total slots NB.. are ones: a token's product over the blocks after
    // its own reads the NB - 1 slots that follow its block's
    for (int e = tid; e < (L::NTOT - NB) * DK; e += NW * 64) sTot[NB * DK + e] = 1.f;

    // q, k, v (helpers) and the gates (every wave) two chunks ahead of the
    // state part.  Every load is issued whether or not its chunk exists (a
    // chunk past the end re-reads the last one and is never used), so the
    // compiler's wait for one set never covers another.
    TilePrefetch<C, DK, NH * 64, IO> pq, pk;
    TilePrefetch<C, DVB, NH * 64, IO> pv;
    float4 pg[GI];   // gates of token `lane`, channels 4 wave + 4 NW i .. +3
    auto load_qkv = [&](int c) {
        const int n = rows(c);
        pq.load(qh + static_cast<size_t>(c * C) * DK, DK, n, htid);
        pk.load(kh + static_cast<size_t>(c * C) * DK, DK, n, htid);
        pv.load(vh + static_cast<size_t>(c * C) * p.d_v, p.d_v, n, htid);
    };
    auto load_gates = [&](int c) {
        const int n = rows(c);
        const float *g = gh + static_cast<size_t>(c * C + (lane < n ? lane : n - 1)) * DK + 4 * wave;
#pragma unroll
        for (int i = 0; i < GI; ++i)
            if (4 * wave + 4 * NW * i < DK) pg[i] = *reinterpret_cast<const float4 *>(g + 4 * NW * i);
    };
    // GDMA, helper waves: chunk c's gate tile by direct loads, 16-byte slot s
    // of the tile (GLD / 4 slots a row, the last one padding) receiving the
    // four gates of its row and column group (rows past the end re-read the
    // last row; their gates are replaced by 1)
    auto dma_gates = [&](int c) {
        constexpr int GRS = GLD / 4, GNI = (C * GRS + 63) / 64;
        const int n = rows(c);
        const float *src0 = gh + static_cast<size_t>(c * C) * DK;
        const unsigned base = lds_addr(sG);
        for (int j = wave - WS; j < GNI; j += NH) {
            const int slot = 64 * j + lane, row = slot / GRS, col = slot % GRS;
            if ((C * GRS) % 64 == 0 || slot < C * GRS)
                lds_dma16(src0 + (row < n ? row : n - 1) * DK + 4 * (col < DK / 4 ? col : 0),
                          __builtin_amdgcn_readfirstlane(base + 1024 * j));
        }
    };
    f32x4 ob[NB];   // state waves: outputs of chunk c, stored in step B
    if (nchunks > 0) {
        if (!state_wave) load_qkv(0);
        if constexpr (!GDMA) load_gates(0);
    }

    // step B, every wave: the gate factors of chunk c+1 (lane = token, four
    // channels per pass; the products along a 16-token block are 16-lane DPP
    // row scans)
    // A whole chunk takes the variant without the selects for tokens past the
    // end (FULL: every token of the tile is on).
    auto gate_pass_n = [&](int c, auto full) {
        constexpr bool FULL = decltype(full)::value;
        const int nb = (c + 1) & 1, n1 = rows(c + 1);
        const int t = lane, I = t >> 4;
        const bool in_tile = t < C, on = FULL ? in_tile : t < n1;
#pragma unroll
        for (int it = 0; it < GI; ++it) {
            const int cc = 4 * wave + 4 * NW * it;
            if (cc >= DK) break;   // uniform: the last pass covers fewer waves
            float g[4] = {1.f, 1.f, 1.f, 1.f}, q[4] = {0.f, 0.f, 0.f, 0.f}, k[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (GDMA) {
                const float4 gv = *reinterpret_cast<const float4 *>(sG + (in_tile ? t : 0) * GLD + cc);
                if (on) { g[0] = gv.x; g[1] = gv.y; g[2] = gv.z; g[3] = gv.w; }   // 1 past the end
            } else {
                if (on) { g[0] = pg[it].x; g[1] = pg[it].y; g[2] = pg[it].z; g[3] = pg[it].w; }
            }
            if (in_tile) {
                Gp::unpack(ld_group(sQ[nb] + t * LDK + cc), q);
                Gp::unpack(ld_group(sK + t * LDK + cc), k);
            }
            float run[4] = {g[0], g[1], g[2], g[3]}, rinv[4];
            row_scan_mul4(run);   // R_t = prod_{16I <= s <= t} g_s
#pragma unroll
            for (int i = 0; i < 4; ++i) rinv[i] = __builtin_amdgcn_rcpf(run[i]);
            // strong decay in these channels (a block product below
            // kGlaWeakBlock): k~ from exclusive suffix products of the gates
            // (never above 1) and exact diagonal tiles for the chunk
            const bool weak = __builtin_amdgcn_ballot_w64(run[0] < kGlaWeakBlock || run[1] < kGlaWeakBlock ||
                                                          run[2] < kGlaWeakBlock || run[3] < kGlaWeakBlock) != 0;
            float sx[4] = {g[0], g[1], g[2], g[3]};
            if (weak) {
                row_suffix_mul4(sx);
#pragma unroll
                for (int i = 0; i < 4; ++i) sx[i] = row_next_or_one(sx[i]);
                if (lane == 0) sWeak = 1;
            }
            {
                // per-chunk factors, from a scan across the block ends: after
                // two DPP row broadcasts lane t holds P_t = prod_{s <= t} g_s, so
                // E_J = P at lane 16J - 1 (J >= 1; E_0 = 1 is never read), D = P at
                // lane 63, and rho_{J1 J0} (blocks strictly between) is the block
                // total of lane 31 or 47, or their product.  Each value is written
                // by the lane that holds it.
                float pre[4] = {run[0], run[1], run[2], run[3]};
                wave_prefix_from_rows4(run, pre);
                if ((lane & 15) == 15 && (lane >> 4) < NB) {
                    const int J = lane >> 4;   // E_{J+1} for J < NB - 1, D for the last block
                    *reinterpret_cast<float4 *>(sE + (J + 1) * DK + cc) = make_float4(pre[0], pre[1], pre[2], pre[3]);
                    // the block's total, for every token of the chunk below
                    *reinterpret_cast<float4 *>(sTot + J * DK + cc) = make_float4(run[0], run[1], run[2], run[3]);
                }
                if constexpr (NB == 4) {
                    // rho_{2,0} = tot_1 (lane 31), rho_{3,1} = tot_2 and rho_{3,0} = tot_1 tot_2 (lane 47)
                    if (lane == 31)
                        *reinterpret_cast<float4 *>(sRho + rho_index(2, 0) * DK + cc) = make_float4(run[0], run[1], run[2], run[3]);
                    float t12[4] = {run[0], run[1], run[2], run[3]};   // row 2: tot_1 (lane 31) times the row's products
                    mul_bcast15_row2_4(run, t12);
                    if (lane == 47) {
                        *reinterpret_cast<float4 *>(sRho + rho_index(3, 1) * DK + cc) = make_float4(run[0], run[1], run[2], run[3]);
                        *reinterpret_cast<float4 *>(sRho + rho_index(3, 0) * DK + cc) = make_float4(t12[0], t12[1], t12[2], t12[3]);
                    }
                }
            }
            // the total of the token's own block and the product of the totals
            // of the blocks after it, read back from the slots the block-end
            // lanes just wrote.  The wave executes its LDS operations in
            // order; the empty asm keeps the compiler from moving these reads
            // (of values other lanes wrote) above those writes.
            asm volatile("" ::: "memory");
            float tb[4], after[4];
            {
                const float4 b = *reinterpret_cast<const float4 *>(sTot + I * DK + cc);
                tb[0] = b.x; tb[1] = b.y; tb[2] = b.z; tb[3] = b.w;
                after[0] = after[1] = after[2] = after[3] = 1.f;
#pragma unroll
                for (int m = 1; m < NB; ++m) {
                    const float4 a = *reinterpret_cast<const float4 *>(sTot + (I + m) * DK + cc);
                    after[0] *= a.x; after[1] *= a.y; after[2] *= a.z; after[3] *= a.w;
                }
            }
            float fq[4], fd[4], fk[4], fa[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // tokens past the end: zero operands (selects, not branches)
                const float rq = on ? run[i] : 0.f, rk = on && !weak ? rinv[i] : 0.f;
                fq[i] = apply_phi<PHI>(q[i]) * rq;
                fd[i] = apply_phi<PHI>(k[i]) * rk;
                fk[i] = weak ? apply_phi<PHI>(k[i]) * (on ? sx[i] : 0.f) : fd[i] * tb[i];
                fa[i] = fk[i] * after[i];
            }
            if (in_tile) {
                st_group(sQ[nb] + t * LDK + cc, Gp::make(fq[0], fq[1], fq[2], fq[3]));
                st_group(sKd + t * LDK + cc, Gp::make(fd[0], fd[1], fd[2], fd[3]));
                st_group(sK + t * LDK + cc, Gp::make(fk[0], fk[1], fk[2], fk[3]));
                st_group(sKt + t * LDK + cc, Gp::make(fa[0], fa[1], fa[2], fa[3]));
            }
        }
    };
    auto gate_pass = [&](int c) {
        if (c + 1 >= nchunks) return;
        if (rows(c + 1) == C) gate_pass_n(c, std::true_type{});
        else gate_pass_n(c, std::false_type{});
    };
    // step C, every wave: the scores of chunk c+1 (16x16 tiles, taken
    // transposed so that a lane writes four consecutive columns of a row)
    auto scores = [&](int c) {
        if (c + 1 >= nchunks) return;
        const int nb = (c + 1) & 1;
        const bool weak = __builtin_amdgcn_readfirstlane(sWeak) != 0;
        auto score_tile = [&](int tt) {   // tile (I, J) = (tt / NB, tt % NB)
            const int I = tt / NB, J = tt % NB;
            const int t = 16 * I + lr, j0 = 16 * J + 4 * lg;
            if (J > I) {
                st_group(sP + t * LDC + j0, Gp::make(0.f, 0.f, 0.f, 0.f));
                return;
            }
            if (J == I && weak) {
                const size_t o = static_cast<size_t>((c + 1) * C) * DK;
                gla_diag_exact<PHI, IO, DK>(qh + o, kh + o, gh + o, rows(c + 1), I, sP + 16 * I * LDC + 16 * I, LDC, lane);
                return;
            }
            f32x4 acc = zero4();
            if (J == I)
                tile_mma_ll<DK>(acc, sKd + 16 * J * LDK, LDK, sQ[nb] + 16 * I * LDK, LDK, lane);
            else if (J == I - 1)
                tile_mma_ll<DK>(acc, sK + 16 * J * LDK, LDK, sQ[nb] + 16 * I * LDK, LDK, lane);
            else
                tile_mma_ll_scaled<DK>(acc, sK + 16 * J * LDK, LDK, sRho + rho_index(I, J) * DK,
                                       sQ[nb] + 16 * I * LDK, LDK, lane);
            st_group(sP + t * LDC + j0, Gp::make(j0 <= t ? acc[0] : 0.f, j0 + 1 <= t ? acc[1] : 0.f,
                                                 j0 + 2 <= t ? acc[2] : 0.f, j0 + 3 <= t ? acc[3] : 0.f));
        };
        if constexpr (NB == 4 && NW == 8) {
            // two tiles per wave (tile ids 4 I + J, a nibble each): the three
            // rho-scaled tiles alone on the state waves (with a zero tile),
            // the other helpers two plain products or one and a zero tile
            // (order 8,1 | 12,2 | 13,3 | 15,6 | 0,4 | 5,9 | 10,7 | 14,11)
            constexpr unsigned long long kOrder = 0xbe7a95406f3d2c18ull;
            score_tile(static_cast<int>((kOrder >> (8 * wave)) & 15));
            score_tile(static_cast<int>((kOrder >> (8 * wave + 4)) & 15));
        } else if constexpr (NB == 4 && NW == 12) {
            // one tile per wave, the rho-scaled ones alone on waves 0-2; waves
            // 3-6 also take a zero tile (second entry 15: none; tile 15 is only
            // ever a first entry)
            constexpr unsigned long long kFirst = 0xb7e94fa50dc8ull, kSecond = 0xfffff6321fffull;
            score_tile(static_cast<int>((kFirst >> (4 * wave)) & 15));
            const int t2 = static_cast<int>((kSecond >> (4 * wave)) & 15);
            if (t2 != 15) score_tile(t2);
        } else {
            for (int tt = wave; tt < NB * NB; tt += NW) score_tile(tt);
        }
    };

    // The two roles run loops of their own with the same three barriers per
    // chunk, so that each role's registers are allocated for its own work (in
    // one loop the staged q, k, v registers were copied at the end of step A,
    // which waited for the loads just issued).
    if (state_wave) {
        for (int c = -1; c < nchunks && nchunks > 0; ++c) {
            const int cur = c & 1;
            // ---- step A: the outputs of chunk c (to registers) and its state update
            if (c >= 0) {
                G4 sb[NCB];
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) sb[cb] = Gp::make(st[cb]);
                // O^T = (Qhat E_I) S0^T + V^T P^T for the NB token blocks I at once
                // (lane: values 16*wave + 4*lg..+3 of token 16 I + lr): each step
                // issues NB independent products, and the V^T operand groups,
                // the same for every block, are read once.  Each accumulator
                // sums in the order of the single-block form.
#pragma unroll
                for (int I = 0; I < NB; ++I) ob[I] = zero4();
                {
                    const int ko = 4 * lg;
                    const Op *qr = sQ[cur] + lr * LDK + ko;
#pragma unroll
                    for (int s2 = 0; s2 + 2 <= NCB; s2 += 2) {
#pragma unroll
                        for (int I = 0; I < NB; ++I) {
                            const Op *q = qr + 16 * I * LDK + 16 * s2;
                            if (I == 0)
                                mma32(ob[I], sb[s2], sb[s2 + 1], ld_group(q), ld_group(q + 16));
                            else
                                mma32(ob[I], sb[s2], sb[s2 + 1], scaled_group(q, sE + I * DK + 16 * s2 + ko),
                                      scaled_group(q + 16, sE + I * DK + 16 * s2 + 16 + ko));
                        }
                    }
                    if constexpr (NCB % 2 == 1) {
#pragma unroll
                        for (int I = 0; I < NB; ++I) {
                            const Op *q = qr + 16 * I * LDK + 16 * (NCB - 1);
                            if (I == 0) mma16(ob[I], sb[NCB - 1], ld_group(q));
                            else mma16(ob[I], sb[NCB - 1], scaled_group(q, sE + I * DK + 16 * (NCB - 1) + ko));
                        }
                    }
#pragma unroll
                    for (int t0 = 0; t0 + 32 <= C; t0 += 32) {
                        const G4 va = kt_group<0>(sV[cur], LDV, t0, 16 * wave, lane);
                        const G4 vb2 = kt_group<0>(sV[cur], LDV, t0 + 16, 16 * wave, lane);
#pragma unroll
                        for (int I = 0; I < NB; ++I) {
                            const Op *prow = sP + (16 * I + lr) * LDC + 4 * lg;
                            mma32(ob[I], va, vb2, ld_group(prow + t0), ld_group(prow + t0 + 16));
                        }
                    }
                    if constexpr (C % 32 == 16) {
                        const G4 va = kt_group<0>(sV[cur], LDV, C - 16, 16 * wave, lane);
#pragma unroll
                        for (int I = 0; I < NB; ++I)
                            mma16(ob[I], va, ld_group(sP + (16 * I + lr) * LDC + 4 * lg + C - 16));
                    }
                }
                // S^T <- S^T diag(D) + K~a^T V, both operands by transposing reads
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) st[cb][i] *= sD[16 * cb + 4 * lg + i];
#pragma unroll
                    for (int s2 = 0; s2 + 2 <= NB; s2 += 2)
                        mma32(st[cb], kt_group<0>(sKt, LDK, 16 * s2, 16 * cb, lane),
                              kt_group<0>(sKt, LDK, 16 * s2 + 16, 16 * cb, lane),
                              kt_group<0>(sV[cur], LDV, 16 * s2, 16 * wave, lane),
                              kt_group<0>(sV[cur], LDV, 16 * s2 + 16, 16 * wave, lane));
                    if constexpr (NB % 2 == 1)
                        mma16(st[cb], kt_group<0>(sKt, LDK, 16 * (NB - 1), 16 * cb, lane),
                              kt_group<0>(sV[cur], LDV, 16 * (NB - 1), 16 * wave, lane));
                }
            }
            __syncthreads();
            // ---- step B: the gate factors of chunk c+1, then chunk c's outputs
            gate_pass(c);
            if (c >= 0) {
                const int n = rows(c);
#pragma unroll
                for (int I = 0; I < NB; ++I) {
                    const int t = 16 * I + lr;
                    if (t < n)
                        st_group(oh + static_cast<size_t>(c * C + t) * p.d_v + vb * DVB + 16 * wave + 4 * lg, Gp::make(ob[I]));
                }
            }
            if constexpr (!GDMA) load_gates(min(c + 2, clast));
            __syncthreads();
            // ---- step C
            scores(c);
            __syncthreads();
        }
    } else {
        for (int c = -1; c < nchunks && nchunks > 0; ++c) {
            const int nb = (c + 1) & 1;
            const bool prep = c + 1 < nchunks;   // chunk c+1 is prepared
            // ---- step A: commit chunk c+1, load its gate tile and chunk c+2's q, k, v
            // committed on every chunk (after the last one into buffers that
            // nothing reads any more), so that every path through the loop
            // consumes the staged registers and the compiler's waits for them
            // stay exact
            pq.store(sQ[nb], LDK, htid);
            pk.store(sK, LDK, htid);
            pv.store(sV[nb], LDV, htid);
            if (htid == 0) sWeak = 0;   // last read in the previous step C
            // GDMA: chunk c+1's gate tile (sG was last read in the previous
            // step B), issued after the stores above, whose waits for the
            // staged registers would otherwise cover these loads too
            if constexpr (GDMA) {
                if (prep) dma_gates(c + 1);
            }
            load_qkv(min(c + 2, clast));
            // GDMA: the gate tile has landed before the barrier; only the q, k,
            // v loads issued after it stay in flight
            if constexpr (GDMA) __builtin_amdgcn_s_waitcnt(wait_vmcnt(pq.PER + pk.PER + pv.PER));
            __syncthreads();
            // ---- step B
            gate_pass(c);
            if constexpr (!GDMA) load_gates(min(c + 2, clast));
            __syncthreads();
            // ---- step C
            scores(c);
            __syncthreads();
        }
    }

    if (p.S_T && state_wave) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            *reinterpret_cast<float4 *>(p.S_T + srow + 16 * cb + 4 * lg) =
                make_float4(st[cb][0], st[cb][1], st[cb][2], st[cb][3]);
    }
}

// ------------------------------------------------------------------ segments
// Normalized and retention variants: their state is a plain sum over the
// tokens (S_C = S0 + V^T phiK, z_C = z0 + phiK^T 1; with a fixed decay each
// term decayed to the end), so the sequence can be cut into segments that run
// concurrently, each entering with the initial state plus the increments of
// the segments before it, decayed by gamma^L per whole segment of L tokens
// in between.  la_segment_state_kernel fills the slots of
// ChunkParams::seg_state: slot 0 of a head is (S0, z0) (zeros when absent),
// slot s >= 1 the increment of segment s - 1,
//   dS = sum_t gamma^(L_s-1-t) v_t phi(k_t)^T,   dz = sum_t gamma^(L_s-1-t) phi(k_t),
// over that segment's L_s tokens t, with the scaled phi(k_t) rounded to the
// operand type before both sums.  Copying S0 here also lets S_T alias S0:
// every read of S0 is done before the chunk kernel starts.  One workgroup per
// (head, slot, DVA-channel value block), four waves; the (value, key) 16x16
// tiles of the block are dealt to the waves round robin.
template <int PHI, class DT, int DK, int DVA, int C>
__global__ void __launch_bounds__(256) la_segment_state_kernel(const ChunkParams p, float *ws) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef Group<Op> Gp;
    constexpr int NKT = DK / 16;
    constexpr int NTILE = (DVA / 16) * NKT;
    constexpr int NT = (NTILE + 3) / 4;          // tiles per wave
    constexpr int PAD = 16 / sizeof(Op);
    constexpr int LDK = DK + PAD, LDV = DVA + PAD;
    __shared__ __align__(16) Op sK[C * LDK];       // phi(K), rows = tokens
    __shared__ __align__(16) Op sV[C * LDV];       // this block's value channels
    __shared__ float sZp[256 * 8];                  // per-thread partial dz, reduced at the end
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int nvb = p.d_v / DVA;
    const int vb = blockIdx.x % nvb, s = (blockIdx.x / nvb) % p.n_seg, bh = blockIdx.x / (nvb * p.n_seg);
    const size_t slot = static_cast<size_t>(p.d_v) * DK + DK;
    float *dst = ws + (static_cast<size_t>(bh) * p.n_seg + s) * slot;
    if (s == 0) {
        for (int e = tid; e < DVA * DK; e += 256) {
            const size_t o = static_cast<size_t>(DVA * vb + e / DK) * DK + e % DK;
            dst[o] = p.S0 ? p.S0[static_cast<size_t>(bh) * p.d_v * DK + o] : 0.f;
        }
        if (vb == 0)
            for (int c = tid; c < DK; c += 256)
                dst[static_cast<size_t>(p.d_v) * DK + c] = p.z0 ? p.z0[static_cast<size_t>(bh) * DK + c] : 0.f;
        return;
    }
    const int tb = (s - 1) * p.seg_len;
    const int Tn = min(p.seg_len, p.T - tb);
    const float l2g = p.gate ? __builtin_amdgcn_logf(p.gate[bh % p.H]) : 0.f;   // fixed decay, 0 = none
    const IO *kh = static_cast<const IO *>(p.k) + (static_cast<size_t>(bh) * p.T + tb) * DK;
    const IO *vh = static_cast<const IO *>(p.v) + (static_cast<size_t>(bh) * p.T + tb) * p.d_v + DVA * vb;
    // the rows of the next two chunks are loaded into registers (two sets,
    // used alternately) while this one is used.  Every load is issued on
    // every path (offsets past the end re-read the last chunk, which a
    // chunk past the end then commits as zeros), so that the compiler's wait
    // for one set never covers the other.
    const int clast = ((Tn - 1) / C) * C;
    TilePrefetch<C, DK, 256, IO> pk[2];
    TilePrefetch<C, DVA, 256, IO> pv[2];
    auto prefetch = [&](int c0, TilePrefetch<C, DK, 256, IO> &k, TilePrefetch<C, DVA, 256, IO> &v) {
        const int n = min(C, Tn - c0);
        k.load(kh + static_cast<size_t>(c0) * DK, DK, n, tid);
        v.load(vh + static_cast<size_t>(c0) * p.d_v, p.d_v, n, tid);
    };
    // one staged 16-byte vector as floats (8 bf16 or 4 f32)
    auto unpack = [](const uint4 &w, float (&x)[8]) {
        if constexpr (sizeof(IO) == 2) {
            x[0] = lo_bf16(w.x); x[1] = hi_bf16(w.x); x[2] = lo_bf16(w.y); x[3] = hi_bf16(w.y);
            x[4] = lo_bf16(w.z); x[5] = hi_bf16(w.z); x[6] = lo_bf16(w.w); x[7] = hi_bf16(w.w);
        } else {
            x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y); x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
        }
    };
    f32x4 acc[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) acc[i] = zero4();
    // dz: each thread sums phi(K) over the rows it commits, for the same
    // VE channels in every chunk (256 is a multiple of the vectors per row)
    float zp[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    auto chunk = [&](int c0, TilePrefetch<C, DK, 256, IO> &k, TilePrefetch<C, DVA, 256, IO> &v) {
        const int n = min(C, Tn - c0);   // <= 0 past the end
        // phi(K) and V rows of the chunk; rows past the segment end are zero
#pragma unroll
        for (int i = 0; i < k.PER; ++i) {
            const int e = tid + i * 256;
            if (k.TOTAL % 256 != 0 && e >= k.TOTAL) continue;
            const int t = e / k.VPR, c = (e % k.VPR) * k.VE;
            const bool ok = ((k.valid >> i) & 1u) && t < n;
            // token c0 + t decays over the Tn - 1 - (c0 + t) tokens after it
            const float w = l2g != 0.f ? __builtin_amdgcn_exp2f(static_cast<float>(Tn - 1 - c0 - t) * l2g) : 1.f;
            float x[8];
            unpack(k.r[i], x);
#pragma unroll
            for (int j = 0; j < k.VE; ++j) x[j] = ok ? apply_phi<PHI>(x[j]) * w : 0.f;
#pragma unroll
            for (int j = 0; j < k.VE; j += 4) {
                const typename Gp::type g = Gp::make(x[j], x[j + 1], x[j + 2], x[j + 3]);
                st_group(sK + t * LDK + c + j, g);
                float r[4];
                Gp::unpack(g, r);   // the rounded values the products use
#pragma unroll
                for (int u = 0; u < 4; ++u) zp[j + u] += r[u];
            }
        }
#pragma unroll
        for (int i = 0; i < v.PER; ++i) {
            const int e = tid + i * 256;
            if (v.TOTAL % 256 != 0 && e >= v.TOTAL) continue;
            const int t = e / v.VPR, c = (e % v.VPR) * v.VE;
            const bool ok = ((v.valid >> i) & 1u) && t < n;
            float x[8];
            unpack(v.r[i], x);
#pragma unroll
            for (int j = 0; j < v.VE; j += 4)
                st_group(sV + t * LDV + c + j, Gp::make(ok ? x[j] : 0.f, ok ? x[j + 1] : 0.f, ok ? x[j + 2] : 0.f, ok ? x[j + 3] : 0.f));
        }
        __syncthreads();
        prefetch(min(c0 + 2 * C, clast), k, v);
        // dS tiles (value tile vt x key tile kt): both operands by transposing
        // reads of the token-major tiles (contraction over the tokens)
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int tile = wave + 4 * i, vt = tile / NKT, kt = tile % NKT;
            if (tile < NTILE) {
#pragma unroll
                for (int t0 = 0; t0 + 32 <= C; t0 += 32)
                    mma32(acc[i], kt_group<0>(sV, LDV, t0, 16 * vt, lane), kt_group<0>(sV, LDV, t0 + 16, 16 * vt, lane),
                          kt_group<0>(sK, LDK, t0, 16 * kt, lane), kt_group<0>(sK, LDK, t0 + 16, 16 * kt, lane));
                if constexpr (C % 32 == 16)
                    mma16(acc[i], kt_group<0>(sV, LDV, C - 16, 16 * vt, lane), kt_group<0>(sK, LDK, C - 16, 16 * kt, lane));
            }
        }
        __syncthreads();
    };
    prefetch(0, pk[0], pv[0]);
    prefetch(min(C, clast), pk[1], pv[1]);
    for (int c0 = 0; c0 < Tn; c0 += 2 * C) {
        chunk(c0, pk[0], pv[0]);
        chunk(c0 + C, pk[1], pv[1]);
    }
#pragma unroll
    for (int i = 0; i < NT; ++i) {
        const int tile = wave + 4 * i, vt = tile / NKT, kt = tile % NKT;
        if (tile < NTILE) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                dst[static_cast<size_t>(DVA * vb + 16 * vt + 4 * lg + r) * DK + 16 * kt + lr] = acc[i][r];
        }
    }
    if (vb == 0) {
        // dz[c]: the partials of the threads that committed channel c, in thread order
        constexpr int VPR = DK / (16 / (int)sizeof(IO)), VE = 16 / (int)sizeof(IO);
#pragma unroll
        for (int j = 0; j < VE; ++j) sZp[j * 256 + tid] = zp[j];
        __syncthreads();
        if (tid < DK) {
            const int g = tid / VE, j = tid % VE;   // threads g, g + VPR, ... hold channel tid
            float z = 0.f;
            for (int th = g; th < 256; th += VPR) z += sZp[j * 256 + th];
            dst[static_cast<size_t>(p.d_v) * DK + tid] = z;
        }
    }
}

// ------------------------------------------------------------------ dispatch

constexpr int kLinearWaves = 8;   // waves per workgroup
constexpr int kGlaWaves = 12;     // waves per workgroup of the pipelined gated kernel (three per SIMD)

constexpr int kComputeUnits = 256;

// Work split of the normalized variant: its state is a plain sum over the
// tokens, so a sequence can run as concurrent segments.  When the heads (with
// value blocks of up to 64 channels, the fewest duplicated state-independent
// passes) give fewer workgroups than compute units, the sequence is cut into
// enough segments for about one workgroup per unit, each at least two chunks
// long (chunks are at least 16 tokens).  max_segments bounds the count for
// any chunk length; it sizes the workspace.
static int64_t linear_max_segments(const ChunkArgs &a) {
    if ((a.variant != LA_NORMALIZED && a.variant != LA_RETENTION) || a.T <= 0) return 1;
    const int64_t wgs = static_cast<int64_t>(a.B) * a.H * (a.d_v / std::min(a.d_v, 64));
    if (wgs <= 0 || wgs >= kComputeUnits) return 1;
    return std::max<int64_t>(1, std::min<int64_t>((kComputeUnits + wgs - 1) / wgs, (a.T + 15) / 16 / 2));
}
static int linear_segment_chunks(const ChunkArgs &a, int C) {   // chunks per segment
    const int nchunks = (a.T + C - 1) / C;
    const int64_t n = std::min<int64_t>(linear_max_segments(a), nchunks / 2);
    return n < 2 ? nchunks : static_cast<int>((nchunks + n - 1) / n);
}

// Value-block width: with segments, up to 64 channels; otherwise the widest
// block that still gives about one workgroup per compute unit.
static int linear_value_block(const ChunkArgs &a) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    const int nchunks = (a.T + a.chunk - 1) / a.chunk;
    if (linear_segment_chunks(a, a.chunk) < nchunks) return std::min(a.d_v, 64);
    if (a.d_v >= 64 && heads * (a.d_v / 64) >= kComputeUnits) return 64;
    if (a.d_v >= 32 && heads * (a.d_v / 32) >= kComputeUnits) return 32;
    return 16;
}

template <bool GATED, int PHI, class DT, int DK, int DVB, int C>
static hipError_t launch_linear_t(const ChunkArgs &a) {
    ChunkParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate; p.beta = nullptr; p.S0 = a.S0; p.z0 = a.z0;
    p.out = a.out; p.S_T = a.S_T; p.z_T = a.z_T;
    p.T = a.T; p.d_v = a.d_v; p.n_vblk = a.d_v / DVB; p.n_heads = a.B * a.H;
    p.H = a.H;
    p.normalize = a.variant == LA_NORMALIZED;
    if constexpr (!GATED) {
        const int per = linear_segment_chunks(a, C);
        const int nchunks = (a.T + C - 1) / C;
        if (a.T > 0 && per < nchunks) {
            p.seg_len = per * C;
            p.n_seg = (nchunks + per - 1) / per;
            p.seg_state = static_cast<const float *>(a.workspace);
            const int64_t sblocks = static_cast<int64_t>(p.n_heads) * p.n_seg * (a.d_v / DVB);
            hipLaunchKernelGGL((la_segment_state_kernel<PHI, DT, DK, DVB, C>), dim3(static_cast<uint32_t>(sblocks)), dim3(256), 0,
                               a.stream, p, static_cast<float *>(a.workspace));
        } else if (p.normalize && a.T > 0 && p.n_vblk > 1 && a.z0 && a.z_T == a.z0) {
            // one pass, several value blocks per head, z_T in place of z0: every
            // value block's workgroup reads z0 but only block 0 writes z_T, and a
            // workgroup may start after block 0 has finished, so the blocks read
            // a copy of z0 staged in the workspace
            const size_t zbytes = static_cast<size_t>(p.n_heads) * a.d_k * sizeof(float);
            hipError_t e = hipMemcpyAsync(a.workspace, a.z0, zbytes, hipMemcpyDeviceToDevice, a.stream);
            if (e != hipSuccess) return e;
            p.z0 = static_cast<const float *>(a.workspace);
        }
    }
    const int64_t blocks = static_cast<int64_t>(p.n_heads) * p.n_vblk * p.n_seg;
    if constexpr (GATED && GlaLds<DT, DK, DVB, C, kGlaWaves>::FITS) {
        hipLaunchKernelGGL((gla_pipelined_kernel<PHI, DT, DK, DVB, C, kGlaWaves>), dim3(static_cast<uint32_t>(blocks)),
                           dim3(kGlaWaves * 64), 0, a.stream, p);
    } else {
        hipLaunchKernelGGL((linear_chunk_kernel<GATED, PHI, DT, DK, DVB, C, kLinearWaves>),
                           dim3(static_cast<uint32_t>(blocks)), dim3(kLinearWaves * 64), 0, a.stream, p);
    }
    return hipGetLastError();
}

// Largest chunk <= the requested one whose LDS tiles fit (the result does not
// depend on the chunk length).
template <bool GATED, class DT, int DK, int DVB, int C>
constexpr int fit_chunk() {
    if constexpr (C > 16 && LinearLds<GATED, DT, DK, DVB, C>::BYTES > 160 * 1024) return fit_chunk<GATED, DT, DK, DVB, C / 2>();
    else return C;
}

template <bool GATED, int PHI, class DT, int DK, int DVB>
static hipError_t linear_chunk(const ChunkArgs &a) {
    switch (a.chunk) {
        case 16: return launch_linear_t<GATED, PHI, DT, DK, DVB, 16>(a);
        case 32: return launch_linear_t<GATED, PHI, DT, DK, DVB, fit_chunk<GATED, DT, DK, DVB, 32>()>(a);
        case 64: return launch_linear_t<GATED, PHI, DT, DK, DVB, fit_chunk<GATED, DT, DK, DVB, 64>()>(a);
        // 128-token tiles of these kernels exceed the LDS of a compute unit;
        // the result does not depend on the chunk length
        case 128: return launch_linear_t<GATED, PHI, DT, DK, DVB, fit_chunk<GATED, DT, DK, DVB, 64>()>(a);
    }
    return hipErrorInvalidValue;
}

template <bool GATED, int PHI, class DT, int DK>
static hipError_t linear_dvb(const ChunkArgs &a) {
    switch (linear_value_block(a)) {
        case 64: return linear_chunk<GATED, PHI, DT, DK, 64>(a);
        case 32: return linear_chunk<GATED, PHI, DT, DK, 32>(a);
    }
    return linear_chunk<GATED, PHI, DT, DK, 16>(a);
}

template <bool GATED, int PHI, class DT>
static hipError_t linear_dk(const ChunkArgs &a) {
    switch (a.d_k) {
        case 16: return linear_dvb<GATED, PHI, DT, 16>(a);
        case 32: return linear_dvb<GATED, PHI, DT, 32>(a);
        case 64: return linear_dvb<GATED, PHI, DT, 64>(a);
        case 128: return linear_dvb<GATED, PHI, DT, 128>(a);
    }
    return hipErrorInvalidValue;
}

template <class DT>
static hipError_t linear_variant(const ChunkArgs &a) {
    // normalized and retention share the ungated kernels (the normalizer is a
    // runtime switch; the normalized variant always uses elu+1)
    if (a.variant == LA_NORMALIZED || (a.variant == LA_RETENTION && a.phi == LA_PHI_ELU1))
        return linear_dk<false, LA_PHI_ELU1, DT>(a);
    if (a.variant == LA_RETENTION) return linear_dk<false, LA_PHI_IDENTITY, DT>(a);
    if (a.phi == LA_PHI_ELU1) return linear_dk<true, LA_PHI_ELU1, DT>(a);
    return linear_dk<true, LA_PHI_IDENTITY, DT>(a);
}

// Workspace of the chunked forward: the segment slots of the normalized
// variant (none for the other variants).
size_t chunk_workspace_bytes(const ChunkArgs &a) {
    if (a.variant == LA_KDA) return kda_workspace_bytes(a);
    int seg_len, n_seg;
    if (seg_plan(a, seg_len, n_seg)) return seg_workspace_bytes(a);
    if ((a.variant != LA_NORMALIZED && a.variant != LA_RETENTION) || a.T <= 0) return 0;
    const int64_t n = linear_max_segments(a);
    const size_t heads = static_cast<size_t>(a.B) * a.H;
    // segment slots, or (normalized, one pass) a staged copy of z0 for z_T aliasing it
    const size_t zstage = a.variant == LA_NORMALIZED ? heads * a.d_k * sizeof(float) : 0;
    if (n < 2) return zstage;
    return std::max(zstage, heads * n * (static_cast<size_t>(a.d_v) * a.d_k + a.d_k) * sizeof(float));
}

hipError_t launch_chunk_linear(const ChunkArgs &a) {
    int seg_len, n_seg;
    if (seg_plan(a, seg_len, n_seg)) return launch_seg(a);
    if (a.dtype == LA_BF16) return linear_variant<BF16>(a);
    return linear_variant<F32>(a);
}

}  // namespace la
