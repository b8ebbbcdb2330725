// la_chunk_linear.hip -- chunked forward of normalized and gated linear
// attention (gfx950).
//
// Normalized (page "Beyond -- Linear attention and recurrent memory",
// section "The big idea"; page "Ch. 11 Linear attention and Hyena", 11.2):
// with phi = elu+1 and a chunk of C tokens entering with (S0, z0),
//   P   = M o (phiQ phiK^T)                       (M: j <= t, a token sees itself)
//   O   = (phiQ S0^T + P V) / (phiQ z0 + P 1)
//   S_C = S0 + V^T phiK,   z_C = z0 + phiK^T 1.
// The denominator uses the same rounded P as the numerator.
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
    static constexpr int P_BYTES = C * LDC * (int)sizeof(Op);
    static constexpr int G_BYTES = GATED ? C * LDG * 4 : 0;
    static constexpr int PG_BYTES = P_BYTES > G_BYTES ? P_BYTES : G_BYTES;
    static constexpr int F_FLOATS = GATED ? (NB + 1 + NRHO) * DK : DK + C;
    static constexpr int KT_ELEMS = GATED ? C * LDK : DK * LDC;   // state-update key operand
    static constexpr int BYTES = (GATED ? 3 : 2) * C * LDK * (int)sizeof(Op) + KT_ELEMS * (int)sizeof(Op) +
                                 DVB * LDC * (int)sizeof(Op) + PG_BYTES + F_FLOATS * 4;
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
    constexpr int LDK = L::LDK, LDC = L::LDC, LDG = L::LDG;
    constexpr int VE = 16 / sizeof(IO);                   // elements per 16-byte vector
    static_assert(C <= 64 && C % 16 == 0 && DK % 16 == 0 && DVB % 16 == 0 && WS <= NW, "tiling");
    static_assert(L::BYTES <= 160 * 1024, "LDS budget");

    __shared__ __align__(16) Op sQ[C * LDK];                 // phi(Q) | Qhat
    __shared__ __align__(16) Op sK[C * LDK];                 // phi(K) | k~ (off-diagonal reference)
    __shared__ __align__(16) Op sKd[GATED ? C * LDK : 8];    // kd (diagonal reference)
    __shared__ __align__(16) Op sKt[L::KT_ELEMS];            // key operand of the state update:
                                                             // gated [t][c], normalized [c][t]
    __shared__ __align__(16) Op sVt[DVB * LDC];              // this block's values, [v][t]
    __shared__ __align__(16) unsigned char sPG[L::PG_BYTES]; // gates (f32), then P
    __shared__ __align__(16) float sF[L::F_FLOATS];
    Op *sP = reinterpret_cast<Op *>(sPG);
    float *sG = reinterpret_cast<float *>(sPG);
    float *sE = sF;                       // gated: prod of the chunk's gates before block I, [NB][DK]
    float *sD = sF + NB * DK;             // gated: prod of all the chunk's gates, [DK]
    float *sRho = sF + (NB + 1) * DK;     // gated: prod of the blocks strictly between J and I, [NRHO][DK]
    float *sZ = sF;                       // normalized: running z, [DK]
    float *sDen = sF + DK;                // normalized: denominators, [C]

    // the wave index is uniform: role branches compile to scalar branches
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    int bh, vb;
    block_to_head(blockIdx.x, p.n_heads, p.n_vblk, bh, vb);
    const int vloc = 16 * wave + lr;
    const int vch = vb * DVB + vloc;
    const size_t tok0 = static_cast<size_t>(bh) * p.T;
    const IO *qh = static_cast<const IO *>(p.q) + tok0 * DK;
    const IO *kh = static_cast<const IO *>(p.k) + tok0 * DK;
    const IO *vh = static_cast<const IO *>(p.v) + tok0 * p.d_v + vb * DVB;
    IO *oh = static_cast<IO *>(p.out) + tok0 * p.d_v;
    const float *gh = GATED ? p.gate + tok0 * DK : nullptr;

    f32x4 st[NCB];
    const size_t srow = (static_cast<size_t>(bh) * p.d_v + (wave < WS ? vch : 0)) * DK;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        st[cb] = zero4();
        if (p.S0 && wave < WS) {
            const float4 s = *reinterpret_cast<const float4 *>(p.S0 + srow + 16 * cb + 4 * lg);
            st[cb] = f32x4{s.x, s.y, s.z, s.w};
        }
    }
    if constexpr (!GATED) {
        for (int c = tid; c < DK; c += NTHR) sZ[c] = p.z0 ? p.z0[static_cast<size_t>(bh) * DK + c] : 0.f;
    }
    // the entering state is in registers before any tile load is issued, so
    // the loop never waits on the global-memory counter for it
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // chunk inputs staged one chunk ahead in registers
    TilePrefetch<C, DK, NTHR, IO> pq, pk;
    TilePrefetch<C, DVB, NTHR, IO> pv;
    TilePrefetch<C, GATED ? DK : 4, NTHR, float> pgt;
    auto prefetch = [&](int c0) {
        const int n = min(C, p.T - c0);
        pq.load(qh + static_cast<size_t>(c0) * DK, DK, n, tid);
        pk.load(kh + static_cast<size_t>(c0) * DK, DK, n, tid);
        pv.load(vh + static_cast<size_t>(c0) * p.d_v, p.d_v, n, tid);
        if constexpr (GATED) pgt.load(gh + static_cast<size_t>(c0) * DK, DK, n, tid);
    };
    if (p.T > 0) prefetch(0);

    // The state waves keep a chunk's outputs in registers and store them after
    // the next chunk's commit: the commit's wait on the global-memory counter
    // (for the staged loads) then never waits for just-issued output stores.
    f32x4 ob[NB];
    auto store_outputs = [&](int oc0) {
        const int on = min(C, p.T - oc0);
#pragma unroll
        for (int I = 0; I < NB; ++I) {
            const int t = 16 * I + lr;
            if (t < on) st_group(oh + static_cast<size_t>(oc0 + t) * p.d_v + vb * DVB + 16 * wave + 4 * lg, Gp::make(ob[I]));
        }
    };

    for (int c0 = 0; c0 < p.T; c0 += C) {
        const int n = min(C, p.T - c0);

        // ---- commit the staged chunk.  Values transposed; queries/keys raw
        // (gated) or with phi applied and keys also transposed (normalized);
        // gates as float32 with padded tokens set to 1 (no decay).
#pragma unroll
        for (int i = 0; i < pv.PER; ++i) {
            const int e = tid + i * NTHR;
            if (pv.TOTAL % NTHR != 0 && e >= pv.TOTAL) continue;
            const int t = e / pv.VPR, v = (e % pv.VPR) * VE;
            const uint4 w = pv.r[i];
            if constexpr (VE == 8) {
                const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sVt[(v + 2 * j) * LDC + t] = static_cast<bf16_t>(u[j] & 0xffffu);
                    sVt[(v + 2 * j + 1) * LDC + t] = static_cast<bf16_t>(u[j] >> 16);
                }
            } else {
                sVt[(v + 0) * LDC + t] = __uint_as_float(w.x);
                sVt[(v + 1) * LDC + t] = __uint_as_float(w.y);
                sVt[(v + 2) * LDC + t] = __uint_as_float(w.z);
                sVt[(v + 3) * LDC + t] = __uint_as_float(w.w);
            }
        }
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
#pragma unroll
                for (int j = 0; j < VE; ++j) {
                    const float fq = on ? apply_phi<PHI>(xq[j]) : 0.f;
                    const float fk = on ? apply_phi<PHI>(xk[j]) : 0.f;
                    from_f32(sQ[t * LDK + c + j], fq);
                    from_f32(sK[t * LDK + c + j], fk);
                    from_f32(sKt[(c + j) * LDC + t], fk);
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
        if (wave < WS && c0 > 0) store_outputs(c0 - C);
        if (c0 + C < p.T) prefetch(c0 + C);

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
                    fd[i] = on ? apply_phi<PHI>(k[i]) * rinv[i] : 0.f;
                    fk[i] = fd[i] * tb;
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
        for (int tt = wave; tt < NB * NB; tt += NW) {
            const int I = tt / NB, J = tt % NB;
            const int t = 16 * I + lr, j0 = 16 * J + 4 * lg;
            if (J > I) {
                st_group(sP + t * LDC + j0, Gp::make(0.f, 0.f, 0.f, 0.f));
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
            }
            st_group(sP + t * LDC + j0, Gp::make(j0 <= t ? acc[0] : 0.f, j0 + 1 <= t ? acc[1] : 0.f,
                                                 j0 + 2 <= t ? acc[2] : 0.f, j0 + 3 <= t ? acc[3] : 0.f));
        }
        __syncthreads();

        if constexpr (!GATED) {
            // ---- denominators phi(q_t).z0 + sum_j P_tj (the rounded P of the
            // numerator); 8 lanes per token
            for (int e = tid; e < 8 * C; e += NTHR) {
                const int t = e >> 3, part = e & 7;
                float d = 0.f;
                for (int c = part; c < DK; c += 8) d += to_f32(sQ[t * LDK + c]) * sZ[c];
                for (int j = part; j <= t; j += 8) d += to_f32(sP[t * LDC + j]);
                d = group_sum<8>(d);
                if (part == 0) sDen[t] = d;
            }
            __syncthreads();
            // z_C = z0 + phiK^T 1 (after every denominator has read z0)
            for (int c = tid; c < DK; c += NTHR) {
                float s = 0.f;
#pragma unroll 8
                for (int t = 0; t < C; ++t) s += to_f32(sKt[c * LDC + t]);
                sZ[c] += s;
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
                }
                tile_mma_ll<C>(o, sVt + 16 * wave * LDC, LDC, sP + 16 * I * LDC, LDC, lane);
                if constexpr (!GATED) {
                    const float inv = 1.f / sDen[16 * I + lr];
#pragma unroll
                    for (int i = 0; i < 4; ++i) o[i] *= inv;
                }
                ob[I] = o;
            }
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                if constexpr (GATED) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) st[cb][i] *= sD[16 * cb + 4 * lg + i];
                }
                if constexpr (GATED) {
                    // K^T from the natural-layout operand tile by transposing reads
                    const Op *vrow = sVt + (16 * wave + lr) * LDC + 4 * lg;
#pragma unroll
                    for (int s2 = 0; s2 + 2 <= NB; s2 += 2)
                        mma32(st[cb], kt_group<0>(sKt, LDK, 16 * s2, 16 * cb, lane),
                              kt_group<0>(sKt, LDK, 16 * s2 + 16, 16 * cb, lane), ld_group(vrow + 16 * s2),
                              ld_group(vrow + 16 * s2 + 16));
                    if constexpr (NB % 2 == 1)
                        mma16(st[cb], kt_group<0>(sKt, LDK, 16 * (NB - 1), 16 * cb, lane), ld_group(vrow + 16 * (NB - 1)));
                } else {
                    tile_mma_ll<C>(st[cb], sKt + 16 * cb * LDC, LDC, sVt + 16 * wave * LDC, LDC, lane);
                }
            }
        }
        __syncthreads();
    }

    if (wave < WS && p.T > 0) store_outputs(((p.T - 1) / C) * C);
    if (p.S_T && wave < WS) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            *reinterpret_cast<float4 *>(p.S_T + srow + 16 * cb + 4 * lg) =
                make_float4(st[cb][0], st[cb][1], st[cb][2], st[cb][3]);
    }
    if constexpr (!GATED) {
        if (p.z_T && vb == 0)
            for (int c = tid; c < DK; c += NTHR) p.z_T[static_cast<size_t>(bh) * DK + c] = sZ[c];
    }
}

// ------------------------------------------------------------------ dispatch

constexpr int kLinearWaves = 8;   // waves per workgroup

template <bool GATED, int PHI, class DT, int DK, int DVB, int C>
static hipError_t launch_linear_t(const ChunkArgs &a) {
    ChunkParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate; p.beta = nullptr; p.S0 = a.S0; p.z0 = a.z0;
    p.out = a.out; p.S_T = a.S_T; p.z_T = a.z_T;
    p.T = a.T; p.d_v = a.d_v; p.n_vblk = a.d_v / DVB; p.n_heads = a.B * a.H;
    const int64_t blocks = static_cast<int64_t>(p.n_heads) * p.n_vblk;
    hipLaunchKernelGGL((linear_chunk_kernel<GATED, PHI, DT, DK, DVB, C, kLinearWaves>),
                       dim3(static_cast<uint32_t>(blocks)), dim3(kLinearWaves * 64), 0, a.stream, p);
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
    }
    return hipErrorInvalidValue;
}

// Value-block width: the widest block (fewest duplicated state-independent
// passes per head) that still gives about one workgroup per compute unit.
constexpr int kComputeUnits = 256;

template <bool GATED, int PHI, class DT, int DK>
static hipError_t linear_dvb(const ChunkArgs &a) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    if (a.d_v >= 64 && heads * (a.d_v / 64) >= kComputeUnits) return linear_chunk<GATED, PHI, DT, DK, 64>(a);
    if (a.d_v >= 32 && heads * (a.d_v / 32) >= kComputeUnits) return linear_chunk<GATED, PHI, DT, DK, 32>(a);
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
    if (a.variant == LA_NORMALIZED) return linear_dk<false, LA_PHI_ELU1, DT>(a);
    if (a.phi == LA_PHI_ELU1) return linear_dk<true, LA_PHI_ELU1, DT>(a);
    return linear_dk<true, LA_PHI_IDENTITY, DT>(a);
}

hipError_t launch_chunk_linear(const ChunkArgs &a) {
    if (a.dtype == LA_BF16) return linear_variant<BF16>(a);
    return linear_variant<F32>(a);
}

}  // namespace la
