// la_chunk_gdr.hip -- chunked forward of the gated delta rule (gfx950).
//
// Recurrence (page "Linear Attention", gated-delta-rule formulation; page
// "Module 18 Beyond attention", section 18.2), state S is d_v x d_k:
//   S_t = g_t S_{t-1} + u_t k_t^T,  u_t = beta_t (v_t - g_t S_{t-1} k_t),
//   o_t = S_t q_t.
// Within a chunk of C tokens entering with state S0, let b_t be the
// chunk-local cumulative sum of log g and Gamma_tj = exp(b_t - b_j).
// Unrolling gives S_t = e^{b_t} S0 + sum_{j<=t} Gamma_tj u_j k_j^T, and
// substituting it into u_t turns the chunk's dependencies into one
// unit-lower-triangular system
//   (I + A) U = diag(beta) (V - diag(e^b) K S0^T),
//   A_tj = beta_t Gamma_tj (k_t . k_j)  for j < t,
// after which
//   O   = diag(e^b) Q S0^T + (M o Gamma o Q K^T) U        (M: j <= t)
//   S_C = e^{b_C} S0 + U^T diag(e^{b_C - b}) K.
// Every exponent used is <= 0 (the kernel keeps b in base 2 and evaluates
// each factor with one hardware exp2).  T = (I + A)^{-1} depends on K, g and beta
// only; it is formed per chunk from 16x16 blocks: each diagonal block from its
// 8x8 diagonal halves (forward substitution) and its lower-left 8x8
// -T_11 A_10 T_00, the off-diagonal blocks by
// T_ij = -T_ii sum_{j<=m<i} A_im T_mj, all in float32.
//
// Work decomposition: one workgroup per (b, h, block of DVB value channels);
// each wave owns 16 value channels and keeps its slice of the state
// (d_k x 16, transposed) in matrix-core accumulators for the whole sequence,
// so the state-dependent chain of a chunk (K S0^T, the solve's right-hand
// side, T Y, P U, the state update) runs from registers.  The
// state-independent work (Q K^T, K K^T, masks, the triangular inverse, the
// scaled K^T) is shared through LDS.
#include "la_chunk_common.hpp"

namespace la {

// LDS bytes of one workgroup of gdr_chunk_kernel<DT, DK, DVB, C>: Q, P and the
// gate values of two chunks, K of three, V and the inverse T of one, the
// float32 solve tile, and either the output staging tile or the published
// state and U^T.
// Layout of the Q and K tiles in LDS.  Two access patterns read them: row
// reads (16 rows x 16 bytes per half wave, the matrix-core A/B operands) and,
// for bfloat16 K, transposing reads (8 consecutive rows x 32 bytes per half
// wave).  bfloat16 rows are 288 bytes apart (32 bytes of padding) and the
// 16-byte column chunks of every row with bit 3 set are swapped in pairs
// (element column c is stored at c ^ 8): both patterns then touch each of the
// 64 four-byte banks once.  float32 tiles keep 16 bytes of padding and no swap.
template <class Op>
constexpr int gdr_kpad() { return sizeof(Op) == 2 ? 16 : 16 / (int)sizeof(Op); }
template <class Op>
constexpr int gdr_kswap() { return sizeof(Op) == 2 ? 8 : 0; }
__device__ __forceinline__ int swap_col(int row, int col, int sw) { return col ^ (sw * ((row >> 3) & 1)); }

// acc += X[0:16, 0:K] Y[0:16, 0:K]^T for two tiles in the Q/K layout above,
// each starting at a row that is a multiple of 16.
template <int K, int SW, class Op>
__device__ __forceinline__ void tile_mma_qk(f32x4 &acc, const Op *x, const Op *y, int ld, int lane) {
    const int off = (lane & 15) * ld + swap_col(lane & 15, 4 * (lane >> 4), SW);
    const Op *xr = x + off, *yr = y + off;
#pragma unroll
    for (int k = 0; k + 32 <= K; k += 32)
        mma32(acc, ld_group(xr + k), ld_group(xr + k + 16), ld_group(yr + k), ld_group(yr + k + 16));
    if constexpr (K % 32 == 16) mma16(acc, ld_group(xr + K - 16), ld_group(yr + K - 16));
}

// With bfloat16, 32- or 64-token chunks and 32-channel value blocks the
// outputs Q S0^T and P U are formed by helper waves from copies of the state
// and of U^T that the state waves publish in LDS (instead of an output tile).
template <class Op, int DVB, int C>
constexpr bool gdr_helper_outputs() { return sizeof(Op) == 2 && C % 32 == 0 && DVB == 32; }

// The state waves read their value channels of the V tile with transposing
// reads (four tokens of one channel per lane) when the tile is bfloat16 and
// 32 channels wide; its rows are then 96 bytes apart, so the eight rows of a
// half-wave read touch each bank once.
template <class Op, int DVB>
constexpr bool gdr_v_transposed() { return sizeof(Op) == 2 && DVB == 32; }
template <class Op, int DVB>
constexpr int gdr_ldv() { return gdr_v_transposed<Op, DVB>() ? DVB + 16 : DVB + 16 / (int)sizeof(Op); }

template <class DT, int DK, int DVB, int C>
constexpr int gdr_lds_bytes() {
    typedef typename OpOf<DT>::type Op;
    constexpr int PAD = 16 / sizeof(Op);
    constexpr int tail = gdr_helper_outputs<Op, DVB, C>() ? DVB * (DK + gdr_kpad<Op>()) + DVB * (C + PAD)
                                                          : C * (DVB + PAD);
    return (5 * C * (DK + gdr_kpad<Op>()) + 3 * C * (C + PAD) + C * gdr_ldv<Op, DVB>() + tail) * (int)sizeof(Op) +
           C * (C + 4) * 4 + 2 * (4 * C + 1) * 4;
}

template <class DT, int DK, int DVB, int C, int NW>
__global__ void __launch_bounds__(NW * 64) gdr_chunk_kernel(const ChunkParams p) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef Group<Op> Gp;
    typedef typename Gp::type G4;
    constexpr int WS = DVB / 16;         // state waves; wave w < WS owns value channels [16w, 16w + 16)
    constexpr int NHW = NW - WS;         // helper waves: the state-independent work of the next chunk
    constexpr int NTHR = NW * 64;
    constexpr int NB = C / 16;           // 16-token blocks per chunk
    constexpr int NCB = DK / 16;         // 16-channel key blocks
    constexpr int PAD = 16 / sizeof(Op);
    constexpr int LDK = DK + gdr_kpad<Op>();   // row strides (elements) of the LDS tiles
    constexpr int KSW = gdr_kswap<Op>();
    constexpr int LDC = C + PAD;
    constexpr int LDV = DVB + PAD;
    constexpr bool VTR = gdr_v_transposed<Op, DVB>();
    constexpr int LDVV = gdr_ldv<Op, DVB>();   // row stride of the V tile
    constexpr int LDA = C + 4;
    constexpr int VE = 16 / sizeof(Op);
    constexpr int NLOW = NB * (NB + 1) / 2;
    constexpr bool S32 = sizeof(Op) == 2 && C % 32 == 0;   // scores in 32x32 jobs
    constexpr int NJ32 = (C / 32) * (C / 32 + 1) / 2;   // score jobs: one per 32-block pair
    static_assert(!S32 || NJ32 <= NHW, "one helper wave per score job");
    constexpr bool HO = gdr_helper_outputs<Op, DVB, C>();   // outputs on helper waves
    constexpr int NJO = C / 32;                     // output jobs of 32 tokens (HO)
    constexpr int OJ0 = NHW - NJO;                  // helper index of the first output job
    constexpr int LDU = C + PAD;
    static_assert(!HO || OJ0 >= NB, "output jobs need helpers of their own in step 2");
    static_assert(C <= 64 && C % 16 == 0 && DK % 16 == 0 && DVB % 16 == 0 && NHW >= 1, "tiling");
    static_assert(gdr_lds_bytes<DT, DK, DVB, C>() <= 160 * 1024, "LDS budget");

    __shared__ __align__(16) Op sQ[2][C * LDK];
    __shared__ __align__(16) Op sK[3][C * LDK];    // chunk c in buffer c % 3
    __shared__ __align__(16) Op sV[C * LDVV];      // this block's value channels of chunk c (read in step 1)
    __shared__ __align__(16) Op sP[2][C * LDC];    // M o Gamma o Q K^T
    __shared__ __align__(16) Op sT[C * LDC];       // (I + A)^{-1}: chunk c+1's replaces chunk c's in step 3
    __shared__ __align__(16) Op sO[HO ? VE : C * LDV];     // output tile, staged for 16-byte stores
    __shared__ __align__(16) Op sS0[HO ? DVB * LDK : VE];  // entering state, rows = values (Q/K layout)
    __shared__ __align__(16) Op sUT[HO ? DVB * LDU : VE];  // U^T, rows = values
    __shared__ __align__(16) float sA[C * LDA];    // A, then the blocks of T, in float32 during the solve
    __shared__ __align__(16) float sB[2][C], sEB[2][C], sBeta[2][C], sEBC[2][C];
    __shared__ float sDecay[2];

    // the wave index is uniform: role branches compile to scalar branches
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const bool state_wave = wave < WS;
    const int hw = wave - WS;                      // helper index (valid when !state_wave)
    const int htid = tid - WS * 64;                // helper thread index
    int bh, vb;
    block_to_head(blockIdx.x, p.n_heads, p.n_vblk, bh, vb);
    const int vloc = 16 * wave + lr;               // value channel within the block (state waves)
    const int vch = vb * DVB + vloc;
    const size_t tok0 = static_cast<size_t>(bh) * p.T;
    const IO *qh = static_cast<const IO *>(p.q) + tok0 * DK;
    const IO *kh = static_cast<const IO *>(p.k) + tok0 * DK;
    const IO *vh = static_cast<const IO *>(p.v) + tok0 * p.d_v + vb * DVB;
    IO *oh = static_cast<IO *>(p.out) + tok0 * p.d_v;
    const float *gh = p.gate + tok0;
    const float *bth = p.beta + tok0;
    const int nchunks = (p.T + C - 1) / C;

    // state slice S^T[c][v] for c in key block cb, v = this lane's column (state waves)
    f32x4 st[NCB];
    const size_t srow = (static_cast<size_t>(bh) * p.d_v + (state_wave ? vch : 0)) * DK;
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        st[cb] = zero4();
        if (p.S0 && state_wave) {
            const float4 s4 = *reinterpret_cast<const float4 *>(p.S0 + srow + 16 * cb + 4 * lg);
            st[cb] = f32x4{s4.x, s4.y, s4.z, s4.w};
        }
    }
    // Wait for the entering state here, before any tile load is issued: the
    // compiler cannot tell that a wave keeps its role, so a state register still
    // pending at the loop entry would cost a full wait on the global-memory
    // counter (including the tile prefetch in flight) inside every chunk.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    // ---------------------------------------------------------------- stages
    // All waves stage the tiles, in step 3: register prefetch one chunk ahead,
    // then LDS (Q, K and the gate values two chunks ahead, V one chunk ahead).
    // K: with two or more state waves they stage it alone, at the end of step
    // 1, where they wait for the score jobs anyway (chunk c+2's K goes to the
    // buffer chunk c-1's used, free for the whole of chunk c)
    // bfloat16: they fill the K tile by direct global->LDS loads (no registers,
    // no LDS write instructions), in the layout above: 16-byte slot s of the
    // tile (LDK/8 slots a row, the last two padding) receives the column chunk
    // of its row that the swap puts there; rows past the end of the sequence
    // re-read its last row (their solve rows and columns carry beta = 0 and
    // their scores are masked).  The loads of chunk c+2 are issued in step 1
    // of chunk c and waited for before its last barrier.
    constexpr bool KSTATE = WS >= 2;
    constexpr int KRS = LDK * (int)sizeof(Op) / 16;   // 16-byte slots per K tile row
    constexpr int KNI = C * KRS / 64;                  // direct loads per K tile
    constexpr bool KDMA = KSTATE && sizeof(Op) == 2 && (C * KRS) % 64 == 0;
    constexpr int KTHR = KSTATE ? WS * 64 : NTHR;
    TilePrefetch<C, DK, NTHR, IO> pq;
    TilePrefetch<C, DK, KTHR, IO> pk;
    TilePrefetch<C, DVB, NTHR, IO> pv;
    // the gate scan runs on the last wave, which has no block column of the
    // off-diagonal inverse to work on
    constexpr int SCAN_WAVE = NW - 1;
    static_assert(NHW >= NB + 1 || NB == 1, "a helper wave must be free for the gate scan");
    // SCAN_WAVE, lane t: gate and beta of token t of the staged chunk (lanes past
    // its end read token 0; the scan treats them as g = 1, beta = 0)
    float pg = 1.f, pb = 0.f;
    auto rows = [&](int c) { return min(C, p.T - c * C); };
    auto load_q = [&](int c) {
        const int c0 = c * C, n = rows(c);
        pq.load(qh + static_cast<size_t>(c0) * DK, DK, n, tid);
        if (wave == SCAN_WAVE) {
            pg = gh[c0 + (lane < n ? lane : 0)];
            pb = bth[c0 + (lane < n ? lane : 0)];
        }
    };
    auto load_k = [&](int c) { pk.load(kh + static_cast<size_t>(c * C) * DK, DK, rows(c), tid); };   // KSTATE: state waves
    auto load_v = [&](int c) { pv.load(vh + static_cast<size_t>(c * C) * p.d_v, p.d_v, rows(c), tid); };
    auto store_q = [&](int buf) { pq.template store<KSW>(sQ[buf], LDK, tid); };
    auto store_k = [&](int kbuf) { pk.template store<KSW>(sK[kbuf], LDK, tid); };
    auto store_v = [&]() { pv.store(sV, LDVV, tid); };
    // a state wave issues the direct loads j = wave, wave + WS, ... of a tile;
    // for a whole chunk their per-lane byte offsets are the same in every
    // chunk, so they are formed once and each load moves only a scalar base
    constexpr int KPW = (KNI + WS - 1) / WS;
    uint32_t koff[KDMA ? KPW : 1];
    auto k_slot = [&](int j, int n) {   // element offset of slot 64 j + lane in a chunk of n rows
        const int slot = 64 * j + lane, row = slot / KRS, pc = slot % KRS;
        const int lc = pc < DK / 8 ? pc ^ (KSW / 8 * ((row >> 3) & 1)) : 0;
        return (row < n ? row : n - 1) * DK + 8 * lc;
    };
    if constexpr (KDMA) {
#pragma unroll
        for (int jj = 0; jj < KPW; ++jj) koff[jj] = k_slot(wave + WS * jj, C) * sizeof(IO);
    }
    auto dma_k = [&](int c, int kbuf) {   // KDMA, state waves
        const int n = rows(c);
        const IO *src0 = kh + static_cast<size_t>(c * C) * DK;
        const unsigned base = lds_addr(sK[kbuf]);
        if (n == C) {
#pragma unroll
            for (int jj = 0; jj < KPW; ++jj) {
                const int j = wave + WS * jj;
                if (KNI % WS != 0 && j >= KNI) break;
                lds_dma16(src0, koff[jj], __builtin_amdgcn_readfirstlane(base + 1024 * j));
            }
        } else {   // the last, partial chunk
#pragma unroll
            for (int jj = 0; jj < KPW; ++jj) {
                const int j = wave + WS * jj;
                if (KNI % WS != 0 && j >= KNI) break;
                lds_dma16(src0 + k_slot(j, n), __builtin_amdgcn_readfirstlane(base + 1024 * j));
            }
        }
    };
    // SCAN_WAVE: cumulative log2-gates of the staged chunk c into buffer `buf`
    // (b and every factor below in base 2: e^{b_t - b_j} = 2^{b2_t - b2_j})
    auto scan = [&](int buf, int c) {
        if (wave == SCAN_WAVE) {
            const bool in = lane < min(C, p.T - c * C);
            // b in log2 units: every factor is then one hardware exp2
            const float b = wave_inclusive_sum(in ? __builtin_amdgcn_logf(pg) : 0.f, lane);
            const float bC = read_lane(b, C - 1);
            if (lane < C) {
                sB[buf][lane] = b;
                sEB[buf][lane] = __builtin_amdgcn_exp2f(b);
                sEBC[buf][lane] = __builtin_amdgcn_exp2f(bC - b);
                sBeta[buf][lane] = in ? pb : 0.f;
            }
            if (lane == 0) sDecay[buf] = __builtin_amdgcn_exp2f(bC);
        }
    };
    // lower score tiles of buffer `buf`, work split over waves [w0, w0 + nw):
    // isK: A = diag(beta) (Gamma o K K^T), strictly lower, in float32 for the
    // inverse; else P = M o Gamma o Q K^T in the operand type.  Tiles above the
    // block diagonal are never read (the products below stop at the diagonal).
    auto score_tiles = [&](int buf, int kbuf, bool isK, int w0, int nw) {
        const Op *X = isK ? sK[kbuf] : sQ[buf], *K = sK[kbuf];
        const float *bb = sB[buf], *beta = sBeta[buf];
        Op *P = sP[buf];
        for (int tt = wave - w0; tt < NLOW; tt += nw) {
            int I = 0;
            while ((I + 1) * (I + 2) / 2 <= tt) ++I;
            const int J = tt - I * (I + 1) / 2;
            // the product is taken transposed (K_J X_I^T), so that each lane holds
            // four consecutive columns s of one row t and writes them at once
            const int t = 16 * I + lr, s0 = 16 * J + 4 * lg;
            f32x4 acc = zero4();
            tile_mma_qk<DK, KSW>(acc, K + 16 * J * LDK, X + 16 * I * LDK, LDK, lane);
            const float bt = bb[t];
            const float4 bs = *reinterpret_cast<const float4 *>(bb + s0);
            const float g0 = __builtin_amdgcn_exp2f(fminf(bt - bs.x, 0.f)), g1 = __builtin_amdgcn_exp2f(fminf(bt - bs.y, 0.f));
            const float g2 = __builtin_amdgcn_exp2f(fminf(bt - bs.z, 0.f)), g3 = __builtin_amdgcn_exp2f(fminf(bt - bs.w, 0.f));
            if (isK) {
                const float be = beta[t];
                *reinterpret_cast<float4 *>(sA + t * LDA + s0) =
                    make_float4(s0 < t ? be * g0 * acc[0] : 0.f, s0 + 1 < t ? be * g1 * acc[1] : 0.f,
                                s0 + 2 < t ? be * g2 * acc[2] : 0.f, s0 + 3 < t ? be * g3 * acc[3] : 0.f);
            } else {
                st_group(P + t * LDC + s0,
                         Gp::make(s0 <= t ? g0 * acc[0] : 0.f, s0 + 1 <= t ? g1 * acc[1] : 0.f,
                                  s0 + 2 <= t ? g2 * acc[2] : 0.f, s0 + 3 <= t ? g3 * acc[3] : 0.f));
            }
        }
    };
    // bfloat16 chunks of 32 or 64 tokens: the scores in 32x32 jobs, one per
    // 32-token block pair (I, J), I >= J, given by `pair`: K_J Q_I^T (P) and
    // K_J K_I^T (A; on the diagonal K_J is both operands), so that K_J is read
    // once for both and the decay factors are formed once.  Each lane then
    // holds sixteen columns s of one row t of each, written four at a time.
    auto score_pair32 = [&](int buf, int kbuf, int pair) {
        if constexpr (S32) {
            int I = 0;
            while ((I + 1) * (I + 2) / 2 <= pair) ++I;
            const int J = pair - I * (I + 1) / 2;
            const int r = lane & 31, h = lane >> 5;
            const int off = r * LDK + swap_col(r, 8 * h, KSW);
            const Op *aJ = sK[kbuf] + 32 * J * LDK + off;
            const Op *qI = sQ[buf] + 32 * I * LDK + off;
            const Op *kI = sK[kbuf] + 32 * I * LDK + off;
            f32x16 accP = {}, accA = {};
            if (I == J) {
#pragma unroll
                for (int kk = 0; kk < DK / 16; ++kk) {
                    const uint4 a = *reinterpret_cast<const uint4 *>(aJ + 16 * kk);
                    mma32x32(accP, a, *reinterpret_cast<const uint4 *>(qI + 16 * kk));
                    mma32x32(accA, a, a);
                }
            } else {
#pragma unroll
                for (int kk = 0; kk < DK / 16; ++kk) {
                    const uint4 a = *reinterpret_cast<const uint4 *>(aJ + 16 * kk);
                    mma32x32(accP, a, *reinterpret_cast<const uint4 *>(qI + 16 * kk));
                    mma32x32(accA, a, *reinterpret_cast<const uint4 *>(kI + 16 * kk));
                }
            }
            const int t = 32 * I + r;
            const float bt = sB[buf][t], be = sBeta[buf][t];
            // e^{b_t - b_s} <= 1 for s <= t (b does not increase); above the
            // diagonal the factor may overflow, and the select drops it
            auto out = [&](bool diag) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int s0 = 32 * J + 8 * q + 4 * h;
                    const float4 bs = *reinterpret_cast<const float4 *>(sB[buf] + s0);
                    const float g[4] = {__builtin_amdgcn_exp2f(bt - bs.x), __builtin_amdgcn_exp2f(bt - bs.y),
                                        __builtin_amdgcn_exp2f(bt - bs.z), __builtin_amdgcn_exp2f(bt - bs.w)};
                    float a[4], pp[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        a[i] = !diag || s0 + i < t ? be * g[i] * accA[4 * q + i] : 0.f;
                        pp[i] = !diag || s0 + i <= t ? g[i] * accP[4 * q + i] : 0.f;
                    }
                    *reinterpret_cast<float4 *>(sA + t * LDA + s0) = make_float4(a[0], a[1], a[2], a[3]);
                    st_group(sP[buf] + t * LDC + s0, Gp::make(pp[0], pp[1], pp[2], pp[3]));
                }
            };
            if (I == J) out(true);
            else out(false);   // every column s precedes the row t
        }
    };
    // diagonal 16x16 block `blk` of T = (I + A)^{-1}, written over A's block,
    // one wave per block, in 8x8 halves: with A = [[A00, 0], [A10, A11]],
    // T = [[T00, 0], [-T11 A10 T00, T11]], Thh = (I + Ahh)^{-1}.
    auto diag_block = [&](int blk) {
        float *Ab = sA + 16 * blk * LDA + 16 * blk;
        {
            // T00 and T11 by forward substitution, one per half wave: lane
            // 32h + 4n + pp owns rows 2pp, 2pp + 1 of column n of half h, so
            // each step's row-times-column product is two multiply-adds and a
            // sum over the lane quad (two DPP adds)
            const int h = lane >> 5, n = (lane >> 2) & 7, pp = lane & 3, o = 8 * h;
            float x[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) x[i] = 2 * pp + i == n ? 1.f : 0.f;
            // every row's two entries are read up front: one LDS latency instead
            // of one per step
            float2 rows[7];
#pragma unroll
            for (int t = 1; t < 8; ++t) rows[t - 1] = *reinterpret_cast<const float2 *>(Ab + (o + t) * LDA + o + 2 * pp);
#pragma unroll
            for (int t = 1; t < 8; ++t) {
                // A's diagonal and upper part are zero, so the not yet computed
                // entries (zero) and x[n] = 1 above row t add nothing
                float part = rows[t - 1].x * x[0] + rows[t - 1].y * x[1];
                part += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(part), 0xB1, 0xF, 0xF, true));  // lanes ^1
                part += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(part), 0x4E, 0xF, 0xF, true));  // lanes ^2
                if (pp == (t >> 1) && t > n) x[t & 1] = -part;
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) Ab[(o + 2 * pp + i) * LDA + o + n] = x[i];
        }
        // the lower-left 8x8, lane 8r + c owning entry (r, c): Y = A10 T00, then
        // -T11 Y.  Lanes read what other lanes of the wave wrote just before;
        // the wave's LDS accesses complete in order, and the empty asm
        // statements keep the compiler from reordering them.
        asm volatile("" ::: "memory");
        const int r = lane >> 3, c = lane & 7;
        const float *row = Ab + (8 + r) * LDA;
        const float4 a0 = *reinterpret_cast<const float4 *>(row), a1 = *reinterpret_cast<const float4 *>(row + 4);
        const float4 u0 = *reinterpret_cast<const float4 *>(row + 8), u1 = *reinterpret_cast<const float4 *>(row + 12);
        float col[8];
#pragma unroll
        for (int b = 0; b < 8; ++b) col[b] = Ab[b * LDA + c];
        const float y = ((a0.x * col[0] + a0.y * col[1]) + (a0.z * col[2] + a0.w * col[3])) +
                        ((a1.x * col[4] + a1.y * col[5]) + (a1.z * col[6] + a1.w * col[7]));
        asm volatile("" ::: "memory");
        Ab[(8 + r) * LDA + c] = y;
        asm volatile("" ::: "memory");
#pragma unroll
        for (int b = 0; b < 8; ++b) col[b] = Ab[(8 + b) * LDA + c];
        const float z = ((u0.x * col[0] + u0.y * col[1]) + (u0.z * col[2] + u0.w * col[3])) +
                        ((u1.x * col[4] + u1.y * col[5]) + (u1.z * col[6] + u1.w * col[7]));
        asm volatile("" ::: "memory");
        Ab[(8 + r) * LDA + c] = -z;
    };
    // off-diagonal blocks of T into buffer `buf`, one block column per helper wave:
    // T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj (matrix cores in the operand type)
    auto offdiag = [&](int w0, int nw) {
        Op *Tt = sT;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if (j % nw != wave - w0) continue;
            G4 tb[NB];
            {
                f32x4 d;
#pragma unroll
                for (int i = 0; i < 4; ++i) d[i] = sA[(16 * j + 4 * lg + i) * LDA + 16 * j + lr];
                tb[j] = Gp::make(d);
#pragma unroll
                for (int i = 0; i < 4; ++i) from_f32(Tt[(16 * j + 4 * lg + i) * LDC + 16 * j + lr], d[i]);
            }
#pragma unroll
            for (int i = j + 1; i < NB; ++i) {
                const float *ar = sA + (16 * i + lr) * LDA + 4 * lg;
                auto agroup = [&](int m) {
                    const float4 f = *reinterpret_cast<const float4 *>(ar + 16 * m);
                    return Gp::make(f.x, f.y, f.z, f.w);
                };
                // every index below is a compile-time constant once the loops are
                // unrolled, so tb stays in registers
                f32x4 acc = zero4();
#pragma unroll
                for (int m = j; m < i; m += 2) {
                    if (m + 1 < i) mma32(acc, agroup(m), agroup(m + 1), tb[m], tb[m + 1]);
                    else mma16(acc, agroup(m), tb[m]);
                }
                f32x4 tij = zero4();
                mma16(tij, agroup(i), Gp::make(acc));
#pragma unroll
                for (int r = 0; r < 4; ++r) tij[r] = -tij[r];
                tb[i] = Gp::make(tij);
#pragma unroll
                for (int r = 0; r < 4; ++r) from_f32(Tt[(16 * i + 4 * lg + r) * LDC + 16 * j + lr], tij[r]);
            }
        }
    };

    // output rows of chunk c (staged in sO), 16 bytes per lane, by the helpers
    auto copy_out = [&](int c) {
        const int c0 = c * C, n = min(C, p.T - c0);
        for (int e = htid; e < n * (DVB / VE); e += NHW * 64) {
            const int t = e / (DVB / VE), v = (e % (DVB / VE)) * VE;
            *reinterpret_cast<uint4 *>(oh + static_cast<size_t>(c0 + t) * p.d_v + vb * DVB + v) =
                *reinterpret_cast<const uint4 *>(sO + t * LDV + v);
        }
    };

    // HO: the state waves publish the entering state (bfloat16, rows = values)
    auto publish_s0 = [&]() {
        if constexpr (HO) {
            const int v = 16 * wave + lr;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                st_group(sS0 + v * LDK + swap_col(v, 16 * cb + 4 * lg, KSW), Gp::make(st[cb]));
        }
    };
    // HO, step 2: S0 Q_I^T for the 32 tokens of output job I (lane: token
    // 32 I + lane%32, values 8q + 4(lane/32) + i in acc[4q + i]) and e^{b_t}
    auto qs_job = [&](int cur, int I, f32x16 &acc, float &ebt) {
        if constexpr (HO) {
            const int r = lane & 31, h = lane >> 5;
            const int off = r * LDK + swap_col(r, 8 * h, KSW);
            const Op *a = sS0 + off, *b = sQ[cur] + 32 * I * LDK + off;
            acc = f32x16{};
#pragma unroll
            for (int kk = 0; kk < DK / 16; ++kk)
                mma32x32(acc, *reinterpret_cast<const uint4 *>(a + 16 * kk), *reinterpret_cast<const uint4 *>(b + 16 * kk));
            ebt = sEB[cur][32 * I + r];
        }
    };
    // HO, step 3: O^T = U^T P_I^T + S0 Q_I^T diag(e^b) for job I, straight to
    // global memory (four values of one token per store)
    auto out_job = [&](int c, int cur, int I, const f32x16 &qs, float ebt) {
        if constexpr (HO) {
            const int r = lane & 31, h = lane >> 5;
            const Op *a = sUT + r * LDU + 8 * h, *b = sP[cur] + (32 * I + r) * LDC + 8 * h;
            f32x16 acc = {};
#pragma unroll
            for (int kk = 0; kk < 2 * NJO; ++kk)
                if (kk < 2 * (I + 1))
                    mma32x32(acc, *reinterpret_cast<const uint4 *>(a + 16 * kk), *reinterpret_cast<const uint4 *>(b + 16 * kk));
            const int t = c * C + 32 * I + r;
            if (t < p.T) {
                IO *orow = oh + static_cast<size_t>(t) * p.d_v + vb * DVB + 4 * h;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    st_group(orow + 8 * q, Gp::make(acc[4 * q] + ebt * qs[4 * q], acc[4 * q + 1] + ebt * qs[4 * q + 1],
                                                    acc[4 * q + 2] + ebt * qs[4 * q + 2], acc[4 * q + 3] + ebt * qs[4 * q + 3]));
            }
        }
    };

    // ---------------------------------------------------------------- prologue
    // staging: everyone; chunk 0's tiles and gates, then chunk 0's scores and
    // inverse, chunk 1's Q, K and gates; the registers then hold K(2), V(1),
    // Q(2), issued in this order, the order in which a chunk of the loop below
    // leaves them in flight.
    // The loads are issued whether or not their chunk exists (a chunk past the
    // end re-reads the last one and is never stored): every path through the
    // loop then issues the same loads in the same order, and the compiler's
    // wait for one tile covers that tile alone, not the loads issued after it.
    const bool k_stager = !KSTATE || (state_wave && !KDMA);   // register staging of K
    const int clast = nchunks - 1;
    auto stage = [&](int c) {
        if (c + 1 < nchunks) store_v();
        if (c + 2 < nchunks) {
            store_q(c & 1);
            if constexpr (!KSTATE) store_k((c + 2) % 3);
            scan(c & 1, c + 2);
        }
        load_v(min(c + 2, clast));
        load_q(min(c + 3, clast));
        if constexpr (!KSTATE) load_k(min(c + 3, clast));
    };
    // KSTATE, state waves, end of step 1: chunk c+2's K (KDMA: the direct
    // loads; registers: stored, and chunk c+3's loaded)
    auto stage_k = [&](int c) {
        if constexpr (KDMA) {
            if (c + 2 < nchunks) dma_k(c + 2, (c + 2) % 3);
        } else if constexpr (KSTATE) {
            if (c + 2 < nchunks) store_k((c + 2) % 3);
            load_k(min(c + 3, clast));
        }
    };
    if (nchunks > 0) {
        load_q(0);
        if (k_stager) load_k(0);
        load_v(0);
        if (KDMA && state_wave) dma_k(0, 0);
        store_q(0);
        if (k_stager) store_k(0);
        store_v();
        scan(0, 0);
        if (state_wave) publish_s0();
        if constexpr (KDMA) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        load_q(min(1, clast));
        if (k_stager) load_k(min(1, clast));
        if (KDMA && state_wave && nchunks > 1) dma_k(1, 1);
        if constexpr (S32) {
            if (wave < NJ32) score_pair32(0, 0, wave);
        } else {
            if (wave < NW / 2) score_tiles(0, 0, true, 0, NW / 2);
            else score_tiles(0, 0, false, NW / 2, NW - NW / 2);
        }
        __syncthreads();
        if (wave < NB) diag_block(wave);
        __syncthreads();
        offdiag(0, NW);
        __syncthreads();
        if (nchunks > 1) {
            store_q(1);
            if (k_stager) store_k(1);
            scan(1, 1);
        }
        if constexpr (KDMA) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
        __syncthreads();
        if (k_stager) load_k(min(2, clast));
        load_v(min(1, clast));
        load_q(min(2, clast));

        // ---------------------------------------------------------------- chunk loop
        // The two roles run loops of their own with the same three barriers per
        // chunk, so that each role's registers are allocated for its own work.
        if (state_wave) {
            for (int c = 0; c < nchunks; ++c) {
                const int cur = c & 1, kc = c % 3;

                // step 1: K S0^T, Q S0^T and the solve's right-hand side Y of chunk c
                G4 yb[NB];
                f32x4 qs[NB];   // S0 Q^T: lane holds values 4*lg..+3 of token 16 I + lr
                {
                    G4 sb[NCB];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) sb[cb] = Gp::make(st[cb]);
                    f32x4 ks[NB];
#pragma unroll
                    for (int I = 0; I < NB; ++I) { ks[I] = zero4(); qs[I] = zero4(); }   // qs: unused with HO
                    const int ko = swap_col(lr, 4 * lg, KSW);   // rows 16 I + lr
#pragma unroll
                    for (int s2 = 0; s2 + 2 <= NCB; s2 += 2) {
#pragma unroll
                        for (int I = 0; I < NB; ++I) {
                            const Op *kr = sK[kc] + (16 * I + lr) * LDK + ko + 16 * s2;
                            const Op *qr = sQ[cur] + (16 * I + lr) * LDK + ko + 16 * s2;
                            mma32(ks[I], ld_group(kr), ld_group(kr + 16), sb[s2], sb[s2 + 1]);
                            if constexpr (!HO) mma32(qs[I], sb[s2], sb[s2 + 1], ld_group(qr), ld_group(qr + 16));
                        }
                    }
                    if constexpr (NCB % 2 == 1) {
#pragma unroll
                        for (int I = 0; I < NB; ++I) {
                            mma16(ks[I], ld_group(sK[kc] + (16 * I + lr) * LDK + ko + 16 * (NCB - 1)), sb[NCB - 1]);
                            if constexpr (!HO) mma16(qs[I], sb[NCB - 1], ld_group(sQ[cur] + (16 * I + lr) * LDK + ko + 16 * (NCB - 1)));
                        }
                    }
#pragma unroll
                    for (int I = 0; I < NB; ++I) {
                        const float4 be = *reinterpret_cast<const float4 *>(&sBeta[cur][16 * I + 4 * lg]);
                        const float4 eb = *reinterpret_cast<const float4 *>(&sEB[cur][16 * I + 4 * lg]);
                        // v of tokens 16 I + 4 lg .. +3, this lane's channel
                        float v4[4];
                        if constexpr (VTR) {
                            const uint2 w = kt_group<0>(sV, LDVV, 16 * I, 16 * wave, lane);
                            v4[0] = lo_bf16(w.x); v4[1] = hi_bf16(w.x); v4[2] = lo_bf16(w.y); v4[3] = hi_bf16(w.y);
                        } else {
                            const Op *vr = sV + (16 * I + 4 * lg) * LDVV + vloc;
#pragma unroll
                            for (int i = 0; i < 4; ++i) v4[i] = to_f32(vr[i * LDVV]);
                        }
                        f32x4 y;
                        y[0] = be.x * (v4[0] - eb.x * ks[I][0]);
                        y[1] = be.y * (v4[1] - eb.y * ks[I][1]);
                        y[2] = be.z * (v4[2] - eb.z * ks[I][2]);
                        y[3] = be.w * (v4[3] - eb.w * ks[I][3]);
                        yb[I] = Gp::make(y);
                    }
                }
                stage_k(c);
                __syncthreads();

                // step 2: U = T Y and (not HO) the outputs of chunk c
                G4 usb[NB];   // U diag(e^{b_C - b}) for the state update
                float decay;
                {
                    decay = sDecay[cur];
                    G4 ub[NB];
#pragma unroll
                    for (int I = 0; I < NB; ++I) {
                        f32x4 u = zero4();
                        tile_mma_lr_n<NB>(u, sT + 16 * I * LDC, LDC, yb, I + 1, lane);
                        ub[I] = Gp::make(u);
                        // HO: U^T for the output jobs (rows = values, four tokens per write)
                        if constexpr (HO) st_group(sUT + vloc * LDU + 16 * I + 4 * lg, ub[I]);
                        const float4 ec = *reinterpret_cast<const float4 *>(&sEBC[cur][16 * I + 4 * lg]);
                        usb[I] = Gp::make(u[0] * ec.x, u[1] * ec.y, u[2] * ec.z, u[3] * ec.w);
                    }
                    if constexpr (!HO) {
#pragma unroll
                        for (int I = 0; I < NB; ++I) {
                            // O^T = U^T P^T: lane holds values 16*wave + 4*lg..+3 of token 16 I + lr
                            f32x4 o = zero4();
                            tile_mma_rl_n<NB>(o, ub, sP[cur] + 16 * I * LDC, LDC, I + 1, lane);
                            const float eb = sEB[cur][16 * I + lr];
                            st_group(sO + (16 * I + lr) * LDV + 16 * wave + 4 * lg,
                                     Gp::make(o[0] + eb * qs[I][0], o[1] + eb * qs[I][1], o[2] + eb * qs[I][2],
                                              o[3] + eb * qs[I][3]));
                        }
                    }
                }
                __syncthreads();

                // step 3: S <- e^{b_C} S + K^T (U e^{b_C - b})
                {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) st[cb][i] *= decay;
#pragma unroll
                        for (int s2 = 0; s2 + 2 <= NB; s2 += 2)
                            mma32(st[cb], kt_group<KSW>(sK[kc], LDK, 16 * s2, 16 * cb, lane),
                                  kt_group<KSW>(sK[kc], LDK, 16 * s2 + 16, 16 * cb, lane), usb[s2], usb[s2 + 1]);
                        if constexpr (NB % 2 == 1) mma16(st[cb], kt_group<KSW>(sK[kc], LDK, 16 * (NB - 1), 16 * cb, lane), usb[NB - 1]);
                    }
                    publish_s0();   // HO: entering state of chunk c+1
                }
                // KDMA: chunk c+2's K tile has landed before this wave's last
                // barrier of the chunk
                if constexpr (KDMA) __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
                stage(c);
                __syncthreads();
            }
        } else {
            f32x16 oqs = {};   // HO output jobs: S0 Q_I^T of the current chunk and e^{b_t}
            float oeb = 0.f;
            for (int c = 0; c < nchunks; ++c) {
                const int cur = c & 1, nxt = cur ^ 1;
                const int kn = (c + 1) % 3;   // K buffer of chunk c+1
                const bool has_next = c + 1 < nchunks;

                // step 1: the scores of chunk c+1 (only its K K^T tiles with 16x16
                // tiles); without HO the staged outputs of chunk c-1 leave
                if constexpr (!HO) {
                    if (c > 0) copy_out(c - 1);
                }
                if constexpr (S32) {
                    if (has_next && hw < NJ32) {
                        // the score jobs bound step 1: raised issue priority
                        __builtin_amdgcn_s_setprio(1);
                        score_pair32(nxt, kn, hw);
                        __builtin_amdgcn_s_setprio(0);
                    }
                } else {
                    if (has_next) score_tiles(nxt, kn, true, WS, NHW);
                }
                __syncthreads();

                // step 2: one wave per diagonal block of chunk c+1's inverse; with 16x16
                // tiles, the other helpers: its Q K^T tiles; HO: S0 Q^T of chunk c
                if (has_next) {
                    if (hw < NB) {
                        // the diagonal blocks bound step 2: raised issue priority
                        // over the waves they share a SIMD with
                        __builtin_amdgcn_s_setprio(1);
                        diag_block(hw);
                        __builtin_amdgcn_s_setprio(0);
                    }
                    else if constexpr (!S32) score_tiles(nxt, kn, false, WS + NB, NHW - NB);
                }
                if (HO && hw >= OJ0) qs_job(cur, hw - OJ0, oqs, oeb);
                __syncthreads();

                // step 3: first the off-diagonal inverse of chunk c+1 (over chunk
                // c's T, last read in step 2), then the staging (the loads it stores
                // arrived during the previous chunk): V of chunk c+1 over chunk c's,
                // chunk c+2's gate values -> gate buffer cur and its Q (and K) into
                // buffers no step reads any more (Q of chunk c, K of chunk c-1), then
                // the loads of V(c+2) and Q (K) of chunk c+3; HO: the outputs of
                // chunk c.
                if (has_next) {
                    // the off-diagonal inverse is the longest task of the step: raised
                    // issue priority over the waves it shares a SIMD with
                    __builtin_amdgcn_s_setprio(1);
                    offdiag(WS, NHW);
                    __builtin_amdgcn_s_setprio(0);
                }
                stage(c);
                if (HO && hw >= OJ0) out_job(c, cur, hw - OJ0, oqs, oeb);
                __syncthreads();
            }
            if constexpr (!HO) {
                copy_out(clast);
            }
        }
    }

    if (p.S_T && state_wave) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            *reinterpret_cast<float4 *>(p.S_T + srow + 16 * cb + 4 * lg) =
                make_float4(st[cb][0], st[cb][1], st[cb][2], st[cb][3]);
    }
}

// ------------------------------------------------------------------ dispatch

constexpr int kGdrWaves = 8;   // waves per workgroup

template <class DT, int DK, int DVB, int C>
static hipError_t launch_gdr_t(const ChunkArgs &a) {
    ChunkParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate; p.beta = a.beta; p.S0 = a.S0; p.z0 = nullptr;
    p.out = a.out; p.S_T = a.S_T; p.z_T = nullptr;
    p.T = a.T; p.d_v = a.d_v; p.n_vblk = a.d_v / DVB; p.n_heads = a.B * a.H;
    const int64_t blocks = static_cast<int64_t>(p.n_heads) * p.n_vblk;
    hipLaunchKernelGGL((gdr_chunk_kernel<DT, DK, DVB, C, kGdrWaves>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kGdrWaves * 64), 0, a.stream, p);
    return hipGetLastError();
}

// Largest chunk <= C whose LDS tiles fit (the result does not depend on the
// chunk length).
template <class DT, int DK, int DVB, int C>
constexpr int gdr_fit_chunk() {
    if constexpr (C > 16 && gdr_lds_bytes<DT, DK, DVB, C>() > 160 * 1024) return gdr_fit_chunk<DT, DK, DVB, C / 2>();
    else return C;
}

template <class DT, int DK, int C>
static hipError_t gdr_dvb(const ChunkArgs &a) {
    if (a.d_v >= 32) return launch_gdr_t<DT, DK, 32, gdr_fit_chunk<DT, DK, 32, C>()>(a);
    return launch_gdr_t<DT, DK, 16, gdr_fit_chunk<DT, DK, 16, C>()>(a);
}

template <class DT, int DK>
static hipError_t gdr_chunk(const ChunkArgs &a) {
    switch (a.chunk) {
        case 16: return gdr_dvb<DT, DK, 16>(a);
        case 32: return gdr_dvb<DT, DK, 32>(a);
        case 64: return gdr_dvb<DT, DK, 64>(a);
        // 128-token tiles of this kernel exceed the LDS of a compute unit; the
        // result does not depend on the chunk length, so they run as 64
        case 128: return gdr_dvb<DT, DK, 64>(a);
    }
    return hipErrorInvalidValue;
}

template <class DT>
static hipError_t gdr_dk(const ChunkArgs &a) {
    switch (a.d_k) {
        case 16: return gdr_chunk<DT, 16>(a);
        case 32: return gdr_chunk<DT, 32>(a);
        case 64: return gdr_chunk<DT, 64>(a);
        case 128: return gdr_chunk<DT, 128>(a);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_linear(const ChunkArgs &a);
hipError_t launch_chunk_gdr(const ChunkArgs &a);
hipError_t launch_chunk(const ChunkArgs &a) {
    if (a.variant == LA_GATED_DELTA) return launch_chunk_gdr(a);
    if (a.variant == LA_KDA) return launch_chunk_kda(a);
    return launch_chunk_linear(a);
}

hipError_t launch_chunk_gdr(const ChunkArgs &a) {
    if (a.dtype == LA_BF16) return gdr_dk<BF16>(a);
    return gdr_dk<F32>(a);
}

}  // namespace la
