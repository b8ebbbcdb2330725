// la_chunk_kda.hip -- chunked forward of the delta rule with a per-key-channel
// (diagonal) decay, the finer-grained gate of page "Beyond -- Linear attention
// and recurrent memory", section "From fixed decay to KDA's gated delta write"
// (gfx950).
//
// Recurrence (decay first, as page "Module 18 Beyond attention", 18.2 orders
// the scalar-gate rule), d_v x d_k state:
//   S_t = S_{t-1} diag(alpha_t) + u_t k_t^T,
//   u_t = beta_t (v_t - S_{t-1} diag(alpha_t) k_t),   o_t = S_t q_t.
// Within a chunk entering with S0, let b_tc be the chunk-local cumulative sum
// of log alpha_c and D_tjc = prod_{j < i <= t} alpha_ic = e^{b_tc - b_jc}.
// Unrolling gives S_t = S0 diag(e^{b_t}) + sum_{j<=t} u_j (k_j o D_tj)^T, and
// substituting it into u_t gives one unit-lower-triangular system
//   (I + A) U = diag(beta) V - diag(beta) (K o e^b) S0^T,
//   A_tj = beta_t sum_c k_tc k_jc D_tjc  (j < t),
// so that with W = (I + A)^{-1} diag(beta) (K o e^b) and
// U' = (I + A)^{-1} diag(beta) V (neither depends on S0):
//   U   = U' - W S0^T
//   O   = (Q o e^b) S0^T + P U,   P_tj = sum_c q_tc k_jc D_tjc  (j <= t)
//   S_C = S0 diag(e^{b_n}) + U^T (K o e^{b_n - b})   (n tokens in the chunk).
// Every factor used is at most 1.
//
// Two kernels:
//   kda_prep_kernel  one workgroup per chunk of one head, all chunks at once:
//     the scores (off the 16-token block diagonal through a reference token
//     between query and key, so both operand factors are at most 1; on it
//     exactly, from running products of the gates), the triangular solve for
//     W and U' by 16-token blocks (the inverse of each diagonal block by
//     forward substitution, then X_I = T_II (R_I - sum_{J<I} A_IJ X_J), each
//     wave solving its own 16-column tiles), and the scaled tiles, written to
//     a workspace record per chunk.  The score and solve products take float32
//     operands (float32 matrix cores) for float32 inputs and split bf16
//     operands x = hi + lo (bf16 matrix cores) for bf16 inputs;
//   kda_chain_kernel one workgroup per (head, block of value channels), the
//     chunks in order: the state-dependent products only, the state slice of
//     each wave held in matrix-core accumulators for the whole sequence.
#include "la_chunk_common.hpp"

namespace la {

// Workspace record of one chunk of one head (element type Op of the matrix
// cores: float32 for float32 inputs, bfloat16 otherwise).
template <class Op, int DK, int DV, int C>
struct KdaRec {
    static constexpr size_t QT = 0;                                 // Q o e^b,            C x DK
    static constexpr size_t WT = QT + C * DK * sizeof(Op);          // W,                  C x DK
    static constexpr size_t KT = WT + C * DK * sizeof(Op);          // K o e^{b_n - b},    C x DK
    static constexpr size_t UP = KT + C * DK * sizeof(Op);          // U',                 C x DV
    static constexpr size_t PT = UP + C * DV * sizeof(Op);          // P (blocks J <= I),  C x C
    static constexpr size_t EC = PT + C * C * sizeof(Op);           // e^{b_n},            DK float32
    static constexpr size_t BYTES = (EC + DK * 4 + 255) / 256 * 256;
};

constexpr int kKdaPrepThreads = 1024;   // sixteen waves

// ------------------------------------------------------------------ prep
template <class DT, int DK, int DV, int C>
__global__ void __launch_bounds__(kKdaPrepThreads) kda_prep_kernel(const ChunkParams p, unsigned char *ws) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef Group<Op> Gp;
    typedef KdaRec<Op, DK, DV, C> R;
    constexpr int NTHR = kKdaPrepThreads;
    constexpr int NB = C / 16;
    constexpr int LDQ = DK + 16 / (int)sizeof(Op);   // raw q, k rows
    constexpr int LDB = DK + 4;                       // cumulative log2 gates (16-byte rows)
    constexpr int LDA = C + 4;                        // A and P, float32
    static_assert(DK + DV <= NTHR && C <= 64 && C % 16 == 0 && DK % 16 == 0, "prep tiling");

    constexpr int LDT = 16 + 4;                       // inverses of the diagonal blocks, float32
    __shared__ __align__(16) Op sQ[C * LDQ];
    __shared__ __align__(16) Op sK[C * LDQ];
    // values staged in LDS for bf16 inputs (float32 tiles at d = 128 would not fit)
    constexpr bool STAGE_V = sizeof(Op) == 2;
    __shared__ __align__(16) Op sV[STAGE_V ? C * (DV + 16 / (int)sizeof(Op)) : 8];
    __shared__ __align__(16) float sB[C * LDB];
    __shared__ __align__(16) float sA[C * LDA];      // A (strict lower), float32
    __shared__ __align__(16) float sP[C * LDA];      // P (lower), float32
    __shared__ __align__(16) float sT[NB * 16 * LDT]; // (I + A_II)^{-1}, float32
    __shared__ float sBeta[C];
    // bf16 inputs: the solve's products take A (off-diagonal blocks) and the
    // diagonal inverses as split operands x = hi + lo (both bf16), two bf16
    // matrix-core steps per 16 x 16 x 16 product instead of four fp32 ones
    constexpr bool SPL = sizeof(Op) == 2;
    constexpr int LDA2 = C + 4, LDT2 = 16 + 4;        // bf16 rows, 2 mod 4 dwords apart
    __shared__ __align__(16) Op sAh[SPL ? C * LDA2 : 4], sAl[SPL ? C * LDA2 : 4];
    __shared__ __align__(16) Op sTh[SPL ? NB * 16 * LDT2 : 4], sTl[SPL ? NB * 16 * LDT2 : 4];
    constexpr int LDVV = DV + 16 / (int)sizeof(Op);

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int nchunks = (p.T + C - 1) / C;
    const int bh = blockIdx.x / nchunks, c = blockIdx.x % nchunks;
    const int t0 = c * C, n = min(C, p.T - t0);
    const size_t tok0 = static_cast<size_t>(bh) * p.T + t0;
    const IO *qh = static_cast<const IO *>(p.q) + tok0 * DK;
    const IO *kh = static_cast<const IO *>(p.k) + tok0 * DK;
    const IO *vh = static_cast<const IO *>(p.v) + tok0 * DV;
    const float *ah = p.gate + tok0 * DK;             // alpha, per token and key channel
    unsigned char *rec = ws + (static_cast<size_t>(bh) * nchunks + c) * R::BYTES;

    // ---- stage q, k, v (rows past n zero), beta (0 past n), and b = cumulative
    // log2 alpha per channel (flat past n: the gates there count as 1).  Every
    // global load is issued before the first LDS write.
    {
        TilePrefetch<C, DK, NTHR, IO> pq, pk;
        TilePrefetch<C, DV, NTHR, IO> pv;
        TilePrefetch<C, DK, NTHR, float> pg;
        pq.load(qh, DK, n, tid);
        pk.load(kh, DK, n, tid);
        if constexpr (STAGE_V) pv.load(vh, DV, n, tid);
        pg.load(ah, DK, n, tid);
        const float beta = tid < C && tid < n ? p.beta[tok0 + tid] : 0.f;
        pq.store(sQ, LDQ, tid);
        pk.store(sK, LDQ, tid);
        if constexpr (STAGE_V) pv.store(sV, LDVV, tid);
        if (tid < C) sBeta[tid] = beta;
#pragma unroll
        for (int i = 0; i < pg.PER; ++i) {
            const int e = tid + i * NTHR;
            if (pg.TOTAL % NTHR != 0 && e >= pg.TOTAL) continue;
            const int t = e / pg.VPR, ch = (e % pg.VPR) * 4;
            float4 g = make_float4(1.f, 1.f, 1.f, 1.f);   // rows past n: no decay
            if ((pg.valid >> i) & 1u) g = *reinterpret_cast<const float4 *>(&pg.r[i]);
            *reinterpret_cast<float4 *>(sB + t * LDB + ch) = g;
        }
    }
    __syncthreads();
    // cumulative log2 per channel: one column per thread, in registers
    for (int ch = tid; ch < DK; ch += NTHR) {
        float col[C];
#pragma unroll
        for (int t = 0; t < C; ++t) col[t] = __builtin_amdgcn_logf(sB[t * LDB + ch]);
#pragma unroll
        for (int t = 1; t < C; ++t) col[t] += col[t - 1];
#pragma unroll
        for (int t = 0; t < C; ++t) sB[t * LDB + ch] = col[t];
    }
    __syncthreads();

    // ---- scores P and A by 16 x 16 tiles (I, J), J <= I, dealt to the waves
    // round robin along the diagonals (the diagonal tiles first)
    const int lr = lane & 15, lg = lane >> 4;
    for (int tt = wave; tt < NB * (NB + 1) / 2; tt += NTHR / 64) {
        int dgl = 0, first = 0;                        // tile tt lies on sub-diagonal dgl
        while (first + (NB - dgl) <= tt) first += NB - dgl++;
        const int J = tt - first, I = J + dgl;
        // Off the diagonal (J < I) the reference token is the last of key block
        // J: for query t > r and key j <= r, D_tj = e^{b_t - b_r} e^{b_r - b_j},
        // both factors <= 1.  On the diagonal the reference is the token
        // before the block (b = 0 before the chunk): the query factor is <= 1,
        // the key factor e^{b_r - b_j} >= 1 is bounded by the channel's decay
        // over the block, so this form is taken only while every channel's
        // decay over the block stays within 2^64 (`fast`), else the exact
        // routine below.
        const bool diag = J == I;
        const int r = diag ? 16 * I - 1 : 16 * J + 15;
        bool fast = !diag;
        if (diag) {
            bool weak = false;
            for (int ch = lane; ch < DK; ch += 64)
                weak |= (r >= 0 ? sB[r * LDB + ch] : 0.f) - sB[(16 * I + 15) * LDB + ch] > 64.f;
            fast = __builtin_amdgcn_ballot_w64(weak) == 0;
        }
        if (fast) {
            const int t = 16 * I + lr, j = 16 * J + lr;
            f32x4 accP = zero4(), accA = zero4();
            // the scaled operands of channels ch .. ch + 3 (f32)
            auto operands = [&](int ch, float (&qs)[4], float (&ks)[4], float (&kj)[4]) {
                // four channels of each row at once (16-byte rows of b, 8- or
                // 16-byte groups of q and k)
                const float4 b4t = *reinterpret_cast<const float4 *>(sB + t * LDB + ch);
                const float4 b4j = *reinterpret_cast<const float4 *>(sB + j * LDB + ch);
                const float4 b4r = r >= 0 ? *reinterpret_cast<const float4 *>(sB + r * LDB + ch) : make_float4(0.f, 0.f, 0.f, 0.f);
                float xq[4], xt[4], xj[4];
                Gp::unpack(ld_group(sQ + t * LDQ + ch), xq);
                Gp::unpack(ld_group(sK + t * LDQ + ch), xt);
                Gp::unpack(ld_group(sK + j * LDQ + ch), xj);
                const float bt[4] = {b4t.x, b4t.y, b4t.z, b4t.w}, bjv[4] = {b4j.x, b4j.y, b4j.z, b4j.w};
                const float brv[4] = {b4r.x, b4r.y, b4r.z, b4r.w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ft = __builtin_amdgcn_exp2f(bt[i] - brv[i]);
                    const float fj = __builtin_amdgcn_exp2f(brv[i] - bjv[i]);
                    qs[i] = xq[i] * ft;
                    ks[i] = xt[i] * ft;
                    kj[i] = xj[i] * fj;
                }
            };
            // the scaled operands are not exact in bf16, and rounding them once
            // would be amplified where q.k cancels: float32 operands for float32
            // inputs; for bf16 inputs split operands x = hi + lo (both bf16,
            // ~16 significant bits), hi hi + lo hi + hi lo on bf16 matrix cores
            if constexpr (SPL && DK % 32 == 0) {
                auto split = [&](const float (&x)[4], uint2 &h, uint2 &l) {
                    float rr[4];
                    h = Gp::make(x[0], x[1], x[2], x[3]);
                    Gp::unpack(h, rr);
                    l = Gp::make(x[0] - rr[0], x[1] - rr[1], x[2] - rr[2], x[3] - rr[3]);
                };
#pragma unroll
                for (int k0 = 0; k0 < DK; k0 += 32) {
                    float qs0[4], ks0[4], kj0[4], qs1[4], ks1[4], kj1[4];
                    operands(k0 + 4 * lg, qs0, ks0, kj0);
                    operands(k0 + 16 + 4 * lg, qs1, ks1, kj1);
                    uint2 qh0, ql0, qh1, ql1, sh0, sl0, sh1, sl1, jh0, jl0, jh1, jl1;
                    split(qs0, qh0, ql0); split(qs1, qh1, ql1);
                    split(ks0, sh0, sl0); split(ks1, sh1, sl1);
                    split(kj0, jh0, jl0); split(kj1, jh1, jl1);
                    mma32(accP, qh0, qh1, jh0, jh1);
                    mma32(accP, ql0, ql1, jh0, jh1);
                    mma32(accP, qh0, qh1, jl0, jl1);
                    mma32(accA, sh0, sh1, jh0, jh1);
                    mma32(accA, sl0, sl1, jh0, jh1);
                    mma32(accA, sh0, sh1, jl0, jl1);
                }
            } else {
#pragma unroll
                for (int k0 = 0; k0 < DK; k0 += 16) {
                    float qs[4], ks[4], kj[4];
                    operands(k0 + 4 * lg, qs, ks, kj);
                    const float4 gk = make_float4(kj[0], kj[1], kj[2], kj[3]);
                    mma16(accP, make_float4(qs[0], qs[1], qs[2], qs[3]), gk);
                    mma16(accA, make_float4(ks[0], ks[1], ks[2], ks[3]), gk);
                }
            }
            // result layout: lane holds rows (queries) 16 I + 4 lg + i of column
            // (key) 16 J + lr; on the diagonal keep j <= t (P) and j < t (A)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tq = 16 * I + 4 * lg + i, jk = 16 * J + lr;
                sP[tq * LDA + jk] = !diag || jk <= tq ? accP[i] : 0.f;
                const float va = !diag || jk < tq ? sBeta[tq] * accA[i] : 0.f;
                sA[tq * LDA + jk] = va;
                if constexpr (SPL) {
                    if (!diag) {
                        Op h;
                        from_f32(h, va);
                        sAh[tq * LDA2 + jk] = h;
                        from_f32(sAl[tq * LDA2 + jk], va - to_f32(h));
                    }
                }
            }
        } else {
            // diagonal block: exact.  Lane (j, cq): key token j of the block and
            // a group of channels; for each query token t >= j the decay factor
            // e^{b_tc - b_jc} (exponent <= 0) is formed directly
            constexpr int NQ = DK / 8 < 4 ? DK / 8 : 4;
            constexpr int CPL = DK / NQ;
            const int j = lr, cq = lg;
            const bool act = cq < NQ;
            const int ch0 = (act ? cq : 0) * CPL;
            const int rj = 16 * I + j;
            float kj[CPL], bj[CPL];
#pragma unroll
            for (int i = 0; i < CPL; ++i) {
                kj[i] = act ? to_f32(sK[rj * LDQ + ch0 + i]) : 0.f;
                bj[i] = sB[rj * LDB + ch0 + i];
            }
#pragma unroll 1
            for (int t = 0; t < 16; ++t) {
                const int rt = 16 * I + t;
                float sp = 0.f, sa = 0.f;
#pragma unroll
                for (int i = 0; i < CPL; ++i) {
                    // t < j: the exponent is positive, but those entries are masked below
                    const float kd = kj[i] * __builtin_amdgcn_exp2f(fminf(sB[rt * LDB + ch0 + i] - bj[i], 0.f));
                    sp += to_f32(sQ[rt * LDQ + ch0 + i]) * kd;
                    sa += to_f32(sK[rt * LDQ + ch0 + i]) * kd;
                }
                sp += __shfl_xor(sp, 16);
                sp += __shfl_xor(sp, 32);
                sa += __shfl_xor(sa, 16);
                sa += __shfl_xor(sa, 32);
                if (cq == 0) {
                    sP[rt * LDA + 16 * I + j] = t >= j ? sp : 0.f;
                    sA[rt * LDA + 16 * I + j] = t > j ? sBeta[rt] * sa : 0.f;
                }
            }
        }
    }
    __syncthreads();

    // ---- T_II = (I + A_II)^{-1} of the diagonal blocks: wave I, lane c < 16
    // forms column c by forward substitution (unit lower triangular)
    for (int I = wave; I < NB; I += NTHR / 64) {
        if (lane < 16) {
            const float *ab = sA + 16 * I * LDA + 16 * I;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s0 = i == lane ? 1.f : 0.f, s1 = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) {
                    if (m & 1) s1 -= ab[i * LDA + m] * x[m];
                    else s0 -= ab[i * LDA + m] * x[m];
                }
                x[i] = s0 + s1;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                sT[(16 * I + i) * LDT + lane] = x[i];
                if constexpr (SPL) {
                    Op h;
                    from_f32(h, x[i]);
                    sTh[(16 * I + i) * LDT2 + lane] = h;
                    from_f32(sTl[(16 * I + i) * LDT2 + lane], x[i] - to_f32(h));
                }
            }
        }
    }
    __syncthreads();

    // ---- W and U': X = [W | U'] solves (I + A) X = R, R = [beta o (K o e^b) |
    // beta o V], by 16-token block rows: X_I = T_II (R_I - sum_{J<I} A_IJ X_J).
    // The columns are independent, so each wave solves its own 16-column tiles
    // with no barrier; a result tile (rows = tokens) is already the B operand
    // of the next product.  float32 inputs: float32 matrix cores; bf16 inputs:
    // split operands (hi hi + lo hi + hi lo), float32 accumulation.
    {
        const int lr = lane & 15, lg = lane >> 4;
        constexpr int NCT = (DK + DV) / 16;
        for (int ct = wave; ct < NCT; ct += NTHR / 64) {
            const int col = 16 * ct + lr;
            const bool wcol = col < DK;
            f32x4 X[NB];
            typename Gp::type xh[NB], xl[NB];   // SPL: X as split B operands
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                f32x4 y;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = 16 * I + 4 * lg + r;
                    float vv = 0.f;
                    if (!wcol) {
                        if constexpr (STAGE_V) vv = to_f32(sV[t * LDVV + col - DK]);
                        else vv = t < n ? load1(vh + static_cast<size_t>(t) * DV + col - DK) : 0.f;
                    }
                    y[r] = wcol ? sBeta[t] * to_f32(sK[t * LDQ + col]) * __builtin_amdgcn_exp2f(sB[t * LDB + col])
                                : sBeta[t] * vv;
                }
                X[I] = zero4();
                if constexpr (SPL) {
                    // y - A_IJ X_J with -A_IJ (sign bits flipped), then T_II y
#pragma unroll
                    for (int J = 0; J < I; ++J) {
                        uint2 ah = ld_group(sAh + (16 * I + lr) * LDA2 + 16 * J + 4 * lg);
                        uint2 al = ld_group(sAl + (16 * I + lr) * LDA2 + 16 * J + 4 * lg);
                        ah.x ^= 0x80008000u; ah.y ^= 0x80008000u; al.x ^= 0x80008000u; al.y ^= 0x80008000u;
                        mma32(y, ah, al, xh[J], xh[J]);
                        mma16(y, ah, xl[J]);
                    }
                    const uint2 th = ld_group(sTh + (16 * I + lr) * LDT2 + 4 * lg);
                    const uint2 tl = ld_group(sTl + (16 * I + lr) * LDT2 + 4 * lg);
                    float r[4];
                    const uint2 yh = Gp::make(y[0], y[1], y[2], y[3]);
                    Gp::unpack(yh, r);
                    const uint2 yl = Gp::make(y[0] - r[0], y[1] - r[1], y[2] - r[2], y[3] - r[3]);
                    mma32(X[I], th, tl, yh, yh);
                    mma16(X[I], th, yl);
                    xh[I] = Gp::make(X[I][0], X[I][1], X[I][2], X[I][3]);
                    Gp::unpack(xh[I], r);
                    xl[I] = Gp::make(X[I][0] - r[0], X[I][1] - r[1], X[I][2] - r[2], X[I][3] - r[3]);
                } else {
#pragma unroll
                    for (int J = 0; J < I; ++J) {
                        const float4 a = *reinterpret_cast<const float4 *>(sA + (16 * I + lr) * LDA + 16 * J + 4 * lg);
                        mma16(y, make_float4(-a.x, -a.y, -a.z, -a.w), make_float4(X[J][0], X[J][1], X[J][2], X[J][3]));
                    }
                    mma16(X[I], *reinterpret_cast<const float4 *>(sT + (16 * I + lr) * LDT + 4 * lg),
                          make_float4(y[0], y[1], y[2], y[3]));
                }
            }
            // rows 16 I + 4 lg + r of column col, to the record
            Op *dst = wcol ? reinterpret_cast<Op *>(rec + R::WT) + col : reinterpret_cast<Op *>(rec + R::UP) + (col - DK);
            const int ld = wcol ? DK : DV;
#pragma unroll
            for (int I = 0; I < NB; ++I)
#pragma unroll
                for (int r = 0; r < 4; ++r) from_f32(dst[(16 * I + 4 * lg + r) * ld], X[I][r]);
        }
    }

    // ---- Q o e^b, K o e^{b_n - b}, e^{b_n} and P (its lower blocks)
    {
        // four channels (tokens) per thread and store
        Op *qt = reinterpret_cast<Op *>(rec + R::QT);
        Op *kt = reinterpret_cast<Op *>(rec + R::KT);
        for (int e = tid; e < C * DK / 4; e += NTHR) {
            const int t = e / (DK / 4), ch = (e % (DK / 4)) * 4;
            const float4 b4 = *reinterpret_cast<const float4 *>(sB + t * LDB + ch);
            const float4 n4 = *reinterpret_cast<const float4 *>(sB + (n - 1) * LDB + ch);
            const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, bn[4] = {n4.x, n4.y, n4.z, n4.w};
            float xq[4], xk[4];
            Gp::unpack(ld_group(sQ + t * LDQ + ch), xq);
            Gp::unpack(ld_group(sK + t * LDQ + ch), xk);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                xq[i] *= __builtin_amdgcn_exp2f(bb[i]);
                xk[i] *= __builtin_amdgcn_exp2f(bn[i] - bb[i]);
            }
            st_group(qt + t * DK + ch, Gp::make(xq[0], xq[1], xq[2], xq[3]));
            st_group(kt + t * DK + ch, Gp::make(xk[0], xk[1], xk[2], xk[3]));
        }
        float *ec = reinterpret_cast<float *>(rec + R::EC);
        for (int ch = tid; ch < DK; ch += NTHR) ec[ch] = __builtin_amdgcn_exp2f(sB[(n - 1) * LDB + ch]);
        Op *pt = reinterpret_cast<Op *>(rec + R::PT);
        for (int e = tid; e < C * C / 4; e += NTHR) {
            const int t = e / (C / 4), j = (e % (C / 4)) * 4;
            if (j / 16 <= t / 16) {
                const float4 x = *reinterpret_cast<const float4 *>(sP + t * LDA + j);
                st_group(pt + t * C + j, Gp::make(x.x, x.y, x.z, x.w));
            }
        }
    }
}

// ------------------------------------------------------------------ chain
// One workgroup per (head, DVB value channels): NW waves, the first DVB / 16
// of them state waves (16 value channels each).  When two copies of a chunk's
// tiles fit in LDS, the other waves stage chunk c + 1 into the second copy while
// the state waves work on chunk c (one barrier per chunk); otherwise every wave
// loads the next chunk's record into registers during the state work and
// stores it to LDS after a barrier.
template <class DT, int DK, int DV, int DVB, int C, int NW>
__global__ void __launch_bounds__(NW * 64) kda_chain_kernel(const ChunkParams p, const unsigned char *ws) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef Group<Op> Gp;
    typedef typename Gp::type G4;
    typedef KdaRec<Op, DK, DV, C> R;
    constexpr int WS = DVB / 16;
    constexpr int NTHR = NW * 64;
    constexpr int NB = C / 16, NCB = DK / 16;
    constexpr int PAD = 16 / sizeof(Op);
    constexpr int LDK = DK + PAD, LDU = DVB + PAD, LDC = C + PAD;
    static_assert(WS <= NW && C <= 64 && C % 16 == 0, "chain tiling");
    constexpr int TILE_BYTES = (3 * C * LDK + C * LDU + C * LDC) * (int)sizeof(Op) + DK * 4;
    constexpr int NBUF = WS < NW && 2 * TILE_BYTES <= 150 * 1024 ? 2 : 1;
    // staging threads: the non-state waves with two buffers, else all
    constexpr int LTHR = NBUF == 2 ? (NW - WS) * 64 : NTHR;

    __shared__ __align__(16) Op sQt[NBUF * C * LDK];
    __shared__ __align__(16) Op sWt[NBUF * C * LDK];
    __shared__ __align__(16) Op sKt[NBUF * C * LDK];
    __shared__ __align__(16) Op sUp[NBUF * C * LDU];
    __shared__ __align__(16) Op sPt[NBUF * C * LDC];
    __shared__ __align__(16) float sEC[NBUF * DK];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    int bh, vb;
    block_to_head(blockIdx.x, p.n_heads, p.n_vblk, bh, vb);
    const int nchunks = (p.T + C - 1) / C;
    const bool state_wave = wave < WS;
    const int vloc = 16 * wave + lr;
    const int vch = vb * DVB + vloc;
    const size_t srow = (static_cast<size_t>(bh) * DV + (state_wave ? vch : 0)) * DK;
    IO *oh = static_cast<IO *>(p.out) + static_cast<size_t>(bh) * p.T * DV;

    f32x4 st[NCB];   // S^T[c][v]: key channels 16 cb + 4 lg + i of this lane's value column
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) {
        st[cb] = zero4();
        if (p.S0 && state_wave) {
            const float4 s4 = *reinterpret_cast<const float4 *>(p.S0 + srow + 16 * cb + 4 * lg);
            st[cb] = f32x4{s4.x, s4.y, s4.z, s4.w};
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    const bool loader = NBUF == 1 || !state_wave;
    const int ltid = NBUF == 2 ? tid - WS * 64 : tid;
    TilePrefetch<C, DK, LTHR, Op> pq, pw, pk;
    TilePrefetch<C, DVB, LTHR, Op> pu;
    TilePrefetch<C, C, LTHR, Op> pp;
    float4 pe = make_float4(0.f, 0.f, 0.f, 0.f);
    auto load = [&](int c) {
        const unsigned char *rec = ws + (static_cast<size_t>(bh) * nchunks + c) * R::BYTES;
        pq.load(reinterpret_cast<const Op *>(rec + R::QT), DK, C, ltid);
        pw.load(reinterpret_cast<const Op *>(rec + R::WT), DK, C, ltid);
        pk.load(reinterpret_cast<const Op *>(rec + R::KT), DK, C, ltid);
        pu.load(reinterpret_cast<const Op *>(rec + R::UP) + vb * DVB, DV, C, ltid);
        pp.load(reinterpret_cast<const Op *>(rec + R::PT), C, C, ltid);
        if (ltid < DK / 4) pe = reinterpret_cast<const float4 *>(rec + R::EC)[ltid];
    };
    auto store = [&](int b) {
        pq.store(sQt + b * C * LDK, LDK, ltid);
        pw.store(sWt + b * C * LDK, LDK, ltid);
        pk.store(sKt + b * C * LDK, LDK, ltid);
        pu.store(sUp + b * C * LDU, LDU, ltid);
        pp.store(sPt + b * C * LDC, LDC, ltid);
        if (ltid < DK / 4) reinterpret_cast<float4 *>(sEC + b * DK)[ltid] = pe;
    };

    if (nchunks > 0) {
        if (loader) {
            load(0);
            store(0);
            // two buffers: the staging waves hold chunk c + 1 in registers from
            // step c - 1 on, so its loads have a whole step to land
            if (NBUF == 2 && nchunks > 1) load(1);
        }
        __syncthreads();
    }
    for (int c = 0; c < nchunks; ++c) {
        const int b = NBUF == 2 ? (c & 1) : 0;
        if constexpr (NBUF == 2) {
            if (loader && c + 1 < nchunks) {
                store(b ^ 1);                        // buffer b ^ 1 was last read in chunk c - 1
                if (c + 2 < nchunks) load(c + 2);    // registers free once stored
            }
        } else {
            if (loader && c + 1 < nchunks) load(c + 1);
        }
        if (state_wave) {
            const Op *sQc = sQt + b * C * LDK, *sWc = sWt + b * C * LDK, *sKc = sKt + b * C * LDK;
            const Op *sUc = sUp + b * C * LDU, *sPc = sPt + b * C * LDC;
            const float *sEc = sEC + b * DK;
            G4 sb[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) sb[cb] = Gp::make(st[cb]);
            // X^T = S0 (Q o e^b)^T (lane: values 4 lg .. of token 16 I + lr) and
            // W S0^T (lane: tokens 16 I + 4 lg + i of value lr)
            f32x4 xs[NB], wsv[NB];
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                xs[I] = zero4();
                wsv[I] = zero4();
                const Op *qr = sQc + (16 * I + lr) * LDK + 4 * lg;
                const Op *wr = sWc + (16 * I + lr) * LDK + 4 * lg;
#pragma unroll
                for (int s2 = 0; s2 + 2 <= NCB; s2 += 2) {
                    mma32(xs[I], sb[s2], sb[s2 + 1], ld_group(qr + 16 * s2), ld_group(qr + 16 * s2 + 16));
                    mma32(wsv[I], ld_group(wr + 16 * s2), ld_group(wr + 16 * s2 + 16), sb[s2], sb[s2 + 1]);
                }
                if constexpr (NCB % 2 == 1) {
                    mma16(xs[I], sb[NCB - 1], ld_group(qr + 16 * (NCB - 1)));
                    mma16(wsv[I], ld_group(wr + 16 * (NCB - 1)), sb[NCB - 1]);
                }
            }
            // U = U' - W S0^T, as operand groups (rows: tokens)
            G4 ub[NB];
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                f32x4 u;
#pragma unroll
                for (int i = 0; i < 4; ++i) u[i] = to_f32(sUc[(16 * I + 4 * lg + i) * LDU + vloc]) - wsv[I][i];
                ub[I] = Gp::make(u);
            }
            // O^T = X^T + U^T P^T, stored four values of a token at a time
            const int n = min(C, p.T - c * C);
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                f32x4 o = xs[I];
                tile_mma_rl_n<NB>(o, ub, sPc + 16 * I * LDC, LDC, I + 1, lane);
                const int t = 16 * I + lr;
                if (t < n) st_group(oh + static_cast<size_t>(c * C + t) * DV + vb * DVB + 16 * wave + 4 * lg, Gp::make(o));
            }
            // S^T <- diag(e^{b_n}) S^T + (K o e^{b_n - b})^T U
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const float4 e4 = *reinterpret_cast<const float4 *>(sEc + 16 * cb + 4 * lg);
                st[cb][0] *= e4.x; st[cb][1] *= e4.y; st[cb][2] *= e4.z; st[cb][3] *= e4.w;
#pragma unroll
                for (int s2 = 0; s2 + 2 <= NB; s2 += 2)
                    mma32(st[cb], kt_group<0>(sKc, LDK, 16 * s2, 16 * cb, lane),
                          kt_group<0>(sKc, LDK, 16 * s2 + 16, 16 * cb, lane), ub[s2], ub[s2 + 1]);
                if constexpr (NB % 2 == 1) mma16(st[cb], kt_group<0>(sKc, LDK, 16 * (NB - 1), 16 * cb, lane), ub[NB - 1]);
            }
        }
        __syncthreads();
        if constexpr (NBUF == 1) {
            if (c + 1 < nchunks) store(0);
            __syncthreads();
        }
    }

    if (p.S_T && state_wave) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
            *reinterpret_cast<float4 *>(p.S_T + srow + 16 * cb + 4 * lg) = make_float4(st[cb][0], st[cb][1], st[cb][2], st[cb][3]);
    }
}

// ------------------------------------------------------------------ dispatch

constexpr int kKdaChainWaves = 6;

template <class DT, int DK, int DV, int C>
static constexpr size_t kda_rec_bytes() { return KdaRec<typename OpOf<DT>::type, DK, DV, C>::BYTES; }

template <class DT, int DK, int DV, int C>
static hipError_t launch_kda_t(const ChunkArgs &a) {
    ChunkParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.gate = a.gate; p.beta = a.beta; p.S0 = a.S0; p.z0 = nullptr;
    p.out = a.out; p.S_T = a.S_T; p.z_T = nullptr;
    p.T = a.T; p.d_v = DV; p.n_heads = a.B * a.H;
    constexpr int DVB = DV >= 32 ? 32 : 16;
    p.n_vblk = DV / DVB;
    const int nchunks = (a.T + C - 1) / C;
    unsigned char *ws = static_cast<unsigned char *>(a.workspace);
    if (nchunks > 0) {
        const int64_t prep_blocks = static_cast<int64_t>(p.n_heads) * nchunks;
        hipLaunchKernelGGL((kda_prep_kernel<DT, DK, DV, C>), dim3(static_cast<uint32_t>(prep_blocks)),
                           dim3(kKdaPrepThreads), 0, a.stream, p, ws);
    }
    const int64_t blocks = static_cast<int64_t>(p.n_heads) * p.n_vblk;
    hipLaunchKernelGGL((kda_chain_kernel<DT, DK, DV, DVB, C, kKdaChainWaves>), dim3(static_cast<uint32_t>(blocks)),
                       dim3(kKdaChainWaves * 64), 0, a.stream, p, static_cast<const unsigned char *>(ws));
    return hipGetLastError();
}

// chunk lengths of this path: 16, 32 or 64 (128 runs as 64)
static int kda_chunk(int chunk) { return chunk == 16 ? 16 : chunk == 32 ? 32 : 64; }

template <class DT, int DK, int DV>
static hipError_t kda_c(const ChunkArgs &a) {
    switch (kda_chunk(a.chunk)) {
        case 16: return launch_kda_t<DT, DK, DV, 16>(a);
        case 32: return launch_kda_t<DT, DK, DV, 32>(a);
    }
    return launch_kda_t<DT, DK, DV, 64>(a);
}

template <class DT, int DK>
static hipError_t kda_dv(const ChunkArgs &a) {
    switch (a.d_v) {
        case 16: return kda_c<DT, DK, 16>(a);
        case 32: return kda_c<DT, DK, 32>(a);
        case 64: return kda_c<DT, DK, 64>(a);
        case 128: return kda_c<DT, DK, 128>(a);
    }
    return hipErrorInvalidValue;
}

template <class DT>
static hipError_t kda_dk(const ChunkArgs &a) {
    switch (a.d_k) {
        case 16: return kda_dv<DT, 16>(a);
        case 32: return kda_dv<DT, 32>(a);
        case 64: return kda_dv<DT, 64>(a);
        case 128: return kda_dv<DT, 128>(a);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_kda(const ChunkArgs &a) {
    if (a.dtype == LA_BF16) return kda_dk<BF16>(a);
    return kda_dk<F32>(a);
}

// Workspace of the per-channel-decay path: one record per chunk and head.
size_t kda_workspace_bytes(const ChunkArgs &a) {
    if (a.T <= 0) return 0;
    const int C = kda_chunk(a.chunk);
    const size_t op = a.dtype == LA_BF16 ? 2 : 4;
    const size_t rec = ((3 * static_cast<size_t>(C) * a.d_k + static_cast<size_t>(C) * a.d_v +
                         static_cast<size_t>(C) * C) * op + a.d_k * 4 + 255) / 256 * 256;
    return static_cast<size_t>(a.B) * a.H * ((a.T + C - 1) / C) * rec;
}

}  // namespace la
