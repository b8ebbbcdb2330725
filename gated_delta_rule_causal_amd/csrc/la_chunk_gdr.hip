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
// Every exponent used is <= 0.  T = (I + A)^{-1} depends on K, g and beta
// only; it is formed per chunk from 16x16 blocks: the diagonal blocks by
// forward substitution, the off-diagonal blocks by
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

// LDS bytes of one workgroup of gdr_chunk_kernel<DT, DK, DVB, C>.
template <class DT, int DK, int DVB, int C>
constexpr int gdr_lds_bytes() {
    typedef typename OpOf<DT>::type Op;
    constexpr int PAD = 16 / sizeof(Op);
    return (2 * C * (DK + PAD) + 2 * C * (C + PAD) + 2 * C * (DVB + PAD) + DK * (C + PAD)) * (int)sizeof(Op) +
           C * (C + 4) * 4 + 4 * C * 4 + 4;
}

template <class DT, int DK, int DVB, int C, int NW>
__global__ void __launch_bounds__(NW * 64) gdr_chunk_kernel(const ChunkParams p) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef Group<Op> Gp;
    typedef typename Gp::type G4;
    constexpr int WS = DVB / 16;         // state waves; wave w < WS owns value channels [16w, 16w + 16)
    constexpr int NTHR = NW * 64;
    constexpr int NB = C / 16;           // 16-token blocks per chunk
    constexpr int NCB = DK / 16;         // 16-channel key blocks
    constexpr int PAD = 16 / sizeof(Op);
    constexpr int LDK = DK + PAD;        // row strides (elements) of the LDS tiles
    constexpr int LDC = C + PAD;
    constexpr int LDV = DVB + PAD;
    constexpr int LDA = C + 4;
    constexpr int LDO = DVB + PAD;
    constexpr int VE = 16 / sizeof(Op);
    static_assert(C <= 64 && C % 16 == 0 && DK % 16 == 0 && DVB % 16 == 0 && WS <= NW, "tiling");
    static_assert(gdr_lds_bytes<DT, DK, DVB, C>() <= 160 * 1024, "LDS budget");

    __shared__ __align__(16) Op sQ[C * LDK];
    __shared__ __align__(16) Op sK[C * LDK];
    __shared__ __align__(16) Op sP[C * LDC];     // M o Gamma o Q K^T
    __shared__ __align__(16) Op sT[C * LDC];     // (I + A)^{-1}
    __shared__ __align__(16) Op sV[C * LDV];     // this block's value channels
    __shared__ __align__(16) Op sO[C * LDO];     // output tile of the block, staged for 16-byte stores
    __shared__ __align__(16) Op sKt[DK * LDC];   // K^T diag(e^{b_C - b}), operand of the state update
    __shared__ __align__(16) float sA[C * LDA];  // A, then T, in float32 during the solve
    __shared__ float sB[C], sEB[C], sBeta[C], sEBC[C];
    __shared__ float sDecay;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    int bh, vb;
    block_to_head(blockIdx.x, p.n_heads, p.n_vblk, bh, vb);
    const int vloc = 16 * wave + lr;               // value channel within the block (state waves)
    const int vch = vb * DVB + vloc;               // value channel of this lane's column
    const size_t tok0 = static_cast<size_t>(bh) * p.T;
    const IO *qh = static_cast<const IO *>(p.q) + tok0 * DK;
    const IO *kh = static_cast<const IO *>(p.k) + tok0 * DK;
    const IO *vh = static_cast<const IO *>(p.v) + tok0 * p.d_v + vb * DVB;
    IO *oh = static_cast<IO *>(p.out) + tok0 * p.d_v;
    const float *gh = p.gate + tok0;
    const float *bth = p.beta + tok0;

    // state slice S^T[c][v] for c in key block cb, v = this lane's column (state waves)
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

    // chunk inputs staged one chunk ahead in registers
    TilePrefetch<C, DK, NTHR, IO> pq, pk;
    TilePrefetch<C, DVB, NTHR, IO> pv;
    float pg = 1.f, pb = 0.f;   // wave 0, lane t: gate and beta of token t (padding: g = 1, beta = 0)
    auto prefetch = [&](int c0) {
        const int n = min(C, p.T - c0);
        pq.load(qh + static_cast<size_t>(c0) * DK, DK, n, tid);
        pk.load(kh + static_cast<size_t>(c0) * DK, DK, n, tid);
        pv.load(vh + static_cast<size_t>(c0) * p.d_v, p.d_v, n, tid);
        if (wave == 0) {
            pg = lane < n ? gh[c0 + lane] : 1.f;
            pb = lane < n ? bth[c0 + lane] : 0.f;
        }
    };
    if (p.T > 0) prefetch(0);

    for (int c0 = 0; c0 < p.T; c0 += C) {
        const int n = min(C, p.T - c0);

        // ---- commit the staged chunk; gate scan on wave 0
        pq.store(sQ, LDK, tid);
        pk.store(sK, LDK, tid);
        pv.store(sV, LDV, tid);
        if (wave == 0) {
            const float b = wave_inclusive_sum(__logf(pg), lane);
            const float bC = __shfl(b, C - 1, 64);
            if (lane < C) {
                sB[lane] = b;
                sEB[lane] = __expf(b);
                sEBC[lane] = __expf(bC - b);
                sBeta[lane] = pb;
            }
            if (lane == 0) sDecay = __expf(bC);
        }
        __syncthreads();
        if (c0 + C < p.T) prefetch(c0 + C);

        // ---- scores: P = M o Gamma o Q K^T and A = strict(beta Gamma o K K^T), the
        // NB(NB+1)/2 lower 16x16 tiles; one wave computes the Q and K tiles of a
        // (I, J) pair from the same K fragments.  Upper tiles are zero.
        constexpr int NLOW = NB * (NB + 1) / 2;
        for (int tt = wave; tt < NLOW; tt += NW) {
            int I = 0;
            while ((I + 1) * (I + 2) / 2 <= tt) ++I;
            const int J = tt - I * (I + 1) / 2;
            const int row = 16 * I + 4 * lg, col = 16 * J + lr;
            f32x4 aq = zero4(), ak = zero4();
            {
                const Op *qr = sQ + (16 * I + lr) * LDK + 4 * lg;
                const Op *kr = sK + (16 * I + lr) * LDK + 4 * lg;
                const Op *br = sK + (16 * J + lr) * LDK + 4 * lg;
#pragma unroll
                for (int k = 0; k + 32 <= DK; k += 32) {
                    const auto b0 = ld_group(br + k), b1 = ld_group(br + k + 16);
                    mma32(aq, ld_group(qr + k), ld_group(qr + k + 16), b0, b1);
                    mma32(ak, ld_group(kr + k), ld_group(kr + k + 16), b0, b1);
                }
                if constexpr (DK % 32 == 16) {
                    const auto b0 = ld_group(br + DK - 16);
                    mma16(aq, ld_group(qr + DK - 16), b0);
                    mma16(ak, ld_group(kr + DK - 16), b0);
                }
            }
            const float bj = sB[col];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = row + i;
                const float gam = __expf(fminf(sB[t] - bj, 0.f));
                sA[t * LDA + col] = col < t ? sBeta[t] * gam * ak[i] : 0.f;
                from_f32(sP[t * LDC + col], col <= t ? gam * aq[i] : 0.f);
            }
        }
        // zero tiles above the block diagonal of P and T
        for (int e = tid; e < NB * NB * 16 * 2; e += NTHR) {
            const int tile = e / 32, r16 = (e % 32) / 2, half = e & 1;
            const int I = tile / NB, J = tile % NB;
            if (J <= I) continue;
            Op *pr = sP + (16 * I + r16) * LDC + 16 * J + 8 * half;
            Op *trow = sT + (16 * I + r16) * LDC + 16 * J + 8 * half;
#pragma unroll
            for (int z = 0; z < 8; ++z) { pr[z] = Op(0); trow[z] = Op(0); }
        }
        // K^T diag(e^{b_C - b}) for the state update: a lane takes two tokens of
        // eight key channels and writes token pairs as one 32-bit word per channel
        for (int e = tid; e < (C / 2) * (DK / 8); e += NTHR) {
            const int tp = e % (C / 2), cg = e / (C / 2);
            const int t0 = 2 * tp;
            const float s0 = sEBC[t0], s1 = sEBC[t0 + 1];
            float x0[8], x1[8];
            if constexpr (VE == 8) {
                load8(reinterpret_cast<const bf16_t *>(sK + t0 * LDK + 8 * cg), x0);
                load8(reinterpret_cast<const bf16_t *>(sK + (t0 + 1) * LDK + 8 * cg), x1);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<uint32_t *>(sKt + (8 * cg + i) * LDC + t0) = pack_bf16x2(x0[i] * s0, x1[i] * s1);
            } else {
                load8(reinterpret_cast<const float *>(sK + t0 * LDK + 8 * cg), x0);
                load8(reinterpret_cast<const float *>(sK + (t0 + 1) * LDK + 8 * cg), x1);
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    *reinterpret_cast<float2 *>(sKt + (8 * cg + i) * LDC + t0) = make_float2(x0[i] * s0, x1[i] * s1);
            }
        }
        __syncthreads();

        // ---- T = (I + A)^{-1}: diagonal 16x16 blocks by forward substitution (wave 0,
        // one lane per column of each block), written over A's diagonal blocks
        if (wave == 0 && lane < 16 * NB) {
            const int blk = lane >> 4, nn = lane & 15;
            float *Ab = sA + 16 * blk * LDA + 16 * blk;
            float x[16];
#pragma unroll
            for (int m = 0; m < 16; ++m) x[m] = m == nn ? 1.f : 0.f;
#pragma unroll
            for (int t = 1; t < 16; ++t) {
                float s4[4] = {0.f, 0.f, 0.f, 0.f};   // four partial sums: shorter dependency chains
#pragma unroll
                for (int m = 0; m < t; ++m) s4[m & 3] += Ab[t * LDA + m] * x[m];
                if (t > nn) x[t] = -((s4[0] + s4[1]) + (s4[2] + s4[3]));
            }
#pragma unroll
            for (int t = 0; t < 16; ++t) Ab[t * LDA + nn] = x[t];
        }
        __syncthreads();

        // off-diagonal blocks, one block column per wave: T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            if (j % NW != wave) continue;
            float4 tb[NB];  // T_mj as B-operand groups (result layout), m >= j
            {
                f32x4 d;
#pragma unroll
                for (int i = 0; i < 4; ++i) d[i] = sA[(16 * j + 4 * lg + i) * LDA + 16 * j + lr];
                tb[j] = Group<float>::make(d);
#pragma unroll
                for (int i = 0; i < 4; ++i) from_f32(sT[(16 * j + 4 * lg + i) * LDC + 16 * j + lr], d[i]);
            }
#pragma unroll
            for (int i = j + 1; i < NB; ++i) {
                f32x4 acc = zero4();
#pragma unroll
                for (int m = j; m < i; ++m) mma16(acc, ld_group(sA + (16 * i + lr) * LDA + 16 * m + 4 * lg), tb[m]);
                f32x4 tij = zero4();
                mma16(tij, ld_group(sA + (16 * i + lr) * LDA + 16 * i + 4 * lg), Group<float>::make(acc));
#pragma unroll
                for (int r = 0; r < 4; ++r) tij[r] = -tij[r];
                tb[i] = Group<float>::make(tij);
#pragma unroll
                for (int r = 0; r < 4; ++r) from_f32(sT[(16 * i + 4 * lg + r) * LDC + 16 * j + lr], tij[r]);
            }
        }
        __syncthreads();

        // ---- state-dependent part: this wave's 16 value channels, from registers
        if (wave < WS) {
            G4 sb[NCB];
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) sb[cb] = Gp::make(st[cb]);
            G4 yb[NB];
            f32x4 qs[NB];
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                f32x4 ks = zero4();
                tile_mma_lr<NCB>(ks, sK + 16 * I * LDK, LDK, sb, lane);
                qs[I] = zero4();
                tile_mma_lr<NCB>(qs[I], sQ + 16 * I * LDK, LDK, sb, lane);
                f32x4 y;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * I + 4 * lg + i;
                    y[i] = sBeta[t] * (to_f32(sV[t * LDV + vloc]) - sEB[t] * ks[i]);
                }
                yb[I] = Gp::make(y);
            }
            G4 ub[NB];
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                f32x4 u = zero4();
                tile_mma_lr_n<NB>(u, sT + 16 * I * LDC, LDC, yb, I + 1, lane);
                ub[I] = Gp::make(u);
            }
#pragma unroll
            for (int I = 0; I < NB; ++I) {
                f32x4 o = zero4();
                tile_mma_lr_n<NB>(o, sP + 16 * I * LDC, LDC, ub, I + 1, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * I + 4 * lg + i;
                    from_f32(sO[t * LDO + vloc], o[i] + sEB[t] * qs[I][i]);
                }
            }
            const float decay = sDecay;
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
                for (int i = 0; i < 4; ++i) st[cb][i] *= decay;
                tile_mma_lr<NB>(st[cb], sKt + 16 * cb * LDC, LDC, ub, lane);
            }
        }
        __syncthreads();
        // the block's output rows, 16 bytes per lane
        for (int e = tid; e < n * (DVB / VE); e += NTHR) {
            const int t = e / (DVB / VE), v = (e % (DVB / VE)) * VE;
            *reinterpret_cast<uint4 *>(oh + static_cast<size_t>(c0 + t) * p.d_v + vb * DVB + v) =
                *reinterpret_cast<const uint4 *>(sO + t * LDO + v);
        }
    }

    if (p.S_T && wave < WS) {
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
size_t chunk_workspace_bytes(const ChunkArgs &) { return 0; }
hipError_t launch_chunk(const ChunkArgs &a) {
    return a.variant == LA_GATED_DELTA ? launch_chunk_gdr(a) : launch_chunk_linear(a);
}

hipError_t launch_chunk_gdr(const ChunkArgs &a) {
    if (a.dtype == LA_BF16) return gdr_dk<BF16>(a);
    return gdr_dk<F32>(a);
}

}  // namespace la
