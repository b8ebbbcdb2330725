// la_chunk_segment.hip -- normalized linear attention and retention over
// sequence segments held whole in LDS (gfx950).
//
// Page "Beyond -- Linear attention and recurrent memory", sections "The big
// idea" and "Fixed decay versus an input-dependent gate"; page "Ch. 11 Linear
// attention and Hyena", 11.2 and 11.3 (RetNet bullet).  The state of these
// variants is a (decayed) sum over the tokens, so a sequence cut into
// segments of L tokens runs all its segments at once:
//
//   seg_increment_kernel, one workgroup per (head, segment s), n_s tokens:
//       dS_s = sum_t gamma^(n_s-1-t) v_t phi(k_t)^T,
//       dz_s = sum_t gamma^(n_s-1-t) phi(k_t)
//     into slot s+1 of the workspace; segment 0's workgroup also copies
//     (S0, z0) into slot 0 (so that S_T may alias S0).
//
//   seg_attention_kernel, one workgroup per (head, segment s): the entering
//   state S_s = gamma^(sL) S0 + sum_{i<s} gamma^((s-1-i)L) dS_i (z likewise),
//   and the segment's outputs in the masked-parallel form, t and j counted
//   from the segment start,
//       P_tj = [j <= t] gamma^(t-j) phi(q_t).phi(k_j)
//       O    = (gamma^(t+1) phiQ S_s^T + P V) / (gamma^(t+1) phiQ z_s + P 1);
//   the last segment also writes S_T = gamma^(n_s) S_s + dS_s (z_T likewise).
//
// Every 16 x 16 tile of P is formed on the matrix cores as (phiK_J)(phiQ_I)^T,
// whose result layout is the B operand of the next product, so P never goes
// through LDS: it is rounded to the operand type once and feeds both V^T P^T
// and the denominator, a product with a tile of ones (the denominator uses
// the same rounded P as the numerator).  The normalizer's state term is the
// same product with 16 copies of z appended below the state rows.  Every
// decay power is at most 1: gamma^(t-j) of an off-diagonal tile is formed as
// gamma^(lr + 16 - j_in) * gamma^(16 (I - J - 1)), both exponents >= 0.
#include <algorithm>

#include "la_chunk_common.hpp"

namespace la {

struct SegParams {
    const void *q, *k, *v;
    const float *gamma;       // fixed per-head decay (H,), or null (none)
    const float *S0, *z0;     // initial state, or null (zeros)
    void *out;
    float *S_T, *z_T;         // final state, or null
    float *slots;             // [head][n_seg + 1][d_v * d_k + d_k] float32
    int T, H, n_heads, seg_len, n_seg;
};

// LDS row strides (elements).  bf16 tiles read a row per lane, 8 bytes at a
// time, 16 rows per 16-lane group (Q, K and the state in the output kernel):
// a stride of 2 mod 4 dwords puts the 16 rows on distinct bank pairs.  bf16
// tiles read transposed (ds_read_b64_tr_b16: four rows of 32 bytes per
// 16-lane group): a stride of 8 mod 32 dwords puts the four rows on distinct
// banks, and keeps rows 16-byte aligned for the staging stores.  float32
// tiles: 16 bytes of padding.
template <class Op, int D>
struct SegStride {
    static constexpr int ROW = sizeof(Op) == 2 ? D + 4 : D + 4;    // row-wise reads
    static constexpr int TR = sizeof(Op) == 2 ? D + 16 : D + 4;    // transposed reads
};

template <class DT, int DK, int DV, int L>
struct SegLds {
    typedef typename OpOf<DT>::type Op;
    static constexpr int LDK = SegStride<Op, DK>::ROW, LDV = SegStride<Op, DV>::TR;
    static constexpr int SROWS = DV + 16;   // state rows, then 16 copies of z
    static constexpr int BYTES = (2 * L * LDK + L * LDV + SROWS * LDK) * (int)sizeof(Op);
    static constexpr bool FITS = BYTES <= 160 * 1024;
    // the increment kernel reads both of its tiles transposed
    static constexpr int ILDK = SegStride<Op, DK>::TR, ILDV = SegStride<Op, DV>::TR;
};

// Longest segment whose tiles fit in LDS (0: none of 64, 128, 256 does).
template <class DT, int DK, int DV>
constexpr int seg_lmax() {
    return SegLds<DT, DK, DV, 256>::FITS ? 256 : SegLds<DT, DK, DV, 128>::FITS ? 128
                                                 : SegLds<DT, DK, DV, 64>::FITS ? 64 : 0;
}

constexpr int kSegIncrThreads = 1024;   // increment kernel: sixteen waves
constexpr int kSegThreads = 512;        // output kernel: eight waves

// workgroup -> (segment, head): segments in order of the workgroup id, the
// heads of a segment dealt so that one head's segments share an XCD
__device__ __forceinline__ void seg_block(int bid, int n_heads, int &s, int &bh) {
    s = bid / n_heads;
    int vb;
    block_to_head(bid - s * n_heads, n_heads, 1, bh, vb);
}

__device__ __forceinline__ float uniform_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}

// log2 of head bh's decay (0 without one)
__device__ __forceinline__ float seg_log2_gamma(const SegParams &p, int bh) {
    return uniform_f(p.gamma ? __builtin_amdgcn_logf(p.gamma[bh % p.H]) : 0.f);
}

// Commit a staged token-major tile to LDS with phi applied and each row t
// scaled by w(t); rows past the valid ones (and padding lanes) hold zeros.
template <int PHI, int NTHR, class IO, class Op, class TP, class W>
__device__ __forceinline__ void commit_phi(const TP &tp, Op *dst, int ld, int tid, W w) {
    typedef Group<Op> Gp;
#pragma unroll
    for (int i = 0; i < TP::PER; ++i) {
        const int e = tid + i * NTHR;
        if (TP::TOTAL % NTHR != 0 && e >= TP::TOTAL) continue;
        const int t = e / TP::VPR, c = (e % TP::VPR) * TP::VE;
        const bool ok = (tp.valid >> i) & 1u;
        const uint4 r = tp.r[i];
        float x[8];
        if constexpr (sizeof(IO) == 2) {
            x[0] = lo_bf16(r.x); x[1] = hi_bf16(r.x); x[2] = lo_bf16(r.y); x[3] = hi_bf16(r.y);
            x[4] = lo_bf16(r.z); x[5] = hi_bf16(r.z); x[6] = lo_bf16(r.w); x[7] = hi_bf16(r.w);
        } else {
            x[0] = __uint_as_float(r.x); x[1] = __uint_as_float(r.y);
            x[2] = __uint_as_float(r.z); x[3] = __uint_as_float(r.w);
        }
        const float s = ok ? w(t) : 0.f;
#pragma unroll
        for (int j = 0; j < TP::VE; ++j) x[j] = ok ? apply_phi<PHI>(x[j]) * s : 0.f;
#pragma unroll
        for (int j = 0; j < TP::VE; j += 4) st_group(dst + t * ld + c + j, Gp::make(x[j], x[j + 1], x[j + 2], x[j + 3]));
    }
}

// ------------------------------------------------------------------ increments
// dS_s (value tile vt x key tile kt, contraction over the segment's tokens,
// both operands by transposing reads of the token-major tiles) and, with the
// normalizer, dz_s as the product of a tile of ones with phi(K).  The 16x16
// tiles are dealt to the sixteen waves round robin.
template <int PHI, bool NORM, class DT, int DK, int DV, int L>
__global__ void __launch_bounds__(kSegIncrThreads) seg_increment_kernel(const SegParams p) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef Group<Op> Gp;
    typedef SegLds<DT, DK, DV, L> Lds;
    constexpr int NTHR = kSegIncrThreads, LDK = Lds::ILDK, LDV = Lds::ILDV;
    constexpr int NKT = DK / 16, NVO = DV / 16, NVT = NVO + (NORM ? 1 : 0);
    constexpr int NTILE = NVT * NKT, TPW = (NTILE + 15) / 16;
    __shared__ __align__(16) Op sK[L * LDK];
    __shared__ __align__(16) Op sV[L * LDV];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    int s, bh;
    seg_block(blockIdx.x, p.n_heads, s, bh);
    const size_t slot = static_cast<size_t>(DV) * DK + DK;
    float *base = p.slots + static_cast<size_t>(bh) * (p.n_seg + 1) * slot;
    const int tb = s * p.seg_len, n = min(p.seg_len, p.T - tb);
    const size_t tok0 = static_cast<size_t>(bh) * p.T + tb;

    TilePrefetch<L, DK, NTHR, IO> pk;
    TilePrefetch<L, DV, NTHR, IO> pv;
    pk.load(static_cast<const IO *>(p.k) + tok0 * DK, DK, n, tid);
    pv.load(static_cast<const IO *>(p.v) + tok0 * DV, DV, n, tid);

    if (s == 0) {
        // slot 0: the initial state (zeros when absent)
        const float4 *S0 = p.S0 ? reinterpret_cast<const float4 *>(p.S0 + static_cast<size_t>(bh) * DV * DK) : nullptr;
        for (int e = tid; e < DV * DK / 4; e += NTHR)
            reinterpret_cast<float4 *>(base)[e] = S0 ? S0[e] : make_float4(0.f, 0.f, 0.f, 0.f);
        for (int c = tid; c < DK; c += NTHR) base[DV * DK + c] = p.z0 ? p.z0[static_cast<size_t>(bh) * DK + c] : 0.f;
    }

    // phi(k_t) gamma^(n-1-t), rounded to the operand type once for both sums
    const float l2g = seg_log2_gamma(p, bh);
    const bool decay = l2g != 0.f;
    commit_phi<PHI, NTHR, IO>(pk, sK, LDK, tid, [&](int t) {
        return decay ? __builtin_amdgcn_exp2f(static_cast<float>(n - 1 - t) * l2g) : 1.f;
    });
    pv.store(sV, LDV, tid);
    __syncthreads();

    const int nst = (n + 15) >> 4;   // 16-token steps that hold tokens
    typename Gp::type ones = Gp::make(1.f, 1.f, 1.f, 1.f);
    float *dst = base + static_cast<size_t>(s + 1) * slot;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int tile = wave + 16 * i;
        if (tile >= NTILE) break;
        const int vt = tile / NKT, kt = tile % NKT;
        const bool zt = NORM && vt == NVO;
        f32x4 acc = zero4();
        int st = 0;
        for (; st + 2 <= nst; st += 2) {
            const int t0 = 16 * st;
            const auto a0 = zt ? ones : kt_group<0>(sV, LDV, t0, 16 * (zt ? 0 : vt), lane);
            const auto a1 = zt ? ones : kt_group<0>(sV, LDV, t0 + 16, 16 * (zt ? 0 : vt), lane);
            mma32(acc, a0, a1, kt_group<0>(sK, LDK, t0, 16 * kt, lane), kt_group<0>(sK, LDK, t0 + 16, 16 * kt, lane));
        }
        if (st < nst) {
            const int t0 = 16 * st;
            mma16(acc, zt ? ones : kt_group<0>(sV, LDV, t0, 16 * (zt ? 0 : vt), lane), kt_group<0>(sK, LDK, t0, 16 * kt, lane));
        }
        if (!zt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[static_cast<size_t>(16 * vt + 4 * lg + r) * DK + 16 * kt + lr] = acc[r];
        } else if (lg == 0) {
            dst[static_cast<size_t>(DV) * DK + 16 * kt + lr] = acc[0];   // every row of the tile is the sum
        }
    }
}

// ------------------------------------------------------------------ outputs
// Eight waves, two per SIMD.  A segment of L tokens has L/32 pairs of query
// tiles; wave w takes the pair seg_qpair(w) (two independent chains of
// matrix-core steps that share every key and value operand read) and, when
// there are fewer than eight pairs, one of 8/(L/32) equal shares of the value
// tiles (each share forms the pair's scores itself).  The work of pair p
// grows with p + 1; the pairs are dealt so that both waves of a SIMD carry
// the same total.
__device__ __forceinline__ void seg_qpair(int w, int npair, int &pair, int &split) {
    const int s = w & 3, m = w >> 2;   // SIMD of the wave, its slot on that SIMD
    if (npair == 8) {
        pair = m == 0 ? s : 7 - s;
        split = 0;
    } else if (npair == 4) {
        pair = m == 0 ? s : 3 - s;
        split = m;
    } else {
        pair = m;
        split = s;
    }
}

template <int PHI, bool NORM, class DT, int DK, int DV, int L>
__global__ void __launch_bounds__(kSegThreads) seg_attention_kernel(const SegParams p) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef Group<Op> Gp;
    typedef typename Gp::type G4;
    typedef SegLds<DT, DK, DV, L> Lds;
    constexpr int NTHR = kSegThreads, LDK = Lds::LDK, LDV = Lds::LDV;
    constexpr int NQP = L / 32;                    // query tile pairs of a whole segment
    static_assert(NQP == 2 || NQP == 4 || NQP == 8, "segment length");
    constexpr int NSPLIT = 8 / NQP;                // waves per pair
    constexpr int NVO = DV / 16, NVW = NVO / NSPLIT;   // value tiles, per wave
    static_assert(NVW >= 1 && NVW * NSPLIT == NVO, "value split");
    constexpr int NACC = NVW + (NORM ? 1 : 0);
    constexpr int NKG = DK / 16;                   // operand groups along d_k
    constexpr bool KPF = DK == 64;                 // key operands loaded a pair ahead
    static_assert(DV * DK % (4 * NTHR) == 0, "state split");
    constexpr int SPER = DV * DK / (4 * NTHR);     // float4 of one slot's state per thread
    constexpr int NSB = 16 / SPER;                 // slots per batch of loads
    static_assert(NSB >= 1, "slot batch");
    __shared__ __align__(16) Op sQ[L * LDK];
    __shared__ __align__(16) Op sK[L * LDK];
    __shared__ __align__(16) Op sV[L * LDV];
    __shared__ __align__(16) Op sS[Lds::SROWS * LDK];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    int s, bh;
    seg_block(blockIdx.x, p.n_heads, s, bh);
    const bool last = s == p.n_seg - 1;
    const int tb = s * p.seg_len, n = min(p.seg_len, p.T - tb);
    const size_t tok0 = static_cast<size_t>(bh) * p.T + tb;
    const size_t slot = static_cast<size_t>(DV) * DK + DK;
    const float *base = p.slots + static_cast<size_t>(bh) * (p.n_seg + 1) * slot;

    // ---- stage the segment: phi(Q), phi(K) and V, rows past n zero
    {
        TilePrefetch<L, DK, NTHR, IO> pq, pk;
        TilePrefetch<L, DV, NTHR, IO> pv;
        pq.load(static_cast<const IO *>(p.q) + tok0 * DK, DK, n, tid);
        pk.load(static_cast<const IO *>(p.k) + tok0 * DK, DK, n, tid);
        pv.load(static_cast<const IO *>(p.v) + tok0 * DV, DV, n, tid);
        commit_phi<PHI, NTHR, IO>(pq, sQ, LDK, tid, [](int) { return 1.f; });
        commit_phi<PHI, NTHR, IO>(pk, sK, LDK, tid, [](int) { return 1.f; });
        pv.store(sV, LDV, tid);
    }
    __syncthreads();

    // ---- slots of the entering state (and, in the last segment, its own
    // increment): loaded NSB at a time, every load issued on every path
    // (indices past the last slot re-read it and are not used)
    const int nread = s + 1 + (last ? 1 : 0);
    float4 sb[NSB][SPER];
    float zb[NSB];   // z element tid (threads below d_k)
    auto issue = [&](int i0) {
#pragma unroll
        for (int j = 0; j < NSB; ++j) {
            const float *src = base + static_cast<size_t>(min(i0 + j, nread - 1)) * slot;
#pragma unroll
            for (int u = 0; u < SPER; ++u) sb[j][u] = reinterpret_cast<const float4 *>(src)[tid + u * NTHR];
            zb[j] = src[DV * DK + min(tid, DK - 1)];
        }
    };
    issue(0);

    const float l2g = seg_log2_gamma(p, bh);
    const bool decay = l2g != 0.f;
    // per-lane decay factors of P tile entries (key row 4lg + r of block J,
    // query column lr of block I): diagonal tiles gamma^(lr - 4lg - r) (zero
    // above the diagonal), off-diagonal tiles gamma^(lr + 16 - 4lg - r) times
    // the uniform gamma^(16 (I - J - 1))
    float fdiag[4], foff[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int dd = lr - 4 * lg - r;
        fdiag[r] = dd < 0 ? 0.f : (decay ? __builtin_amdgcn_exp2f(static_cast<float>(dd) * l2g) : 1.f);
        foff[r] = decay ? __builtin_amdgcn_exp2f(static_cast<float>(dd + 16) * l2g) : 1.f;
    }
    const float g16 = decay ? __builtin_amdgcn_exp2f(16.f * l2g) : 1.f;   // gamma^16
    const G4 ones = Gp::make(1.f, 1.f, 1.f, 1.f);

    int pr, split;
    seg_qpair(wave, NQP, pr, split);
    const int I0 = 2 * pr;            // query tiles I0 and I0 + 1
    const bool active = 16 * I0 < n;  // the pair holds tokens
    const int vt0 = split * NVW;      // first value tile of this wave

    // ---- within the segment: O^T += V^T P^T, den += 1^T P^T.  Key blocks
    // J < I0 go in pairs (one k32 step of the value product per pair), below
    // the diagonal of both tiles, with the next pair's key operands loaded a
    // pair ahead; blocks I0 and I0 + 1 come last.
    f32x4 o0[NACC], o1[NACC];
#pragma unroll
    for (int a = 0; a < NACC; ++a) o0[a] = o1[a] = zero4();
    G4 q0[NKG], q1[NKG];   // phi(Q) operand groups of the two tiles
    if (active) {
        {
            const Op *qrow = sQ + (16 * I0 + lr) * LDK + 4 * lg;
#pragma unroll
            for (int g = 0; g < NKG; ++g) {
                q0[g] = ld_group(qrow + 16 * g);
                q1[g] = ld_group(qrow + 16 * LDK + 16 * g);
            }
        }
        auto kload = [&](int J, G4 (&kg)[NKG]) {
            const Op *krow = sK + (16 * J + lr) * LDK + 4 * lg;
#pragma unroll
            for (int g = 0; g < NKG; ++g) kg[g] = ld_group(krow + 16 * g);
        };
        // P_IJ^T (rows = keys of block J, columns = queries of block I) from
        // key and query groups, times the decay factors f * blk
        auto score = [&](const G4 (&kg)[NKG], const G4 (&qg)[NKG], const float (&f)[4], float blk) {
            f32x4 acc = zero4();
#pragma unroll
            for (int g = 0; g + 2 <= NKG; g += 2) mma32(acc, kg[g], kg[g + 1], qg[g], qg[g + 1]);
            if constexpr (NKG % 2 == 1) mma16(acc, kg[NKG - 1], qg[NKG - 1]);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] *= f[r] * blk;
            return Gp::make(acc);
        };
        auto vload = [&](int J, G4 (&vg)[NVW]) {
#pragma unroll
            for (int a = 0; a < NVW; ++a) vg[a] = kt_group<0>(sV, LDV, 16 * J, 16 * (vt0 + a), lane);
        };
        G4 kA[NKG], kB[NKG];
        kload(0, kA);
        kload(1, kB);
        for (int J = 0; J < I0; J += 2) {
            // this pair's value operands, then the next pair's key operands
            // (d_k = 128: loaded at the top of each pair instead, for registers)
            G4 va[NVW], vb[NVW];
            vload(J, va);
            vload(J + 1, vb);
            G4 nA[NKG], nB[NKG];
            if constexpr (KPF) {
                kload(J + 2, nA);
                kload(J + 3, nB);
            } else if (J > 0) {
                kload(J, kA);
                kload(J + 1, kB);
            }
            // gamma^(16 (I0 - J - 1)) and gamma^(16 (I0 - J - 2)) for blocks J and
            // J + 1 against tile I0 (both exponents >= 0); tile I0 + 1 has one
            // more block of decay
            const float blk = decay ? __builtin_amdgcn_exp2f(static_cast<float>(16 * (I0 - J - 1)) * l2g) : 1.f;
            const float blkB = decay ? __builtin_amdgcn_exp2f(static_cast<float>(16 * (I0 - J - 2)) * l2g) : 1.f;
            const G4 a0 = score(kA, q0, foff, blk), b0 = score(kB, q0, foff, blkB);
            const G4 a1 = score(kA, q1, foff, blk * g16), b1 = score(kB, q1, foff, blkB * g16);
#pragma unroll
            for (int a = 0; a < NVW; ++a) {
                mma32(o0[a], va[a], vb[a], a0, b0);
                mma32(o1[a], va[a], vb[a], a1, b1);
            }
            if constexpr (NORM) {
                mma32(o0[NVW], ones, ones, a0, b0);
                mma32(o1[NVW], ones, ones, a1, b1);
            }
            if constexpr (KPF) {
#pragma unroll
                for (int g = 0; g < NKG; ++g) {
                    kA[g] = nA[g];
                    kB[g] = nB[g];
                }
            }
        }
        if constexpr (!KPF) {
            if (I0 > 0) {
                kload(I0, kA);
                kload(I0 + 1, kB);
            }
        }
        // kA, kB hold key blocks I0 and I0 + 1: tile I0 takes block I0 on its
        // diagonal; tile I0 + 1 takes block I0 just below its diagonal and
        // block I0 + 1 on it
        G4 va[NVW], vb[NVW];
        vload(I0, va);
        vload(I0 + 1, vb);
        const G4 d0 = score(kA, q0, fdiag, 1.f);
        const G4 a1 = score(kA, q1, foff, 1.f), b1 = score(kB, q1, fdiag, 1.f);
#pragma unroll
        for (int a = 0; a < NVW; ++a) {
            mma16(o0[a], va[a], d0);
            mma32(o1[a], va[a], vb[a], a1, b1);
        }
        if constexpr (NORM) {
            mma16(o0[NVW], ones, d0);
            mma32(o1[NVW], ones, ones, a1, b1);
        }
    }

    // ---- entering state S_s = sum_{i <= s} w_i slot_i in float32 (slot 0 the
    // initial state, weight gamma^(sL); slot i the increment of segment i-1,
    // weight gamma^((s-i)L)); the last segment keeps its own increment apart
    float4 se[SPER], own[SPER];
    float ze = 0.f, zown = 0.f;
#pragma unroll
    for (int u = 0; u < SPER; ++u) se[u] = own[u] = make_float4(0.f, 0.f, 0.f, 0.f);
    auto add4 = [](float4 &d, const float4 &x, float w) {
        d.x += w * x.x; d.y += w * x.y; d.z += w * x.z; d.w += w * x.w;
    };
    auto accumulate = [&](int i0) {
#pragma unroll
        for (int j = 0; j < NSB; ++j) {
            const int i = i0 + j;
            if (i <= s) {
                const int steps = i == 0 ? s : s - i;   // whole segments of decay
                const float w = decay ? __builtin_amdgcn_exp2f(static_cast<float>(steps * p.seg_len) * l2g) : 1.f;
#pragma unroll
                for (int u = 0; u < SPER; ++u) add4(se[u], sb[j][u], w);
                ze += w * zb[j];
            } else if (i == s + 1 && last) {
#pragma unroll
                for (int u = 0; u < SPER; ++u) own[u] = sb[j][u];
                zown = zb[j];
            }
        }
    };
    accumulate(0);
    for (int i0 = NSB; i0 < nread; i0 += NSB) {
        issue(i0);
        accumulate(i0);
    }
    // the state rows (value-major, key channels contiguous) and, with the
    // normalizer, 16 copies of z below them, as matrix-core operands
#pragma unroll
    for (int u = 0; u < SPER; ++u) {
        const int e = 4 * (tid + u * NTHR), vr = e / DK, c = e % DK;
        st_group(sS + vr * LDK + c, Gp::make(se[u].x, se[u].y, se[u].z, se[u].w));
    }
    if constexpr (NORM) {
        if (tid < DK) {
            Op zo;
            from_f32(zo, ze);
#pragma unroll
            for (int r = 0; r < 16; ++r) sS[(DV + r) * LDK + tid] = zo;
        }
    }
    if (last) {
        // S_T = gamma^n S_s + dS_s, z_T likewise (float32 throughout)
        const float wn = decay ? __builtin_amdgcn_exp2f(static_cast<float>(n) * l2g) : 1.f;
        if (p.S_T) {
            float4 *dstS = reinterpret_cast<float4 *>(p.S_T + static_cast<size_t>(bh) * DV * DK);
#pragma unroll
            for (int u = 0; u < SPER; ++u) {
                float4 x = own[u];
                add4(x, se[u], wn);
                dstS[tid + u * NTHR] = x;
            }
        }
        if (NORM && p.z_T && tid < DK) p.z_T[static_cast<size_t>(bh) * DK + tid] = zown + wn * ze;
    }
    __syncthreads();

    // ---- state term gamma^(t+1) S_s phi(q_t) (and phiQ z_s), normalize, store
    if (active) {
        const int t0 = 16 * I0 + lr, t1 = t0 + 16;
        const float lead0 = decay ? __builtin_amdgcn_exp2f(static_cast<float>(t0 + 1) * l2g) : 1.f;
        const float lead1 = lead0 * g16;
#pragma unroll
        for (int a = 0; a < NACC; ++a) {
            // state rows of value tile vt0 + a, or the z rows for the denominator
            const int row0 = (NORM && a == NVW) ? DV : 16 * (vt0 + a);
            G4 sg[NKG];
            const Op *srow = sS + (row0 + lr) * LDK + 4 * lg;
#pragma unroll
            for (int g = 0; g < NKG; ++g) sg[g] = ld_group(srow + 16 * g);
            auto term = [&](f32x4 &x0, f32x4 &x1) {
#pragma unroll
                for (int g = 0; g + 2 <= NKG; g += 2) {
                    mma32(x0, sg[g], sg[g + 1], q0[g], q0[g + 1]);
                    mma32(x1, sg[g], sg[g + 1], q1[g], q1[g + 1]);
                }
                if constexpr (NKG % 2 == 1) {
                    mma16(x0, sg[NKG - 1], q0[NKG - 1]);
                    mma16(x1, sg[NKG - 1], q1[NKG - 1]);
                }
            };
            if (decay) {
                f32x4 x0 = zero4(), x1 = zero4();
                term(x0, x1);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    o0[a][r] += lead0 * x0[r];
                    o1[a][r] += lead1 * x1[r];
                }
            } else {
                term(o0[a], o1[a]);   // no decay: straight into the accumulators
            }
        }
        // the denominators are positive (phi > 0): hardware reciprocal (1 ulp)
        const float inv0 = NORM ? __builtin_amdgcn_rcpf(o0[NACC - 1][0]) : 1.f;
        const float inv1 = NORM ? __builtin_amdgcn_rcpf(o1[NACC - 1][0]) : 1.f;
        IO *orow = static_cast<IO *>(p.out) + (tok0 + t0) * DV + 16 * vt0 + 4 * lg;
        if (t0 < n) {
#pragma unroll
            for (int a = 0; a < NVW; ++a)
                st_group(orow + 16 * a, Gp::make(o0[a][0] * inv0, o0[a][1] * inv0, o0[a][2] * inv0, o0[a][3] * inv0));
        }
        if (t1 < n) {
#pragma unroll
            for (int a = 0; a < NVW; ++a)
                st_group(orow + 16 * DV + 16 * a,
                         Gp::make(o1[a][0] * inv1, o1[a][1] * inv1, o1[a][2] * inv1, o1[a][3] * inv1));
        }
    }
}

// ------------------------------------------------------------------ dispatch

namespace {

// float4 of one slot's state per thread of the output kernel
int seg_slot_quads(const ChunkArgs &a) { return a.d_v * a.d_k / (4 * kSegThreads); }
// slots per batch of loads of the output kernel
int seg_slot_batch(const ChunkArgs &a) { return 16 / seg_slot_quads(a); }

int seg_lmax_rt(const ChunkArgs &a) {
    const bool bf = a.dtype == LA_BF16;
    if (a.d_k == 64 && a.d_v == 64) return bf ? seg_lmax<BF16, 64, 64>() : seg_lmax<F32, 64, 64>();
    if (a.d_k == 64 && a.d_v == 128) return bf ? seg_lmax<BF16, 64, 128>() : seg_lmax<F32, 64, 128>();
    if (a.d_k == 128 && a.d_v == 64) return bf ? seg_lmax<BF16, 128, 64>() : seg_lmax<F32, 128, 64>();
    if (a.d_k == 128 && a.d_v == 128) return bf ? seg_lmax<BF16, 128, 128>() : seg_lmax<F32, 128, 128>();
    return 0;
}

}  // namespace

// The segment path serves the normalized and retention variants (d_k, d_v in
// {64, 128}) when the heads alone leave most compute units idle (fewer than
// 256 workgroups of up to 64 value channels) and the slots a workgroup sums
// stay few: segments as long as LDS allows, halved (down to 64 tokens) while
// that still gives at most one workgroup per compute unit.
bool seg_plan(const ChunkArgs &a, int &seg_len, int &n_seg) {
    if ((a.variant != LA_NORMALIZED && a.variant != LA_RETENTION) || a.T <= 0) return false;
    const int lmax = seg_lmax_rt(a);
    if (lmax == 0) return false;
    const int64_t heads = static_cast<int64_t>(a.B) * a.H;
    if (heads * (a.d_v / std::min(a.d_v, 64)) >= 256) return false;
    // a workgroup loads at most two batches of slots (the last segment reads
    // n_seg + 1 of them)
    const int max_slots = 2 * seg_slot_batch(a);
    int L = lmax;
    while (L > 64) {
        const int64_t ns2 = (a.T + L / 2 - 1) / (L / 2);
        if (heads * ns2 > 256 || ns2 + 1 > max_slots) break;
        L /= 2;
    }
    const int ns = (a.T + L - 1) / L;
    if (ns + 1 > max_slots) return false;
    seg_len = L;
    n_seg = ns;
    return true;
}

size_t seg_workspace_bytes(const ChunkArgs &a) {
    int L, ns;
    if (!seg_plan(a, L, ns)) return 0;
    return static_cast<size_t>(a.B) * a.H * (ns + 1) * (static_cast<size_t>(a.d_v) * a.d_k + a.d_k) * sizeof(float);
}

template <int PHI, bool NORM, class DT, int DK, int DV>
static hipError_t launch_seg_t(const ChunkArgs &a, int seg_len, int n_seg) {
    constexpr int L = seg_lmax<DT, DK, DV>();
    if constexpr (L == 0) {
        return hipErrorInvalidValue;
    } else {
        SegParams p;
        p.q = a.q; p.k = a.k; p.v = a.v;
        p.gamma = a.gate; p.S0 = a.S0; p.z0 = NORM ? a.z0 : nullptr;
        p.out = a.out; p.S_T = a.S_T; p.z_T = NORM ? a.z_T : nullptr;
        p.slots = static_cast<float *>(a.workspace);
        p.T = a.T; p.H = a.H; p.n_heads = a.B * a.H; p.seg_len = seg_len; p.n_seg = n_seg;
        const dim3 grid(static_cast<uint32_t>(p.n_heads * n_seg));
        hipLaunchKernelGGL((seg_increment_kernel<PHI, NORM, DT, DK, DV, L>), grid, dim3(kSegIncrThreads), 0, a.stream, p);
        hipLaunchKernelGGL((seg_attention_kernel<PHI, NORM, DT, DK, DV, L>), grid, dim3(kSegThreads), 0, a.stream, p);
        return hipGetLastError();
    }
}

template <int PHI, bool NORM, class DT>
static hipError_t launch_seg_dt(const ChunkArgs &a, int L, int ns) {
    if (a.d_k == 64 && a.d_v == 64) return launch_seg_t<PHI, NORM, DT, 64, 64>(a, L, ns);
    if (a.d_k == 64 && a.d_v == 128) return launch_seg_t<PHI, NORM, DT, 64, 128>(a, L, ns);
    if (a.d_k == 128 && a.d_v == 64) return launch_seg_t<PHI, NORM, DT, 128, 64>(a, L, ns);
    if (a.d_k == 128 && a.d_v == 128) return launch_seg_t<PHI, NORM, DT, 128, 128>(a, L, ns);
    return hipErrorInvalidValue;
}

template <int PHI, bool NORM>
static hipError_t launch_seg_v(const ChunkArgs &a, int L, int ns) {
    if (a.dtype == LA_BF16) return launch_seg_dt<PHI, NORM, BF16>(a, L, ns);
    return launch_seg_dt<PHI, NORM, F32>(a, L, ns);
}

hipError_t launch_seg(const ChunkArgs &a) {
    int L, ns;
    if (!seg_plan(a, L, ns)) return hipErrorInvalidValue;
    // normalized attention always uses elu+1; retention takes the caller's map
    if (a.variant == LA_NORMALIZED) return launch_seg_v<LA_PHI_ELU1, true>(a, L, ns);
    if (a.phi == LA_PHI_ELU1) return launch_seg_v<LA_PHI_ELU1, false>(a, L, ns);
    return launch_seg_v<LA_PHI_IDENTITY, false>(a, L, ns);
}

}  // namespace la
