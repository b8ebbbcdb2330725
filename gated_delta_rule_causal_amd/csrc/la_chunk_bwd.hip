// la_chunk_bwd.hip -- chunked backward (gradients) of normalized linear
// attention and of retention (gfx950).
//
// Both recurrences (page "Beyond -- Linear attention and recurrent memory",
// sections "The big idea" and "Fixed decay versus an input-dependent gate";
// page "Ch. 11 Linear attention and Hyena", 11.3, RetNet bullet) are linear
// in their state, and the pages name chunkwise training as the reason chunked
// kernels exist without giving one.  The gradient below is derived from the
// recurrence.  Values are augmented with a constant 1, so that the
// normalizer z is one more state column (normalized variant only); for a
// chunk of n tokens that enters with state S'_c and leaves with cotangent
// dS'_{c+1}, and with D_tj = gamma^(t-j) for j <= t (0 above):
//   dO'   = [dO / den, -(dO . o) / den]     (retention: dO' = dO)
//   A     = D o (phiQ phiK^T),   G = D o (dO' V'^T)
//   dphiQ = G phiK + diag(gamma^(t+1)) (dO' S'_c)
//   dphiK = G^T phiQ + diag(gamma^(n-1-j)) (V' dS'_{c+1})
//   dV    = A^T dO'[:, :d_v] + diag(gamma^(n-1-j)) phiK dS_{c+1}^T
//   S'_{c+1} = gamma^n S'_c + phiK^T diag(gamma^(n-1-j)) V'
//   dS'_c    = gamma^n dS'_{c+1} + phiQ^T diag(gamma^(t+1)) dO'
// and dq = dphiQ phi'(q), dk = dphiK phi'(k).  The decay's gradient, chunk
// by chunk with the entering state held fixed (every term below has a
// non-negative weight):
//   d(ln gamma) = sum_t (t+1) phi(q_t).X_t + sum_{j<=t} (t-j) A_tj H_tj
//               + sum_j (n-1-j) phi(k_j).Y_j + n gamma^n <dS'_{c+1}, S'_c>
// with H = dO' V'^T and X, Y the state terms of dphiQ and dphiK.
//
// Launches, in order:
//   1. bwd_increments_kernel (one workgroup per chunk): the chunk's state
//      increment phiK^T diag(gamma^(n-1-j)) V' on the matrix cores, and for
//      retention also its cotangent increment phiQ^T diag(gamma^(t+1)) dO;
//   2. bwd_scan_kernel (one lane per state element of a head): the forward
//      scan turns the increments into the state entering every chunk, in
//      place (retention: the reverse scan of step 4 in the same launch);
//   3. normalized only, bwd_normalizer_kernel (one workgroup per chunk): every
//      token's output and denominator again, in float32 from float32 features
//      and the entering state, hence 1/den_t and dden_t, and the chunk's
//      cotangent increment.  The gradient with respect to q nearly cancels
//      between its value and normalizer parts (phi(x) = elu(x) + 1 is close to
//      1 for small x), so the output it uses must be this exact; the forward's
//      rounded output would not do;
//   4. bwd_scan_kernel: the reverse scan turns the cotangent increments into
//      the cotangent leaving every chunk, in place, and ends in dS0, dz0;
//   5. bwd_grad_kernel (one workgroup per chunk; retention in bf16: persistent,
//      one workgroup per CU, the next chunk's loads in flight): dq, dk, dv and
//      the chunk's share of d(ln gamma);
//   6. bwd_dgate_kernel (one workgroup per head, only when the decay's
//      gradient is asked for): the shares summed over batch and chunks.
// The states are float32 in the workspace, key-major ([key channel][value
// channel], then z): the layout in which the gradient kernel reads them as
// matrix-core operands.
#include <algorithm>

#include "la_chunk_common.hpp"

namespace la {

struct BwdParams {
    const void *q, *k, *v, *dout;
    const float *gate, *S0, *z0, *dS_T, *dz_T;
    void *dq, *dk, *dv;
    float *dS0, *dz0, *dgate;
    // workspace: states, cotangents, decay-gradient shares, and (normalized)
    // 1/den_t and dden_t of every token
    float *slot_f, *slot_r, *part, *tok;
    int B, H, T, n_chunk, normalize, elu;
};

namespace {

__device__ __forceinline__ float phi_rt(float x, bool elu) { return elu ? phi_elu1(x) : x; }
// derivative of the feature map: 1 above zero and e^x at or below for elu + 1
__device__ __forceinline__ float dphi_rt(float x, bool elu) { return elu && !(x > 0.f) ? __expf(x) : 1.f; }

__device__ __forceinline__ float uniform_f(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, x)));
}
// log2 of the head's fixed decay, 0 without one
__device__ __forceinline__ float head_l2g(const BwdParams &p, int bh) {
    return uniform_f(p.gate ? __builtin_amdgcn_logf(p.gate[bh % p.H]) : 0.f);
}

// one 16-byte vector of elements as floats (4 float32 or 8 bf16)
__device__ __forceinline__ void load16(const float *p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void load16(const bf16_t *p, float (&x)[8]) { load8(p, x); }
// four consecutive elements
__device__ __forceinline__ void load4(const float *p, float (&x)[4]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
}
__device__ __forceinline__ void load4(const bf16_t *p, float (&x)[4]) {
    const uint2 w = *reinterpret_cast<const uint2 *>(p);
    x[0] = lo_bf16(w.x); x[1] = hi_bf16(w.x); x[2] = lo_bf16(w.y); x[3] = hi_bf16(w.y);
}
__device__ __forceinline__ void store4(float *p, const float (&x)[4]) {
    *reinterpret_cast<float4 *>(p) = make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store4(bf16_t *p, const float (&x)[4]) {
    *reinterpret_cast<uint2 *>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
}

// one staged 16-byte vector as floats (4 float32 or 8 bf16)
__device__ __forceinline__ void unpack16(const uint4 &w, float (&x)[8], float) {
    x[0] = __uint_as_float(w.x); x[1] = __uint_as_float(w.y); x[2] = __uint_as_float(w.z); x[3] = __uint_as_float(w.w);
}
__device__ __forceinline__ void unpack16(const uint4 &w, float (&x)[8], bf16_t) {
    x[0] = lo_bf16(w.x); x[1] = hi_bf16(w.x); x[2] = lo_bf16(w.y); x[3] = hi_bf16(w.y);
    x[4] = lo_bf16(w.z); x[5] = hi_bf16(w.z); x[6] = lo_bf16(w.w); x[7] = hi_bf16(w.w);
}

// Commit a tile staged in registers (TilePrefetch: every global load of the
// tile issued at once) to LDS rows `ld` apart as the operand type, element x
// of row t becoming f(t, x); rows the staging marked invalid (past the
// chunk's tokens: a padded token carries no feature, phi(0) would be 1)
// become zero.  With `lo`, also the low operand part Op(f - Op(f)).
template <int NTHR, class TP, class Op, class F>
__device__ __forceinline__ void commit_tile(const TP &tp, Op *dst, Op *lo, int ld, int tid, F f) {
    typedef Group<Op> Gp;
#pragma unroll
    for (int i = 0; i < TP::PER; ++i) {
        const int e = tid + i * NTHR;
        if (TP::TOTAL % NTHR != 0 && e >= TP::TOTAL) continue;
        const int t = e / TP::VPR, c = (e % TP::VPR) * TP::VE;
        float x[8];
        unpack16(tp.r[i], x, decltype(tp.tag){});
        const bool ok = (tp.valid >> i) & 1u;
#pragma unroll
        for (int j = 0; j < TP::VE; ++j) x[j] = ok ? f(t, x[j]) : 0.f;
#pragma unroll
        for (int j = 0; j < TP::VE; j += 4) {
            const typename Gp::type h = Gp::make(x[j], x[j + 1], x[j + 2], x[j + 3]);
            st_group(dst + t * ld + c + j, h);
            if (lo) {
                float r[4];
                Gp::unpack(h, r);
                st_group(lo + t * ld + c + j, Gp::make(x[j] - r[0], x[j + 1] - r[1], x[j + 2] - r[2], x[j + 3] - r[3]));
            }
        }
    }
}

// TilePrefetch with its element type visible to commit_tile
template <int R, int D, int NTHR, class E>
struct Staged : TilePrefetch<R, D, NTHR, E> {
    E tag;
};

template <class DT, bool NORM>
constexpr bool split_operands() { return NORM && sizeof(typename OpOf<DT>::type) == 2; }

template <class DT, int DK, int DV, int C, bool NORM>
struct BwdLds {
    typedef typename OpOf<DT>::type Op;
    static constexpr int PAD = 16 / sizeof(Op);
    static constexpr int LDK = DK + PAD, LDV = DV + PAD, LDC = C + PAD;
    static constexpr int F_FLOATS = (C + 1) + 2 * C + 2 * DK + 16;   // powers, 1/den, dden, z, dz, reduction
    static constexpr int SPLIT_ELEMS = split_operands<DT, NORM>() ? C * LDK + C * LDC : 0;   // low parts of phiK, G
    // retention with bf16 data: the entering state as an LDS operand tile
    static constexpr bool STAGE_S = !NORM && sizeof(Op) == 2;
    static constexpr int STATE_ELEMS = STAGE_S ? DK * LDV : 0;
    static constexpr int GRAD_BYTES =
        (2 * C * LDK + 2 * C * LDV + 2 * C * LDC + DK * LDV + SPLIT_ELEMS + STATE_ELEMS) *
            static_cast<int>(sizeof(Op)) +
        F_FLOATS * 4;
};

template <class DT, int DK, int DV, int C>
struct NormLds {
    typedef typename OpOf<DT>::type Op;
    static constexpr int PAD = 16 / sizeof(Op);
    static constexpr int LFK = DK + 4, LFC = C + 4;          // float32 rows
    static constexpr int LDK = DK + PAD, LDV = DV + PAD;     // operand rows
    static constexpr int BYTES = (2 * C * LFK + C * LFC) * 4 + 2 * C * LDV * static_cast<int>(sizeof(Op)) +
                                 (C + 1 + DK + 3 * C + C * (DV / 16)) * 4;
};


// Chunk length of the backward: the largest of 64, 32, 16 whose tiles fit a
// compute unit's LDS in every kernel of the pass.
template <class DT, int DK, int DV, bool NORM, int C>
constexpr bool bwd_fits() {
    return BwdLds<DT, DK, DV, C, NORM>::GRAD_BYTES <= 160 * 1024 &&
           (!NORM || NormLds<DT, DK, DV, C>::BYTES <= 160 * 1024);
}
template <class DT, int DK, int DV, bool NORM>
constexpr int bwd_chunk() {
    if (bwd_fits<DT, DK, DV, NORM, 64>()) return 64;
    if (bwd_fits<DT, DK, DV, NORM, 32>()) return 32;
    return 16;
}

constexpr int kBwdWaves = 8;
constexpr uint32_t kGradPersistWGs = 256;   // MI355X compute units

// ------------------------------------------------------------- increments

// Retention (NORM false) also forms the cotangent increments here (its dO'
// is dO); the normalized variant forms them in bwd_normalizer_kernel.  With
// bf16 data the decay-weighted token operands carry a low part (x = hi + lo,
// both bf16): the chunk states feed the decay's gradient, which is badly
// conditioned when the decay is close to 1 over long sequences.
template <class DT, int DK, int DV, int C, bool NORM>
__global__ void __launch_bounds__(kBwdWaves * 64) bwd_increments_kernel(const BwdParams p) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef BwdLds<DT, DK, DV, C, NORM> L;
    constexpr bool REV = !NORM, SPLIT = sizeof(Op) == 2;
    constexpr int NTHR = kBwdWaves * 64, NCB = DK / 16, NIB = DV / 16;
    constexpr int LDK = L::LDK, LDV = L::LDV;
    __shared__ __align__(16) Op sQ[REV ? C * LDK : 8];               // gamma^(t+1) phi(q_t)
    __shared__ __align__(16) Op sQl[REV && SPLIT ? C * LDK : 8];     // its low part
    __shared__ __align__(16) Op sK[C * LDK];                         // gamma^(n-1-t) phi(k_t)
    __shared__ __align__(16) Op sKl[SPLIT ? C * LDK : 8];            // its low part
    __shared__ __align__(16) Op sV[C * LDV];
    __shared__ __align__(16) Op sO[REV ? C * LDV : 8];               // dO

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int N = p.n_chunk;
    const int bh = blockIdx.x / N, ch = blockIdx.x - bh * N;
    const int n = min(C, p.T - ch * C);
    const size_t tok0 = static_cast<size_t>(bh) * p.T + static_cast<size_t>(ch) * C;
    const float l2g = head_l2g(p, bh);
    const bool elu = p.elu;

    // every global load of the chunk first, then the LDS commits
    Staged<C, DK, NTHR, IO> pk, pq;
    Staged<C, DV, NTHR, IO> pv, po;
    pk.load(static_cast<const IO *>(p.k) + tok0 * DK, DK, n, tid);
    pv.load(static_cast<const IO *>(p.v) + tok0 * DV, DV, n, tid);
    if constexpr (REV) {
        pq.load(static_cast<const IO *>(p.q) + tok0 * DK, DK, n, tid);
        po.load(static_cast<const IO *>(p.dout) + tok0 * DV, DV, n, tid);
    }
    commit_tile<NTHR>(pk, sK, SPLIT ? sKl : static_cast<Op *>(nullptr), LDK, tid, [&](int t, float x) {
        return phi_rt(x, elu) * __builtin_amdgcn_exp2f(static_cast<float>(n - 1 - t) * l2g);
    });
    commit_tile<NTHR>(pv, sV, static_cast<Op *>(nullptr), LDV, tid, [](int, float x) { return x; });
    if constexpr (REV) {
        commit_tile<NTHR>(pq, sQ, SPLIT ? sQl : static_cast<Op *>(nullptr), LDK, tid, [&](int t, float x) {
            return phi_rt(x, elu) * __builtin_amdgcn_exp2f(static_cast<float>(t + 1) * l2g);
        });
        commit_tile<NTHR>(po, sO, static_cast<Op *>(nullptr), LDV, tid, [](int, float x) { return x; });
    }
    __syncthreads();

    const size_t E = static_cast<size_t>(DK) * DV + (NORM ? DK : 0);
    float *sf = p.slot_f + (static_cast<size_t>(bh) * N + ch) * E;
    float *sr = p.slot_r + (static_cast<size_t>(bh) * N + ch) * E;
    // (key block cb, value block ib) tiles of phiK^T V (forward) and
    // phiQ^T dO (reverse), contracting over the tokens: both operands by
    // transposing reads of the token-major tiles
    for (int u = wave; u < (REV ? 2 : 1) * NCB * NIB; u += kBwdWaves) {
        const bool rev = u >= NCB * NIB;
        const int w = rev ? u - NCB * NIB : u;
        const int cb = w % NCB, ib = w / NCB;
        const Op *A = rev ? sQ : sK;
        const Op *Al = rev ? sQl : sKl;
        const Op *Bm = rev ? sO : sV;
        f32x4 acc = zero4();
#pragma unroll
        for (int t0 = 0; t0 + 32 <= C; t0 += 32) {
            const auto b0 = kt_group<0>(Bm, LDV, t0, 16 * ib, lane), b1 = kt_group<0>(Bm, LDV, t0 + 16, 16 * ib, lane);
            mma32(acc, kt_group<0>(A, LDK, t0, 16 * cb, lane), kt_group<0>(A, LDK, t0 + 16, 16 * cb, lane), b0, b1);
            if constexpr (SPLIT)
                mma32(acc, kt_group<0>(Al, LDK, t0, 16 * cb, lane), kt_group<0>(Al, LDK, t0 + 16, 16 * cb, lane), b0, b1);
        }
        if constexpr (C % 32 == 16) {
            const auto b0 = kt_group<0>(Bm, LDV, C - 16, 16 * ib, lane);
            mma16(acc, kt_group<0>(A, LDK, C - 16, 16 * cb, lane), b0);
            if constexpr (SPLIT) mma16(acc, kt_group<0>(Al, LDK, C - 16, 16 * cb, lane), b0);
        }
        float *dst = (rev ? sr : sf) + static_cast<size_t>(16 * cb + 4 * lg) * DV + 16 * ib + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r * DV] = acc[r];
    }
    if constexpr (NORM) {
        // z increment from the same operands
        for (int c = tid; c < DK; c += NTHR) {
            float zf = 0.f;
            for (int t = 0; t < n; ++t) zf += to_f32(sK[t * LDK + c]) + (SPLIT ? to_f32(sKl[t * LDK + c]) : 0.f);
            sf[static_cast<size_t>(DK) * DV + c] = zf;
        }
    }
}

// ------------------------------------------------- normalizer (normalized)

template <class DT, int DK, int DV, int C>
__global__ void __launch_bounds__(kBwdWaves * 64) bwd_normalizer_kernel(const BwdParams p) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef Group<Op> Gp;
    typedef NormLds<DT, DK, DV, C> L;
    constexpr int NTHR = kBwdWaves * 64, NB = C / 16, NCB = DK / 16, NIB = DV / 16;
    constexpr int LFK = L::LFK, LFC = L::LFC, LDK = L::LDK, LDV = L::LDV;
    static_assert(L::BYTES <= 160 * 1024, "LDS budget");
    static_assert(C * LDK * sizeof(Op) <= C * LFK * sizeof(float), "operand tile fits the key tile");
    __shared__ __align__(16) float fQ[C * LFK];   // phi(q), float32
    __shared__ __align__(16) float fK[C * LFK];   // phi(k), float32; then the cotangent-increment operand
    __shared__ __align__(16) float fP[C * LFC];   // D o (phiQ phiK^T), float32
    __shared__ __align__(16) Op sV[C * LDV];
    __shared__ __align__(16) Op sO[C * LDV];      // dO
    __shared__ float sPow[C + 1], sZ[DK], sDen[C], sInv[C], sE[C], sDot[C * NIB];
    // gamma^(t+1) phi(q_t) / den_t as a high and (bf16) a low operand part,
    // in the key and score tiles once those are dead
    constexpr bool SPLIT = sizeof(Op) == 2;
    Op *sQr = reinterpret_cast<Op *>(fK);
    Op *sQrl = reinterpret_cast<Op *>(fP);
    static_assert(!SPLIT || C * LDK * sizeof(Op) <= C * LFC * sizeof(float), "low part fits the score tile");

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int N = p.n_chunk;
    const int bh = blockIdx.x / N, ch = blockIdx.x - bh * N;
    const int n = min(C, p.T - ch * C);
    const size_t tok0 = static_cast<size_t>(bh) * p.T + static_cast<size_t>(ch) * C;
    const float l2g = head_l2g(p, bh);
    const bool elu = p.elu;
    const size_t E = static_cast<size_t>(DK) * DV + DK;
    const float *sf = p.slot_f + (static_cast<size_t>(bh) * N + ch) * E;   // state entering the chunk
    float *sr = p.slot_r + (static_cast<size_t>(bh) * N + ch) * E;

    for (int e = tid; e <= C; e += NTHR) sPow[e] = __builtin_amdgcn_exp2f(static_cast<float>(e) * l2g);
    for (int c = tid; c < DK; c += NTHR) sZ[c] = sf[static_cast<size_t>(DK) * DV + c];
    {
        // every global load of the chunk first; float32 features, padded tokens zero
        Staged<C, DK, NTHR, IO> pq, pk;
        Staged<C, DV, NTHR, IO> pv, po;
        pq.load(static_cast<const IO *>(p.q) + tok0 * DK, DK, n, tid);
        pk.load(static_cast<const IO *>(p.k) + tok0 * DK, DK, n, tid);
        pv.load(static_cast<const IO *>(p.v) + tok0 * DV, DV, n, tid);
        po.load(static_cast<const IO *>(p.dout) + tok0 * DV, DV, n, tid);
        commit_tile<NTHR>(pq, fQ, static_cast<float *>(nullptr), LFK, tid, [&](int, float x) { return phi_rt(x, elu); });
        commit_tile<NTHR>(pk, fK, static_cast<float *>(nullptr), LFK, tid, [&](int, float x) { return phi_rt(x, elu); });
        commit_tile<NTHR>(pv, sV, static_cast<Op *>(nullptr), LDV, tid, [](int, float x) { return x; });
        commit_tile<NTHR>(po, sO, static_cast<Op *>(nullptr), LDV, tid, [](int, float x) { return x; });
    }
    __syncthreads();

    // scores on the float32 matrix cores; a lane holds four keys j of query t
    for (int tt = wave; tt < NB * NB; tt += kBwdWaves) {
        const int I = tt / NB, J = tt % NB;
        const int t = 16 * I + lr, j0 = 16 * J + 4 * lg;
        f32x4 acc = zero4();
        if (J <= I) {
#pragma unroll
            for (int c0 = 0; c0 < DK; c0 += 16)
                mma16(acc, *reinterpret_cast<const float4 *>(fK + (16 * J + lr) * LFK + c0 + 4 * lg),
                      *reinterpret_cast<const float4 *>(fQ + t * LFK + c0 + 4 * lg));
        }
        float pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = j0 + i;
            pv[i] = j <= t && j < n ? sPow[t - j] * acc[i] : 0.f;
        }
        *reinterpret_cast<float4 *>(fP + t * LFC + j0) = make_float4(pv[0], pv[1], pv[2], pv[3]);
    }
    __syncthreads();

    // denominators gamma^(t+1) phi(q_t).z_c + sum_j P_tj, eight lanes per token
    for (int e = tid; e < 8 * C; e += NTHR) {
        const int t = e >> 3, part = e & 7;
        float dz = 0.f, dp = 0.f;
        for (int c = part; c < DK; c += 8) dz += fQ[t * LFK + c] * sZ[c];
        for (int j = part; j < C; j += 8) dp += fP[t * LFC + j];
        const float d = group_sum<8>(sPow[t + 1] * dz + dp);
        if (part == 0) sDen[t] = d;
    }
    // numerators dotted with dO: tiles (token block I, value block ib), a lane
    // holding num[16 I + 4 lg + r][16 ib + lr]
    for (int u = wave; u < NB * NIB; u += kBwdWaves) {
        const int I = u / NIB, ib = u % NIB;
        f32x4 acc = zero4(), st = zero4();
#pragma unroll
        for (int J = 0; J < NB; ++J) {
            if (J <= I) {
                float v4[4];
                Gp::unpack(kt_group<0>(sV, LDV, 16 * J, 16 * ib, lane), v4);
                mma16(acc, *reinterpret_cast<const float4 *>(fP + (16 * I + lr) * LFC + 16 * J + 4 * lg),
                      make_float4(v4[0], v4[1], v4[2], v4[3]));
            }
        }
#pragma unroll
        for (int c0 = 0; c0 < DK; c0 += 16) {
            const float *sp = sf + static_cast<size_t>(c0 + 4 * lg) * DV + 16 * ib + lr;
            mma16(st, *reinterpret_cast<const float4 *>(fQ + (16 * I + lr) * LFK + c0 + 4 * lg),
                  make_float4(sp[0], sp[DV], sp[2 * DV], sp[3 * DV]));
        }
        float d4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * I + 4 * lg + r;
            d4[r] = group_sum<16>(to_f32(sO[t * LDV + 16 * ib + lr]) * (acc[r] + sPow[t + 1] * st[r]));
        }
        if (lr == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) sDot[(16 * I + 4 * lg + r) * NIB + ib] = d4[r];
        }
    }
    __syncthreads();

    // per token: 1/den_t and dden_t = -(dO_t . num_t) / den_t^2, kept for the
    // gradient kernel
    for (int t = tid; t < C; t += NTHR) {
        float dot = 0.f;
        for (int ib = 0; ib < NIB; ++ib) dot += sDot[t * NIB + ib];
        const float inv = t < n ? 1.f / sDen[t] : 0.f;
        sInv[t] = inv;
        sE[t] = -dot * inv;   // -(dO_t . o_t)
        if (t < n) {
            p.tok[2 * (tok0 + t)] = inv;
            p.tok[2 * (tok0 + t) + 1] = -dot * inv * inv;
        }
    }
    __syncthreads();
    // the cotangent increment's token operand (the key tile is dead)
    for (int e = tid; e < C * (DK / 4); e += NTHR) {
        const int t = e / (DK / 4), c = (e % (DK / 4)) * 4;
        const float4 f = *reinterpret_cast<const float4 *>(fQ + t * LFK + c);
        const float w = sPow[t + 1] * sInv[t];
        const float x[4] = {f.x * w, f.y * w, f.z * w, f.w * w};
        const auto h = Gp::make(x[0], x[1], x[2], x[3]);
        st_group(sQr + t * LDK + c, h);
        if constexpr (SPLIT) {
            float r[4];
            Gp::unpack(h, r);
            st_group(sQrl + t * LDK + c, Gp::make(x[0] - r[0], x[1] - r[1], x[2] - r[2], x[3] - r[3]));
        }
    }
    __syncthreads();
    // dS'_c increment: (key block cb, value block ib) tiles of
    // sum_t gamma^(t+1) phi(q_t) dO_t^T / den_t, and its normalizer part
    // sum_t gamma^(t+1) phi(q_t) dden_t
    for (int u = wave; u < NCB * NIB; u += kBwdWaves) {
        const int cb = u % NCB, ib = u / NCB;
        f32x4 acc = zero4();
#pragma unroll
        for (int t0 = 0; t0 + 32 <= C; t0 += 32) {
            const auto b0 = kt_group<0>(sO, LDV, t0, 16 * ib, lane), b1 = kt_group<0>(sO, LDV, t0 + 16, 16 * ib, lane);
            mma32(acc, kt_group<0>(sQr, LDK, t0, 16 * cb, lane), kt_group<0>(sQr, LDK, t0 + 16, 16 * cb, lane), b0, b1);
            if constexpr (SPLIT)
                mma32(acc, kt_group<0>(sQrl, LDK, t0, 16 * cb, lane), kt_group<0>(sQrl, LDK, t0 + 16, 16 * cb, lane), b0,
                      b1);
        }
        if constexpr (C % 32 == 16) {
            const auto b0 = kt_group<0>(sO, LDV, C - 16, 16 * ib, lane);
            mma16(acc, kt_group<0>(sQr, LDK, C - 16, 16 * cb, lane), b0);
            if constexpr (SPLIT) mma16(acc, kt_group<0>(sQrl, LDK, C - 16, 16 * cb, lane), b0);
        }
        float *dst = sr + static_cast<size_t>(16 * cb + 4 * lg) * DV + 16 * ib + lr;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r * DV] = acc[r];
    }
    for (int c = tid; c < DK; c += NTHR) {
        float zr = 0.f;
        for (int t = 0; t < n; ++t) zr += (to_f32(sQr[t * LDK + c]) + (SPLIT ? to_f32(sQrl[t * LDK + c]) : 0.f)) * sE[t];
        sr[static_cast<size_t>(DK) * DV + c] = zr;
    }
}

// ------------------------------------------------------------------- scans

// Lane (head bh, element e of its state): e < d_k d_v is key channel e / d_v,
// value channel e % d_v; the normalized variant's z follows.
// dirs: bit 0 the forward scan, bit 1 the reverse scan.
__global__ void __launch_bounds__(256) bwd_scan_kernel(const BwdParams p, int DK, int DV, int C, int dirs) {
    const size_t KV = static_cast<size_t>(DK) * DV;
    const size_t E = KV + (p.normalize ? DK : 0);
    const size_t gid = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
    const size_t heads = static_cast<size_t>(p.B) * p.H;
    if (gid >= heads * E) return;
    const size_t bh = gid / E, e = gid - bh * E;
    const int N = p.n_chunk;
    const float l2g = p.gate ? __builtin_amdgcn_logf(p.gate[bh % p.H]) : 0.f;
    const float gC = __builtin_amdgcn_exp2f(static_cast<float>(C) * l2g);
    const float gL = __builtin_amdgcn_exp2f(static_cast<float>(p.T - (N - 1) * C) * l2g);   // the last chunk
    const bool is_z = e >= KV;
    const size_t kc = is_z ? e - KV : e / DV, vc = is_z ? 0 : e % DV;
    // library layout of the state: (d_v, d_k), row = value channel
    const size_t lib = (bh * DV + vc) * DK + kc, zlib = bh * DK + kc;

    // forward: slot c becomes the state entering chunk c
    float s = is_z ? (p.z0 ? p.z0[zlib] : 0.f) : (p.S0 ? p.S0[lib] : 0.f);
    float *f = p.slot_f + bh * N * E + e;
    for (int c = 0; c < ((dirs & 1) ? N : 0); c += 8) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = c + j < N ? f[static_cast<size_t>(c + j) * E] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (c + j < N) {
                f[static_cast<size_t>(c + j) * E] = s;
                s = (c + j == N - 1 ? gL : gC) * s + x[j];
            }
    }
    if (!(dirs & 2)) return;
    // reverse: slot c becomes the cotangent leaving chunk c
    float d = is_z ? (p.dz_T ? p.dz_T[zlib] : 0.f) : (p.dS_T ? p.dS_T[lib] : 0.f);
    float *r = p.slot_r + bh * N * E + e;
    for (int c = N - 1; c >= 0; c -= 8) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = c - j >= 0 ? r[static_cast<size_t>(c - j) * E] : 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (c - j >= 0) {
                r[static_cast<size_t>(c - j) * E] = d;
                d = (c - j == N - 1 ? gL : gC) * d + x[j];
            }
    }
    if (is_z) {
        if (p.dz0) p.dz0[zlib] = d;
    } else if (p.dS0) {
        p.dS0[lib] = d;
    }
}

// ----------------------------------------------------- chained states

// Retention over many chunks: launches 1 and 2 as one chain per (head,
// direction, block of VB value channels).  The workgroup keeps its columns of
// the state (forward) or of the cotangent (reverse) in matrix-core
// accumulators, walks the chunks in order, writes each chunk's entering state
// (leaving cotangent) to its slot and adds the chunk's increment on the
// matrix cores, with the same split operands as bwd_increments_kernel:
//   forward  S_{c+1}  = gamma^n S_c + phiK^T diag(gamma^(n-1-j)) V,  from S0,
//   reverse  dS_c     = gamma^n dS_{c+1} + phiQ^T diag(gamma^(t+1)) dO, from dS_T,
// ending in dS0.  The slots are written once, and no increment goes through
// memory.  Eight waves; wave w keeps the (key, value) 16x16 tiles w, w + 8, ...
// The chunk operands sit in two LDS copies: each wave commits chunk i + 1 to
// one while the matrix-core work of chunk i reads the other (one barrier per
// chunk).
constexpr int kChainWaves = 8;
constexpr int kChainMinChunks = 16;   // fewer chunks: increments + scan

template <class DT, int DK, int DV, int C, int VB>
__global__ void __launch_bounds__(kChainWaves * 64) bwd_chain_kernel(const BwdParams p) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    constexpr bool SPLIT = sizeof(Op) == 2;
    constexpr int NTHR = kChainWaves * 64, NCB = DK / 16, NIB = VB / 16;
    constexpr int NT = NCB * NIB, TPW = (NT + kChainWaves - 1) / kChainWaves;
    constexpr int PAD = 16 / sizeof(Op), LDK = DK + PAD, LDV = VB + PAD;
    constexpr int NVB = DV / VB;
    static_assert(DV % VB == 0 && VB % 16 == 0, "value blocks");
    __shared__ __align__(16) Op sA[2 * C * LDK];                 // weighted phi(k) (forward) or phi(q) (reverse)
    __shared__ __align__(16) Op sAl[SPLIT ? 2 * C * LDK : 8];     // its low part
    __shared__ __align__(16) Op sB[2 * C * LDV];                 // this block's v (forward) or dO (reverse)

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    // workgroup -> (head, direction, value block); with a multiple of 8 heads
    // the workgroups that read one head's keys (or queries) share an XCD
    const int heads = p.B * p.H;
    int bh, rev, vb;
    {
        const int bid = blockIdx.x;
        if ((heads & 7) == 0) {
            const int x = bid & 7, r = bid >> 3;
            vb = r % NVB;
            rev = (r / NVB) & 1;
            bh = (r / NVB >> 1) * 8 + x;
        } else {
            vb = bid % NVB;
            rev = (bid / NVB) & 1;
            bh = bid / (2 * NVB);
        }
    }
    const int N = p.n_chunk;
    const float l2g = head_l2g(p, bh);
    const bool elu = p.elu;
    const size_t E = static_cast<size_t>(DK) * DV;
    float *slots = (rev ? p.slot_r : p.slot_f) + static_cast<size_t>(bh) * N * E;
    const IO *ah = static_cast<const IO *>(rev ? p.q : p.k) + static_cast<size_t>(bh) * p.T * DK;
    const IO *bhp = static_cast<const IO *>(rev ? p.dout : p.v) + static_cast<size_t>(bh) * p.T * DV + vb * VB;
    const float *init = rev ? p.dS_T : p.S0;   // library layout (d_v, d_k)

    // the tiles of this wave: acc[i][r] = element (key 16 cb + 4 lg + r,
    // value 16 ib + lr of the block)
    f32x4 acc[TPW];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        acc[i] = zero4();
        const int u = wave + kChainWaves * i;
        if (u < NT && init) {
            const int cb = u % NCB, ib = u / NCB;
            const float *src = init + (static_cast<size_t>(bh) * DV + vb * VB + 16 * ib + lr) * DK + 16 * cb + 4 * lg;
            const float4 x = *reinterpret_cast<const float4 *>(src);
            acc[i] = f32x4{x.x, x.y, x.z, x.w};
        }
    }
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

    Staged<C, DK, NTHR, IO> pa;
    Staged<C, VB, NTHR, IO> pb;
    auto chunk_of = [&](int i) { return rev ? N - 1 - i : i; };   // i-th chunk of the walk
    auto load = [&](int c) {
        const int n = min(C, p.T - c * C);
        pa.load(ah + static_cast<size_t>(c) * C * DK, DK, n, tid);
        pb.load(bhp + static_cast<size_t>(c) * C * DV, DV, n, tid);
    };
    // slot stores per thread and chunk, issued after the next chunk's loads
    constexpr int NST = (NT % kChainWaves == 0 ? TPW : 0) * 4;
    // the chunk's token operands into copy b, decay-weighted as in bwd_increments_kernel
    auto commit = [&](int c, int b) {
        const int n = min(C, p.T - c * C);
        commit_tile<NTHR>(pa, sA + b * C * LDK, SPLIT ? sAl + b * C * LDK : static_cast<Op *>(nullptr), LDK, tid,
                          [&](int t, float x) {
                              return phi_rt(x, elu) * __builtin_amdgcn_exp2f(static_cast<float>(rev ? t + 1 : n - 1 - t) * l2g);
                          });
        commit_tile<NTHR>(pb, sB + b * C * LDV, static_cast<Op *>(nullptr), LDV, tid, [](int, float x) { return x; });
    };
    load(chunk_of(0));
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    commit(chunk_of(0), 0);
    __syncthreads();
    for (int i = 0; i < N; ++i) {
        const int c = chunk_of(i);
        const int n = min(C, p.T - c * C);
        const int b = i & 1;
        const Op *cA = sA + b * C * LDK, *cAl = sAl + (SPLIT ? b * C * LDK : 0), *cB = sB + b * C * LDV;
        // the next chunk's loads (the last one re-read at the end), then the
        // slot stores, which the commit's wait for those loads leaves in
        // flight: the state entering (cotangent leaving) chunk c
        load(chunk_of(min(i + 1, N - 1)));
        float *slot = slots + static_cast<size_t>(c) * E + vb * VB;
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int u = wave + kChainWaves * j;
            if (NT % kChainWaves == 0 || u < NT) {
                const int cb = u % NCB, ib = u / NCB;
                float *dst = slot + static_cast<size_t>(16 * cb + 4 * lg) * DV + 16 * ib + lr;
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[r * DV] = acc[j][r];
            }
        }
        const float gn = __builtin_amdgcn_exp2f(static_cast<float>(n) * l2g);
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int u = wave + kChainWaves * j;
            if (NT % kChainWaves != 0 && u >= NT) break;
            const int cb = u % NCB, ib = u / NCB;
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[j][r] *= gn;
#pragma unroll
            for (int t0 = 0; t0 + 32 <= C; t0 += 32) {
                const auto b0 = kt_group<0>(cB, LDV, t0, 16 * ib, lane), b1 = kt_group<0>(cB, LDV, t0 + 16, 16 * ib, lane);
                mma32(acc[j], kt_group<0>(cA, LDK, t0, 16 * cb, lane), kt_group<0>(cA, LDK, t0 + 16, 16 * cb, lane), b0, b1);
                if constexpr (SPLIT)
                    mma32(acc[j], kt_group<0>(cAl, LDK, t0, 16 * cb, lane), kt_group<0>(cAl, LDK, t0 + 16, 16 * cb, lane), b0, b1);
            }
            if constexpr (C % 32 == 16) {
                const auto b0 = kt_group<0>(cB, LDV, C - 16, 16 * ib, lane);
                mma16(acc[j], kt_group<0>(cA, LDK, C - 16, 16 * cb, lane), b0);
                if constexpr (SPLIT) mma16(acc[j], kt_group<0>(cAl, LDK, C - 16, 16 * cb, lane), b0);
            }
        }
        // chunk i + 1 into the other copy, last read by chunk i - 1 (before the
        // previous barrier); its loads have landed, the slot stores stay in flight
        __builtin_amdgcn_s_waitcnt(wait_vmcnt(NST));
        if (i + 1 < N) commit(chunk_of(i + 1), b ^ 1);
        __syncthreads();
    }
    if (rev && p.dS0) {
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
            const int u = wave + kChainWaves * j;
            if (u < NT) {
                const int cb = u % NCB, ib = u / NCB;
                float *dst = p.dS0 + (static_cast<size_t>(bh) * DV + vb * VB + 16 * ib + lr) * DK + 16 * cb + 4 * lg;
                *reinterpret_cast<float4 *>(dst) = make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
            }
        }
    }
}

// --------------------------------------------------------------- gradients

template <class DT, int DK, int DV, int C, bool NORM>
__global__ void __launch_bounds__(kBwdWaves * 64) bwd_grad_kernel(const BwdParams p) {
    typedef typename DT::storage IO;
    typedef typename OpOf<DT>::type Op;
    typedef Group<Op> Gp;
    typedef BwdLds<DT, DK, DV, C, NORM> L;
    constexpr bool SPLIT = split_operands<DT, NORM>(), STAGE_S = L::STAGE_S;
    constexpr int NTHR = kBwdWaves * 64, NB = C / 16, NCB = DK / 16, NIB = DV / 16;
    constexpr int LDK = L::LDK, LDV = L::LDV, LDC = L::LDC;
    static_assert(L::GRAD_BYTES <= 160 * 1024, "LDS budget");
    __shared__ __align__(16) Op sQ[C * LDK];    // phi(q)
    __shared__ __align__(16) Op sK[C * LDK];    // phi(k)
    __shared__ __align__(16) Op sV[C * LDV];
    __shared__ __align__(16) Op sO[C * LDV];    // dO
    __shared__ __align__(16) Op sA[C * LDC];    // D o (phiQ phiK^T) / den_t
    __shared__ __align__(16) Op sG[C * LDC];    // D o (dO' V'^T)
    __shared__ __align__(16) Op sdS[DK * LDV];  // cotangent leaving the chunk, [key][value]
    __shared__ __align__(16) Op sKl[SPLIT ? C * LDK : 8];   // low parts of phi(k) and of G
    __shared__ __align__(16) Op sGl[SPLIT ? C * LDC : 8];
    __shared__ __align__(16) Op sS[STAGE_S ? DK * LDV : 8];   // retention, bf16: the entering state, [key][value]
    __shared__ float sPow[C + 1], sInv[C], sDd[C], sZ[DK], sdZ[DK], sRed[16];

    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int lr = lane & 15, lg = lane >> 4;
    const int N = p.n_chunk;
    const int jobs = p.B * p.H * N;
    const bool elu = p.elu, want_dg = p.dgate != nullptr;
    constexpr bool norm = NORM;
    const size_t E = static_cast<size_t>(DK) * DV + (norm ? DK : 0);
    // With the states staged in LDS (retention, bf16) no product of a chunk
    // reads global memory, so the workgroups are persistent and each keeps the
    // next chunk's loads in flight during the current chunk's products.
    // The derivative of phi = elu + 1 is min(phi, 1): with PF it is taken from
    // the staged phi (bf16, relative error <= 2^-8) instead of a global load.
    constexpr bool PF = STAGE_S;

    Staged<C, DK, NTHR, IO> pq, pk;
    Staged<C, DV, NTHR, IO> pv, po;
    Staged<DK, DV, NTHR, float> pd, ps;
    // every global load of a chunk (inputs, and the float32 state and
    // cotangent rows), issued before any LDS commit
    auto load_job = [&](int job) {
        const int bh = job / N, ch = job - bh * N;
        const int n = min(C, p.T - ch * C);
        const size_t tok0 = static_cast<size_t>(bh) * p.T + static_cast<size_t>(ch) * C;
        pq.load(static_cast<const IO *>(p.q) + tok0 * DK, DK, n, tid);
        pk.load(static_cast<const IO *>(p.k) + tok0 * DK, DK, n, tid);
        pv.load(static_cast<const IO *>(p.v) + tok0 * DV, DV, n, tid);
        po.load(static_cast<const IO *>(p.dout) + tok0 * DV, DV, n, tid);
        pd.load(p.slot_r + static_cast<size_t>(job) * E, DV, DK, tid);
        if (STAGE_S || want_dg) ps.load(p.slot_f + static_cast<size_t>(job) * E, DV, DK, tid);
    };
    if (PF && static_cast<int>(blockIdx.x) < jobs) load_job(blockIdx.x);

    for (int job = blockIdx.x; job < jobs; job += gridDim.x) {
        const int bh = job / N, ch = job - bh * N;
        const int n = min(C, p.T - ch * C);
        const size_t tok0 = static_cast<size_t>(bh) * p.T + static_cast<size_t>(ch) * C;
        const float l2g = head_l2g(p, bh);
        const IO *qh = static_cast<const IO *>(p.q) + tok0 * DK;
        const IO *kh = static_cast<const IO *>(p.k) + tok0 * DK;
        const float *sf = p.slot_f + (static_cast<size_t>(bh) * N + ch) * E;   // state entering the chunk
        const float *sr = p.slot_r + (static_cast<size_t>(bh) * N + ch) * E;   // cotangent leaving it
        float dl = 0.f;   // this lane's share of the chunk's d(ln gamma)

        for (int e = tid; e <= C; e += NTHR) sPow[e] = __builtin_amdgcn_exp2f(static_cast<float>(e) * l2g);
        if (norm)
            for (int t = tid; t < C; t += NTHR) {
                sInv[t] = t < n ? p.tok[2 * (tok0 + t)] : 0.f;
                sDd[t] = t < n ? p.tok[2 * (tok0 + t) + 1] : 0.f;
            }
        {
            // the chunk's loads (issued during the previous chunk's products
            // with PF), then the LDS commits.  dO goes in as it is: 1/den_t is
            // applied in float32 to the products (the value and normalizer
            // parts of the normalized gradient nearly cancel).
            if (!PF) load_job(job);
            const bool need_s = STAGE_S || want_dg;
            commit_tile<NTHR>(pq, sQ, static_cast<Op *>(nullptr), LDK, tid, [&](int, float x) { return phi_rt(x, elu); });
            commit_tile<NTHR>(pk, sK, SPLIT ? sKl : static_cast<Op *>(nullptr), LDK, tid,
                              [&](int, float x) { return phi_rt(x, elu); });
            commit_tile<NTHR>(pv, sV, static_cast<Op *>(nullptr), LDV, tid, [](int, float x) { return x; });
            commit_tile<NTHR>(po, sO, static_cast<Op *>(nullptr), LDV, tid, [](int, float x) { return x; });
            commit_tile<NTHR>(pd, sdS, static_cast<Op *>(nullptr), LDV, tid, [](int, float x) { return x; });
            if (need_s) {
                if constexpr (STAGE_S) commit_tile<NTHR>(ps, sS, static_cast<Op *>(nullptr), LDV, tid, [](int, float x) { return x; });
                if (want_dg) {
                    // the state-coupling term n gamma^n <dS'_{c+1}, S'_c>, float32
                    const float wf = static_cast<float>(n) * __builtin_amdgcn_exp2f(static_cast<float>(n) * l2g);
#pragma unroll
                    for (int i = 0; i < pd.PER; ++i) {
                        if (!((pd.valid >> i) & 1u)) continue;   // lanes past the tile re-read its last vector
                        const uint4 a4 = pd.r[i], b4 = ps.r[i];
                        dl += wf * (__uint_as_float(a4.x) * __uint_as_float(b4.x) + __uint_as_float(a4.y) * __uint_as_float(b4.y) +
                                    __uint_as_float(a4.z) * __uint_as_float(b4.z) + __uint_as_float(a4.w) * __uint_as_float(b4.w));
                    }
                }
            }
            if (norm)
                for (int c = tid; c < DK; c += NTHR) {
                    const float z = sf[static_cast<size_t>(DK) * DV + c], dz = sr[static_cast<size_t>(DK) * DV + c];
                    sZ[c] = z;
                    sdZ[c] = dz;
                    if (want_dg) dl += static_cast<float>(n) * __builtin_amdgcn_exp2f(static_cast<float>(n) * l2g) * z * dz;
                }
        }
        __syncthreads();
        if (PF && job + static_cast<int>(gridDim.x) < jobs) load_job(job + gridDim.x);

        // ---- score tiles A and G (16 x 16, lower block triangle), taken
        // transposed so that a lane holds four consecutive keys j of one query t
        for (int tt = wave; tt < NB * NB; tt += kBwdWaves) {
            const int I = tt / NB, J = tt % NB;
            const int t = 16 * I + lr, j0 = 16 * J + 4 * lg;
            if (J > I) {
                st_group(sA + t * LDC + j0, Gp::make(0.f, 0.f, 0.f, 0.f));
                st_group(sG + t * LDC + j0, Gp::make(0.f, 0.f, 0.f, 0.f));
                if constexpr (SPLIT) st_group(sGl + t * LDC + j0, Gp::make(0.f, 0.f, 0.f, 0.f));
                continue;
            }
            f32x4 a = zero4(), h = zero4();
            tile_mma_ll<DK>(a, sK + 16 * J * LDK, LDK, sQ + 16 * I * LDK, LDK, lane);
            tile_mma_ll<DV>(h, sV + 16 * J * LDV, LDV, sO + 16 * I * LDV, LDV, lane);
            const float inv = norm ? sInv[t] : 1.f, dd = norm ? sDd[t] : 0.f;
            float av[4], gv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = j0 + i;
                const bool on = j <= t && j < n;
                const float w = on ? sPow[t - j] : 0.f;
                const float hv = h[i] * inv + dd;   // dO'_t . v'_j
                av[i] = w * a[i];
                gv[i] = w * hv;
                if (want_dg) dl += static_cast<float>(t - j) * av[i] * hv;
                av[i] *= inv;   // dV = (A / den)^T dO
            }
            st_group(sA + t * LDC + j0, Gp::make(av[0], av[1], av[2], av[3]));
            const auto gh = Gp::make(gv[0], gv[1], gv[2], gv[3]);
            st_group(sG + t * LDC + j0, gh);
            if constexpr (SPLIT) {
                float r[4];
                Gp::unpack(gh, r);
                st_group(sGl + t * LDC + j0, Gp::make(gv[0] - r[0], gv[1] - r[1], gv[2] - r[2], gv[3] - r[3]));
            }
        }
        __syncthreads();

        // ---- dq: tiles (key block cb, query block I) of dphiQ^T; a lane ends
        // with four consecutive key channels of one query token
        for (int u = wave; u < NCB * NB; u += kBwdWaves) {
            const int cb = u % NCB, I = u / NCB;
            const int t = 16 * I + lr;
            f32x4 acc = zero4(), xs = zero4();
            // G phiK over key blocks J <= I (split operands: Gh Kh + Gh Kl + Gl Kh)
#pragma unroll
            for (int J = 0; J < NB; J += 2) {
                if (J + 1 <= I) {
                    const auto k0 = kt_group<0>(sK, LDK, 16 * J, 16 * cb, lane), k1 = kt_group<0>(sK, LDK, 16 * J + 16, 16 * cb, lane);
                    const auto g0 = ld_group(sG + t * LDC + 16 * J + 4 * lg), g1 = ld_group(sG + t * LDC + 16 * J + 16 + 4 * lg);
                    mma32(acc, k0, k1, g0, g1);
                    if constexpr (SPLIT) {
                        mma32(acc, kt_group<0>(sKl, LDK, 16 * J, 16 * cb, lane), kt_group<0>(sKl, LDK, 16 * J + 16, 16 * cb, lane),
                              g0, g1);
                        mma32(acc, k0, k1, ld_group(sGl + t * LDC + 16 * J + 4 * lg),
                              ld_group(sGl + t * LDC + 16 * J + 16 + 4 * lg));
                    }
                } else if (J <= I) {
                    const auto k0 = kt_group<0>(sK, LDK, 16 * J, 16 * cb, lane);
                    const auto g0 = ld_group(sG + t * LDC + 16 * J + 4 * lg);
                    mma16(acc, k0, g0);
                    if constexpr (SPLIT) {
                        mma16(acc, kt_group<0>(sKl, LDK, 16 * J, 16 * cb, lane), g0);
                        mma16(acc, k0, ld_group(sGl + t * LDC + 16 * J + 4 * lg));
                    }
                }
            }
            if constexpr (!STAGE_S) {
                // the entering state: S'_c (key-major rows, float32 in the
                // workspace) times dO_t, on the float32 matrix cores (normalized:
                // it nearly cancels against the normalizer term below)
                const float *srow = sf + static_cast<size_t>(16 * cb + lr) * DV + 4 * lg;
#pragma unroll
                for (int i0 = 0; i0 < DV; i0 += 16) {
                    float o4[4];
                    Gp::unpack(ld_group(sO + t * LDV + i0 + 4 * lg), o4);
                    mma16(xs, *reinterpret_cast<const float4 *>(srow + i0), make_float4(o4[0], o4[1], o4[2], o4[3]));
                }
            } else {
                // retention, bf16: S_c rows from LDS times dO_t
                const Op *srow = sS + (16 * cb + lr) * LDV + 4 * lg;
                const Op *orow = sO + t * LDV + 4 * lg;
#pragma unroll
                for (int i0 = 0; i0 + 32 <= DV; i0 += 32)
                    mma32(xs, ld_group(srow + i0), ld_group(srow + i0 + 16), ld_group(orow + i0), ld_group(orow + i0 + 16));
                if constexpr (DV % 32 == 16) mma16(xs, ld_group(srow + DV - 16), ld_group(orow + DV - 16));
            }
            if (t < n) {
                const int c0 = 16 * cb + 4 * lg;
                const float wq = sPow[t + 1], inv = norm ? sInv[t] : 1.f, dd = norm ? sDd[t] : 0.f;
                float dph[4], g[4];
                if constexpr (PF) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) dph[r] = elu ? fminf(to_f32(sQ[t * LDK + c0 + r]), 1.f) : 1.f;
                } else {
                    float raw[4];
                    load4(qh + static_cast<size_t>(t) * DK + c0, raw);
#pragma unroll
                    for (int r = 0; r < 4; ++r) dph[r] = dphi_rt(raw[r], elu);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float X = wq * (xs[r] * inv + (norm ? dd * sZ[c0 + r] : 0.f));
                    if (want_dg) dl += static_cast<float>(t + 1) * to_f32(sQ[t * LDK + c0 + r]) * X;
                    g[r] = (acc[r] + X) * dph[r];
                }
                store4(static_cast<IO *>(p.dq) + (tok0 + t) * DK + c0, g);
            }
        }

        // ---- dk: tiles (key block cb, key-token block J) of dphiK^T
        for (int u = wave; u < NCB * NB; u += kBwdWaves) {
            const int cb = u % NCB, J = u / NCB;
            const int j = 16 * J + lr;
            f32x4 acc = zero4(), ys = zero4();
            // G^T phiQ over query blocks I >= J
#pragma unroll
            for (int s = 0; s < NB; s += 2) {
                const int I = J + s;
                if (I + 1 < NB)
                    mma32(acc, kt_group<0>(sQ, LDK, 16 * I, 16 * cb, lane), kt_group<0>(sQ, LDK, 16 * I + 16, 16 * cb, lane),
                          kt_group<0>(sG, LDC, 16 * I, 16 * J, lane), kt_group<0>(sG, LDC, 16 * I + 16, 16 * J, lane));
                else if (I < NB)
                    mma16(acc, kt_group<0>(sQ, LDK, 16 * I, 16 * cb, lane), kt_group<0>(sG, LDC, 16 * I, 16 * J, lane));
            }
            const Op *vrow = sV + j * LDV + 4 * lg;
            if constexpr (!STAGE_S) {
                // the leaving cotangent: dS'_{c+1} rows (key-major, float32 in the
                // workspace) times v_j, on the float32 matrix cores (normalized:
                // it nearly cancels against dz below)
                const float *drow = sr + static_cast<size_t>(16 * cb + lr) * DV + 4 * lg;
#pragma unroll
                for (int i0 = 0; i0 < DV; i0 += 16) {
                    float v4[4];
                    Gp::unpack(ld_group(vrow + i0), v4);
                    mma16(ys, *reinterpret_cast<const float4 *>(drow + i0), make_float4(v4[0], v4[1], v4[2], v4[3]));
                }
            } else {
                // retention, bf16: dS_{c+1} rows from LDS times v_j
                const Op *drow = sdS + (16 * cb + lr) * LDV + 4 * lg;
#pragma unroll
                for (int i0 = 0; i0 + 32 <= DV; i0 += 32)
                    mma32(ys, ld_group(drow + i0), ld_group(drow + i0 + 16), ld_group(vrow + i0), ld_group(vrow + i0 + 16));
                if constexpr (DV % 32 == 16) mma16(ys, ld_group(drow + DV - 16), ld_group(vrow + DV - 16));
            }
            if (j < n) {
                const int c0 = 16 * cb + 4 * lg;
                const float wk = sPow[n - 1 - j];
                float dph[4], g[4];
                if constexpr (PF) {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        dph[r] = elu ? fminf(to_f32(sK[j * LDK + c0 + r]) + (SPLIT ? to_f32(sKl[j * LDK + c0 + r]) : 0.f), 1.f) : 1.f;
                } else {
                    float raw[4];
                    load4(kh + static_cast<size_t>(j) * DK + c0, raw);
#pragma unroll
                    for (int r = 0; r < 4; ++r) dph[r] = dphi_rt(raw[r], elu);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float Y = wk * (ys[r] + (norm ? sdZ[c0 + r] : 0.f));
                    if (want_dg)
                        dl += static_cast<float>(n - 1 - j) *
                              (to_f32(sK[j * LDK + c0 + r]) + (SPLIT ? to_f32(sKl[j * LDK + c0 + r]) : 0.f)) * Y;
                    g[r] = (acc[r] + Y) * dph[r];
                }
                store4(static_cast<IO *>(p.dk) + (tok0 + j) * DK + c0, g);
            }
        }

        // ---- dv: tiles (value block ib, token block J) of dV^T
        for (int u = wave; u < NIB * NB; u += kBwdWaves) {
            const int ib = u % NIB, J = u / NIB;
            const int j = 16 * J + lr;
            f32x4 acc = zero4(), vs = zero4();
            // (A / den)^T dO over query blocks I >= J
#pragma unroll
            for (int s = 0; s < NB; s += 2) {
                const int I = J + s;
                if (I + 1 < NB)
                    mma32(acc, kt_group<0>(sO, LDV, 16 * I, 16 * ib, lane), kt_group<0>(sO, LDV, 16 * I + 16, 16 * ib, lane),
                          kt_group<0>(sA, LDC, 16 * I, 16 * J, lane), kt_group<0>(sA, LDC, 16 * I + 16, 16 * J, lane));
                else if (I < NB)
                    mma16(acc, kt_group<0>(sO, LDV, 16 * I, 16 * ib, lane), kt_group<0>(sA, LDC, 16 * I, 16 * J, lane));
            }
            // dS_{c+1} phi(k_j): the cotangent's value rows by transposing reads
            const Op *krow = sK + j * LDK + 4 * lg;
#pragma unroll
            for (int c0 = 0; c0 + 32 <= DK; c0 += 32)
                mma32(vs, kt_group<0>(sdS, LDV, c0, 16 * ib, lane), kt_group<0>(sdS, LDV, c0 + 16, 16 * ib, lane),
                      ld_group(krow + c0), ld_group(krow + c0 + 16));
            if constexpr (DK % 32 == 16) mma16(vs, kt_group<0>(sdS, LDV, DK - 16, 16 * ib, lane), ld_group(krow + DK - 16));
            if (j < n) {
                const float wk = sPow[n - 1 - j];
                float g[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) g[r] = acc[r] + wk * vs[r];
                store4(static_cast<IO *>(p.dv) + (tok0 + j) * DV + 16 * ib + 4 * lg, g);
            }
        }

        if (want_dg) {
            dl = group_sum<64>(dl);
            if (lane == 0) sRed[wave] = dl;
            __syncthreads();
            if (tid == 0) {
                float s = 0.f;
                for (int w = 0; w < kBwdWaves; ++w) s += sRed[w];
                p.part[static_cast<size_t>(bh) * N + ch] = s;
            }
        }
        __syncthreads();   // the next chunk overwrites every LDS tile and sRed
    }
}

// d gamma_h = (1 / gamma_h) * the chunks' shares of d(ln gamma), summed over
// the batch and the chunks in a fixed order.
__global__ void __launch_bounds__(256) bwd_dgate_kernel(const BwdParams p) {
    __shared__ float red[4];
    const int h = blockIdx.x, tid = threadIdx.x, N = p.n_chunk;
    float s = 0.f;
    for (int e = tid; e < p.B * N; e += 256) {
        const int b = e / N, c = e - b * N;
        s += p.part[(static_cast<size_t>(b) * p.H + h) * N + c];
    }
    s = group_sum<64>(s);
    if ((tid & 63) == 0) red[tid >> 6] = s;
    __syncthreads();
    if (tid == 0) p.dgate[h] = (red[0] + red[1] + red[2] + red[3]) / p.gate[h];
}

template <class DT, int DK, int DV, bool NORM>
hipError_t bwd_launch(const BwdArgs &a) {
    constexpr int C = bwd_chunk<DT, DK, DV, NORM>();
    BwdParams p;
    p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.dout;
    p.gate = a.gate; p.S0 = a.S0; p.z0 = a.z0; p.dS_T = a.dS_T; p.dz_T = a.dz_T;
    p.dq = a.dq; p.dk = a.dk; p.dv = a.dv; p.dS0 = a.dS0; p.dz0 = a.dz0; p.dgate = a.dgate;
    p.B = a.B; p.H = a.H; p.T = a.T;
    p.n_chunk = (a.T + C - 1) / C;
    p.normalize = a.variant == LA_NORMALIZED;
    p.elu = a.phi == LA_PHI_ELU1;
    const size_t heads = static_cast<size_t>(a.B) * a.H;
    const size_t E = static_cast<size_t>(DK) * DV + (p.normalize ? DK : 0);
    const size_t slots = heads * p.n_chunk * E;
    p.slot_f = static_cast<float *>(a.workspace);
    p.slot_r = p.slot_f + slots;
    p.part = p.slot_r + slots;
    p.tok = p.part + heads * p.n_chunk;
    const uint32_t wgs = static_cast<uint32_t>(heads * p.n_chunk);
    const uint32_t scan_blocks = static_cast<uint32_t>((heads * E + 255) / 256);
    const dim3 blk(kBwdWaves * 64);
    if constexpr (NORM) {
        if (wgs) hipLaunchKernelGGL((bwd_increments_kernel<DT, DK, DV, C, true>), dim3(wgs), blk, 0, a.stream, p);
        hipLaunchKernelGGL(bwd_scan_kernel, dim3(scan_blocks), dim3(256), 0, a.stream, p, DK, DV, C, 1);
        if (wgs) hipLaunchKernelGGL((bwd_normalizer_kernel<DT, DK, DV, C>), dim3(wgs), blk, 0, a.stream, p);
        hipLaunchKernelGGL(bwd_scan_kernel, dim3(scan_blocks), dim3(256), 0, a.stream, p, DK, DV, C, 2);
    } else if (p.n_chunk >= kChainMinChunks) {
        constexpr int VB = DV >= 64 ? 64 : DV;
        const uint32_t chains = static_cast<uint32_t>(heads * 2 * (DV / VB));
        hipLaunchKernelGGL((bwd_chain_kernel<DT, DK, DV, C, VB>), dim3(chains), dim3(kChainWaves * 64), 0, a.stream, p);
    } else {
        if (wgs) hipLaunchKernelGGL((bwd_increments_kernel<DT, DK, DV, C, false>), dim3(wgs), blk, 0, a.stream, p);
        hipLaunchKernelGGL(bwd_scan_kernel, dim3(scan_blocks), dim3(256), 0, a.stream, p, DK, DV, C, 3);
    }
    // the retention bf16 gradient kernel is persistent: one workgroup per CU
    // (its LDS allows one), each walking the chunks with a stride of the grid
    const uint32_t grad_wgs = BwdLds<DT, DK, DV, C, NORM>::STAGE_S ? std::min<uint32_t>(wgs, kGradPersistWGs) : wgs;
    if (wgs) hipLaunchKernelGGL((bwd_grad_kernel<DT, DK, DV, C, NORM>), dim3(grad_wgs), blk, 0, a.stream, p);
    if (a.dgate) hipLaunchKernelGGL(bwd_dgate_kernel, dim3(a.H), dim3(256), 0, a.stream, p);
    return hipGetLastError();
}

template <class DT, int DK, int DV>
hipError_t bwd_variant(const BwdArgs &a) {
    if (a.variant == LA_NORMALIZED) return bwd_launch<DT, DK, DV, true>(a);
    return bwd_launch<DT, DK, DV, false>(a);
}

template <class DT, int DK>
hipError_t bwd_dv(const BwdArgs &a) {
    switch (a.d_v) {
        case 16: return bwd_variant<DT, DK, 16>(a);
        case 32: return bwd_variant<DT, DK, 32>(a);
        case 64: return bwd_variant<DT, DK, 64>(a);
        case 128: return bwd_variant<DT, DK, 128>(a);
    }
    return hipErrorInvalidValue;
}

template <class DT>
hipError_t bwd_dk(const BwdArgs &a) {
    switch (a.d_k) {
        case 16: return bwd_dv<DT, 16>(a);
        case 32: return bwd_dv<DT, 32>(a);
        case 64: return bwd_dv<DT, 64>(a);
        case 128: return bwd_dv<DT, 128>(a);
    }
    return hipErrorInvalidValue;
}

template <class DT, int DK, int DV>
int chunk_norm(bool norm) {
    return norm ? bwd_chunk<DT, DK, DV, true>() : bwd_chunk<DT, DK, DV, false>();
}
template <class DT, int DK>
int chunk_dv(int d_v, bool norm) {
    switch (d_v) {
        case 16: return chunk_norm<DT, DK, 16>(norm);
        case 32: return chunk_norm<DT, DK, 32>(norm);
        case 64: return chunk_norm<DT, DK, 64>(norm);
    }
    return chunk_norm<DT, DK, 128>(norm);
}
template <class DT>
int chunk_dk(int d_k, int d_v, bool norm) {
    switch (d_k) {
        case 16: return chunk_dv<DT, 16>(d_v, norm);
        case 32: return chunk_dv<DT, 32>(d_v, norm);
        case 64: return chunk_dv<DT, 64>(d_v, norm);
    }
    return chunk_dv<DT, 128>(d_v, norm);
}

}  // namespace

int bwd_chunk_length(const BwdArgs &a) {
    const bool norm = a.variant == LA_NORMALIZED;
    return a.dtype == LA_BF16 ? chunk_dk<BF16>(a.d_k, a.d_v, norm) : chunk_dk<F32>(a.d_k, a.d_v, norm);
}

// Workspace: the state and cotangent of every chunk (float32, d_k d_v + d_k
// with the normalizer), one decay-gradient share per chunk, and (normalized)
// 1/den_t and dden_t of every token.
size_t bwd_workspace_bytes(const BwdArgs &a) {
    const int C = bwd_chunk_length(a);
    const size_t heads = static_cast<size_t>(a.B) * a.H;
    const size_t N = a.T > 0 ? (static_cast<size_t>(a.T) + C - 1) / C : 0;
    const size_t E = static_cast<size_t>(a.d_k) * a.d_v + (a.variant == LA_NORMALIZED ? a.d_k : 0);
    const size_t tok = a.variant == LA_NORMALIZED ? 2 * heads * static_cast<size_t>(a.T > 0 ? a.T : 0) : 0;
    const size_t bytes = (2 * heads * N * E + heads * N + tok) * sizeof(float);
    return (bytes + 255) / 256 * 256;
}

hipError_t launch_chunk_bwd(const BwdArgs &a) {
    if (a.dtype == LA_BF16) return bwd_dk<BF16>(a);
    return bwd_dk<F32>(a);
}

}  // namespace la
