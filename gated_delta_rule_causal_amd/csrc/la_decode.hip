// la_decode.hip -- one-token recurrent step for the three variants (gfx950).
//
// The step is bandwidth-bound: every head's d_v x d_k float32 state is read
// once and written once, with O(d_k d_v) arithmetic (page "Beyond -- Linear
// attention and recurrent memory", section "The big idea": per-token state
// work independent of history length).  The kernel streams the state through
// registers: a state row of d_k floats is split over G = d_k/8 lanes (eight
// consecutive floats, two 16-byte loads per lane), every row of a workgroup
// is loaded before any arithmetic so that all of a lane's loads are in
// flight together, and the two row dot products a step needs are reduced
// across the G lanes with lane shuffles.  Workgroups of 1024 lanes keep at
// most two rows per lane (few registers, many waves in flight); the new state
// is written with non-temporal stores.  No LDS, and no barrier except the one
// the normalized variant needs before it overwrites the shared z.
//
// Per-row arithmetic (row i of the d_v x d_k state, all in float32):
//   gated delta rule (page "Linear Attention", decay first, then predict):
//     p = S_i.k, r = S_i.q, u = beta (v_i - g p),
//     S_i <- g S_i + u k,  o_i = g r + u (k.q)      (= S_new,i . q)
//   gated linear attention (page "Ch. 11 Linear attention and Hyena", 11.3):
//     r = S_i.(gamma o phi(q)),  S_i <- S_i o gamma + v_i phi(k),
//     o_i = r + v_i (phi(k).phi(q))                 (= S_new,i . phi(q))
//   normalized (page "Beyond -- Linear attention and recurrent memory"),
//   with the head's fixed decay gamma (1 without one; section "Fixed decay
//   versus an input-dependent gate"):
//     r = gamma S_i.phi(q),  S_i <- gamma S_i + v_i phi(k),  z <- gamma z + phi(k),
//     o_i = (r + v_i (phi(k).phi(q))) / (gamma z_old.phi(q) + phi(k).phi(q))
//   retention (page "Ch. 11 Linear attention and Hyena", 11.3, RetNet bullet):
//     the same without z: o_i = r + v_i (phi(k).phi(q))
//   delta rule with a per-channel decay alpha (page "Beyond -- Linear
//   attention and recurrent memory", "From fixed decay to KDA's gated delta
//   write"; decay first as above): with a = alpha o k, b = alpha o q,
//     p = S_i.a, r = S_i.b, u = beta (v_i - p),
//     S_i <- S_i o alpha + u k,  o_i = r + u (k.q)
#include "la_internal.hpp"

namespace la {

constexpr int kDecodeThreads = 1024;

template <int VAR, class DT, int DK, int DV, int PHI>
__global__ __launch_bounds__(kDecodeThreads) void decode_kernel(
    const typename DT::storage *__restrict__ q, const typename DT::storage *__restrict__ k,
    const typename DT::storage *__restrict__ v, const float *__restrict__ gate,
    const float *__restrict__ beta, float *__restrict__ S, float *__restrict__ z,
    typename DT::storage *__restrict__ out, int64_t n_heads, int H) {
    constexpr int G = DK / 8;                                // lanes per state row
    constexpr int GROUPS = kDecodeThreads / G;               // row groups per workgroup
    constexpr int HPW = GROUPS >= DV ? GROUPS / DV : 1;      // heads per workgroup
    constexpr int GPH = GROUPS / HPW;                        // groups per head
    constexpr int RPG = DV / GPH;                            // rows per group
    static_assert(DK % 8 == 0 && G <= 64 && RPG >= 1 && RPG * GPH == DV, "decode tiling");

    const int tid = threadIdx.x;
    const int grp = tid / G;
    const int c0 = (tid % G) * 8;
    const int64_t head = static_cast<int64_t>(blockIdx.x) * HPW + grp / GPH;
    const int row0 = grp % GPH;
    const bool active = head < n_heads;
    const int64_t h = active ? head : 0;   // inactive lanes compute on head 0 and store nothing

    float kk[8], qq[8];
    load8(k + h * DK + c0, kk);
    load8(q + h * DK + c0, qq);
    float s[RPG][8];
    float vv[RPG];
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        load8(S + (h * DV + row0 + r * GPH) * DK + c0, s[r]);
        vv[r] = load1(v + h * DV + row0 + r * GPH);
    }

    if constexpr (VAR == LA_KDA) {
        float al[8], ak[8], aq[8];
        load8(gate + h * DK + c0, al);
        const float b = beta[h];
        float kq = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) { kq += kk[c] * qq[c]; ak[c] = al[c] * kk[c]; aq[c] = al[c] * qq[c]; }
        kq = group_sum<G>(kq);
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            float p = 0.f, rq = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) { p += s[r][c] * ak[c]; rq += s[r][c] * aq[c]; }
            p = group_sum<G>(p);
            rq = group_sum<G>(rq);
            const float u = b * (vv[r] - p);
#pragma unroll
            for (int c = 0; c < 8; ++c) s[r][c] = s[r][c] * al[c] + u * kk[c];
            vv[r] = rq + u * kq;
        }
    } else if constexpr (VAR == LA_GATED_DELTA) {
        const float g = gate[h];
        const float b = beta[h];
        float kq = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) kq += kk[c] * qq[c];
        kq = group_sum<G>(kq);
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            float p = 0.f, rq = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) { p += s[r][c] * kk[c]; rq += s[r][c] * qq[c]; }
            p = group_sum<G>(p);
            rq = group_sum<G>(rq);
            const float u = b * (vv[r] - g * p);
#pragma unroll
            for (int c = 0; c < 8; ++c) s[r][c] = g * s[r][c] + u * kk[c];
            vv[r] = g * rq + u * kq;   // output
        }
    } else {
        float fk[8], fq[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) { fk[c] = apply_phi<PHI>(kk[c]); fq[c] = apply_phi<PHI>(qq[c]); }
        float kq = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) kq += fk[c] * fq[c];
        kq = group_sum<G>(kq);
        if constexpr (VAR == LA_GATED) {
            float gm[8], rq_w[8];
            load8(gate + h * DK + c0, gm);
#pragma unroll
            for (int c = 0; c < 8; ++c) rq_w[c] = gm[c] * fq[c];
#pragma unroll
            for (int r = 0; r < RPG; ++r) {
                float rq = 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) rq += s[r][c] * rq_w[c];
                rq = group_sum<G>(rq);
#pragma unroll
                for (int c = 0; c < 8; ++c) s[r][c] = s[r][c] * gm[c] + vv[r] * fk[c];
                vv[r] = rq + vv[r] * kq;
            }
        } else if constexpr (VAR == LA_RETENTION) {
            const float gm = gate ? gate[h % H] : 1.f;
#pragma unroll
            for (int r = 0; r < RPG; ++r) {
                float rq = 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) rq += s[r][c] * fq[c];
                rq = group_sum<G>(rq);
#pragma unroll
                for (int c = 0; c < 8; ++c) s[r][c] = gm * s[r][c] + vv[r] * fk[c];
                vv[r] = gm * rq + vv[r] * kq;
            }
        } else {
            const float gm = gate ? gate[h % H] : 1.f;
            float zz[8];
            load8(z + h * DK + c0, zz);
            float zq = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) zq += zz[c] * fq[c];
            zq = group_sum<G>(zq);
            const float inv_den = 1.f / (gm * zq + kq);
#pragma unroll
            for (int r = 0; r < RPG; ++r) {
                float rq = 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) rq += s[r][c] * fq[c];
                rq = group_sum<G>(rq);
#pragma unroll
                for (int c = 0; c < 8; ++c) s[r][c] = gm * s[r][c] + vv[r] * fk[c];
                vv[r] = (gm * rq + vv[r] * kq) * inv_den;
            }
            // every group of the head has read z; only then may row 0's group overwrite it
            __syncthreads();
            if (active && row0 == 0) {
                float4 *zp = reinterpret_cast<float4 *>(z + h * DK + c0);
                zp[0] = make_float4(gm * zz[0] + fk[0], gm * zz[1] + fk[1], gm * zz[2] + fk[2], gm * zz[3] + fk[3]);
                zp[1] = make_float4(gm * zz[4] + fk[4], gm * zz[5] + fk[5], gm * zz[6] + fk[6], gm * zz[7] + fk[7]);
            }
        }
    }

    if (!active) return;
#pragma unroll
    for (int r = 0; r < RPG; ++r) {
        f32x4_t *sp = reinterpret_cast<f32x4_t *>(S + (h * DV + row0 + r * GPH) * DK + c0);
        __builtin_nontemporal_store(f32x4_t{s[r][0], s[r][1], s[r][2], s[r][3]}, sp);
        __builtin_nontemporal_store(f32x4_t{s[r][4], s[r][5], s[r][6], s[r][7]}, sp + 1);
        if (c0 == 0) store1(out + h * DV + row0 + r * GPH, vv[r]);
    }
}

// ------------------------------------------------------------------ multi-token
// Speculative decoding by checkpoint plus input replay (page "Beyond --
// Linear attention and recurrent memory", section "What we don't cover",
// recurrent-state commit and rollback): a fixed state has no token rows to
// truncate, so draft tokens are verified from the checkpointed state without
// changing it, and the accepted prefix is then replayed into it.
//   COMMIT = false (verify): T tokens from S (and z), outputs of every token,
//            S and z untouched;
//   COMMIT = true (commit):  the first accepted[b] tokens of sequence b
//            (clamped to [0, T]) applied to S (and z) in place, no outputs.
// The state rows stay in registers for all the tokens, so either call reads
// the state once (commit writes it once); the per-token arithmetic is the
// step of decode_kernel above.  The normalizer z is kept per lane in
// registers (every row group of a head updates its own copy identically) and
// written after a barrier, once every group has read it.
template <int VAR, class DT, int DK, int DV, int PHI, bool COMMIT>
__global__ __launch_bounds__(kDecodeThreads) void decode_multi_kernel(
    const typename DT::storage *__restrict__ q, const typename DT::storage *__restrict__ k,
    const typename DT::storage *__restrict__ v, const float *__restrict__ gate,
    const float *__restrict__ beta, float *__restrict__ S, float *__restrict__ z,
    typename DT::storage *__restrict__ out, const int32_t *__restrict__ accepted, int64_t n_heads, int H, int T) {
    constexpr int G = DK / 8;
    constexpr int GROUPS = kDecodeThreads / G;
    constexpr int HPW = GROUPS >= DV ? GROUPS / DV : 1;
    constexpr int GPH = GROUPS / HPW;
    constexpr int RPG = DV / GPH;
    static_assert(DK % 8 == 0 && G <= 64 && RPG >= 1 && RPG * GPH == DV, "decode tiling");

    const int tid = threadIdx.x;
    const int grp = tid / G;
    const int c0 = (tid % G) * 8;
    const int64_t head = static_cast<int64_t>(blockIdx.x) * HPW + grp / GPH;
    const int row0 = grp % GPH;
    const bool active = head < n_heads;
    const int64_t h = active ? head : 0;
    // tokens to apply: all T to verify; the sequence's accepted count to commit
    const int n = COMMIT ? min(max(accepted[h / H], 0), T) : T;

    float s[RPG][8];
#pragma unroll
    for (int r = 0; r < RPG; ++r) load8(S + (h * DV + row0 + r * GPH) * DK + c0, s[r]);
    float zz[8];
    if constexpr (VAR == LA_NORMALIZED) load8(z + h * DK + c0, zz);
    const float gh = (VAR == LA_NORMALIZED || VAR == LA_RETENTION) && gate ? gate[h % H] : 1.f;

    for (int t = 0; t < n; ++t) {
        const int64_t tok = h * T + t;
        float kk[8], qq[8], vv[RPG];
        load8(k + tok * DK + c0, kk);
        if constexpr (!COMMIT) load8(q + tok * DK + c0, qq);
#pragma unroll
        for (int r = 0; r < RPG; ++r) vv[r] = load1(v + tok * DV + row0 + r * GPH);

        if constexpr (VAR == LA_KDA) {
            float al[8], ak[8], aq[8];
            load8(gate + tok * DK + c0, al);
            const float b = beta[tok];
            float kq = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                ak[c] = al[c] * kk[c];
                aq[c] = COMMIT ? 0.f : al[c] * qq[c];
                if constexpr (!COMMIT) kq += kk[c] * qq[c];
            }
            if constexpr (!COMMIT) kq = group_sum<G>(kq);
#pragma unroll
            for (int r = 0; r < RPG; ++r) {
                float p = 0.f, rq = 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    p += s[r][c] * ak[c];
                    if constexpr (!COMMIT) rq += s[r][c] * aq[c];
                }
                p = group_sum<G>(p);
                if constexpr (!COMMIT) rq = group_sum<G>(rq);
                const float u = b * (vv[r] - p);
#pragma unroll
                for (int c = 0; c < 8; ++c) s[r][c] = s[r][c] * al[c] + u * kk[c];
                vv[r] = rq + u * kq;
            }
        } else if constexpr (VAR == LA_GATED_DELTA) {
            const float g = gate[tok], b = beta[tok];
            float kq = 0.f;
            if constexpr (!COMMIT) {
#pragma unroll
                for (int c = 0; c < 8; ++c) kq += kk[c] * qq[c];
                kq = group_sum<G>(kq);
            }
#pragma unroll
            for (int r = 0; r < RPG; ++r) {
                float p = 0.f, rq = 0.f;
#pragma unroll
                for (int c = 0; c < 8; ++c) {
                    p += s[r][c] * kk[c];
                    if constexpr (!COMMIT) rq += s[r][c] * qq[c];
                }
                p = group_sum<G>(p);
                if constexpr (!COMMIT) rq = group_sum<G>(rq);
                const float u = b * (vv[r] - g * p);
#pragma unroll
                for (int c = 0; c < 8; ++c) s[r][c] = g * s[r][c] + u * kk[c];
                vv[r] = g * rq + u * kq;
            }
        } else {
            float fk[8], fq[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                fk[c] = apply_phi<PHI>(kk[c]);
                fq[c] = COMMIT ? 0.f : apply_phi<PHI>(qq[c]);
            }
            float kq = 0.f;
            if constexpr (!COMMIT) {
#pragma unroll
                for (int c = 0; c < 8; ++c) kq += fk[c] * fq[c];
                kq = group_sum<G>(kq);
            }
            if constexpr (VAR == LA_GATED) {
                float gm[8];
                load8(gate + tok * DK + c0, gm);
#pragma unroll
                for (int r = 0; r < RPG; ++r) {
                    float rq = 0.f;
                    if constexpr (!COMMIT) {
#pragma unroll
                        for (int c = 0; c < 8; ++c) rq += s[r][c] * gm[c] * fq[c];
                        rq = group_sum<G>(rq);
                    }
#pragma unroll
                    for (int c = 0; c < 8; ++c) s[r][c] = s[r][c] * gm[c] + vv[r] * fk[c];
                    vv[r] = rq + vv[r] * kq;
                }
            } else {
                float inv_den = 1.f;
                if constexpr (VAR == LA_NORMALIZED && !COMMIT) {
                    float zq = 0.f;
#pragma unroll
                    for (int c = 0; c < 8; ++c) zq += zz[c] * fq[c];
                    zq = group_sum<G>(zq);
                    inv_den = 1.f / (gh * zq + kq);
                }
#pragma unroll
                for (int r = 0; r < RPG; ++r) {
                    float rq = 0.f;
                    if constexpr (!COMMIT) {
#pragma unroll
                        for (int c = 0; c < 8; ++c) rq += s[r][c] * fq[c];
                        rq = group_sum<G>(rq);
                    }
#pragma unroll
                    for (int c = 0; c < 8; ++c) s[r][c] = gh * s[r][c] + vv[r] * fk[c];
                    vv[r] = (gh * rq + vv[r] * kq) * inv_den;
                }
                if constexpr (VAR == LA_NORMALIZED) {
#pragma unroll
                    for (int c = 0; c < 8; ++c) zz[c] = gh * zz[c] + fk[c];
                }
            }
        }
        if constexpr (!COMMIT) {
            if (active && c0 == 0) {
#pragma unroll
                for (int r = 0; r < RPG; ++r) store1(out + tok * DV + row0 + r * GPH, vv[r]);
            }
        }
    }

    if constexpr (COMMIT) {
        // every group of the head has read z (at the start); only then may row
        // 0's group overwrite it
        if constexpr (VAR == LA_NORMALIZED) __syncthreads();
        if (!active || n == 0) return;
#pragma unroll
        for (int r = 0; r < RPG; ++r) {
            f32x4_t *sp = reinterpret_cast<f32x4_t *>(S + (h * DV + row0 + r * GPH) * DK + c0);
            __builtin_nontemporal_store(f32x4_t{s[r][0], s[r][1], s[r][2], s[r][3]}, sp);
            __builtin_nontemporal_store(f32x4_t{s[r][4], s[r][5], s[r][6], s[r][7]}, sp + 1);
        }
        if constexpr (VAR == LA_NORMALIZED) {
            if (row0 == 0) {
                float4 *zp = reinterpret_cast<float4 *>(z + h * DK + c0);
                zp[0] = make_float4(zz[0], zz[1], zz[2], zz[3]);
                zp[1] = make_float4(zz[4], zz[5], zz[6], zz[7]);
            }
        }
    }
}

// ------------------------------------------------------------------ dispatch

template <int VAR, class DT, int DK, int DV, int PHI>
static hipError_t launch_decode_t(const DecodeArgs &a) {
    constexpr int G = DK / 8;
    constexpr int GROUPS = kDecodeThreads / G;
    constexpr int HPW = GROUPS >= DV ? GROUPS / DV : 1;
    const int64_t n_heads = static_cast<int64_t>(a.B) * a.H;
    const int64_t blocks = (n_heads + HPW - 1) / HPW;
    typedef typename DT::storage T;
    const dim3 grid(static_cast<uint32_t>(blocks)), block(kDecodeThreads);
    const T *q = static_cast<const T *>(a.q), *k = static_cast<const T *>(a.k), *v = static_cast<const T *>(a.v);
    T *out = static_cast<T *>(a.out);
    if (a.mode == DECODE_STEP)
        hipLaunchKernelGGL((decode_kernel<VAR, DT, DK, DV, PHI>), grid, block, 0, a.stream, q, k, v, a.gate, a.beta,
                           a.S, a.z, out, n_heads, a.H);
    else if (a.mode == DECODE_VERIFY)
        hipLaunchKernelGGL((decode_multi_kernel<VAR, DT, DK, DV, PHI, false>), grid, block, 0, a.stream, q, k, v,
                           a.gate, a.beta, a.S, a.z, out, a.accepted, n_heads, a.H, a.T);
    else
        hipLaunchKernelGGL((decode_multi_kernel<VAR, DT, DK, DV, PHI, true>), grid, block, 0, a.stream, q, k, v,
                           a.gate, a.beta, a.S, a.z, out, a.accepted, n_heads, a.H, a.T);
    return hipGetLastError();
}

template <int VAR, class DT, int DK, int PHI>
static hipError_t decode_dv(const DecodeArgs &a) {
    switch (a.d_v) {
        case 16: return launch_decode_t<VAR, DT, DK, 16, PHI>(a);
        case 32: return launch_decode_t<VAR, DT, DK, 32, PHI>(a);
        case 64: return launch_decode_t<VAR, DT, DK, 64, PHI>(a);
        case 128: return launch_decode_t<VAR, DT, DK, 128, PHI>(a);
    }
    return hipErrorInvalidValue;
}

template <int VAR, class DT, int PHI>
static hipError_t decode_dk(const DecodeArgs &a) {
    switch (a.d_k) {
        case 16: return decode_dv<VAR, DT, 16, PHI>(a);
        case 32: return decode_dv<VAR, DT, 32, PHI>(a);
        case 64: return decode_dv<VAR, DT, 64, PHI>(a);
        case 128: return decode_dv<VAR, DT, 128, PHI>(a);
    }
    return hipErrorInvalidValue;
}

template <class DT>
static hipError_t decode_variant(const DecodeArgs &a) {
    if (a.variant == LA_NORMALIZED) return decode_dk<LA_NORMALIZED, DT, LA_PHI_ELU1>(a);
    if (a.variant == LA_GATED_DELTA) return decode_dk<LA_GATED_DELTA, DT, LA_PHI_IDENTITY>(a);
    if (a.variant == LA_KDA) return decode_dk<LA_KDA, DT, LA_PHI_IDENTITY>(a);
    if (a.variant == LA_RETENTION) {
        if (a.phi == LA_PHI_ELU1) return decode_dk<LA_RETENTION, DT, LA_PHI_ELU1>(a);
        return decode_dk<LA_RETENTION, DT, LA_PHI_IDENTITY>(a);
    }
    if (a.phi == LA_PHI_ELU1) return decode_dk<LA_GATED, DT, LA_PHI_ELU1>(a);
    return decode_dk<LA_GATED, DT, LA_PHI_IDENTITY>(a);
}

hipError_t launch_decode(const DecodeArgs &a) {
    if (a.dtype == LA_BF16) return decode_variant<BF16>(a);
    return decode_variant<F32>(a);
}

}  // namespace la
