/*
 * oracle.c -- float64 CPU oracle for causal linear attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously-correct
 * reference that the GPU path is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header or constant with the HIP library.
 *
 * Every sequence is processed token by token, exactly as the pages state
 * the recurrences, in double precision.  Each token is "update first, then
 * read" (page "Beyond -- Linear attention and recurrent memory", section
 * "Pitfalls to expect": updating the state before reading lets a token
 * attend to itself, matching the parallel form).
 *
 * Variants (integer codes used by the ctypes wrapper):
 *   0  normalized linear attention
 *        page "Beyond -- Linear attention and recurrent memory",
 *        section "The big idea":
 *          S_t = S_{t-1} + phi(k_t) v_t^T      (d_k x d_v)
 *          z_t = z_{t-1} + phi(k_t)
 *          out_t = (phi(q_t) . S_t) / (phi(q_t) . z_t)
 *        also page "Linear Attention" (normalized kernel formulation) and
 *        "Ch. 11 Linear attention and Hyena", section 11.2.
 *   1  gated linear attention (per-step, per-key-channel gate gamma_t)
 *        page "Ch. 11 Linear attention and Hyena", section 11.3 and the
 *        solution to Exercise 11.5: the gate multiplies the d_k rows of
 *        the d_k x d_v state, S_t = diag(gamma_t) S_{t-1} + phi(k_t) v_t^T,
 *        read without a normalizer, y_t = S_t^T phi(q_t).
 *   2  gated delta rule (d_v x d_k state, unit-norm keys)
 *        page "Linear Attention", gated-delta-rule formulation:
 *          S~_t = alpha_t S_{t-1}
 *          S_t  = S~_t + beta_t (v_t - S~_t k_t) k_t^T,   o_t = S_t q_t
 *        equal to page "Module 18 Beyond attention", section 18.2,
 *          S_t = g_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T.
 *
 *      With a per-head decay gamma_h (gate of shape (H,), shared by the
 *      batch; NULL means gamma_h = 1) both accumulators decay before the
 *      write, page "Beyond -- Linear attention and recurrent memory",
 *      section "Fixed decay versus an input-dependent gate":
 *          S_t = gamma_h S_{t-1} + phi(k_t) v_t^T
 *          z_t = gamma_h z_{t-1} + phi(k_t)
 *   3  retention: the same fixed per-head decay without a normalizer, the
 *      constant gate of page "Ch. 11 Linear attention and Hyena", section
 *      11.3 (RetNet bullet):
 *          S_t = gamma_h S_{t-1} + phi(k_t) v_t^T,   y_t = S_t^T phi(q_t)
 *      (gate (H,) or NULL = 1; phi identity by default).
 *   4  gated delta rule with a per-key-channel (diagonal) decay alpha_t,
 *      the finer-grained gate of page "Beyond -- Linear attention and
 *      recurrent memory", section "From fixed decay to KDA's gated delta
 *      write", in the decay-first order of variant 2 (d_v x d_k state):
 *          S~_t = S_{t-1} diag(alpha_t)
 *          S_t  = S~_t + beta_t (v_t - S~_t k_t) k_t^T,   o_t = S_t q_t
 *      (gate alpha (B, H, T, d_k), beta (B, H, T)).
 *
 * phi codes: 0 identity, 1 elu(x)+1 (page "Beyond -- Linear attention and
 * recurrent memory", section "The big idea": phi(x) = elu(x) + 1).
 *
 * External state layout for every variant: S is (B, H, d_v, d_k) row-major
 * (row = value index, column = key index), z is (B, H, d_k).  Variants 0
 * and 1 keep their state internally in the pages' own d_k x d_v
 * orientation and transpose only when reading S0 / writing S_T.
 *
 * Per-token tensors are (B, H, T, d) row-major.  gate: variant 0 and 3 ->
 * gamma_h (H,) or NULL; variant 1 -> gamma (B, H, T, d_k); variant 2 -> g
 * (B, H, T); variant 4 -> alpha (B, H, T, d_k).  beta: variants 2 and 4 ->
 * (B, H, T).
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double phi_apply(int phi, double x)
{
    /* elu(x) + 1:  x + 1 for x > 0,  exp(x) for x <= 0 */
    if (phi == 1)
        return x > 0.0 ? x + 1.0 : exp(x);
    return x;
}

double oracle_phi(int phi, double x) { return phi_apply(phi, x); }

/* One head, T tokens.  Pointers are already offset to this head. */
static void head_forward(int variant, int phi, int T, int dk, int dv,
                         const double *q, const double *k, const double *v,
                         const double *gate, const double *beta,
                         const double *S0, const double *z0,
                         double *out, double *ST, double *zT,
                         double *work /* dk*dv + 3*dk + dv doubles */)
{
    double *S = work;             /* variant 0/1/3: [c][i] (d_k x d_v); variant 2/4: [i][c] */
    double *z = S + (size_t)dk * dv;
    double *fq = z + dk;
    double *fk = fq + dk;
    double *pred = fk + dk;       /* d_v */

    /* initial state */
    for (int i = 0; i < dv; ++i)
        for (int c = 0; c < dk; ++c) {
            double s = S0 ? S0[(size_t)i * dk + c] : 0.0;
            if (variant == 2 || variant == 4) S[(size_t)i * dk + c] = s;
            else                              S[(size_t)c * dv + i] = s;
        }
    for (int c = 0; c < dk; ++c) z[c] = z0 ? z0[c] : 0.0;

    for (int t = 0; t < T; ++t) {
        const double *qt = q + (size_t)t * dk;
        const double *kt = k + (size_t)t * dk;
        const double *vt = v + (size_t)t * dv;
        double *ot = out + (size_t)t * dv;

        if (variant == 0) {
            for (int c = 0; c < dk; ++c) { fq[c] = phi_apply(phi, qt[c]); fk[c] = phi_apply(phi, kt[c]); }
            /* S_t = gamma_h S_{t-1} + phi(k_t) v_t^T ;  z_t = gamma_h z_{t-1} + phi(k_t)
               (gamma_h = 1 without a gate) */
            const double gam = gate ? gate[0] : 1.0;
            for (int c = 0; c < dk; ++c) {
                for (int i = 0; i < dv; ++i) S[(size_t)c * dv + i] = gam * S[(size_t)c * dv + i] + fk[c] * vt[i];
                z[c] = gam * z[c] + fk[c];
            }
            /* out_t = phi(q_t)^T S_t / phi(q_t)^T z_t */
            double den = 0.0;
            for (int c = 0; c < dk; ++c) den += fq[c] * z[c];
            for (int i = 0; i < dv; ++i) {
                double num = 0.0;
                for (int c = 0; c < dk; ++c) num += fq[c] * S[(size_t)c * dv + i];
                ot[i] = num / den;
            }
        } else if (variant == 1) {
            const double *gt = gate + (size_t)t * dk;
            for (int c = 0; c < dk; ++c) { fq[c] = phi_apply(phi, qt[c]); fk[c] = phi_apply(phi, kt[c]); }
            /* S_t = diag(gamma_t) S_{t-1} + phi(k_t) v_t^T */
            for (int c = 0; c < dk; ++c)
                for (int i = 0; i < dv; ++i)
                    S[(size_t)c * dv + i] = gt[c] * S[(size_t)c * dv + i] + fk[c] * vt[i];
            /* y_t = S_t^T phi(q_t) */
            for (int i = 0; i < dv; ++i) {
                double y = 0.0;
                for (int c = 0; c < dk; ++c) y += fq[c] * S[(size_t)c * dv + i];
                ot[i] = y;
            }
        } else if (variant == 3) {
            for (int c = 0; c < dk; ++c) { fq[c] = phi_apply(phi, qt[c]); fk[c] = phi_apply(phi, kt[c]); }
            /* S_t = gamma_h S_{t-1} + phi(k_t) v_t^T */
            const double gam = gate ? gate[0] : 1.0;
            for (int c = 0; c < dk; ++c)
                for (int i = 0; i < dv; ++i)
                    S[(size_t)c * dv + i] = gam * S[(size_t)c * dv + i] + fk[c] * vt[i];
            /* y_t = S_t^T phi(q_t) */
            for (int i = 0; i < dv; ++i) {
                double y = 0.0;
                for (int c = 0; c < dk; ++c) y += fq[c] * S[(size_t)c * dv + i];
                ot[i] = y;
            }
        } else if (variant == 4) {
            const double *alpha = gate + (size_t)t * dk;
            const double bw = beta[t];
            /* S~ = S_{t-1} diag(alpha_t): key channel c of every row decays by alpha_tc */
            for (int i = 0; i < dv; ++i)
                for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] *= alpha[c];
            /* prediction S~ k_t */
            for (int i = 0; i < dv; ++i) {
                double acc = 0.0;
                for (int c = 0; c < dk; ++c) acc += S[(size_t)i * dk + c] * kt[c];
                pred[i] = acc;
            }
            /* S_t = S~ + beta_t (v_t - S~ k_t) k_t^T */
            for (int i = 0; i < dv; ++i) {
                const double err = bw * (vt[i] - pred[i]);
                for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] += err * kt[c];
            }
            /* o_t = S_t q_t */
            for (int i = 0; i < dv; ++i) {
                double acc = 0.0;
                for (int c = 0; c < dk; ++c) acc += S[(size_t)i * dk + c] * qt[c];
                ot[i] = acc;
            }
        } else {
            const double a = gate[t];
            const double b = beta[t];
            /* S~ = alpha_t S_{t-1} */
            for (size_t e = 0; e < (size_t)dv * dk; ++e) S[e] *= a;
            /* prediction S~ k_t */
            for (int i = 0; i < dv; ++i) {
                double p = 0.0;
                for (int c = 0; c < dk; ++c) p += S[(size_t)i * dk + c] * kt[c];
                pred[i] = p;
            }
            /* S_t = S~ + beta_t (v_t - S~ k_t) k_t^T */
            for (int i = 0; i < dv; ++i) {
                double e = b * (vt[i] - pred[i]);
                for (int c = 0; c < dk; ++c) S[(size_t)i * dk + c] += e * kt[c];
            }
            /* o_t = S_t q_t */
            for (int i = 0; i < dv; ++i) {
                double o = 0.0;
                for (int c = 0; c < dk; ++c) o += S[(size_t)i * dk + c] * qt[c];
                ot[i] = o;
            }
        }
    }

    if (ST)
        for (int i = 0; i < dv; ++i)
            for (int c = 0; c < dk; ++c)
                ST[(size_t)i * dk + c] = (variant == 2 || variant == 4) ? S[(size_t)i * dk + c] : S[(size_t)c * dv + i];
    if (zT)
        for (int c = 0; c < dk; ++c) zT[c] = z[c];
}

static int check_args(int variant, int phi, int B, int H, int T, int dk, int dv,
                      const double *q, const double *k, const double *v,
                      const double *gate, const double *beta, const double *out)
{
    if (variant < 0 || variant > 4 || phi < 0 || phi > 1) return 1;
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return 1;
    if ((size_t)B * H * T > 0 && (!q || !k || !v || !out)) return 1;
    if (variant == 1 && T > 0 && !gate) return 1;
    if ((variant == 2 || variant == 4) && T > 0 && (!gate || !beta)) return 1;
    return 0;
}

/* The gate values of flat head h = b * H + hh: per token and channel
   (variants 1, 4), per token (variant 2), or the head's one decay (variants
   0 and 3, shared by the batch; NULL = no decay). */
static const double *head_gate(int variant, const double *gate, long h, int H, int T, int dk)
{
    if (!gate) return NULL;
    if (variant == 1 || variant == 4) return gate + (size_t)h * T * dk;
    if (variant == 2) return gate + (size_t)h * T;
    return gate + (h % H);
}

/*
 * Whole-sequence forward: B*H independent heads, each processed token by
 * token.  S0 / z0 may be NULL (zeros).  S_T / z_T may be NULL (not
 * returned) and may alias S0 / z0.  nthreads <= 0 uses the OpenMP default.
 * Returns 0 on success, 1 on bad arguments, 2 on allocation failure.
 */
int oracle_forward(int variant, int phi, int B, int H, int T, int dk, int dv,
                   const double *q, const double *k, const double *v,
                   const double *gate, const double *beta,
                   const double *S0, const double *z0,
                   double *out, double *S_T, double *z_T, int nthreads)
{
    if (check_args(variant, phi, B, H, T, dk, dv, q, k, v, gate, beta, out)) return 1;
    const long nh = (long)B * H;
    const size_t wsz = (size_t)dk * dv + 3 * (size_t)dk + dv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads) reduction(| : failed)
#endif
    {
        double *work = (double *)malloc(wsz * sizeof(double));
        if (!work) failed = 1;
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
        for (long h = 0; h < nh; ++h) {
            if (!work) continue;
            head_forward(variant, phi, T, dk, dv,
                         q + (size_t)h * T * dk, k + (size_t)h * T * dk, v + (size_t)h * T * dv,
                         head_gate(variant, gate, h, H, T, dk),
                         (variant == 2 || variant == 4) ? beta + (size_t)h * T : NULL,
                         S0 ? S0 + (size_t)h * dv * dk : NULL,
                         (variant == 0 && z0) ? z0 + (size_t)h * dk : NULL,
                         out + (size_t)h * T * dv,
                         S_T ? S_T + (size_t)h * dv * dk : NULL,
                         (variant == 0 && z_T) ? z_T + (size_t)h * dk : NULL,
                         work);
        }
        free(work);
    }
    return failed ? 2 : 0;
}

/*
 * One recurrent decode step for every head, in place on S (and z for
 * variant 0): the same token update as oracle_forward with T = 1.
 * q, k: (B,H,d_k); v, out: (B,H,d_v); gate: variant 1 (B,H,d_k),
 * variant 2 (B,H); beta: variant 2 (B,H).
 */
int oracle_decode_step(int variant, int phi, int B, int H, int dk, int dv,
                       const double *q, const double *k, const double *v,
                       const double *gate, const double *beta,
                       double *S, double *z, double *out, int nthreads)
{
    if (!S || (variant == 0 && !z)) return 1;
    return oracle_forward(variant, phi, B, H, 1, dk, dv, q, k, v, gate, beta,
                          S, variant == 0 ? z : NULL, out, S, variant == 0 ? z : NULL, nthreads);
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Gradients of oracle_forward for variants 0 (normalized, optional per-head
 * decay) and 3 (retention): reverse-mode differentiation of the token
 * recurrence, token by token from the last to the first, in double
 * precision.  The recurrence (page "Beyond -- Linear attention and
 * recurrent memory", sections "The big idea" and "Fixed decay versus an
 * input-dependent gate"), update first, then read:
 *     S_t = gamma S_{t-1} + phi(k_t) v_t^T,   z_t = gamma z_{t-1} + phi(k_t),
 *     variant 0: out_t = S_t^T phi(q_t) / (z_t . phi(q_t));
 *     variant 3: out_t = S_t^T phi(q_t).
 * Going back from token t, with num_t = S_t^T phi(q_t) and den_t = z_t.phi(q_t):
 *     d num = d out / den,  d den = -(d out . out) / den      (variant 0)
 *     dS_t += phi(q_t) d num^T,  dz_t += d den phi(q_t),
 *     d phi(q_t) = S_t d num + d den z_t,
 *     d v_t = dS_t^T phi(k_t),  d phi(k_t) = dS_t v_t + dz_t,
 *     d gamma += <dS_t, S_{t-1}> + dz_t . z_{t-1},
 *     dS_{t-1} = gamma dS_t,  dz_{t-1} = gamma dz_t,
 * and dq = d phi(q) phi'(q), dk = d phi(k) phi'(k) (phi' = 1 for the identity;
 * for elu + 1, 1 above zero and e^x at or below).  The states S_t, z_t of the
 * forward pass are kept for every token (small problems only).
 *
 * Layouts as oracle_forward; dS_T, dz_T may be NULL (zero).  Outputs dq, dk
 * (B,H,T,d_k), dv (B,H,T,d_v), dS0 (B,H,d_v,d_k), dz0 (B,H,d_k) (variant 0)
 * and dgate (H,) summed over the batch (only when gate is given; otherwise
 * may be NULL).  Returns 0 on success, 1 on bad arguments, 2 on allocation
 * failure.  Runs on one thread (the decay gradient sums over heads).
 */
static double phi_prime(int phi, double x)
{
    if (phi == 1)
        return x > 0.0 ? 1.0 : exp(x);
    return 1.0;
}

int oracle_backward(int variant, int phi, int B, int H, int T, int dk, int dv,
                    const double *q, const double *k, const double *v, const double *gate,
                    const double *S0, const double *z0,
                    const double *dout, const double *dS_T, const double *dz_T,
                    double *dq, double *dk_out, double *dv_out, double *dgate,
                    double *dS0, double *dz0)
{
    if (variant != 0 && variant != 3) return 1;
    if (B < 0 || H < 0 || T < 0 || dk <= 0 || dv <= 0) return 1;
    const size_t sz = (size_t)dk * dv;
    double *Sall = (double *)malloc(((size_t)T + 1) * sz * sizeof(double));   /* S_{-1} .. S_{T-1}, [c][i] */
    double *zall = (double *)malloc(((size_t)T + 1) * dk * sizeof(double));
    double *dS = (double *)malloc(sz * sizeof(double));
    double *dz = (double *)malloc((size_t)dk * sizeof(double));
    double *fq = (double *)malloc((size_t)dk * sizeof(double));
    double *fk = (double *)malloc((size_t)dk * sizeof(double));
    double *dnum = (double *)malloc((size_t)dv * sizeof(double));
    double *num = (double *)malloc((size_t)dv * sizeof(double));
    if (!Sall || !zall || !dS || !dz || !fq || !fk || !dnum || !num) {
        free(Sall); free(zall); free(dS); free(dz); free(fq); free(fk); free(dnum); free(num);
        return 2;
    }
    if (gate)
        for (int h = 0; h < H; ++h) dgate[h] = 0.0;
    for (long bh = 0; bh < (long)B * H; ++bh) {
        const double gam = gate ? gate[bh % H] : 1.0;
        const double *qh = q + (size_t)bh * T * dk, *kh = k + (size_t)bh * T * dk, *vh = v + (size_t)bh * T * dv;
        const double *doh = dout + (size_t)bh * T * dv;
        /* forward, keeping every state (internal layout [c][i], d_k x d_v) */
        for (int i = 0; i < dv; ++i)
            for (int c = 0; c < dk; ++c) Sall[(size_t)c * dv + i] = S0 ? S0[(size_t)bh * sz + (size_t)i * dk + c] : 0.0;
        for (int c = 0; c < dk; ++c) zall[c] = (variant == 0 && z0) ? z0[(size_t)bh * dk + c] : 0.0;
        for (int t = 0; t < T; ++t) {
            const double *Sp = Sall + (size_t)t * sz, *zp = zall + (size_t)t * dk;
            double *Sn = Sall + (size_t)(t + 1) * sz, *zn = zall + (size_t)(t + 1) * dk;
            for (int c = 0; c < dk; ++c) {
                const double f = phi_apply(phi, kh[(size_t)t * dk + c]);
                for (int i = 0; i < dv; ++i) Sn[(size_t)c * dv + i] = gam * Sp[(size_t)c * dv + i] + f * vh[(size_t)t * dv + i];
                zn[c] = gam * zp[c] + f;
            }
        }
        /* backward */
        for (int i = 0; i < dv; ++i)
            for (int c = 0; c < dk; ++c) dS[(size_t)c * dv + i] = dS_T ? dS_T[(size_t)bh * sz + (size_t)i * dk + c] : 0.0;
        for (int c = 0; c < dk; ++c) dz[c] = (variant == 0 && dz_T) ? dz_T[(size_t)bh * dk + c] : 0.0;
        double dg = 0.0;
        for (int t = T - 1; t >= 0; --t) {
            const double *St = Sall + (size_t)(t + 1) * sz, *zt = zall + (size_t)(t + 1) * dk;
            const double *Sp = Sall + (size_t)t * sz, *zp = zall + (size_t)t * dk;
            const double *dot = doh + (size_t)t * dv;
            for (int c = 0; c < dk; ++c) {
                fq[c] = phi_apply(phi, qh[(size_t)t * dk + c]);
                fk[c] = phi_apply(phi, kh[(size_t)t * dk + c]);
            }
            double dden = 0.0;
            if (variant == 0) {
                double den = 0.0;
                for (int c = 0; c < dk; ++c) den += zt[c] * fq[c];
                double dot_o = 0.0;
                for (int i = 0; i < dv; ++i) {
                    double s = 0.0;
                    for (int c = 0; c < dk; ++c) s += St[(size_t)c * dv + i] * fq[c];
                    num[i] = s;
                    dot_o += dot[i] * (s / den);
                    dnum[i] = dot[i] / den;
                }
                dden = -dot_o / den;
            } else {
                for (int i = 0; i < dv; ++i) dnum[i] = dot[i];
            }
            /* the read of token t: dS_t += phi(q) dnum^T, dz_t += dden phi(q) */
            for (int c = 0; c < dk; ++c) {
                for (int i = 0; i < dv; ++i) dS[(size_t)c * dv + i] += fq[c] * dnum[i];
                dz[c] += dden * fq[c];
            }
            /* d phi(q_t) = S_t dnum + dden z_t */
            for (int c = 0; c < dk; ++c) {
                double s = 0.0;
                for (int i = 0; i < dv; ++i) s += St[(size_t)c * dv + i] * dnum[i];
                s += dden * zt[c];
                dq[((size_t)bh * T + t) * dk + c] = s * phi_prime(phi, qh[(size_t)t * dk + c]);
            }
            /* the write of token t */
            for (int i = 0; i < dv; ++i) {
                double s = 0.0;
                for (int c = 0; c < dk; ++c) s += dS[(size_t)c * dv + i] * fk[c];
                dv_out[((size_t)bh * T + t) * dv + i] = s;
            }
            for (int c = 0; c < dk; ++c) {
                double s = 0.0;
                for (int i = 0; i < dv; ++i) s += dS[(size_t)c * dv + i] * vh[(size_t)t * dv + i];
                s += dz[c];
                dk_out[((size_t)bh * T + t) * dk + c] = s * phi_prime(phi, kh[(size_t)t * dk + c]);
            }
            /* the decay of token t */
            for (size_t e = 0; e < sz; ++e) dg += dS[e] * Sp[e];
            for (int c = 0; c < dk; ++c) dg += dz[c] * zp[c];
            for (size_t e = 0; e < sz; ++e) dS[e] *= gam;
            for (int c = 0; c < dk; ++c) dz[c] *= gam;
        }
        if (gate) dgate[bh % H] += dg;
        if (dS0)
            for (int i = 0; i < dv; ++i)
                for (int c = 0; c < dk; ++c) dS0[(size_t)bh * sz + (size_t)i * dk + c] = dS[(size_t)c * dv + i];
        if (dz0 && variant == 0)
            for (int c = 0; c < dk; ++c) dz0[(size_t)bh * dk + c] = dz[c];
    }
    free(Sall); free(zall); free(dS); free(dz); free(fq); free(fk); free(dnum); free(num);
    return 0;
}
