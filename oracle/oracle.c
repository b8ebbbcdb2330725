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
