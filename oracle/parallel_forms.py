"""Explicit T x T masked-parallel forms, float64 numpy -- TEST INFRASTRUCTURE.

These are the "parallel faces" the pages state next to each recurrence.  They
materialize the full T x T score and decay matrices, so they are quadratic in
T and only meant for T up to a few hundred.  Their one job is to pin the
token-by-token oracle in ``oracle.c``: the tests require the two to agree to
1e-12 in float64.  Nothing here is shared with, or imported by, the GPU path.

All functions take ONE head: q, k (T, d_k), v (T, d_v).  States passed in or
returned use the pages' orientation named in each docstring.
"""
from __future__ import annotations

import numpy as np


def phi_elu1(x):
    """elu(x) + 1: x + 1 for x > 0 and exp(x) otherwise.

    Page "Beyond -- Linear attention and recurrent memory", section "The big
    idea"; page "Ch. 11 Linear attention and Hyena", section 11.2.
    """
    x = np.asarray(x, np.float64)
    return np.where(x > 0, x + 1.0, np.exp(np.minimum(x, 0.0)))


def causal_mask(T):
    """L_tj = 1 if j <= t else 0 (diagonal included: a token sees itself)."""
    return np.tril(np.ones((T, T), np.float64))


def la_masked(q, k, v, S0=None, z0=None, phi=phi_elu1):
    """Normalized linear attention, parallel form.

    Page "Ch. 11 Linear attention and Hyena", section 11.2 and the solution
    to Exercise 11.4: the unnormalized output is (L o (Q_phi K_phi^T)) V with
    the causal mask L; the normalizer is the same masked score matrix summed
    over keys.  A nonzero initial state S0 (d_k x d_v, the pages'
    orientation) and z0 (d_k) add phi(q_t)^T S0 and phi(q_t)^T z0, which is
    what unrolling S_t = S_{t-1} + phi(k_t) v_t^T from S0 gives.
    Returns out (T, d_v).
    """
    Qf, Kf = phi(q), phi(k)
    T = q.shape[0]
    scores = causal_mask(T) * (Qf @ Kf.T)
    num = scores @ v
    den = scores.sum(axis=1)
    if S0 is not None:
        num = num + Qf @ S0
    if z0 is not None:
        den = den + Qf @ z0
    return num / den[:, None]


def gla_decay(gamma):
    """D[t, j, c] = prod_{i=j+1}^{t} gamma[i, c] for j <= t, else 0.

    The per-channel decay mask of gated linear attention (page "Ch. 11 Linear
    attention and Hyena", section 11.3, data-dependent gate: L_tj is the
    product of the gates strictly after j up to and including t).  Built
    from explicit running products, not from log-gate differences.
    """
    T, dk = gamma.shape
    D = np.zeros((T, T, dk), np.float64)
    for j in range(T):
        run = np.ones(dk, np.float64)
        D[j, j] = run
        for t in range(j + 1, T):
            run = run * gamma[t]
            D[t, j] = run
    return D


def gla_masked(q, k, v, gamma, S0=None, phi=phi_elu1):
    """Gated linear attention, parallel form with the explicit decay mask.

    Page "Ch. 11 Linear attention and Hyena", solution to Exercise 11.5:
    y_t = sum_{j<=t} v_j sum_c phi(q_t)_c (prod_{i=j+1}^t gamma_{i,c}) phi(k_j)_c.
    A nonzero initial state S0 (d_k x d_v) contributes
    sum_c phi(q_t)_c (prod_{i=1}^t gamma_{i,c}) S0[c, :].
    Returns out (T, d_v).
    """
    Qf, Kf = phi(q), phi(k)
    D = gla_decay(gamma)
    P = np.einsum("tc,tjc,jc->tj", Qf, D, Kf)
    out = P @ v
    if S0 is not None:
        G = np.cumprod(gamma, axis=0)       # prod_{i=1}^{t} gamma_i
        out = out + (Qf * G) @ S0
    return out


def retnet_masked(q, k, v, gamma, phi=phi_elu1):
    """Constant gate gamma_t = gamma: the Toeplitz mask L_tj = gamma^(t-j).

    Page "Ch. 11 Linear attention and Hyena", section 11.3 (RetNet bullet)
    and Exercise 11.3.  Returns out (T, d_v) of y_t = sum_j L_tj
    (phi(q_t).phi(k_j)) v_j, no normalizer.
    """
    T = q.shape[0]
    lag = np.arange(T)[:, None] - np.arange(T)[None, :]
    L = np.where(lag >= 0, float(gamma) ** np.maximum(lag, 0), 0.0)
    return (L * (phi(q) @ phi(k).T)) @ v


def gdr_product_form(q, k, v, g, beta, S0=None):
    """Gated delta rule written with the explicit transition matrix.

    Page "Module 18 Beyond attention", section 18.2:
    S_t = g_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T with the
    d_v x d_k state, read as o_t = S_t q_t (page "Linear Attention").
    Returns (out (T, d_v), S_T (d_v, d_k)).
    """
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
    I = np.eye(dk)
    out = np.empty((T, dv))
    for t in range(T):
        kt = k[t][:, None]
        S = g[t] * S @ (I - beta[t] * (kt @ kt.T)) + beta[t] * (v[t][:, None] @ kt.T)
        out[t] = S @ q[t]
    return out, S


def gdr_ut_form(q, k, v, g, beta, S0=None):
    """Gated delta rule over the whole sequence as one triangular solve.

    Not printed on the pages; derived from the page-2 recurrence by
    unrolling.  With G_tj = prod_{i=j+1}^t g_i and pseudo-values
    u_t = beta_t (v_t - g_t S_{t-1} k_t), the state is
    S_t = (prod_{i<=t} g_i) S0 + sum_{j<=t} G_tj u_j k_j^T, and substituting
    back gives the unit-lower-triangular system
    (I + A) U = diag(beta) V - diag(beta * g_cum) K S0^T,
    A_tj = beta_t G_tj (k_t . k_j) for j < t.  Then
    O = diag(g_cum) Q S0^T + (L o G o Q K^T) U.
    Returns (out (T, d_v), S_T (d_v, d_k)).
    """
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dv, dk)) if S0 is None else np.asarray(S0, np.float64)
    G = np.zeros((T, T))
    for j in range(T):
        run = 1.0
        G[j, j] = 1.0
        for t in range(j + 1, T):
            run *= g[t]
            G[t, j] = run
    gcum = np.cumprod(g)
    A = np.tril(beta[:, None] * G * (k @ k.T), -1)
    rhs = beta[:, None] * v - (beta * gcum)[:, None] * (k @ S0.T)
    U = np.linalg.solve(np.eye(T) + A, rhs)
    out = gcum[:, None] * (q @ S0.T) + (np.tril(G) * (q @ k.T)) @ U
    tail = G[T - 1] if T > 0 else np.zeros(0)          # prod_{i=j+1}^{T} g_i
    S_T = gcum[-1] * S0 + U.T @ (tail[:, None] * k) if T > 0 else S0.copy()
    return out, S_T


def decay_weights(T, gamma):
    """W_tj = gamma^(t-j) for j <= t, else 0: the distance-dependent weights
    of a fixed per-head decay (page "Beyond -- Linear attention and recurrent
    memory", section "Pitfalls to expect": the parallel form applies the
    geometric decay gamma^(t-i))."""
    lag = np.arange(T)[:, None] - np.arange(T)[None, :]
    return np.where(lag >= 0, float(gamma) ** np.maximum(lag, 0), 0.0)


def la_decayed_masked(q, k, v, gamma, S0=None, z0=None, phi=phi_elu1):
    """Normalized linear attention with a fixed per-head decay, parallel form.

    Page "Beyond -- Linear attention and recurrent memory", section "Fixed
    decay versus an input-dependent gate": S and z both decay by gamma before
    each write, so the masked scores carry gamma^(t-j) in numerator and
    denominator alike.  Unrolling from (S0, z0) (d_k x d_v, d_k) adds
    gamma^(t+1) phi(q_t)^T S0 and gamma^(t+1) phi(q_t)^T z0 (t counted from 0).
    Returns out (T, d_v).
    """
    Qf, Kf = phi(q), phi(k)
    T = q.shape[0]
    scores = decay_weights(T, gamma) * (Qf @ Kf.T)
    num = scores @ v
    den = scores.sum(axis=1)
    lead = float(gamma) ** np.arange(1, T + 1)
    if S0 is not None:
        num = num + lead[:, None] * (Qf @ S0)
    if z0 is not None:
        den = den + lead * (Qf @ z0)
    return num / den[:, None]


def retention_masked(q, k, v, gamma, S0=None, phi=None):
    """Constant per-head gate, no normalizer: y = (W o (phi(Q) phi(K)^T)) V with
    the Toeplitz weights gamma^(t-j) (page "Ch. 11 Linear attention and
    Hyena", section 11.3, RetNet bullet), plus gamma^(t+1) phi(q_t)^T S0 for an
    initial state S0 (d_k x d_v).  phi defaults to the identity.
    Returns out (T, d_v).
    """
    f = (lambda x: np.asarray(x, np.float64)) if phi is None else phi
    Qf, Kf = f(q), f(k)
    T = q.shape[0]
    out = (decay_weights(T, gamma) * (Qf @ Kf.T)) @ v
    if S0 is not None:
        out = out + (float(gamma) ** np.arange(1, T + 1))[:, None] * (Qf @ S0)
    return out


def kda_product_form(q, k, v, alpha, beta, S0=None):
    """Gated delta rule with a per-key-channel decay, explicit transition form.

    The decay-first delta write of page "Module 18 Beyond attention", section
    18.2, with the scalar gate replaced by the diagonal one of page "Beyond --
    Linear attention and recurrent memory", section "From fixed decay to KDA's
    gated delta write": S_t = S_{t-1} diag(alpha_t) (I - beta_t k_t k_t^T)
    + beta_t v_t k_t^T (d_v x d_k state), o_t = S_t q_t.
    Returns (out (T, d_v), S_T (d_v, d_k)).
    """
    T, dk = k.shape
    dv = v.shape[1]
    S = np.zeros((dv, dk)) if S0 is None else np.array(S0, np.float64)
    I = np.eye(dk)
    out = np.empty((T, dv))
    for t in range(T):
        kt = k[t][:, None]
        S = S @ np.diag(alpha[t]) @ (I - beta[t] * (kt @ kt.T)) + beta[t] * (v[t][:, None] @ kt.T)
        out[t] = S @ q[t]
    return out, S


def kda_ut_form(q, k, v, alpha, beta, S0=None):
    """The per-channel-decay delta rule over the whole sequence as one
    unit-lower-triangular solve (derived here by unrolling, not printed on
    the pages).  With D_tjc = prod_{i=j+1}^t alpha_ic and A_c = prod_{i<=t}
    alpha_ic, pseudo-values u_t = beta_t (v_t - S_{t-1} diag(alpha_t) k_t)
    give S_t = S0 diag(A_t) + sum_{j<=t} u_j (k_j o D_tj)^T, hence
      (I + A) U = diag(beta) V - diag(beta) (K o A) S0^T,
      A_tj = beta_t sum_c k_tc k_jc D_tjc  (j < t),
      O = (Q o A) S0^T + P U,   P_tj = sum_c q_tc k_jc D_tjc  (j <= t).
    Returns (out (T, d_v), S_T (d_v, d_k)).
    """
    T, dk = k.shape
    dv = v.shape[1]
    S0 = np.zeros((dv, dk)) if S0 is None else np.asarray(S0, np.float64)
    D = gla_decay(alpha)                                # [t, j, c], 0 above the diagonal
    Acum = np.cumprod(alpha, axis=0)                    # prod_{i<=t} alpha_i
    KK = np.einsum("tc,tjc,jc->tj", k, D, k)
    A = np.tril(beta[:, None] * KK, -1)
    rhs = beta[:, None] * (v - (k * Acum) @ S0.T)
    U = np.linalg.solve(np.eye(T) + A, rhs)
    P = np.einsum("tc,tjc,jc->tj", q, D, k)
    out = (q * Acum) @ S0.T + P @ U
    if T == 0:
        return out, S0.copy()
    tail = D[T - 1]                                     # [j, c] = prod_{i=j+1}^{T} alpha_ic
    S_T = S0 * Acum[T - 1][None, :] + U.T @ (k * tail)
    return out, S_T
