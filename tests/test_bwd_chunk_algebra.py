"""The chunked backward's algebra in float64, against the oracle's gradients
(CPU only).

The recurrence of normalized linear attention and of retention (page
"Beyond -- Linear attention and recurrent memory", sections "The big idea"
and "Fixed decay versus an input-dependent gate"; page "Ch. 11 Linear
attention and Hyena", 11.3) is linear in its state, so its gradient splits
by chunk exactly as its forward does.  With the value rows augmented by a
constant 1 (the normalizer is then the last state column), per chunk of n
tokens entering with state S'_c and leaving with cotangent dS'_{c+1}, and
D_tj = gamma^(t-j) for j <= t:
  dO'  = [dO / den, -(dO . o) / den]                      (normalized)
  A    = D o (phiQ phiK^T),   G = D o (dO' V'^T)
  dphiQ = G phiK + diag(gamma^(t+1)) dO' S'_c^T
  dphiK = G^T phiQ + diag(gamma^(n-1-j)) V' dS'_{c+1}^T
  dV    = A^T dO'[:, :d_v] + diag(gamma^(n-1-j)) phiK dS_{c+1}^T
  dS'_c = gamma^n dS'_{c+1} + phiQ^T diag(gamma^(t+1)) dO'
and the decay's gradient, chunk by chunk with the entering state held fixed:
  d(ln gamma) = sum_t (t+1) a_t + sum_tj (t-j) A_tj H_tj
                + sum_j (n-1-j) e_j + n gamma^n <dS'_{c+1}, S'_c>
with H = dO' V'^T, a_t = gamma^(t+1) phi(q_t) . (S'_c dO'_t) and
e_j = gamma^(n-1-j) phi(k_j) . (dS'_{c+1} v'_j).  These tests run exactly
those steps (increments per chunk, forward and reverse scans over the
chunks, then every chunk on its own) and compare with the oracle's
token-by-token reverse pass.
"""
import numpy as np
import pytest

import oracle

NORMALIZED, RETENTION = oracle.NORMALIZED, oracle.RETENTION


def phi(x, kind):
    return np.where(x > 0, x + 1.0, np.exp(x)) if kind == oracle.PHI_ELU1 else x


def dphi(x, kind):
    return np.where(x > 0, 1.0, np.exp(x)) if kind == oracle.PHI_ELU1 else np.ones_like(x)


def chunked_backward(variant, phik, q, k, v, dout, gamma, S0, z0, dS_T, dz_T, C):
    """One head.  State in (d_k, d_v') orientation: column d_v is z."""
    T, dk = q.shape
    dv = v.shape[1]
    norm = variant == NORMALIZED
    Fq, Fk = phi(q, phik), phi(k, phik)
    Vp = np.concatenate([v, np.ones((T, 1))], 1) if norm else v
    S = np.concatenate([S0.T, z0[:, None]], 1) if norm else S0.T.copy()
    dST = np.concatenate([dS_T.T, dz_T[:, None]], 1) if norm else dS_T.T.copy()
    N = (T + C - 1) // C
    ch = [slice(c * C, min(T, (c + 1) * C)) for c in range(N)]
    # the forward's outputs and denominators (what the forward pass saves)
    out, den = np.zeros((T, dv)), np.ones(T)
    St = S.copy()
    for t in range(T):
        St = gamma * St + np.outer(Fk[t], Vp[t])
        r = Fq[t] @ St
        den[t] = r[dv] if norm else 1.0
        out[t] = r[:dv] / den[t]
    # cotangent of the augmented outputs
    dOp = dout / den[:, None]
    if norm:
        dden = -np.sum(dout * out, 1) / den
        dOp = np.concatenate([dOp, dden[:, None]], 1)
    # per-chunk increments, then the scans
    inc_f, inc_r = [], []
    for s in ch:
        n = s.stop - s.start
        w_k = gamma ** (n - 1 - np.arange(n))
        w_q = gamma ** (np.arange(n) + 1)
        inc_f.append((Fk[s] * w_k[:, None]).T @ Vp[s])
        inc_r.append((Fq[s] * w_q[:, None]).T @ dOp[s])
    ck_f, ck_r = [None] * N, [None] * N
    for c in range(N):
        n = ch[c].stop - ch[c].start
        ck_f[c] = S
        S = gamma ** n * S + inc_f[c]
    d = dST
    for c in reversed(range(N)):
        n = ch[c].stop - ch[c].start
        ck_r[c] = d
        d = gamma ** n * d + inc_r[c]
    dS0 = d
    # every chunk on its own
    dq, dk_, dv_ = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    dl = 0.0
    for c, s in enumerate(ch):
        n = s.stop - s.start
        t = np.arange(n)
        D = np.where(t[:, None] >= t[None, :], gamma ** np.clip(t[:, None] - t[None, :], 0, None), 0.0)
        Q, K, V, dO = Fq[s], Fk[s], Vp[s], dOp[s]
        P = Q @ K.T
        Hm = dO @ V.T
        A, G = D * P, D * Hm
        wq = gamma ** (t + 1)
        wk = gamma ** (n - 1 - t)
        X = wq[:, None] * (dO @ ck_f[c].T)          # state part of dphi(q)
        Y = wk[:, None] * (V @ ck_r[c].T)           # state part of dphi(k)
        dFq = G @ K + X
        dFk = G.T @ Q + Y
        dv_[s] = A.T @ dO[:, :dv] + wk[:, None] * (K @ ck_r[c][:, :dv])
        dq[s] = dFq * dphi(q[s], phik)
        dk_[s] = dFk * dphi(k[s], phik)
        dl += np.sum((t + 1) * np.sum(Q * X, 1)) + np.sum((t[:, None] - t[None, :]) * A * Hm)
        dl += np.sum((n - 1 - t) * np.sum(K * Y, 1)) + n * gamma ** n * np.sum(ck_r[c] * ck_f[c])
    res = {"dq": dq, "dk": dk_, "dv": dv_, "dS0": dS0[:, :dv].T, "dlog": dl}
    if norm:
        res["dz0"] = dS0[:, dv]
    return res


CASES = [(NORMALIZED, oracle.PHI_ELU1, 0.9, 16), (NORMALIZED, oracle.PHI_ELU1, 1.0, 16),
         (NORMALIZED, oracle.PHI_ELU1, 0.3, 8), (RETENTION, oracle.PHI_IDENTITY, 0.8, 16),
         (RETENTION, oracle.PHI_ELU1, 0.97, 32)]


@pytest.mark.parametrize("T", [1, 16, 37, 80])
@pytest.mark.parametrize("variant,phik,gamma,C", CASES)
def test_chunked_backward_equals_oracle(variant, phik, gamma, C, T):
    r = np.random.default_rng(1000 + T)
    dk, dv = 6, 5
    q, k = r.standard_normal((T, dk)), r.standard_normal((T, dk))
    v, do = r.standard_normal((T, dv)), r.standard_normal((T, dv))
    S0, dS_T = r.standard_normal((dv, dk)) * 0.3, r.standard_normal((dv, dk))
    z0, dz_T = np.abs(r.standard_normal(dk)) + 1.0, r.standard_normal(dk)
    norm = variant == NORMALIZED
    got = chunked_backward(variant, phik, q, k, v, do, gamma, S0, z0, dS_T, dz_T, C)
    e = lambda a: a[None, None]  # noqa: E731
    ref = oracle.backward(variant, e(q), e(k), e(v), e(do), gate=np.array([gamma]), S0=e(S0),
                          z0=e(z0) if norm else None, dS_T=e(dS_T), dz_T=e(dz_T) if norm else None, phi_kind=phik)
    for name in ("dq", "dk", "dv", "dS0") + (("dz0",) if norm else ()):
        np.testing.assert_allclose(got[name], ref[name][0, 0], rtol=1e-9, atol=1e-10, err_msg=name)
    # d/dgamma = d/d(ln gamma) / gamma
    np.testing.assert_allclose(got["dlog"] / gamma, ref["dgate"][0], rtol=1e-9, atol=1e-10)
