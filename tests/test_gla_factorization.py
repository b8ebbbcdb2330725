"""Float32 emulation of how the gated chunk kernels form one 16-token diagonal
score tile, against its float64 definition (CPU only).

Gated linear attention weighs key j for query t >= j by the product of one
channel's gates strictly after j up to t (page "Ch. 11 Linear attention and
Hyena", 11.3 and the solution to Exercise 11.5; gates anywhere in (0, 1]).
The fast form of the kernels factors that weight through the block start,
Qhat_t = phi(q_t) R_t and kd_j = phi(k_j) / R_j with R the running product of
the gates from the block start; it is only used while every channel's
product over the block stays at or above 2^-64.  Below that the kernels form
the tile from running products of the gates alone (never above 1) and the
off-diagonal key operand from suffix products.  These tests show, in float32
as the kernels compute it, where the fast form leaves the float32 range and
that the exact forms do not.
"""
import numpy as np
import pytest

F = np.float32
WEAK = F(2.0 ** -64)   # the kernels' threshold for a block product


def definition(q, k, g):
    """float64 P_tj = sum_c q_tc k_jc prod_{j < i <= t} g_ic for j <= t."""
    n = q.shape[0]
    P = np.zeros((n, n))
    for t in range(n):
        for j in range(t + 1):
            w = np.prod(g[j + 1:t + 1].astype(np.float64), axis=0)
            P[t, j] = np.sum(q[t].astype(np.float64) * k[j].astype(np.float64) * w)
    return P


def fast_form(q, k, g):
    """Block-start reference in float32: R_t = prod_{i <= t} g_i (within the block)."""
    with np.errstate(over="ignore", divide="ignore", invalid="ignore", under="ignore"):
        R = np.cumprod(g, axis=0, dtype=F)
        Qh = (q * R).astype(F)
        kd = (k / R).astype(F)
        return np.tril(Qh @ kd.T)


def exact_form(q, k, g):
    """The exact tile: for key j, kd_c runs phi(k_jc) * g_(j+1)c * ... in
    float32, one token at a time, and never exceeds phi(k_jc)."""
    n, d = q.shape
    P = np.zeros((n, n), F)
    for j in range(n):
        kd = k[j].astype(F).copy()
        for t in range(j, n):
            if t > j:
                kd = (kd * g[t]).astype(F)
            P[t, j] = np.dot(q[t].astype(F), kd)
    return P


def suffix_key_operand(k, g):
    """k~_j = phi(k_j) prod_{j < i <= 15} g_i from suffix products (float32)."""
    n = k.shape[0]
    suf = np.ones_like(g, dtype=F)
    for j in range(n - 2, -1, -1):
        suf[j] = (suf[j + 1] * g[j + 1]).astype(F)
    return (k * suf).astype(F)


def _inputs(seed, gate):
    r = np.random.default_rng(seed)
    q = np.exp(r.standard_normal((16, 8))).astype(F)     # positive features, as phi gives
    k = np.exp(r.standard_normal((16, 8))).astype(F)
    g = np.full((16, 8), gate, F) if np.isscalar(gate) else gate.astype(F)
    return q, k, g


def _rel(a, b):
    return float(np.max(np.abs(a - b)) / np.max(np.abs(b)))


def test_fast_form_holds_for_mild_gates():
    q, k, g = _inputs(1, 0.6)          # block product 0.6^16 ~ 3e-4
    assert np.prod(g[:, 0].astype(np.float64)) >= WEAK
    assert _rel(fast_form(q, k, g), definition(q, k, g)) < 1e-6


@pytest.mark.parametrize("gate", [0.05, 0.005, 0.001])
def test_fast_form_breaks_past_the_threshold(gate):
    """0.05^16 ~ 1.5e-21, 0.005^16 ~ 1.5e-37 and 0.001^16 = 1e-48 are below
    2^-64: the kernels flag the chunk.  The last is below float32's range: the
    running product underflows, 1/R overflows and the fast form gives inf or
    NaN (0.005 is a hair inside the range); the exact form matches in all three."""
    q, k, g = _inputs(2, gate)
    assert np.prod(g[:, 0].astype(np.float64)) < WEAK
    ref = definition(q, k, g)
    if gate == 0.001:
        assert not np.all(np.isfinite(fast_form(q, k, g)))
    ex = exact_form(q, k, g)
    assert np.all(np.isfinite(ex))
    assert _rel(ex, ref) < 1e-6


def test_one_strong_channel_is_exact():
    """Mild gates everywhere but one channel at 1e-3 (the mixed GPU case)."""
    r = np.random.default_rng(3)
    g = (1.0 / (1.0 + np.exp(-r.normal(3.0, 1.0, (16, 8))))).astype(F)
    g[:, 5] = 1e-3
    q, k, _ = _inputs(3, 0.5)
    assert _rel(exact_form(q, k, g), definition(q, k, g)) < 1e-6


@pytest.mark.parametrize("gate", [0.9, 0.005, 0.001])
def test_suffix_key_operand(gate):
    """The off-diagonal key operand: the fast form kd_j * (block total) is
    0 * inf = NaN once 1/R_j overflows; suffix products stay exact."""
    q, k, g = _inputs(4, gate)
    want = np.stack([k[j].astype(np.float64) * np.prod(g[j + 1:].astype(np.float64), axis=0) for j in range(16)])
    got = suffix_key_operand(k, g)
    assert np.all(np.isfinite(got))
    nz = want > 1e-30
    assert np.max(np.abs(got[nz] - want[nz]) / want[nz]) < 1e-5
    with np.errstate(over="ignore", divide="ignore", invalid="ignore", under="ignore"):
        R = np.cumprod(g, axis=0, dtype=F)
        fast = (k / R * R[-1]).astype(F)
    if gate == 0.001:
        assert not np.all(np.isfinite(fast))
