"""Pins of the float64 oracle against facts the pages fix.

Each ``check_*`` function takes a loaded oracle library and raises
AssertionError when the oracle disagrees with a fact that does not come from
the oracle itself: a worked example printed on the pages, a closed form, an
invariant, or the explicit T x T masked-parallel form the pages state next to
each recurrence (``oracle/parallel_forms.py``).  ``test_oracle_pins.py`` runs
them on the real oracle; ``test_oracle_mutants.py`` runs them on deliberately
broken copies of ``oracle.c`` and requires every copy to fail at least one.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

from oracle import GATED, GATED_DELTA, NORMALIZED, PHI_ELU1, PHI_IDENTITY
from oracle import parallel_forms as pf

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
TOL = 1e-12   # float64 identity pins: the pages' companion threshold


def _rng(seed):
    return np.random.default_rng(seed)


def _maxdiff(a, b):
    return float(np.max(np.abs(np.asarray(a) - np.asarray(b))))


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


# ---------------------------------------------------------------- feature map

def check_phi_closed_form(orc):
    """phi(x) = elu(x) + 1: x + 1 above zero, exp(x) at or below zero."""
    for x in (-3.0, -1.0, -0.25, -1e-9, 0.0, 1e-9, 0.5, 2.0, 7.5):
        want = x + 1.0 if x > 0 else math.exp(x)
        assert abs(orc.phi(x, PHI_ELU1) - want) <= 1e-15 * max(1.0, abs(want)), x
        assert orc.phi(x, PHI_ELU1) > 0.0
        assert orc.phi(x, PHI_IDENTITY) == x
    assert orc.phi(0.0, PHI_ELU1) == 1.0


# ------------------------------------------------- normalized linear attention

def check_la_matches_masked_T64(orc):
    _la_vs_masked(orc, T=64, dk=16, dv=16, seed=101)


def check_la_matches_masked_T512(orc):
    _la_vs_masked(orc, T=512, dk=16, dv=16, seed=102)


def check_la_matches_masked_rect(orc):
    _la_vs_masked(orc, T=48, dk=12, dv=7, seed=103)


def _la_vs_masked(orc, T, dk, dv, seed):
    r = _rng(seed)
    q, k = r.standard_normal((1, 2, T, dk)), r.standard_normal((1, 2, T, dk))
    v = r.standard_normal((1, 2, T, dv))
    out, S_T, z_T = orc.forward(NORMALIZED, q, k, v)
    for h in range(2):
        ref = pf.la_masked(q[0, h], k[0, h], v[0, h])
        assert _maxdiff(out[0, h], ref) <= TOL, _maxdiff(out[0, h], ref)
        Kf = pf.phi_elu1(k[0, h])
        # unrolled state: S_T = sum_j phi(k_j) v_j^T (stored d_v x d_k), z_T = sum_j phi(k_j)
        assert _maxdiff(S_T[0, h], v[0, h].T @ Kf) <= TOL * T
        assert _maxdiff(z_T[0, h], Kf.sum(axis=0)) <= TOL * T


def check_la_initial_state_matches_masked(orc):
    r = _rng(104)
    T, dk, dv = 40, 8, 6
    q, k = r.standard_normal((1, 1, T, dk)), r.standard_normal((1, 1, T, dk))
    v = r.standard_normal((1, 1, T, dv))
    S0 = r.standard_normal((1, 1, dv, dk))
    z0 = np.abs(r.standard_normal((1, 1, dk))) + 1.0
    out, _, _ = orc.forward(NORMALIZED, q, k, v, S0=S0, z0=z0)
    ref = pf.la_masked(q[0, 0], k[0, 0], v[0, 0], S0=S0[0, 0].T, z0=z0[0, 0])
    assert _maxdiff(out[0, 0], ref) <= TOL


def check_la_single_token_returns_value(orc):
    """T = 1 from a zero state: out_1 = (phi(q).phi(k)) v / (phi(q).phi(k)) = v."""
    r = _rng(105)
    q, k, v = (r.standard_normal((2, 3, 1, 16)) for _ in range(3))
    out, _, _ = orc.forward(NORMALIZED, q, k, v)
    # the two sums round in different orders: a few ulps per term
    assert np.max(np.abs(out - v) / np.maximum(np.abs(v), 1e-300)) <= 1e-14


def check_la_equal_keys_give_running_mean(orc):
    """With every key equal the scores are equal, so out_t is the mean of v_1..v_t."""
    r = _rng(106)
    T, d = 33, 8
    q = r.standard_normal((1, 1, T, d))
    k = np.broadcast_to(r.standard_normal(d), (1, 1, T, d)).copy()
    v = r.standard_normal((1, 1, T, d))
    out, _, _ = orc.forward(NORMALIZED, q, k, v)
    mean = np.cumsum(v[0, 0], axis=0) / np.arange(1, T + 1)[:, None]
    assert _maxdiff(out[0, 0], mean) <= TOL


# ------------------------------------------------------ gated linear attention

def check_gla_matches_masked(orc):
    for T, dk, dv, seed in ((64, 16, 16, 201), (96, 10, 6, 202)):
        r = _rng(seed)
        q, k = r.standard_normal((1, 2, T, dk)), r.standard_normal((1, 2, T, dk))
        v = r.standard_normal((1, 2, T, dv))
        gam = _sigmoid(r.normal(2.0, 1.0, (1, 2, T, dk)))
        S0 = r.standard_normal((1, 2, dv, dk))
        for with_state in (False, True):
            out, S_T, _ = orc.forward(GATED, q, k, v, gate=gam, S0=S0 if with_state else None)
            for h in range(2):
                ref = pf.gla_masked(q[0, h], k[0, h], v[0, h], gam[0, h],
                                    S0=S0[0, h].T if with_state else None)
                assert _maxdiff(out[0, h], ref) <= TOL * 10, _maxdiff(out[0, h], ref)


def check_gla_unit_gate_is_unnormalized_la(orc):
    """gamma = 1: the gated form loses its decay and is (L o (Q_phi K_phi^T)) V."""
    r = _rng(203)
    T, d = 50, 8
    q, k, v = (r.standard_normal((1, 1, T, d)) for _ in range(3))
    out, _, _ = orc.forward(GATED, q, k, v, gate=np.ones((1, 1, T, d)))
    ref = pf.causal_mask(T) * (pf.phi_elu1(q[0, 0]) @ pf.phi_elu1(k[0, 0]).T) @ v[0, 0]
    assert _maxdiff(out[0, 0], ref) <= TOL * 10


def check_gla_constant_gate_is_toeplitz(orc):
    """A constant gate gives the Toeplitz mask gamma^(t-j)."""
    r = _rng(204)
    T, d, g = 64, 8, 0.93
    q, k, v = (r.standard_normal((1, 1, T, d)) for _ in range(3))
    out, _, _ = orc.forward(GATED, q, k, v, gate=np.full((1, 1, T, d), g))
    ref = pf.retnet_masked(q[0, 0], k[0, 0], v[0, 0], g)
    assert _maxdiff(out[0, 0], ref) <= TOL * 10


def check_gla_identity_phi_is_plain_regrouping(orc):
    """phi = identity, gamma = 1: sum_{j<=t} (q_t.k_j) v_j, the regrouped sum."""
    r = _rng(205)
    T, dk, dv = 50, 32, 5
    q, k = r.standard_normal((1, 1, T, dk)), r.standard_normal((1, 1, T, dk))
    v = r.standard_normal((1, 1, T, dv))
    out, S_T, _ = orc.forward(GATED, q, k, v, gate=np.ones((1, 1, T, dk)), phi_kind=PHI_IDENTITY)
    for t in (0, 7, T - 1):
        ref = sum((q[0, 0, t] @ k[0, 0, j]) * v[0, 0, j] for j in range(t + 1))
        assert _maxdiff(out[0, 0, t], ref) <= TOL * 10
    assert _maxdiff(S_T[0, 0], v[0, 0].T @ k[0, 0]) <= TOL * 10


# --------------------------------------------------------- gated delta rule

def check_gdr_two_key_example(orc):
    with open(os.path.join(GOLDEN, "delta_rule_two_keys.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        keys = np.array(c["keys"], np.float64)
        vals = np.array(c["values"], np.float64)
        T = len(vals)
        q = np.zeros((1, 1, T, 2))
        _, S_T, _ = orc.forward(GATED_DELTA, q, keys[None, None], vals[None, None, :, None],
                                gate=np.ones((1, 1, T)), beta=np.full((1, 1, T), c["beta"]))
        assert S_T[0, 0, 0].tolist() == c["expected_state"], (c["name"], S_T[0, 0, 0])


def check_gdr_repeated_key_overwrites(orc):
    """A repeated unit key written with beta = 1 recalls only the last value."""
    r = _rng(301)
    dk, dv = 16, 8
    key = _unit(r.standard_normal(dk))
    k = np.stack([key, key])[None, None]
    v = r.standard_normal((1, 1, 2, dv))
    S0 = r.standard_normal((1, 1, dv, dk))
    _, S_T, _ = orc.forward(GATED_DELTA, np.zeros((1, 1, 2, dk)), k, v,
                            gate=np.array([[[0.9, 0.7]]]), beta=np.ones((1, 1, 2)), S0=S0)
    assert _maxdiff(S_T[0, 0] @ key, v[0, 0, 1]) <= TOL


def check_gdr_unit_beta_recalls_value(orc):
    """beta = 1, unit keys: after each write S_t k_t = v_t, for any gate and history."""
    r = _rng(302)
    T, dk, dv = 24, 16, 12
    k = _unit(r.standard_normal((1, 2, T, dk)))
    v = r.standard_normal((1, 2, T, dv))
    q = r.standard_normal((1, 2, T, dk))
    g = r.uniform(0.3, 1.0, (1, 2, T))
    S = np.ascontiguousarray(r.standard_normal((1, 2, dv, dk)))
    for t in range(T):
        orc.decode_step(GATED_DELTA, S, q[:, :, t], k[:, :, t], v[:, :, t],
                        gate=g[:, :, t], beta=np.ones((1, 2)))
        recall = np.einsum("bhvk,bhk->bhv", S, k[:, :, t])
        assert _maxdiff(recall, v[:, :, t]) <= TOL


def check_gdr_zero_beta_is_pure_decay(orc):
    """beta = 0: S_t = g_t S_{t-1}, o_t = S_t q_t."""
    r = _rng(303)
    T, dk, dv = 20, 8, 8
    q, k = r.standard_normal((1, 1, T, dk)), _unit(r.standard_normal((1, 1, T, dk)))
    v = r.standard_normal((1, 1, T, dv))
    g = r.uniform(0.5, 1.0, (1, 1, T))
    S0 = r.standard_normal((1, 1, dv, dk))
    out, S_T, _ = orc.forward(GATED_DELTA, q, k, v, gate=g, beta=np.zeros((1, 1, T)), S0=S0)
    gc = np.cumprod(g[0, 0])
    assert _maxdiff(S_T[0, 0], gc[-1] * S0[0, 0]) <= TOL
    assert _maxdiff(out[0, 0], gc[:, None] * (q[0, 0] @ S0[0, 0].T)) <= TOL


def check_gdr_unit_gate_is_gradient_step(orc):
    """g = 1: S_t = S_{t-1} - beta (S_{t-1} k - v) k^T (one gradient step)."""
    r = _rng(304)
    dk, dv = 12, 9
    S0 = r.standard_normal((dv, dk))
    k = _unit(r.standard_normal(dk))
    v, q = r.standard_normal(dv), r.standard_normal(dk)
    b = 0.37
    _, S_T, _ = orc.forward(GATED_DELTA, q[None, None, None], k[None, None, None],
                            v[None, None, None], gate=np.ones((1, 1, 1)),
                            beta=np.full((1, 1, 1), b), S0=S0[None, None])
    want = S0 - b * np.outer(S0 @ k - v, k)
    assert _maxdiff(S_T[0, 0], want) <= TOL


def check_gdr_matches_product_form(orc):
    for T, dk, dv, seed in ((64, 16, 16, 305), (40, 12, 5, 306)):
        r = _rng(seed)
        q = r.standard_normal((1, 2, T, dk))
        k = _unit(r.standard_normal((1, 2, T, dk)))
        v = r.standard_normal((1, 2, T, dv))
        g = _sigmoid(r.normal(2.0, 1.0, (1, 2, T)))
        b = _sigmoid(r.normal(0.0, 1.0, (1, 2, T)))
        S0 = r.standard_normal((1, 2, dv, dk))
        out, S_T, _ = orc.forward(GATED_DELTA, q, k, v, gate=g, beta=b, S0=S0)
        for h in range(2):
            ro, rS = pf.gdr_product_form(q[0, h], k[0, h], v[0, h], g[0, h], b[0, h], S0[0, h])
            assert _maxdiff(out[0, h], ro) <= TOL
            assert _maxdiff(S_T[0, h], rS) <= TOL


def check_gdr_matches_ut_form(orc):
    r = _rng(307)
    T, dk, dv = 200, 16, 16
    q = r.standard_normal((1, 1, T, dk))
    k = _unit(r.standard_normal((1, 1, T, dk)))
    v = r.standard_normal((1, 1, T, dv))
    g = _sigmoid(r.normal(4.0, 1.0, (1, 1, T)))
    b = _sigmoid(r.normal(0.0, 1.0, (1, 1, T)))
    S0 = r.standard_normal((1, 1, dv, dk))
    out, S_T, _ = orc.forward(GATED_DELTA, q, k, v, gate=g, beta=b, S0=S0)
    ro, rS = pf.gdr_ut_form(q[0, 0], k[0, 0], v[0, 0], g[0, 0], b[0, 0], S0[0, 0])
    assert _maxdiff(out[0, 0], ro) <= TOL
    assert _maxdiff(S_T[0, 0], rS) <= TOL


# ------------------------------------------------ state, decode, split calls

def check_state_accounting(orc):
    """State size H d_h^2 + H d_h, independent of T."""
    with open(os.path.join(GOLDEN, "state_accounting.json")) as f:
        cases = json.load(f)["cases"]
    c0, c1 = cases
    H, d = c0["H"], c0["d_h"]
    r = _rng(401)
    for T in (1, 3, 8):
        q, k, v = (r.standard_normal((1, H, T, d)) * 0.1 for _ in range(3))
        _, S_T, z_T = orc.forward(NORMALIZED, q, k, v, nthreads=1)
        n = S_T.size + z_T.size
        assert n == c0["state_values"] == c0["D"] ** 2 // H + c0["D"]
        assert round(n * 2 / 1e6, 1) == c0["fp16_megabytes_approx"]
        g = np.ones((1, 1, T))
        _, S_T, z_T = orc.forward(GATED_DELTA, q[:, :1], _unit(k[:, :1]), v[:, :1], gate=g, beta=g)
        assert z_T is None and S_T.size == c1["state_values_without_normalizer"]


def _variant_inputs(r, variant, T, dk, dv, B=1, H=2):
    q, k = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk))
    v = r.standard_normal((B, H, T, dv))
    gate = beta = None
    if variant == GATED:
        gate = _sigmoid(r.normal(2.0, 1.0, (B, H, T, dk)))
    elif variant == GATED_DELTA:
        k = _unit(k)
        gate = _sigmoid(r.normal(3.0, 1.0, (B, H, T)))
        beta = _sigmoid(r.normal(0.0, 1.0, (B, H, T)))
    return q, k, v, gate, beta


def check_decode_chain_equals_forward(orc):
    for variant in (NORMALIZED, GATED, GATED_DELTA):
        r = _rng(500 + variant)
        T, dk, dv = 17, 8, 6
        q, k, v, gate, beta = _variant_inputs(r, variant, T, dk, dv)
        S0 = r.standard_normal((1, 2, dv, dk))
        z0 = np.abs(r.standard_normal((1, 2, dk))) + 1.0 if variant == NORMALIZED else None
        out, S_T, z_T = orc.forward(variant, q, k, v, gate=gate, beta=beta, S0=S0, z0=z0)
        S = np.ascontiguousarray(S0.copy())
        z = np.ascontiguousarray(z0.copy()) if z0 is not None else None
        for t in range(T):
            o = orc.decode_step(variant, S, q[:, :, t], k[:, :, t], v[:, :, t],
                                gate=None if gate is None else gate[:, :, t],
                                beta=None if beta is None else beta[:, :, t], z=z)
            assert _maxdiff(o, out[:, :, t]) <= TOL
        assert _maxdiff(S, S_T) <= TOL
        if z is not None:
            assert _maxdiff(z, z_T) <= TOL


def check_split_call_equals_single_call(orc):
    for variant in (NORMALIZED, GATED, GATED_DELTA):
        r = _rng(600 + variant)
        T, T1, dk, dv = 45, 19, 8, 8
        q, k, v, gate, beta = _variant_inputs(r, variant, T, dk, dv)
        sl = lambda a, s: None if a is None else a[:, :, s]  # noqa: E731
        out, S_T, z_T = orc.forward(variant, q, k, v, gate=gate, beta=beta)
        a = slice(0, T1)
        b = slice(T1, T)
        o1, S1, z1 = orc.forward(variant, q[:, :, a], k[:, :, a], v[:, :, a], sl(gate, a), sl(beta, a))
        o2, S2, z2 = orc.forward(variant, q[:, :, b], k[:, :, b], v[:, :, b], sl(gate, b), sl(beta, b),
                                 S0=S1, z0=z1)
        assert _maxdiff(np.concatenate([o1, o2], axis=2), out) <= TOL
        assert _maxdiff(S2, S_T) <= TOL


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_") and callable(v)]
