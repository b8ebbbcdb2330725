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

from oracle import GATED, GATED_DELTA, KDA, NORMALIZED, PHI_ELU1, PHI_IDENTITY, RETENTION
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


# ------------------------------------- fixed per-head decay (normalized, retention)

def check_la_decay_matches_masked(orc):
    """S and z both decay by gamma_h: the decayed T x T form, per head, at T=64
    and T=512, with and without an initial state (B = 2 shares the decays)."""
    for T, dk, dv, seed in ((64, 16, 16, 701), (512, 16, 8, 702)):
        r = _rng(seed)
        B, H = 2, 2
        q, k = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk))
        v = r.standard_normal((B, H, T, dv))
        gam = np.array([0.97, 0.8])
        S0 = r.standard_normal((B, H, dv, dk))
        z0 = np.abs(r.standard_normal((B, H, dk))) + 1.0
        for with_state in (False, True):
            out, S_T, z_T = orc.forward(NORMALIZED, q, k, v, gate=gam, S0=S0 if with_state else None,
                                        z0=z0 if with_state else None)
            for b in range(B):
                for h in range(H):
                    ref = pf.la_decayed_masked(q[b, h], k[b, h], v[b, h], gam[h],
                                               S0=S0[b, h].T if with_state else None,
                                               z0=z0[b, h] if with_state else None)
                    assert _maxdiff(out[b, h], ref) <= TOL, _maxdiff(out[b, h], ref)
                    if not with_state:
                        # unrolled: S_T = sum_j gamma^(T-1-j) v_j phi(k_j)^T, z_T likewise
                        w = gam[h] ** np.arange(T - 1, -1, -1)
                        Kf = pf.phi_elu1(k[b, h])
                        assert _maxdiff(S_T[b, h], (v[b, h] * w[:, None]).T @ Kf) <= TOL * 10
                        assert _maxdiff(z_T[b, h], w @ Kf) <= TOL * 10


def check_la_unit_decay_is_undecayed(orc):
    """gamma_h = 1 reproduces the undecayed normalized variant exactly."""
    r = _rng(703)
    q, k, v = (r.standard_normal((2, 3, 30, 8)) for _ in range(3))
    a = orc.forward(NORMALIZED, q, k, v)
    b = orc.forward(NORMALIZED, q, k, v, gate=np.ones(3))
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def check_la_decay_equal_keys_give_weighted_mean(orc):
    """Equal keys: out_t = sum_i gamma^(t-i) v_i / sum_i gamma^(t-i)."""
    r = _rng(704)
    T, d, g = 40, 8, 0.85
    q = r.standard_normal((1, 1, T, d))
    k = np.broadcast_to(r.standard_normal(d), (1, 1, T, d)).copy()
    v = r.standard_normal((1, 1, T, d))
    out, _, _ = orc.forward(NORMALIZED, q, k, v, gate=np.array([g]))
    for t in (0, 1, 17, T - 1):
        w = g ** np.arange(t, -1, -1)
        assert _maxdiff(out[0, 0, t], (w @ v[0, 0, :t + 1]) / w.sum()) <= TOL


def check_retention_matches_toeplitz(orc):
    for phi_kind, phi in ((PHI_IDENTITY, None), (PHI_ELU1, pf.phi_elu1)):
        r = _rng(705 + phi_kind)
        B, H, T, dk, dv = 2, 2, 64, 12, 7
        q, k = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk))
        v = r.standard_normal((B, H, T, dv))
        gam = np.array([0.9, 0.6])
        S0 = r.standard_normal((B, H, dv, dk))
        out, _, _ = orc.forward(RETENTION, q, k, v, gate=gam, S0=S0, phi_kind=phi_kind)
        for b in range(B):
            for h in range(H):
                ref = pf.retention_masked(q[b, h], k[b, h], v[b, h], gam[h], S0=S0[b, h].T, phi=phi)
                assert _maxdiff(out[b, h], ref) <= TOL * 10, _maxdiff(out[b, h], ref)


def check_retention_is_gla_with_constant_gate(orc):
    """A per-head constant gamma is gated linear attention with that gate everywhere."""
    r = _rng(707)
    B, H, T, dk, dv = 1, 3, 45, 8, 5
    q, k = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk))
    v = r.standard_normal((B, H, T, dv))
    gam = np.array([0.99, 0.5, 0.05])
    S0 = r.standard_normal((B, H, dv, dk))
    a, Sa, _ = orc.forward(RETENTION, q, k, v, gate=gam, S0=S0, phi_kind=PHI_ELU1)
    full = np.broadcast_to(gam[None, :, None, None], (B, H, T, dk)).copy()
    b, Sb, _ = orc.forward(GATED, q, k, v, gate=full, S0=S0, phi_kind=PHI_ELU1)
    assert _maxdiff(a, b) <= TOL and _maxdiff(Sa, Sb) <= TOL


def check_retention_geometric_sum(orc):
    """One key and one value written T times: S_T = v phi(k)^T (1 - g^T) / (1 - g)."""
    r = _rng(708)
    T, dk, dv, g = 25, 6, 4, 0.7
    key, val = r.standard_normal(dk), r.standard_normal(dv)
    k = np.broadcast_to(key, (1, 1, T, dk)).copy()
    v = np.broadcast_to(val, (1, 1, T, dv)).copy()
    _, S_T, _ = orc.forward(RETENTION, np.zeros((1, 1, T, dk)), k, v, gate=np.array([g]))
    assert _maxdiff(S_T[0, 0], np.outer(val, key) * (1 - g ** T) / (1 - g)) <= TOL


# ------------------------------------- delta rule with a per-channel decay (KDA)

def _kda_inputs(r, B, H, T, dk, dv, mean=2.0):
    q = r.standard_normal((B, H, T, dk))
    k = _unit(r.standard_normal((B, H, T, dk)))
    v = r.standard_normal((B, H, T, dv))
    a = _sigmoid(r.normal(mean, 1.0, (B, H, T, dk)))
    b = _sigmoid(r.normal(0.0, 1.0, (B, H, T)))
    return q, k, v, a, b


def check_kda_matches_product_form(orc):
    for T, dk, dv, seed in ((64, 16, 16, 801), (40, 12, 5, 802)):
        r = _rng(seed)
        q, k, v, a, b = _kda_inputs(r, 1, 2, T, dk, dv)
        S0 = r.standard_normal((1, 2, dv, dk))
        out, S_T, _ = orc.forward(KDA, q, k, v, gate=a, beta=b, S0=S0)
        for h in range(2):
            ro, rS = pf.kda_product_form(q[0, h], k[0, h], v[0, h], a[0, h], b[0, h], S0[0, h])
            assert _maxdiff(out[0, h], ro) <= TOL and _maxdiff(S_T[0, h], rS) <= TOL


def check_kda_matches_ut_form(orc):
    r = _rng(803)
    T, dk, dv = 150, 16, 12
    q, k, v, a, b = _kda_inputs(r, 1, 1, T, dk, dv, mean=4.0)
    S0 = r.standard_normal((1, 1, dv, dk))
    out, S_T, _ = orc.forward(KDA, q, k, v, gate=a, beta=b, S0=S0)
    ro, rS = pf.kda_ut_form(q[0, 0], k[0, 0], v[0, 0], a[0, 0], b[0, 0], S0[0, 0])
    assert _maxdiff(out[0, 0], ro) <= TOL and _maxdiff(S_T[0, 0], rS) <= TOL


def check_kda_shared_channel_gate_is_gdr(orc):
    """alpha_t = g_t in every channel: the scalar-gate delta rule."""
    r = _rng(804)
    q, k, v, _, b = _kda_inputs(r, 2, 2, 33, 8, 6)
    g = _sigmoid(r.normal(2.0, 1.0, (2, 2, 33)))
    S0 = r.standard_normal((2, 2, 6, 8))
    a = np.broadcast_to(g[..., None], (2, 2, 33, 8)).copy()
    x = orc.forward(KDA, q, k, v, gate=a, beta=b, S0=S0)
    y = orc.forward(GATED_DELTA, q, k, v, gate=g, beta=b, S0=S0)
    assert _maxdiff(x[0], y[0]) <= TOL and _maxdiff(x[1], y[1]) <= TOL


def check_kda_unit_beta_recalls_value(orc):
    """beta = 1, unit keys: S_t k_t = v_t after every write, whatever the decays."""
    r = _rng(805)
    T, dk, dv = 20, 16, 8
    q, k, v, a, _ = _kda_inputs(r, 1, 2, T, dk, dv, mean=0.0)
    S = np.ascontiguousarray(r.standard_normal((1, 2, dv, dk)))
    for t in range(T):
        orc.decode_step(KDA, S, q[:, :, t], k[:, :, t], v[:, :, t], gate=a[:, :, t], beta=np.ones((1, 2)))
        assert _maxdiff(np.einsum("bhvk,bhk->bhv", S, k[:, :, t]), v[:, :, t]) <= TOL


def check_kda_zero_beta_is_channel_decay(orc):
    """beta = 0: S_T = S0 diag(prod_t alpha_t), o_t = S0 (prod_{i<=t} alpha_i o q_t)."""
    r = _rng(806)
    T, dk, dv = 18, 8, 5
    q, k, v, a, _ = _kda_inputs(r, 1, 1, T, dk, dv)
    S0 = r.standard_normal((1, 1, dv, dk))
    out, S_T, _ = orc.forward(KDA, q, k, v, gate=a, beta=np.zeros((1, 1, T)), S0=S0)
    A = np.cumprod(a[0, 0], axis=0)
    assert _maxdiff(S_T[0, 0], S0[0, 0] * A[-1][None, :]) <= TOL
    assert _maxdiff(out[0, 0], (q[0, 0] * A) @ S0[0, 0].T) <= TOL


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


def _variant_inputs(r, variant, T, dk, dv, B=1, H=2, decay=False):
    q, k = r.standard_normal((B, H, T, dk)), r.standard_normal((B, H, T, dk))
    v = r.standard_normal((B, H, T, dv))
    gate = beta = None
    if variant == GATED:
        gate = _sigmoid(r.normal(2.0, 1.0, (B, H, T, dk)))
    elif variant == GATED_DELTA:
        k = _unit(k)
        gate = _sigmoid(r.normal(3.0, 1.0, (B, H, T)))
        beta = _sigmoid(r.normal(0.0, 1.0, (B, H, T)))
    elif variant == KDA:
        k = _unit(k)
        gate = _sigmoid(r.normal(3.0, 1.0, (B, H, T, dk)))
        beta = _sigmoid(r.normal(0.0, 1.0, (B, H, T)))
    elif variant == RETENTION or decay:
        gate = _sigmoid(r.normal(2.0, 1.0, H))
    return q, k, v, gate, beta


# (variant, per-head decay) cases of the decode and split-call invariants
_INVARIANT_CASES = ((NORMALIZED, False), (NORMALIZED, True), (GATED, False), (GATED_DELTA, False),
                    (RETENTION, True), (KDA, False))


def check_decode_chain_equals_forward(orc):
    for variant, decay in _INVARIANT_CASES:
        r = _rng(500 + variant + 10 * decay)
        T, dk, dv = 17, 8, 6
        q, k, v, gate, beta = _variant_inputs(r, variant, T, dk, dv, B=2, decay=decay)
        per_head = variant in (NORMALIZED, RETENTION)
        S0 = r.standard_normal((2, 2, dv, dk))
        z0 = np.abs(r.standard_normal((2, 2, dk))) + 1.0 if variant == NORMALIZED else None
        out, S_T, z_T = orc.forward(variant, q, k, v, gate=gate, beta=beta, S0=S0, z0=z0)
        S = np.ascontiguousarray(S0.copy())
        z = np.ascontiguousarray(z0.copy()) if z0 is not None else None
        for t in range(T):
            g = gate if (gate is None or per_head) else gate[:, :, t]
            o = orc.decode_step(variant, S, q[:, :, t], k[:, :, t], v[:, :, t], gate=g,
                                beta=None if beta is None else beta[:, :, t], z=z)
            assert _maxdiff(o, out[:, :, t]) <= TOL
        assert _maxdiff(S, S_T) <= TOL
        if z is not None:
            assert _maxdiff(z, z_T) <= TOL


def check_split_call_equals_single_call(orc):
    for variant, decay in _INVARIANT_CASES:
        r = _rng(600 + variant + 10 * decay)
        T, T1, dk, dv = 45, 19, 8, 8
        q, k, v, gate, beta = _variant_inputs(r, variant, T, dk, dv, decay=decay)
        per_head = variant in (NORMALIZED, RETENTION)
        sl = lambda a, s: None if a is None else (a if per_head and a is gate else a[:, :, s])  # noqa: E731
        out, S_T, z_T = orc.forward(variant, q, k, v, gate=gate, beta=beta)
        a = slice(0, T1)
        b = slice(T1, T)
        o1, S1, z1 = orc.forward(variant, q[:, :, a], k[:, :, a], v[:, :, a], sl(gate, a), sl(beta, a))
        o2, S2, z2 = orc.forward(variant, q[:, :, b], k[:, :, b], v[:, :, b], sl(gate, b), sl(beta, b),
                                 S0=S1, z0=z1)
        assert _maxdiff(np.concatenate([o1, o2], axis=2), out) <= TOL
        assert _maxdiff(S2, S_T) <= TOL




# ------------------------------------------------ gradients (training, backward)

def _loss_fd(orc, variant, phi_kind, inp, cot, name, idx, h):
    """Central difference of L = <dout, out> + <dS_T, S_T> + <dz_T, z_T> in one
    input element (the forward pass is the pinned recurrence)."""
    def loss(x):
        a = dict(inp)
        a[name] = x
        out, S_T, z_T = orc.forward(variant, a["q"], a["k"], a["v"], gate=a.get("gate"), S0=a.get("S0"),
                                    z0=a.get("z0"), phi_kind=phi_kind)
        s = float(np.sum(cot["dout"] * out) + np.sum(cot["dS_T"] * S_T))
        if z_T is not None:
            s += float(np.sum(cot["dz_T"] * z_T))
        return s
    xp, xm = inp[name].copy(), inp[name].copy()
    xp[idx] += h
    xm[idx] -= h
    return (loss(xp) - loss(xm)) / (2 * h)


def _bwd_case(r, variant, B, H, T, dk, dv, decay):
    inp = {"q": r.standard_normal((B, H, T, dk)), "k": r.standard_normal((B, H, T, dk)),
           "v": r.standard_normal((B, H, T, dv)), "S0": r.standard_normal((B, H, dv, dk)) * 0.5}
    if variant == NORMALIZED:
        inp["z0"] = np.abs(r.standard_normal((B, H, dk))) + 1.0
    if decay:
        inp["gate"] = r.uniform(0.5, 0.99, H)
    cot = {"dout": r.standard_normal((B, H, T, dv)), "dS_T": r.standard_normal((B, H, dv, dk)),
           "dz_T": r.standard_normal((B, H, dk))}
    return inp, cot


def _check_grads_by_fd(orc, variant, phi_kind, decay, seed):
    r = _rng(seed)
    inp, cot = _bwd_case(r, variant, 2, 2, 7, 3, 2, decay)
    g = orc.backward(variant, inp["q"], inp["k"], inp["v"], cot["dout"], gate=inp.get("gate"), S0=inp["S0"],
                     z0=inp.get("z0"), dS_T=cot["dS_T"], dz_T=cot["dz_T"] if variant == NORMALIZED else None,
                     phi_kind=phi_kind)
    names = {"q": "dq", "k": "dk", "v": "dv", "S0": "dS0", "z0": "dz0", "gate": "dgate"}
    for name, gname in names.items():
        if name not in inp:
            continue
        x = inp[name]
        for idx in np.ndindex(x.shape):
            fd = _loss_fd(orc, variant, phi_kind, inp, cot, name, idx, 1e-6)
            assert abs(g[gname][idx] - fd) <= 1e-6 * max(1.0, abs(fd)), (name, idx, g[gname][idx], fd)


def check_grad_la_by_finite_differences(orc):
    _check_grads_by_fd(orc, NORMALIZED, PHI_ELU1, False, 901)


def check_grad_la_decay_by_finite_differences(orc):
    _check_grads_by_fd(orc, NORMALIZED, PHI_ELU1, True, 902)


def check_grad_retention_by_finite_differences(orc):
    _check_grads_by_fd(orc, RETENTION, PHI_IDENTITY, True, 903)
    _check_grads_by_fd(orc, RETENTION, PHI_ELU1, True, 904)


def check_grad_retention_matches_masked_form(orc):
    """Retention, phi = identity: out = (D o Q K^T) V with D_tj = gamma^(t-j)
    (j <= t), so dV = (D o Q K^T)^T dO, dQ = (D o dO V^T) K, dK = (D o dO V^T)^T Q
    exactly (zero initial state, no state cotangent)."""
    r = _rng(905)
    T, dk, dv, g = 40, 6, 5, 0.8
    q, k, v, do = (r.standard_normal((1, 1, T, d)) for d in (dk, dk, dv, dv))
    gr = orc.backward(RETENTION, q, k, v, do, gate=np.array([g]), phi_kind=PHI_IDENTITY)
    Q, K, V, dO = q[0, 0], k[0, 0], v[0, 0], do[0, 0]
    t = np.arange(T)
    D = np.where(t[:, None] >= t[None, :], g ** (t[:, None] - t[None, :]).clip(min=0), 0.0)
    A = D * (Q @ K.T)
    G = D * (dO @ V.T)
    assert _maxdiff(gr["dv"][0, 0], A.T @ dO) <= TOL * 10
    assert _maxdiff(gr["dq"][0, 0], G @ K) <= TOL * 10
    assert _maxdiff(gr["dk"][0, 0], G.T @ Q) <= TOL * 10
    # dgamma: d/dg of sum_{t>=j} g^(t-j) (q_t.k_j)(dO_t.v_j)
    E = (t[:, None] - t[None, :]).clip(min=0)
    dD = np.where((t[:, None] > t[None, :]), E * g ** (E - 1).clip(min=0), 0.0)
    assert abs(gr["dgate"][0] - np.sum(dD * (Q @ K.T) * (dO @ V.T))) <= TOL * 100


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_") and callable(v)]
