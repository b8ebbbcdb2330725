"""GPU parity of la_decode_step against the float64 oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_causal_amd as la
import oracle
import workloads as wl
from gpu_util import TOL, dev, host64, parity_error, record

pytestmark = pytest.mark.gpu

VARIANTS = [(la.LA_NORMALIZED, la.LA_PHI_ELU1), (la.LA_GATED, la.LA_PHI_ELU1),
            (la.LA_GATED, la.LA_PHI_IDENTITY), (la.LA_GATED_DELTA, la.LA_PHI_IDENTITY)]
DIMS = [(16, 16), (32, 64), (64, 32), (128, 128), (128, 16), (16, 128), (64, 64)]


def run_decode(w, steps, B, H, sample=None, state_dtype_check=True):
    """Run `steps` decode steps on the GPU and in the oracle; return worst errors."""
    S0 = wl.decode_state(w, B=B, H=H)
    S = dev(S0)
    z = dev(wl.decode_normalizer(w, B=B, H=H)) if w.variant == la.LA_NORMALIZED else None
    heads = np.arange(B * H) if sample is None else np.asarray(sample)
    S_ref = np.ascontiguousarray(S0.f64().reshape(B * H, w.d_v, w.d_k)[heads][None])
    z_ref = None
    if z is not None:
        z_ref = np.ascontiguousarray(host64(z).reshape(B * H, w.d_k)[heads][None])
    worst_o = 0.0
    for s in range(steps):
        inp = wl.decode_step_inputs(w, s, B=B, H=H)
        g = dev(inp.get("gate"))
        b = dev(inp.get("beta"))
        o = la.la_decode_step(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), S, variant=w.variant,
                              gate=g, beta=b, z=z, phi=w.phi_kind)
        sel = lambda a, d: None if a is None else a.f64().reshape((B * H,) + a.shape[2:])[heads][None]  # noqa: E731
        o_ref = oracle.decode_step(w.variant, S_ref, sel(inp["q"], 0), sel(inp["k"], 0),
                                   sel(inp["v"], 0), gate=sel(inp.get("gate"), 0),
                                   beta=sel(inp.get("beta"), 0), z=z_ref, phi_kind=w.phi_kind)
        o_gpu = host64(o).reshape((B * H, w.d_v))[heads][None]
        worst_o = max(worst_o, parity_error(o_gpu, o_ref))
    S_gpu = host64(S).reshape(B * H, w.d_v, w.d_k)[heads][None]
    err_S = parity_error(S_gpu, S_ref)
    err_z = 0.0
    if z is not None:
        err_z = parity_error(host64(z).reshape(B * H, w.d_k)[heads][None], z_ref)
    return worst_o, err_S, err_z


@pytest.mark.parametrize("dk,dv", DIMS, ids=lambda x: str(x))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("variant,phi", VARIANTS, ids=["la", "gla", "gla_id", "gdr"])
def test_decode_matches_oracle(variant, phi, dtype, dk, dv):
    w = wl.variant_workload(variant, dtype, dk, dv, S0_std=0.1, phi=phi, seed=17)
    print("decode parity", variant, phi, dtype, dk, dv, flush=True)
    eo, es, ez = run_decode(w, steps=6, B=2, H=5)
    record("decode-%d-%d-%s-dk%d-dv%d" % (variant, phi, dtype, dk, dv), {"o": eo, "S": es, "z": ez}, dtype)
    tol = TOL[dtype]
    assert eo <= tol and es <= tol and ez <= tol, (eo, es, ez)


def test_decode_gdr_full_shape_1000_steps():
    """The B=256, H=16, d=128 decode sequence: 1000 in-place steps on every head,
    compared at every step and on the final state over every 37th head (111
    heads, every residue modulo 8, so every XCD's share of the launch)."""
    w = wl.WORKLOADS["gdr_decode_b256h16d128"]
    sample = list(range(0, w.B * w.H, 37)) + [w.B * w.H - 1]
    print("decode full shape", w.name, "steps", w.T, flush=True)
    eo, es, _ = run_decode(w, steps=w.T, B=w.B, H=w.H, sample=sample)
    record("workload-" + w.name, {"o": eo, "S": es}, w.dtype)
    assert eo <= TOL[w.dtype] and es <= TOL[w.dtype], (eo, es)


def test_decode_gdr_unit_beta_recalls_value():
    """beta = 1 with unit keys: the new state maps k_t to v_t (page 'Module 18
    Beyond attention', section 18.2: the delta rule erases what the state returns
    for k_t before writing)."""
    B, H, d = 4, 8, 128
    gen = torch.Generator().manual_seed(3)
    S = (torch.randn(B, H, d, d, generator=gen) * 0.1).cuda()
    k = torch.nn.functional.normalize(torch.randn(B, H, d, generator=gen, dtype=torch.float64), dim=-1)
    k = k.float().cuda()
    q = torch.randn(B, H, d, generator=gen).cuda()
    v = torch.randn(B, H, d, generator=gen).cuda()
    g = torch.rand(B, H, generator=gen).cuda() * 0.5 + 0.5
    b = torch.ones(B, H).cuda()
    la.la_decode_step(q, k, v, S, variant=la.LA_GATED_DELTA, gate=g, beta=b)
    recall = torch.einsum("bhvk,bhk->bhv", S.double(), k.double())
    # |k| = 1 only to float32 rounding; the recall error is float32-sized
    assert torch.max(torch.abs(recall - v.double())).item() < 1e-4


def test_decode_is_deterministic():
    w = wl.variant_workload(la.LA_GATED_DELTA, "bf16", 128, 128, S0_std=0.1, seed=23)
    S0 = dev(wl.decode_state(w, B=8, H=4))
    inp = wl.decode_step_inputs(w, 0, B=8, H=4)
    outs = []
    for _ in range(2):
        S = S0.clone()
        o = la.la_decode_step(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), S,
                              variant=w.variant, gate=dev(inp["gate"]), beta=dev(inp["beta"]))
        outs.append((o.clone(), S.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
