"""GPU parity of speculative verify and commit (checkpoint plus input replay)
against the float64 oracle, and their invariants."""
import numpy as np
import pytest
import torch

import gated_delta_rule_causal_amd as la
import oracle
import workloads as wl
from gpu_util import TOL, dev, host64, parity_error, record

pytestmark = pytest.mark.gpu

# (name, variant, phi, per-head decay)
KINDS = [("la", la.LA_NORMALIZED, la.LA_PHI_ELU1, False), ("la_decay", la.LA_NORMALIZED, la.LA_PHI_ELU1, True),
         ("gla", la.LA_GATED, la.LA_PHI_ELU1, False), ("gla_id", la.LA_GATED, la.LA_PHI_IDENTITY, False),
         ("gdr", la.LA_GATED_DELTA, la.LA_PHI_IDENTITY, False), ("ret", la.LA_RETENTION, la.LA_PHI_IDENTITY, True)]


def _case(kind, dtype, d, B, H, T, seed):
    name, variant, phi, decay = kind
    w = wl.variant_workload(variant, dtype, d, d, phi=phi, seed=seed)
    inp = wl.chunk_inputs(w, B=B, H=H, T=T, S0_std=0.1, z0=True, head_decay=decay)
    if "z0" not in inp and variant == la.LA_NORMALIZED:
        inp["z0"] = wl.decode_normalizer(w, B=B, H=H)
    return w, inp


def _oracle(w, inp, upto=None):
    """Oracle over the first upto[b] tokens of each sequence (all T if None)."""
    f = {n: inp[n].f64() for n in inp}
    B, H, T = f["q"].shape[:3]
    per_head_gate = w.variant in (la.LA_NORMALIZED, la.LA_RETENTION)
    outs, Ss, zs = [], [], []
    for b in range(B):
        n = T if upto is None else int(upto[b])
        cut = lambda a: None if a is None else a[b:b + 1, :, :n]  # noqa: E731
        gate = f.get("gate")
        g = gate if (gate is None or per_head_gate) else cut(gate)
        o, S, z = oracle.forward(w.variant, cut(f["q"]), cut(f["k"]), cut(f["v"]), gate=g, beta=cut(f.get("beta")),
                                 S0=f["S0"][b:b + 1], z0=None if "z0" not in f or w.variant != la.LA_NORMALIZED
                                 else f["z0"][b:b + 1], phi_kind=w.phi_kind)
        outs.append(o); Ss.append(S); zs.append(z)
    z = None if zs[0] is None else np.concatenate(zs)
    return outs, np.concatenate(Ss), z


def _dev(inp, w):
    d = {k: dev(v) for k, v in inp.items()}
    if w.variant != la.LA_NORMALIZED:
        d.pop("z0", None)
    return d


CASES = [(k, dt, d) for k in KINDS for dt in ("f32", "bf16") for d in (16, 64, 128)]


@pytest.mark.parametrize("T", [1, 4, 9])
@pytest.mark.parametrize("kind,dtype,d", CASES, ids=["%s-%s-%d" % (k[0], dt, d) for k, dt, d in CASES])
def test_verify_then_commit(kind, dtype, d, T):
    w, inp = _case(kind, dtype, d, 3, 2, T, seed=131)
    dd = _dev(inp, w)
    S0, z0 = dd["S0"], dd.get("z0")
    S, z = S0.clone(), (z0.clone() if z0 is not None else None)
    out = la.la_verify(dd["q"], dd["k"], dd["v"], S, variant=w.variant, gate=dd.get("gate"), beta=dd.get("beta"),
                       z=z, phi=w.phi_kind)
    torch.cuda.synchronize()
    assert torch.equal(S, S0) and (z is None or torch.equal(z, z0)), "verify changed the checkpoint"
    ro, _, _ = _oracle(w, inp)
    errs = {"out": parity_error(host64(out), np.concatenate(ro))}
    # commit a different prefix per sequence: 0, T and something in between
    acc = np.array([0, T, min(T, max(1, T // 2 + 1))], np.int32)
    la.la_commit(dd["k"], dd["v"], S, torch.as_tensor(acc, device="cuda"), variant=w.variant, gate=dd.get("gate"),
                 beta=dd.get("beta"), z=z, phi=w.phi_kind)
    torch.cuda.synchronize()
    _, rS, rz = _oracle(w, inp, upto=acc)
    errs["S"] = parity_error(host64(S), rS)
    if z is not None:
        errs["z"] = parity_error(host64(z), rz)
    assert torch.equal(S[0], S0[0]), "accepting nothing must leave the state as it was"
    record("verify-%s-%s-d%d-T%d" % (kind[0], dtype, d, T), errs, dtype)
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("kind", KINDS, ids=[k[0] for k in KINDS])
def test_speculative_loop_equals_decode_chain(kind):
    """Three rounds of verify(4 drafts) + commit(accepted) equal one decode step
    per accepted token, outputs included."""
    w, inp = _case(kind, "f32", 64, 2, 3, 12, seed=137)
    dd = _dev(inp, w)
    S_spec, S_dec = dd["S0"].clone(), dd["S0"].clone()
    z_spec = dd["z0"].clone() if "z0" in dd else None
    z_dec = dd["z0"].clone() if "z0" in dd else None
    per_head = w.variant in (la.LA_NORMALIZED, la.LA_RETENTION)
    sl = lambda a, s: None if a is None else (a if (per_head and a is dd.get("gate")) else a[:, :, s].contiguous())  # noqa: E731
    pos = 0
    for accepted in (3, 0, 4):
        s = slice(pos, pos + 4)
        args = dict(variant=w.variant, gate=sl(dd.get("gate"), s), beta=sl(dd.get("beta"), s), phi=w.phi_kind)
        out = la.la_verify(sl(dd["q"], s), sl(dd["k"], s), sl(dd["v"], s), S_spec, z=z_spec, **args)
        acc = torch.full((2,), accepted, dtype=torch.int32, device="cuda")
        la.la_commit(sl(dd["k"], s), sl(dd["v"], s), S_spec, acc, z=z_spec, **args)
        for t in range(accepted):
            g = dd.get("gate")
            b = dd.get("beta")
            o = la.la_decode_step(dd["q"][:, :, pos + t].contiguous(), dd["k"][:, :, pos + t].contiguous(),
                                  dd["v"][:, :, pos + t].contiguous(), S_dec, variant=w.variant, phi=w.phi_kind,
                                  gate=None if g is None else (g if per_head else g[:, :, pos + t].contiguous()),
                                  beta=None if b is None else b[:, :, pos + t].contiguous(), z=z_dec)
            assert parity_error(host64(out[:, :, t]), host64(o)) <= 1e-5
        assert parity_error(host64(S_spec), host64(S_dec)) <= 1e-5
        pos += accepted
    if z_spec is not None:
        assert parity_error(host64(z_spec), host64(z_dec)) <= 1e-5


def test_verify_commit_decode_workload_shape():
    """The decode workload's shape (B=256 x H=16 heads of 128 x 128 state, bf16
    q/k/v) with 4 draft tokens: verify against the oracle on every 37th head,
    then commit random accepted counts."""
    w = wl.WORKLOADS["gdr_decode_b256h16d128"]
    B, H, T = w.B, w.H, 4
    rng = np.random.default_rng(139)
    steps = [wl.decode_step_inputs(w, s, B=B, H=H) for s in range(T)]
    stack = lambda n: wl.HostTensor(steps[0][n].dtype, np.ascontiguousarray(np.stack([s[n].data for s in steps], 2)))  # noqa: E731
    inp = {n: stack(n) for n in ("q", "k", "v", "gate", "beta")}
    inp["S0"] = wl.decode_state(w)
    dd = {k: dev(v) for k, v in inp.items()}
    S = dd["S0"].clone()
    out = la.la_verify(dd["q"], dd["k"], dd["v"], S, variant=w.variant, gate=dd["gate"], beta=dd["beta"])
    acc = rng.integers(0, T + 1, size=B).astype(np.int32)
    la.la_commit(dd["k"], dd["v"], S, torch.as_tensor(acc, device="cuda"), variant=w.variant, gate=dd["gate"],
                 beta=dd["beta"])
    torch.cuda.synchronize()
    heads = np.arange(0, B * H, 37)
    sel = lambda a: a.f64().reshape((B * H,) + a.shape[2:])[heads][None]  # noqa: E731
    ro, _, _ = oracle.forward(w.variant, sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), gate=sel(inp["gate"]),
                              beta=sel(inp["beta"]), S0=sel(inp["S0"]))
    idx = torch.as_tensor(heads, device="cuda")
    e_out = parity_error(host64(out.reshape(B * H, T, -1)[idx])[None], ro)
    # committed state: the oracle over each sampled head's accepted prefix
    e_S = 0.0
    f = {n: inp[n].f64().reshape((B * H,) + inp[n].shape[2:]) for n in inp}
    for fh in heads:
        n = int(acc[fh // H])
        cut = lambda name: f[name][fh][None, None, :n]  # noqa: E731
        _, rS, _ = oracle.forward(w.variant, cut("q"), cut("k"), cut("v"), gate=cut("gate"), beta=cut("beta"),
                                  S0=f["S0"][fh][None, None])
        e_S = max(e_S, parity_error(host64(S.reshape(B * H, w.d_v, w.d_k)[fh])[None, None], rS))
    record("workload-verify_commit_b256h16d128_T4", {"out": e_out, "S": e_S}, "bf16")
    assert e_out <= TOL["bf16"] and e_S <= TOL["bf16"], (e_out, e_S)
