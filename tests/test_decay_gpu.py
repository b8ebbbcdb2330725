"""GPU parity of the fixed per-head decay: the normalized variant with gamma_h
(S and z both decay) and the retention variant (no normalizer), chunked and
decode, against the float64 oracle, plus their invariants."""
import numpy as np
import pytest
import torch

import gated_delta_rule_causal_amd as la
import oracle
import workloads as wl
from gpu_util import TOL, dev, host64, parity_error, record

pytestmark = pytest.mark.gpu

KINDS = {"la_decay": (la.LA_NORMALIZED, la.LA_PHI_ELU1), "ret": (la.LA_RETENTION, la.LA_PHI_IDENTITY),
         "ret_elu": (la.LA_RETENTION, la.LA_PHI_ELU1)}


def _workload(kind, dtype, dk, dv, chunk=64, seed=101, gate_mean=3.0):
    variant, phi = KINDS[kind]
    return wl.variant_workload(variant, dtype, dk, dv, chunk=chunk, phi=phi, seed=seed, gate_mean=gate_mean)


def _inputs(w, B, H, T, gamma=None):
    inp = wl.chunk_inputs(w, B=B, H=H, T=T, S0_std=0.1, z0=w.variant == la.LA_NORMALIZED, head_decay=True)
    if gamma is not None:
        inp["gate"].data[...] = gamma
    return inp


def run(w, inp, chunk, B, H, sample=None):
    d = {k: dev(v) for k, v in inp.items()}
    out, S_T, z_T = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=w.variant, gate=d["gate"], S0=d.get("S0"),
                                    z0=d.get("z0"), chunk=chunk, phi=w.phi_kind)
    torch.cuda.synchronize()
    heads = np.arange(B * H) if sample is None else np.asarray(sample)
    ro, rS, rz = _oracle_heads(w, inp, B, H, heads)
    idx = torch.as_tensor(heads, device=out.device)
    pick = lambda t: host64(t.reshape((B * H,) + tuple(t.shape[2:]))[idx])[None]  # noqa: E731
    errs = {"out": parity_error(pick(out), ro), "S_T": parity_error(pick(S_T), rS)}
    if rz is not None:
        errs["z_T"] = parity_error(pick(z_T), rz)
    return errs, (out, S_T, z_T)


def _oracle_heads(w, inp, B, H, heads):
    """The oracle on the selected flat heads b*H + h (all heads of a batch row
    run together, with the (H,) decays), stacked as one (1, n, ...) batch."""
    f = {n: inp[n].f64() for n in ("q", "k", "v", "S0", "z0") if n in inp}
    rows = {}
    for b in sorted({int(fh) // H for fh in heads}):
        one = lambda n: None if n not in f else f[n][b:b + 1]  # noqa: E731
        rows[b] = oracle.forward(w.variant, one("q"), one("k"), one("v"), gate=inp["gate"].f64(), S0=one("S0"),
                                 z0=one("z0"), phi_kind=w.phi_kind)
    pick = lambda i: np.stack([rows[int(fh) // H][i][0, int(fh) % H] for fh in heads])[None]  # noqa: E731
    return pick(0), pick(1), (pick(2) if rows[int(heads[0]) // H][2] is not None else None)


SWEEP = [(k, dt, dk, dv, c) for k in KINDS for dt in ("f32", "bf16")
         for (dk, dv) in ((16, 16), (64, 64), (128, 128), (32, 64)) for c in (16, 64)]


@pytest.mark.parametrize("kind,dtype,dk,dv,chunk", SWEEP, ids=["-".join(map(str, c)) for c in SWEEP])
def test_decay_chunk_matches_oracle(kind, dtype, dk, dv, chunk):
    w = _workload(kind, dtype, dk, dv, chunk)
    T = 3 * chunk + 5
    inp = _inputs(w, 2, 2, T)
    print("decay chunk parity", kind, dtype, dk, dv, chunk, "T", T, flush=True)
    errs, _ = run(w, inp, chunk, 2, 2)
    record("decay-%s-%s-dk%d-dv%d-c%d" % (kind, dtype, dk, dv, chunk), errs, dtype)
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("B,H,T,d,chunk", [(1, 1, 64 * 20 + 7, 64, 64), (2, 3, 16 * 9, 32, 16),
                                             (1, 2, 4096, 128, 64)])
def test_decay_segments(kind, B, H, T, d, chunk):
    """Few heads and long sequences run as concurrent segments: each enters
    with the decayed sum of the increments before it."""
    w = _workload(kind, "f32", d, d, chunk, seed=103)
    inp = _inputs(w, B, H, T)
    print("decay segments", kind, B, H, T, d, chunk, flush=True)
    errs, _ = run(w, inp, chunk, B, H)
    record("decay-seg-%s-B%dH%dT%dd%d" % (kind, B, H, T, d), errs, "f32")
    assert max(errs.values()) <= TOL["f32"], errs


@pytest.mark.parametrize("gamma", [0.5, 0.05, 0.005])
@pytest.mark.parametrize("kind", list(KINDS))
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decay_strong(kind, dtype, gamma):
    w = _workload(kind, dtype, 64, 64, 64, seed=107)
    inp = _inputs(w, 1, 2, 300, gamma=gamma)
    errs, (out, S_T, _) = run(w, inp, 64, 1, 2)
    record("decay-strong-%s-%s-%g" % (kind, dtype, gamma), errs, dtype)
    assert torch.isfinite(out).all() and torch.isfinite(S_T).all()
    assert max(errs.values()) <= TOL[dtype], errs


def test_decay_normalized_workload_shape():
    """The normalized workload's shape (B=4, H=8, T=2048, d=64, bf16, chunk 64)
    with per-head decays sigmoid(N(3, 1)), every head against the oracle."""
    w = _workload("la_decay", "bf16", 64, 64, 64, seed=2)
    w = wl.Workload("la_decay_bf16_b4h8t2048d64", w.variant, "bf16", 4, 8, 2048, 64, 64, 64, 64 ** -0.5,
                    gate_mean=3.0, seed=2)
    inp = wl.chunk_inputs(w, head_decay=True)
    errs, _ = run(w, inp, 64, 4, 8)
    record("workload-la_decay_bf16_b4h8t2048d64", errs, "bf16")
    assert max(errs.values()) <= TOL["bf16"], errs


def test_unit_decay_is_the_undecayed_variant():
    """gamma_h = 1 everywhere: the same kernels with every power equal to 1."""
    w = _workload("la_decay", "bf16", 64, 64, 64)
    inp = _inputs(w, 2, 3, 500, gamma=1.0)
    d = {k: dev(v) for k, v in inp.items()}
    a = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=la.LA_NORMALIZED, gate=d["gate"], S0=d["S0"], z0=d["z0"])
    b = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=la.LA_NORMALIZED, S0=d["S0"], z0=d["z0"])
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("kind", list(KINDS))
def test_decay_decode_chain_equals_chunked(kind):
    w = _workload(kind, "f32", 64, 32, seed=109)
    T = 40
    inp = _inputs(w, 2, 3, T)
    d = {k: dev(v) for k, v in inp.items()}
    out, S_T, z_T = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=w.variant, gate=d["gate"], S0=d["S0"],
                                    z0=d.get("z0"), phi=w.phi_kind)
    S = d["S0"].clone()
    z = d["z0"].clone() if "z0" in d else None
    for t in range(T):
        o = la.la_decode_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(),
                              d["v"][:, :, t].contiguous(), S, variant=w.variant, gate=d["gate"], z=z,
                              phi=w.phi_kind)
        assert parity_error(host64(o), host64(out[:, :, t])) <= 1e-4
    assert parity_error(host64(S), host64(S_T)) <= 1e-4
    if z is not None:
        assert parity_error(host64(z), host64(z_T)) <= 1e-4


@pytest.mark.parametrize("kind", list(KINDS))
def test_decay_split_call_and_in_place(kind):
    w = _workload(kind, "f32", 64, 64, seed=113)
    T, T1 = 700, 301
    inp = _inputs(w, 1, 2, T)
    d = {k: dev(v) for k, v in inp.items()}
    kw = dict(variant=w.variant, gate=d["gate"], phi=w.phi_kind)
    full = la.la_chunk_fwd(d["q"], d["k"], d["v"], S0=d["S0"], z0=d.get("z0"), **kw)
    a, b = slice(0, T1), slice(T1, T)
    c = lambda t, s: t[:, :, s].contiguous()  # noqa: E731
    o1, S1, z1 = la.la_chunk_fwd(c(d["q"], a), c(d["k"], a), c(d["v"], a), S0=d["S0"], z0=d.get("z0"), **kw)
    o2, S2, z2 = la.la_chunk_fwd(c(d["q"], b), c(d["k"], b), c(d["v"], b), S0=S1, z0=z1, **kw)
    assert parity_error(host64(torch.cat([o1, o2], dim=2)), host64(full[0])) <= 1e-4
    assert parity_error(host64(S2), host64(full[1])) <= 1e-4
    # in place
    S, z = d["S0"].clone(), (d["z0"].clone() if "z0" in d else None)
    la.la_chunk_fwd(d["q"], d["k"], d["v"], S0=S, z0=z, S_T=S, z_T=z, **kw)
    assert torch.equal(S, full[1])
    if z is not None:
        assert torch.equal(z, full[2])


DEC = [(k, dt, dk, dv) for k in KINDS for dt in ("f32", "bf16") for (dk, dv) in ((16, 16), (128, 128), (64, 32))]


@pytest.mark.parametrize("kind,dtype,dk,dv", DEC, ids=["-".join(map(str, c)) for c in DEC])
def test_decay_decode_matches_oracle(kind, dtype, dk, dv):
    w = _workload(kind, dtype, dk, dv, seed=127)
    w = wl.Workload(w.name, w.variant, dtype, 2, 5, 6, dk, dv, 0, dk ** -0.5, gate_mean=2.0, S0_std=0.1,
                    decode=True, seed=127, phi=w.phi)
    B, H = 2, 5
    S = dev(wl.decode_state(w, B=B, H=H))
    S_ref = np.ascontiguousarray(host64(S))
    g = wl.head_decays(w, H=H)
    gd = dev(g)
    z = dev(wl.decode_normalizer(w, B=B, H=H)) if w.variant == la.LA_NORMALIZED else None
    z_ref = np.ascontiguousarray(host64(z)) if z is not None else None
    worst = 0.0
    for s in range(w.T):
        inp = wl.decode_step_inputs(w, s, B=B, H=H)
        o = la.la_decode_step(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), S, variant=w.variant, gate=gd, z=z,
                              phi=w.phi_kind)
        o_ref = oracle.decode_step(w.variant, S_ref, inp["q"].f64(), inp["k"].f64(), inp["v"].f64(),
                                   gate=g.f64(), z=z_ref, phi_kind=w.phi_kind)
        worst = max(worst, parity_error(host64(o), o_ref))
    errs = {"o": worst, "S": parity_error(host64(S), S_ref)}
    if z is not None:
        errs["z"] = parity_error(host64(z), z_ref)
    record("decode-decay-%s-%s-dk%d-dv%d" % (kind, dtype, dk, dv), errs, dtype)
    assert max(errs.values()) <= TOL[dtype], errs
