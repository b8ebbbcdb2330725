"""GPU parity of la_chunk_fwd against the float64 oracle, and its invariants."""
import numpy as np
import pytest
import torch

import gated_delta_rule_causal_amd as la
import oracle
import workloads as wl
from gpu_util import TOL, dev, host64, parity_error, record

pytestmark = pytest.mark.gpu

VARIANTS = {"la": (la.LA_NORMALIZED, la.LA_PHI_ELU1), "gla": (la.LA_GATED, la.LA_PHI_ELU1),
            "gla_id": (la.LA_GATED, la.LA_PHI_IDENTITY), "gdr": (la.LA_GATED_DELTA, la.LA_PHI_IDENTITY)}


def run_chunk(w, inp, chunk, sample=None, B=None, H=None):
    """GPU forward over every head; oracle on `sample` heads (flat b*H+h indices)."""
    B = w.B if B is None else B
    H = w.H if H is None else H
    d = {k: dev(v) for k, v in inp.items()}
    out, S_T, z_T = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=w.variant, gate=d.get("gate"),
                                    beta=d.get("beta"), S0=d.get("S0"), z0=d.get("z0"), chunk=chunk,
                                    phi=w.phi_kind)
    torch.cuda.synchronize()
    heads = np.arange(B * H) if sample is None else np.asarray(sample)

    def sel(name):
        if name not in inp:
            return None
        a = inp[name]
        raw = a.data.reshape((B * H,) + a.data.shape[2:])[heads]
        return wl.HostTensor(a.dtype, raw).f64()[None]

    ro, rS, rz = oracle.forward(w.variant, sel("q"), sel("k"), sel("v"), gate=sel("gate"), beta=sel("beta"),
                                S0=sel("S0"), z0=sel("z0"), phi_kind=w.phi_kind)
    idx = torch.as_tensor(heads, device=out.device)
    pick = lambda t: host64(t.reshape((B * H,) + tuple(t.shape[2:]))[idx])[None]  # noqa: E731
    errs = {"out": parity_error(pick(out), ro), "S_T": parity_error(pick(S_T), rS)}
    if rz is not None:
        errs["z_T"] = parity_error(pick(z_T), rz)
    return errs, (out, S_T, z_T)


SWEEP = []
for name in VARIANTS:
    for dtype in ("f32", "bf16"):
        for dk, dv in ((16, 16), (32, 64), (64, 32), (128, 128), (64, 16)):
            for chunk in (16, 32, 64, 128):
                SWEEP.append((name, dtype, dk, dv, chunk))


@pytest.mark.parametrize("name,dtype,dk,dv,chunk", SWEEP, ids=["-".join(map(str, c)) for c in SWEEP])
def test_chunk_matches_oracle(name, dtype, dk, dv, chunk):
    """Several tiles per chunk, several chunks, a ragged tail, and an initial state."""
    variant, phi = VARIANTS[name]
    w = wl.variant_workload(variant, dtype, dk, dv, chunk=chunk, phi=phi, seed=31)
    T = 3 * chunk + 5
    inp = wl.chunk_inputs(w, B=2, H=2, T=T, S0_std=0.1, z0=True)
    print("chunk parity", name, dtype, dk, dv, chunk, "T", T, flush=True)
    errs, _ = run_chunk(w, inp, chunk, B=2, H=2)
    record("sweep-%s-%s-dk%d-dv%d-c%d" % (name, dtype, dk, dv, chunk), errs, dtype)
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("wname", ["la_f32_b1h2t64d16", "la_bf16_b4h8t2048d64",
                                   "gla_bf16_b8h16t4096d128", "gdr_bf16_b4h16t8192d128"])
def test_chunk_workload_full_shape(wname):
    """The specified workloads at full size, every head on the GPU and in the
    oracle (the oracle runs the largest, 64 heads x 8192 tokens, in seconds)."""
    w = wl.WORKLOADS[wname]
    inp = wl.chunk_inputs(w)
    print("chunk workload", wname, "all heads", flush=True)
    errs, _ = run_chunk(w, inp, w.chunk)
    record("workload-" + wname, errs, w.dtype)
    assert max(errs.values()) <= TOL[w.dtype], errs


# Strong decay (page "Ch. 11 Linear attention and Hyena", 11.3: any gate in
# (0, 1]): random gates sigmoid(N(-3, 1)) (about 0.05), constant gates down to
# 0.001 (a 16-token block product of 1e-48, below float32's range), and mild
# gates with one channel at 1e-3.  Ragged lengths of one to four chunks.
def _strong_gates(inp, kind):
    g = inp["gate"].data
    if isinstance(kind, float):
        g[...] = kind
    elif kind == "mixed":
        g[..., 5] = 1e-3
    return inp


GLA_STRONG = [(n, dt, d, c) for (n, dt, d, c) in (("gla", "bf16", 128, 64), ("gla", "bf16", 64, 32),
                                                  ("gla_id", "bf16", 64, 64), ("gla", "f32", 64, 64),
                                                  ("gla", "f32", 128, 64), ("gla", "f32", 32, 16))]


@pytest.mark.parametrize("T", [16, 65, 200])
@pytest.mark.parametrize("kind", ["sig-3", 0.5, 0.05, 0.005, 0.001, "mixed"])
@pytest.mark.parametrize("name,dtype,d,chunk", GLA_STRONG, ids=["-".join(map(str, c)) for c in GLA_STRONG])
def test_gla_strong_decay(name, dtype, d, chunk, kind, T):
    variant, phi = VARIANTS[name]
    w = wl.variant_workload(variant, dtype, d, d, chunk=chunk, phi=phi, seed=83,
                            gate_mean=-3.0 if kind == "sig-3" else 3.0)
    inp = _strong_gates(wl.chunk_inputs(w, B=1, H=2, T=T, S0_std=0.1), kind)
    print("gla strong decay", name, dtype, d, chunk, kind, T, flush=True)
    errs, (out, S_T, _) = run_chunk(w, inp, chunk, B=1, H=2)
    record("gla-strong-%s-%s-d%d-c%d-%s-T%d" % (name, dtype, d, chunk, kind, T), errs, dtype)
    assert torch.isfinite(out).all() and torch.isfinite(S_T).all()
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("T", [65, 200])
@pytest.mark.parametrize("kind", ["sig-2", 0.005])
@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 64), ("bf16", 128, 32), ("f32", 64, 64)])
def test_gdr_strong_decay(dtype, d, chunk, kind, T):
    w = wl.variant_workload(la.LA_GATED_DELTA, dtype, d, d, chunk=chunk, seed=89,
                            gate_mean=-2.0 if kind == "sig-2" else 4.0)
    inp = _strong_gates(wl.chunk_inputs(w, B=1, H=2, T=T, S0_std=0.1), kind)
    print("gdr strong decay", dtype, d, chunk, kind, T, flush=True)
    errs, (out, S_T, _) = run_chunk(w, inp, chunk, B=1, H=2)
    record("gdr-strong-%s-d%d-c%d-%s-T%d" % (dtype, d, chunk, kind, T), errs, dtype)
    assert torch.isfinite(out).all() and torch.isfinite(S_T).all()
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("name", list(VARIANTS))
def test_chunk_size_independence(name):
    variant, phi = VARIANTS[name]
    w = wl.variant_workload(variant, "f32", 64, 64, phi=phi, seed=41)
    inp = wl.chunk_inputs(w, B=1, H=3, T=150, S0_std=0.1, z0=True)
    d = {k: dev(v) for k, v in inp.items()}
    res = []
    for chunk in (16, 32, 64, 128):
        out, S_T, _ = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=variant, gate=d.get("gate"),
                                      beta=d.get("beta"), S0=d.get("S0"), z0=d.get("z0"), chunk=chunk, phi=phi)
        res.append((host64(out), host64(S_T)))
    for o, s in res[1:]:
        assert parity_error(o, res[0][0]) <= 1e-4 and parity_error(s, res[0][1]) <= 1e-4


@pytest.mark.parametrize("name", list(VARIANTS))
def test_split_call_equals_single_call(name):
    """The state carries exactly across calls: [0, T1) then [T1, T) equals [0, T)."""
    variant, phi = VARIANTS[name]
    w = wl.variant_workload(variant, "f32", 32, 32, phi=phi, seed=43)
    T, T1 = 200, 77
    inp = wl.chunk_inputs(w, B=2, H=2, T=T)
    d = {k: dev(v) for k, v in inp.items()}
    kw = lambda s: {"gate": None if "gate" not in d else d["gate"][:, :, s].contiguous(),  # noqa: E731
                    "beta": None if "beta" not in d else d["beta"][:, :, s].contiguous()}
    full = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=variant, phi=phi, **kw(slice(0, T)))
    a, b = slice(0, T1), slice(T1, T)
    o1, S1, z1 = la.la_chunk_fwd(d["q"][:, :, a].contiguous(), d["k"][:, :, a].contiguous(),
                                 d["v"][:, :, a].contiguous(), variant=variant, phi=phi, **kw(a))
    o2, S2, z2 = la.la_chunk_fwd(d["q"][:, :, b].contiguous(), d["k"][:, :, b].contiguous(),
                                 d["v"][:, :, b].contiguous(), variant=variant, phi=phi, S0=S1, z0=z1, **kw(b))
    assert parity_error(host64(torch.cat([o1, o2], dim=2)), host64(full[0])) <= 1e-4
    assert parity_error(host64(S2), host64(full[1])) <= 1e-4


@pytest.mark.parametrize("name", list(VARIANTS))
def test_decode_steps_equal_chunked_forward(name):
    """T recurrent decode steps reproduce the chunked forward over the same T tokens."""
    variant, phi = VARIANTS[name]
    w = wl.variant_workload(variant, "f32", 64, 32, phi=phi, seed=47)
    T = 40
    inp = wl.chunk_inputs(w, B=2, H=3, T=T, S0_std=0.1, z0=True)
    d = {k: dev(v) for k, v in inp.items()}
    out, S_T, z_T = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=variant, gate=d.get("gate"),
                                    beta=d.get("beta"), S0=d.get("S0"), z0=d.get("z0"), phi=phi)
    S = d["S0"].clone()
    z = d["z0"].clone() if variant == la.LA_NORMALIZED else None
    for t in range(T):
        g = d.get("gate")
        b = d.get("beta")
        o = la.la_decode_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(),
                              d["v"][:, :, t].contiguous(), S, variant=variant, phi=phi, z=z,
                              gate=None if g is None else g[:, :, t].contiguous(),
                              beta=None if b is None else b[:, :, t].contiguous())
        assert parity_error(host64(o), host64(out[:, :, t])) <= 1e-4
    assert parity_error(host64(S), host64(S_T)) <= 1e-4


@pytest.mark.parametrize("name", list(VARIANTS))
def test_in_place_state_and_empty_sequence(name):
    variant, phi = VARIANTS[name]
    w = wl.variant_workload(variant, "bf16", 64, 64, phi=phi, seed=53)
    # T = 300: five chunks, so the normalized variant runs in two concurrent
    # segments and S_T aliasing S0 crosses them
    inp = wl.chunk_inputs(w, B=1, H=2, T=300, S0_std=0.1, z0=True)
    d = {k: dev(v) for k, v in inp.items()}
    ref = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=variant, gate=d.get("gate"), beta=d.get("beta"),
                          S0=d["S0"], z0=d.get("z0"), phi=phi)
    S = d["S0"].clone()
    z = d["z0"].clone() if "z0" in d else None
    la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=variant, gate=d.get("gate"), beta=d.get("beta"),
                    S0=S, z0=z, S_T=S, z_T=z, phi=phi)
    assert torch.equal(S, ref[1])
    if z is not None:
        assert torch.equal(z, ref[2])
    # T = 0: the final state is the initial state
    e = lambda t: None if t is None else t[:, :, :0].contiguous()  # noqa: E731
    o0, S0o, z0o = la.la_chunk_fwd(e(d["q"]), e(d["k"]), e(d["v"]), variant=variant, gate=e(d.get("gate")),
                                   beta=e(d.get("beta")), S0=d["S0"], z0=d.get("z0"), phi=phi)
    assert o0.numel() == 0 and torch.equal(S0o, d["S0"])
    if z0o is not None:
        assert torch.equal(z0o, d["z0"])


@pytest.mark.parametrize("T", [40, 1000])
def test_la_in_place_one_pass_many_value_blocks(T):
    """Normalized variant on the chained path with several value blocks per
    head (B=1, H=2, d=32 gives two 16-channel blocks; T=40 is too short to
    segment, T=1000 runs as segments), z_T and S_T in place of z0 and S0:
    every block reads z0, one writes z_T."""
    w = wl.variant_workload(la.LA_NORMALIZED, "f32", 32, 32, chunk=16, phi=la.LA_PHI_ELU1, seed=61)
    inp = wl.chunk_inputs(w, B=1, H=2, T=T, S0_std=0.1, z0=True)
    d = {k: dev(v) for k, v in inp.items()}
    ref = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=w.variant, S0=d["S0"], z0=d["z0"], chunk=16)
    S, z = d["S0"].clone(), d["z0"].clone()
    out, _, _ = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=w.variant, S0=S, z0=z, S_T=S, z_T=z, chunk=16)
    assert torch.equal(out, ref[0]) and torch.equal(S, ref[1]) and torch.equal(z, ref[2])
    ro, rS, rz = oracle.forward(w.variant, inp["q"].f64(), inp["k"].f64(), inp["v"].f64(),
                                S0=inp["S0"].f64(), z0=inp["z0"].f64())
    errs = {"out": parity_error(host64(out), ro), "S_T": parity_error(host64(S), rS),
            "z_T": parity_error(host64(z), rz)}
    record("la-in-place-one-pass-T%d" % T, errs, "f32")
    assert max(errs.values()) <= TOL["f32"], errs


@pytest.mark.parametrize("B,H,T,d,chunk", [(1, 1, 64 * 20 + 7, 64, 64), (2, 3, 16 * 9, 32, 16),
                                             (16, 16, 100, 16, 16)])
def test_la_segment_counts(B, H, T, d, chunk):
    """Normalized variant: many concurrent segments with a ragged last one (the
    first two shapes), and enough heads for one unsegmented pass (the last)."""
    w = wl.variant_workload(la.LA_NORMALIZED, "f32", d, d, chunk=chunk, phi=la.LA_PHI_ELU1, seed=67)
    inp = wl.chunk_inputs(w, B=B, H=H, T=T, S0_std=0.1, z0=True)
    nh = B * H
    sample = None if nh <= 8 else [0, 1, nh // 2, nh - 1]
    print("la segments", B, H, T, d, chunk, flush=True)
    errs, _ = run_chunk(w, inp, chunk, sample=sample, B=B, H=H)
    assert max(errs.values()) <= TOL["f32"], errs


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 64), ("bf16", 128, 32), ("f32", 64, 64)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 128, 129, 191, 192, 200])
def test_gdr_chunk_counts(dtype, d, chunk, T):
    """Delta rule at one to four chunks, whole and ragged: the prologue stages
    up to three chunks ahead and the loop's staging re-reads the last chunk
    when the ones ahead do not exist."""
    w = wl.variant_workload(la.LA_GATED_DELTA, dtype, d, d, chunk=chunk, seed=71)
    inp = wl.chunk_inputs(w, B=1, H=2, T=T, S0_std=0.1)
    print("gdr chunk counts", dtype, d, chunk, T, flush=True)
    errs, _ = run_chunk(w, inp, chunk, B=1, H=2)
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 64), ("bf16", 64, 32), ("f32", 64, 64)])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 128, 129, 191, 200])
def test_gla_chunk_counts(dtype, d, chunk, T):
    """Gated linear attention at one to four chunks, whole and ragged: the
    two role loops run one iteration more than there are chunks (the first
    prepares chunk 0), the helpers commit staged tiles even when nothing
    follows, and the gate tile of a ragged last chunk re-reads its last row."""
    w = wl.variant_workload(la.LA_GATED, dtype, d, d, chunk=chunk, phi=la.LA_PHI_ELU1, seed=73)
    inp = wl.chunk_inputs(w, B=1, H=2, T=T, S0_std=0.1)
    print("gla chunk counts", dtype, d, chunk, T, flush=True)
    errs, _ = run_chunk(w, inp, chunk, B=1, H=2)
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 64, 64), ("f32", 32, 32)])
@pytest.mark.parametrize("T", [1, 64, 65, 129, 200])
def test_la_chunk_counts(dtype, d, chunk, T):
    """Normalized linear attention at one to four chunks, whole and ragged (the
    next chunk's loads are issued on every chunk, re-reading the last one past
    the end), with an initial state and normalizer."""
    w = wl.variant_workload(la.LA_NORMALIZED, dtype, d, d, chunk=chunk, phi=la.LA_PHI_ELU1, seed=79)
    inp = wl.chunk_inputs(w, B=1, H=2, T=T, S0_std=0.1, z0=True)
    print("la chunk counts", dtype, d, chunk, T, flush=True)
    errs, _ = run_chunk(w, inp, chunk, B=1, H=2)
    assert max(errs.values()) <= TOL[dtype], errs


def test_chunk_is_deterministic():
    w = wl.WORKLOADS["gdr_bf16_b4h16t8192d128"]
    inp = wl.chunk_inputs(w, B=1, H=4, T=1000)
    d = {k: dev(v) for k, v in inp.items()}
    r = [la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=w.variant, gate=d["gate"], beta=d["beta"])
         for _ in range(2)]
    assert torch.equal(r[0][0], r[1][0]) and torch.equal(r[0][1], r[1][1])


def test_gdr_unit_beta_recall_after_chunk():
    """beta = 1 everywhere: after the sequence, S_T k_T = v_T (the last write is exact)."""
    w = wl.variant_workload(la.LA_GATED_DELTA, "f32", 64, 64, seed=59)
    inp = wl.chunk_inputs(w, B=1, H=2, T=100)
    d = {k: dev(v) for k, v in inp.items()}
    beta = torch.ones_like(d["beta"])
    _, S_T, _ = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=w.variant, gate=d["gate"], beta=beta)
    k_last = d["k"][:, :, -1].double()
    recall = torch.einsum("bhvk,bhk->bhv", S_T.double(), k_last)
    assert torch.max(torch.abs(recall - d["v"][:, :, -1].double())).item() < 1e-3
