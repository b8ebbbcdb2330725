"""GPU parity of the chunked backward pass (normalized linear attention and
retention, with and without the fixed per-head decay) against the float64
oracle's reverse pass through the token recurrence, plus its invariants."""
import numpy as np
import pytest
import torch

import gated_delta_rule_causal_amd as la
import oracle
import workloads as wl
from gpu_util import TOL, dev, host64, parity_error, record

pytestmark = pytest.mark.gpu

# (name, variant, phi, per-head decay)
KINDS = {"la": (la.LA_NORMALIZED, la.LA_PHI_ELU1, False), "la_decay": (la.LA_NORMALIZED, la.LA_PHI_ELU1, True),
         "ret": (la.LA_RETENTION, la.LA_PHI_IDENTITY, True), "ret_elu": (la.LA_RETENTION, la.LA_PHI_ELU1, True)}


def _case(kind, dtype, dk, dv, B, H, T, seed, gamma=None, state=True):
    variant, phi, decay = KINDS[kind]
    w = wl.variant_workload(variant, dtype, dk, dv, phi=phi, seed=seed)
    inp = wl.chunk_inputs(w, B=B, H=H, T=T, S0_std=0.1 if state else 0.0, z0=state, head_decay=decay)
    if gamma is not None:
        inp["gate"].data[...] = gamma
    cot = wl.backward_cotangents(w, B=B, H=H, T=T, state=state)
    return w, inp, cot


def _run_gpu(w, inp, cot):
    d = {n: dev(t) for n, t in inp.items()}
    c = {n: dev(t) for n, t in cot.items()}
    g = la.la_chunk_bwd(d["q"], d["k"], d["v"], c["dout"], variant=w.variant, gate=d.get("gate"), S0=d.get("S0"),
                        z0=d.get("z0"), dS_T=c.get("dS_T"), dz_T=c.get("dz_T"), phi=w.phi_kind)
    torch.cuda.synchronize()
    return dict(zip(("dq", "dk", "dv", "dgate", "dS0", "dz0"), g))


def _oracle(w, inp, cot):
    f = {n: t.f64() for n, t in inp.items()}
    c = {n: t.f64() for n, t in cot.items()}
    return oracle.backward(w.variant, f["q"], f["k"], f["v"], c["dout"], gate=f.get("gate"), S0=f.get("S0"),
                           z0=f.get("z0"), dS_T=c.get("dS_T"), dz_T=c.get("dz_T"), phi_kind=w.phi_kind)


def _errors(got, ref):
    errs = {}
    for n in ("dq", "dk", "dv", "dS0", "dz0"):
        if ref.get(n) is not None and got.get(n) is not None:
            errs[n] = parity_error(host64(got[n]), ref[n])
    if ref.get("dgate") is not None:
        errs["dgate"] = parity_error(host64(got["dgate"])[None], ref["dgate"][None], lead=1)
    return errs


SWEEP = [(k, dt, dk, dv) for k in KINDS for dt in ("f32", "bf16")
         for (dk, dv) in ((16, 16), (64, 64), (128, 128), (32, 64), (64, 16))]


@pytest.mark.parametrize("kind,dtype,dk,dv", SWEEP, ids=["-".join(map(str, c)) for c in SWEEP])
def test_bwd_matches_oracle(kind, dtype, dk, dv):
    T = 3 * 64 + 5   # several chunks of 64 (or of 32) and a ragged tail
    w, inp, cot = _case(kind, dtype, dk, dv, 2, 2, T, seed=211)
    print("bwd parity", kind, dtype, dk, dv, "T", T, flush=True)
    errs = _errors(_run_gpu(w, inp, cot), _oracle(w, inp, cot))
    record("bwd-%s-%s-dk%d-dv%d" % (kind, dtype, dk, dv), errs, dtype)
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("T", [1, 15, 16, 63, 64, 65, 130])
@pytest.mark.parametrize("kind", list(KINDS))
def test_bwd_short_and_ragged(kind, T):
    w, inp, cot = _case(kind, "f32", 64, 32, 1, 3, T, seed=223)
    errs = _errors(_run_gpu(w, inp, cot), _oracle(w, inp, cot))
    record("bwd-ragged-%s-T%d" % (kind, T), errs, "f32")
    assert max(errs.values()) <= TOL["f32"], errs


@pytest.mark.parametrize("gamma", [0.5, 0.05])
@pytest.mark.parametrize("kind", ["la_decay", "ret"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_strong_decay(kind, dtype, gamma):
    w, inp, cot = _case(kind, dtype, 64, 64, 1, 2, 300, seed=227, gamma=gamma)
    got = _run_gpu(w, inp, cot)
    for n in ("dq", "dk", "dv"):
        assert torch.isfinite(got[n]).all()
    errs = _errors(got, _oracle(w, inp, cot))
    record("bwd-strong-%s-%s-%g" % (kind, dtype, gamma), errs, dtype)
    assert max(errs.values()) <= TOL[dtype], errs


def test_bwd_without_initial_state_or_state_cotangent():
    for kind in KINDS:
        w, inp, cot = _case(kind, "f32", 32, 32, 2, 2, 100, seed=229, state=False)
        errs = _errors(_run_gpu(w, inp, cot), _oracle(w, inp, cot))
        assert max(errs.values()) <= TOL["f32"], (kind, errs)


def test_bwd_empty_sequence_passes_the_state_cotangent():
    """T = 0: dS0 = dS_T, dz0 = dz_T and the decay gradient is zero."""
    w, inp, cot = _case("la_decay", "f32", 64, 64, 2, 3, 0, seed=233)
    got = _run_gpu(w, inp, cot)
    assert torch.equal(got["dS0"], dev(cot["dS_T"])) and torch.equal(got["dz0"], dev(cot["dz_T"]))
    assert torch.equal(got["dgate"], torch.zeros_like(got["dgate"]))


def test_bwd_unit_decay_is_the_undecayed_variant():
    """gamma_h = 1 everywhere gives the same dq, dk, dv, dS0 and dz0 as no
    decay (every power is 1)."""
    w, inp, cot = _case("la_decay", "bf16", 64, 64, 2, 3, 200, seed=239, gamma=1.0)
    a = _run_gpu(w, inp, cot)
    inp.pop("gate")
    b = _run_gpu(w, inp, cot)
    for n in ("dq", "dk", "dv", "dS0", "dz0"):
        assert torch.equal(a[n], b[n]), n


@pytest.mark.parametrize("kind", list(KINDS))
def test_bwd_split_sequence_chains_through_the_state(kind):
    """Backward of two consecutive calls (the second starting from the first's
    final state) equals the backward of one call over the whole sequence: the
    second call's dS0 is the first call's dS_T."""
    T, T1 = 300, 131
    w, inp, cot = _case(kind, "f32", 64, 64, 1, 2, T, seed=241)
    d = {n: dev(t) for n, t in inp.items()}
    c = {n: dev(t) for n, t in cot.items()}
    full = _run_gpu(w, inp, cot)
    cut = lambda t, s: t[:, :, s].contiguous()  # noqa: E731
    a, b = slice(0, T1), slice(T1, T)
    kw = dict(variant=w.variant, gate=d.get("gate"), phi=w.phi_kind)
    _, S1, z1 = la.la_chunk_fwd(cut(d["q"], a), cut(d["k"], a), cut(d["v"], a), S0=d["S0"], z0=d.get("z0"), **kw)
    g2 = la.la_chunk_bwd(cut(d["q"], b), cut(d["k"], b), cut(d["v"], b), cut(c["dout"], b), S0=S1, z0=z1,
                         dS_T=c["dS_T"], dz_T=c.get("dz_T"), **kw)
    g1 = la.la_chunk_bwd(cut(d["q"], a), cut(d["k"], a), cut(d["v"], a), cut(c["dout"], a), S0=d["S0"],
                         z0=d.get("z0"), dS_T=g2[4], dz_T=g2[5], **kw)
    for i, n in enumerate(("dq", "dk", "dv")):
        assert parity_error(host64(torch.cat([g1[i], g2[i]], dim=2)), host64(full[n])) <= 1e-4, n
    assert parity_error(host64(g1[4]), host64(full["dS0"])) <= 1e-4
    if full["dgate"] is not None:
        # the second call's decay gradient holds the first call's state fixed;
        # the first call's carries it through S1
        assert parity_error(host64(g1[3] + g2[3])[None], host64(full["dgate"])[None], lead=1) <= 1e-3


def test_bwd_normalized_workload_shape():
    """The normalized workload's shape (B=4, H=8, T=2048, d=64, bf16) with
    per-head decays, every head and every gradient against the oracle."""
    w = wl.Workload("la_decay_bf16_b4h8t2048d64", la.LA_NORMALIZED, "bf16", 4, 8, 2048, 64, 64, 64, 64 ** -0.5,
                    gate_mean=3.0, seed=2)
    inp = wl.chunk_inputs(w, head_decay=True)
    cot = wl.backward_cotangents(w, state=False)
    print("bwd workload", w.name, flush=True)
    errs = _errors(_run_gpu(w, inp, cot), _oracle(w, inp, cot))
    record("workload-bwd-la_decay_bf16_b4h8t2048d64", errs, "bf16")
    assert max(errs.values()) <= TOL["bf16"], errs


def test_bwd_retention_training_shape_sampled_heads():
    """Retention at a training shape (B=4, H=16, T=8192, d=128, bf16): every
    gradient of two heads (all batch rows, so that their decay gradients are
    whole) against the oracle."""
    w = wl.Workload("ret_bf16_b4h16t8192d128", la.LA_RETENTION, "bf16", 4, 16, 8192, 128, 128, 64, 128 ** -0.5,
                    gate_mean=4.0, seed=8, phi=la.LA_PHI_IDENTITY)
    inp = wl.chunk_inputs(w)
    cot = wl.backward_cotangents(w, state=False)
    print("bwd workload", w.name, flush=True)
    got = _run_gpu(w, inp, cot)
    errs = {}
    for h in (0, 9):
        sel = {n: wl.HostTensor(t.dtype, np.ascontiguousarray(t.data[:, h:h + 1])) for n, t in inp.items()
               if n != "gate"}
        sel["gate"] = wl.HostTensor("f32", inp["gate"].data[h:h + 1].copy())
        csel = {n: wl.HostTensor(t.dtype, np.ascontiguousarray(t.data[:, h:h + 1])) for n, t in cot.items()}
        ref = _oracle(w, sel, csel)
        part = {n: (got[n][:, h:h + 1] if n != "dgate" else got[n][h:h + 1]) for n in got if got[n] is not None}
        for n, e in _errors(part, ref).items():
            errs[n] = max(errs.get(n, 0.0), e)
    record("workload-bwd-ret_bf16_b4h16t8192d128-heads0,9", errs, "bf16")
    assert max(errs.values()) <= TOL["bf16"], errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("kind,H,dk,dv", [("ret", 3, 64, 64), ("ret_elu", 8, 128, 32), ("ret", 8, 32, 128),
                                           ("ret_elu", 16, 64, 64)])
def test_bwd_retention_many_chunks(kind, H, dk, dv, dtype):
    """Retention over many chunks (18 of 64 tokens, the last one ragged), where
    the chunk states come from one chain per head, direction and value block:
    every gradient against the oracle, with 3 heads and with 8 (the two
    workgroup orders), and with 16 (288 chunk-heads: the persistent bf16
    gradient kernel's 256 workgroups take two chunks each for some)."""
    T = 17 * 64 + 29
    w, inp, cot = _case(kind, dtype, dk, dv, 1, H, T, seed=251)
    print("bwd chain", kind, dtype, H, dk, dv, "T", T, flush=True)
    errs = _errors(_run_gpu(w, inp, cot), _oracle(w, inp, cot))
    record("bwd-chain-%s-%s-H%d-dk%d-dv%d" % (kind, dtype, H, dk, dv), errs, dtype)
    assert max(errs.values()) <= TOL[dtype], errs
