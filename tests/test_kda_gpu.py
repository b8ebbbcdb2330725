"""GPU parity of the delta rule with a per-key-channel decay (LA_KDA) against
the float64 oracle: chunked forward, decode, verify/commit, and invariants."""
import numpy as np
import pytest
import torch

import gated_delta_rule_causal_amd as la
import oracle
import workloads as wl
from gpu_util import TOL, dev, host64, parity_error, record

pytestmark = pytest.mark.gpu


def _w(dtype, dk, dv, chunk=64, seed=151, gate_mean=3.0):
    return wl.variant_workload(la.LA_KDA, dtype, dk, dv, chunk=chunk, seed=seed, gate_mean=gate_mean)


def run(w, inp, chunk, B, H):
    d = {k: dev(v) for k, v in inp.items()}
    out, S_T, _ = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=la.LA_KDA, gate=d["gate"], beta=d["beta"],
                                  S0=d.get("S0"), chunk=chunk)
    torch.cuda.synchronize()
    f = lambda n: None if n not in inp else inp[n].f64()  # noqa: E731
    ro, rS, _ = oracle.forward(la.LA_KDA, f("q"), f("k"), f("v"), gate=f("gate"), beta=f("beta"), S0=f("S0"))
    return {"out": parity_error(host64(out), ro), "S_T": parity_error(host64(S_T), rS)}, (out, S_T)


SWEEP = [(dt, dk, dv, c) for dt in ("f32", "bf16") for (dk, dv) in ((16, 16), (64, 64), (128, 128), (32, 64), (64, 16))
         for c in (16, 32, 64)]


@pytest.mark.parametrize("dtype,dk,dv,chunk", SWEEP, ids=["-".join(map(str, c)) for c in SWEEP])
def test_kda_chunk_matches_oracle(dtype, dk, dv, chunk):
    w = _w(dtype, dk, dv, chunk)
    T = 3 * chunk + 5
    inp = wl.chunk_inputs(w, B=2, H=2, T=T, S0_std=0.1)
    print("kda chunk parity", dtype, dk, dv, chunk, "T", T, flush=True)
    errs, _ = run(w, inp, chunk, 2, 2)
    record("kda-%s-dk%d-dv%d-c%d" % (dtype, dk, dv, chunk), errs, dtype)
    assert max(errs.values()) <= TOL[dtype], errs


@pytest.mark.parametrize("T", [1, 16, 63, 64, 65, 200])
@pytest.mark.parametrize("kind", ["sig-3", 0.05, 0.001, "mixed"])
@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 64), ("f32", 64, 64), ("bf16", 64, 32)])
def test_kda_strong_decay_and_ragged(dtype, d, chunk, kind, T):
    """Strong per-channel decay (page "Beyond -- Linear attention and recurrent
    memory": any gate in (0, 1]) at one to four chunks, whole and ragged."""
    w = _w(dtype, d, d, chunk, seed=157, gate_mean=-3.0 if kind == "sig-3" else 3.0)
    inp = wl.chunk_inputs(w, B=1, H=2, T=T, S0_std=0.1)
    g = inp["gate"].data
    if isinstance(kind, float):
        g[...] = kind
    elif kind == "mixed":
        g[..., 5] = 1e-3
    errs, (out, S_T) = run(w, inp, chunk, 1, 2)
    record("kda-strong-%s-d%d-c%d-%s-T%d" % (dtype, d, chunk, kind, T), errs, dtype)
    assert torch.isfinite(out).all() and torch.isfinite(S_T).all()
    assert max(errs.values()) <= TOL[dtype], errs


def test_kda_workload_shape():
    """The delta-rule workload's shape (B=4, H=16, T=8192, d=128, bf16, chunk 64)
    with per-channel gates sigmoid(N(4, 1)), every head against the oracle."""
    w = wl.Workload("kda_bf16_b4h16t8192d128", la.LA_KDA, "bf16", 4, 16, 8192, 128, 128, 64, 128 ** -0.5,
                    gate_mean=4.0, seed=6)
    inp = wl.chunk_inputs(w)
    print("kda workload", w.name, flush=True)
    errs, _ = run(w, inp, 64, 4, 16)
    record("workload-kda_bf16_b4h16t8192d128", errs, "bf16")
    assert max(errs.values()) <= TOL["bf16"], errs


def test_kda_shared_channel_gates_match_scalar_rule():
    """alpha_t = g_t in every channel: the per-channel path and the scalar-gate
    delta-rule kernel compute the same recurrence."""
    w = wl.variant_workload(la.LA_GATED_DELTA, "f32", 64, 64, seed=163)
    inp = wl.chunk_inputs(w, B=2, H=2, T=300, S0_std=0.1)
    d = {k: dev(v) for k, v in inp.items()}
    a = d["gate"][..., None].expand(-1, -1, -1, 64).contiguous()
    o1, S1, _ = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=la.LA_KDA, gate=a, beta=d["beta"], S0=d["S0"])
    o2, S2, _ = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=la.LA_GATED_DELTA, gate=d["gate"], beta=d["beta"],
                                S0=d["S0"])
    assert parity_error(host64(o1), host64(o2)) <= 1e-4 and parity_error(host64(S1), host64(S2)) <= 1e-4


def test_kda_chunk_size_independence_and_split():
    w = _w("f32", 64, 64, seed=167)
    T, T1 = 300, 131
    inp = wl.chunk_inputs(w, B=1, H=3, T=T, S0_std=0.1)
    d = {k: dev(v) for k, v in inp.items()}
    kw = dict(variant=la.LA_KDA)
    res = [la.la_chunk_fwd(d["q"], d["k"], d["v"], gate=d["gate"], beta=d["beta"], S0=d["S0"], chunk=c, **kw)
           for c in (16, 32, 64, 128)]
    for o, S, _ in res[1:]:
        assert parity_error(host64(o), host64(res[0][0])) <= 1e-4
        assert parity_error(host64(S), host64(res[0][1])) <= 1e-4
    c = lambda t, s: t[:, :, s].contiguous()  # noqa: E731
    a, b = slice(0, T1), slice(T1, T)
    o1, S1, _ = la.la_chunk_fwd(c(d["q"], a), c(d["k"], a), c(d["v"], a), gate=c(d["gate"], a), beta=c(d["beta"], a),
                                S0=d["S0"], **kw)
    o2, S2, _ = la.la_chunk_fwd(c(d["q"], b), c(d["k"], b), c(d["v"], b), gate=c(d["gate"], b), beta=c(d["beta"], b),
                                S0=S1, **kw)
    assert parity_error(host64(torch.cat([o1, o2], dim=2)), host64(res[2][0])) <= 1e-4
    assert parity_error(host64(S2), host64(res[2][1])) <= 1e-4
    # in place, and T = 0
    S = d["S0"].clone()
    la.la_chunk_fwd(d["q"], d["k"], d["v"], gate=d["gate"], beta=d["beta"], S0=S, S_T=S, **kw)
    assert torch.equal(S, res[2][1])
    e = lambda t: t[:, :, :0].contiguous()  # noqa: E731
    o0, S00, _ = la.la_chunk_fwd(e(d["q"]), e(d["k"]), e(d["v"]), gate=e(d["gate"]), beta=e(d["beta"]), S0=d["S0"], **kw)
    assert o0.numel() == 0 and torch.equal(S00, d["S0"])


def test_kda_decode_chain_equals_chunked():
    w = _w("f32", 64, 32, seed=173)
    T = 40
    inp = wl.chunk_inputs(w, B=2, H=3, T=T, S0_std=0.1)
    d = {k: dev(v) for k, v in inp.items()}
    out, S_T, _ = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=la.LA_KDA, gate=d["gate"], beta=d["beta"],
                                  S0=d["S0"])
    S = d["S0"].clone()
    for t in range(T):
        o = la.la_decode_step(d["q"][:, :, t].contiguous(), d["k"][:, :, t].contiguous(), d["v"][:, :, t].contiguous(),
                              S, variant=la.LA_KDA, gate=d["gate"][:, :, t].contiguous(),
                              beta=d["beta"][:, :, t].contiguous())
        assert parity_error(host64(o), host64(out[:, :, t])) <= 1e-4
    assert parity_error(host64(S), host64(S_T)) <= 1e-4


DEC = [(dt, dk, dv) for dt in ("f32", "bf16") for (dk, dv) in ((16, 16), (128, 128), (64, 32), (32, 64))]


@pytest.mark.parametrize("dtype,dk,dv", DEC, ids=["-".join(map(str, c)) for c in DEC])
def test_kda_decode_matches_oracle(dtype, dk, dv):
    w = wl.Workload("kda_decode", la.LA_KDA, dtype, 2, 5, 6, dk, dv, 0, dk ** -0.5, gate_mean=3.0, S0_std=0.1,
                    decode=True, seed=179)
    B, H = 2, 5
    S = dev(wl.decode_state(w, B=B, H=H))
    S_ref = np.ascontiguousarray(host64(S))
    worst = 0.0
    for s in range(w.T):
        inp = wl.decode_step_inputs(w, s, B=B, H=H)
        o = la.la_decode_step(dev(inp["q"]), dev(inp["k"]), dev(inp["v"]), S, variant=la.LA_KDA, gate=dev(inp["gate"]),
                              beta=dev(inp["beta"]))
        o_ref = oracle.decode_step(la.LA_KDA, S_ref, inp["q"].f64(), inp["k"].f64(), inp["v"].f64(),
                                   gate=inp["gate"].f64(), beta=inp["beta"].f64())
        worst = max(worst, parity_error(host64(o), o_ref))
    errs = {"o": worst, "S": parity_error(host64(S), S_ref)}
    record("decode-kda-%s-dk%d-dv%d" % (dtype, dk, dv), errs, dtype)
    assert max(errs.values()) <= TOL[dtype], errs


def test_kda_verify_commit():
    w = _w("bf16", 128, 128, seed=181)
    B, H, T = 3, 2, 5
    inp = wl.chunk_inputs(w, B=B, H=H, T=T, S0_std=0.1)
    d = {k: dev(v) for k, v in inp.items()}
    S = d["S0"].clone()
    out = la.la_verify(d["q"], d["k"], d["v"], S, variant=la.LA_KDA, gate=d["gate"], beta=d["beta"])
    assert torch.equal(S, d["S0"])
    f = {n: inp[n].f64() for n in inp}
    ro, _, _ = oracle.forward(la.LA_KDA, f["q"], f["k"], f["v"], gate=f["gate"], beta=f["beta"], S0=f["S0"])
    e_out = parity_error(host64(out), ro)
    acc = np.array([0, T, 2], np.int32)
    la.la_commit(d["k"], d["v"], S, torch.as_tensor(acc, device="cuda"), variant=la.LA_KDA, gate=d["gate"],
                 beta=d["beta"])
    e_S = 0.0
    for b in range(B):
        n = int(acc[b])
        cut = lambda a: a[b:b + 1, :, :n]  # noqa: E731
        _, rS, _ = oracle.forward(la.LA_KDA, cut(f["q"]), cut(f["k"]), cut(f["v"]), gate=cut(f["gate"]),
                                  beta=cut(f["beta"]), S0=f["S0"][b:b + 1])
        e_S = max(e_S, parity_error(host64(S[b:b + 1]), rS))
    record("verify-kda-bf16-d128-T5", {"out": e_out, "S": e_S}, "bf16")
    assert e_out <= TOL["bf16"] and e_S <= TOL["bf16"], (e_out, e_S)
