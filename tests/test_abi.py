"""The C ABI on the host: exported symbols and synchronous argument checks.

Every call here fails validation, which happens before any HIP call, so these
tests run without a GPU.  Pointers are fake device addresses that validation
only compares and never dereferences.
"""
import ctypes
import os
import re

import pytest

import gated_delta_rule_causal_amd as la
from gated_delta_rule_causal_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "la.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from gated_delta_rule_causal_amd import build
        build.build()
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(la_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == sorted(_lib.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_abi_version_and_status_strings(lib):
    assert la.la_abi_version() == _lib.LA_ABI_VERSION
    for s in (la.LA_OK, la.LA_EINVAL, la.LA_EUNSUPPORTED, la.LA_EHIP):
        assert la.la_status_str(s).startswith("LA_")
    assert "unknown" in la.la_status_str(99)


BASE = 1 << 32          # fake, 256-byte aligned device addresses
STEP = 1 << 28


def fake(i, off=0):
    return ctypes.c_void_p(BASE + i * STEP + off)


def call_chunk(lib, desc, **kw):
    args = dict(q=fake(0), k=fake(1), v=fake(2), gate=None, beta=None, S0=None, z0=None,
                out=fake(3), S_T=fake(4), z_T=None, ws=None, ws_bytes=0)
    if desc is not None and desc.variant == la.LA_GATED:
        args["gate"] = fake(5)
    if desc is not None and desc.variant == la.LA_GATED_DELTA:
        args["gate"], args["beta"] = fake(5), fake(6)
    args.update(kw)
    d = ctypes.byref(desc) if desc is not None else None
    return lib.la_chunk_fwd(d, args["q"], args["k"], args["v"], args["gate"], args["beta"],
                            args["S0"], args["z0"], args["out"], args["S_T"], args["z_T"],
                            args["ws"], args["ws_bytes"], None)


def call_decode(lib, desc, **kw):
    args = dict(q=fake(0), k=fake(1), v=fake(2), gate=None, beta=None, S=fake(4), z=None,
                out=fake(3))
    if desc.variant == la.LA_NORMALIZED:
        args["z"] = fake(7)
    if desc.variant == la.LA_GATED:
        args["gate"] = fake(5)
    if desc.variant == la.LA_GATED_DELTA:
        args["gate"], args["beta"] = fake(5), fake(6)
    args.update(kw)
    return lib.la_decode_step(ctypes.byref(desc), args["q"], args["k"], args["v"], args["gate"],
                              args["beta"], args["S"], args["z"], args["out"], None)


def D(variant=la.LA_GATED_DELTA, **kw):
    p = dict(dtype=la.LA_BF16, B=2, H=3, T=100, d_k=64, d_v=64, chunk=0, phi=None)
    p.update(kw)
    return la.make_desc(variant, p["dtype"], p["B"], p["H"], p["T"], p["d_k"], p["d_v"],
                        p["chunk"], p["phi"])


CHUNK_CASES = [
    ("null_desc", None, {}, la.LA_EINVAL, "desc"),
    ("bad_variant", D(variant=7), {}, la.LA_EINVAL, "variant"),
    ("bad_dtype", D(dtype=5), {}, la.LA_EINVAL, "dtype"),
    ("bad_phi", D(phi=3), {}, la.LA_EINVAL, "phi"),
    ("normalized_needs_elu1", D(la.LA_NORMALIZED, phi=la.LA_PHI_IDENTITY), {}, la.LA_EINVAL, "LA_PHI_ELU1"),
    ("delta_needs_identity", D(phi=la.LA_PHI_ELU1), {}, la.LA_EINVAL, "LA_PHI_IDENTITY"),
    ("negative_B", D(B=-1), {}, la.LA_EINVAL, "B="),
    ("negative_T", D(T=-5), {}, la.LA_EINVAL, "T="),
    ("zero_dk", D(d_k=0), {}, la.LA_EINVAL, "d_k"),
    ("unsupported_dk", D(d_k=48), {}, la.LA_EUNSUPPORTED, "head sizes"),
    ("unsupported_dv", D(d_v=256), {}, la.LA_EUNSUPPORTED, "head sizes"),
    ("unsupported_chunk", D(chunk=256), {}, la.LA_EUNSUPPORTED, "chunk"),
    ("unsupported_chunk_48", D(chunk=48), {}, la.LA_EUNSUPPORTED, "chunk"),
    ("negative_chunk", D(chunk=-16), {}, la.LA_EINVAL, "chunk"),
    ("missing_q", D(), {"q": None}, la.LA_EINVAL, "required"),
    ("missing_out", D(), {"out": None}, la.LA_EINVAL, "required"),
    ("missing_gate", D(), {"gate": None}, la.LA_EINVAL, "gate"),
    ("missing_beta", D(), {"beta": None}, la.LA_EINVAL, "beta"),
    ("beta_on_normalized", D(la.LA_NORMALIZED), {"beta": fake(6)}, la.LA_EINVAL, "beta"),
    ("beta_on_retention", D(la.LA_RETENTION), {"beta": fake(6)}, la.LA_EINVAL, "beta"),
    ("z0_on_retention", D(la.LA_RETENTION), {"z0": fake(7)}, la.LA_EINVAL, "z"),
    ("misaligned_head_gate", D(la.LA_NORMALIZED), {"gate": fake(5, 2)}, la.LA_EINVAL, "aligned"),
    ("head_gate_overlaps_out", D(la.LA_RETENTION), {"gate": fake(3, 64), "ws": fake(9), "ws_bytes": 1 << 24},
     la.LA_EINVAL, "overlaps"),
    ("bad_variant_5", D(variant=5), {}, la.LA_EINVAL, "variant"),
    ("beta_on_gated", D(la.LA_GATED), {"beta": fake(6)}, la.LA_EINVAL, "beta"),
    ("z0_on_delta", D(), {"z0": fake(7)}, la.LA_EINVAL, "z"),
    ("z_T_on_gated", D(la.LA_GATED), {"z_T": fake(7)}, la.LA_EINVAL, "z"),
    ("misaligned_q", D(), {"q": fake(0, 8)}, la.LA_EINVAL, "aligned"),
    ("misaligned_S0", D(), {"S0": fake(8, 4)}, la.LA_EINVAL, "aligned"),
    ("misaligned_beta", D(), {"beta": fake(6, 2)}, la.LA_EINVAL, "aligned"),
    ("out_overlaps_q", D(), {"out": fake(0, 256)}, la.LA_EINVAL, "overlaps"),
    ("out_overlaps_v", D(), {"out": fake(2)}, la.LA_EINVAL, "overlaps"),
    ("state_partially_overlaps_S0", D(), {"S0": fake(8), "S_T": fake(8, 1024)}, la.LA_EINVAL, "overlaps"),
    ("state_overlaps_out", D(), {"S_T": fake(3, 512)}, la.LA_EINVAL, "overlaps"),
]


@pytest.mark.parametrize("name,desc,kw,status,msg", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_chunk_fwd_rejects(lib, name, desc, kw, status, msg):
    assert call_chunk(lib, desc, **kw) == status
    assert msg in la.la_last_error()


DECODE_CASES = [
    ("normalized_needs_z", D(la.LA_NORMALIZED), {"z": None}, la.LA_EINVAL, "z is required"),
    ("missing_state", D(), {"S": None}, la.LA_EINVAL, "required"),
    ("state_overlaps_k", D(), {"S": fake(1, 64)}, la.LA_EINVAL, "overlaps"),
    ("out_overlaps_state", D(), {"out": fake(4, 128)}, la.LA_EINVAL, "overlaps"),
    ("z_on_gated", D(la.LA_GATED), {"z": fake(7)}, la.LA_EINVAL, "z"),
    ("unsupported_dk", D(d_k=8), {}, la.LA_EUNSUPPORTED, "head sizes"),
    ("z_on_retention", D(la.LA_RETENTION), {"z": fake(7)}, la.LA_EINVAL, "z"),
    ("misaligned_head_gate", D(la.LA_RETENTION), {"gate": fake(5, 1)}, la.LA_EINVAL, "aligned"),
]


@pytest.mark.parametrize("name,desc,kw,status,msg", DECODE_CASES, ids=[c[0] for c in DECODE_CASES])
def test_decode_step_rejects(lib, name, desc, kw, status, msg):
    assert call_decode(lib, desc, **kw) == status
    assert msg in la.la_last_error()


def test_workspace_query_of_invalid_desc_is_zero(lib):
    assert la.la_chunk_fwd_workspace(D(d_k=48)) == 0


def test_workspace_sizes(lib):
    # Only the normalized and retention variants use a workspace, slots of
    # d_v*d_k + d_k floats.  With d_k, d_v in {64, 128} and fewer heads than
    # compute units, the segment path: n_seg + 1 slots per head (slot 0 the
    # initial state), segments of up to 256 tokens (bf16, d = 64; 128 for
    # d = 128) halved while one workgroup per compute unit remains.  Other
    # few-head shapes: the chained path's slots, one per head and segment (the
    # count bounded by 256 / workgroups and by the 16-token chunks over two);
    # otherwise a staged copy of z0, d_k floats per head.
    slot = lambda dk, dv: (dv * dk + dk) * 4  # noqa: E731
    assert la.la_chunk_fwd_workspace(D(la.LA_NORMALIZED, B=4, H=8, T=2048)) == 32 * 9 * slot(64, 64)
    assert la.la_chunk_fwd_workspace(D(la.LA_NORMALIZED, B=1, H=1, T=100, d_k=16, d_v=16)) == 3 * slot(16, 16)
    assert la.la_chunk_fwd_workspace(D(la.LA_NORMALIZED, B=16, H=16, T=2048)) == 256 * 64 * 4   # 256 heads
    assert la.la_chunk_fwd_workspace(D(la.LA_NORMALIZED, T=0)) == 0
    assert la.la_chunk_fwd_workspace(D(la.LA_NORMALIZED, T=31)) == 6 * 2 * slot(64, 64)   # one 64-token segment
    assert la.la_chunk_fwd_workspace(D(la.LA_NORMALIZED, T=31, d_k=32, d_v=32)) == 6 * 32 * 4   # one pass
    # d = 128: 64-token segments, at most three per head (four slots a workgroup)
    assert la.la_chunk_fwd_workspace(D(la.LA_NORMALIZED, T=100, d_k=128, d_v=128)) == 6 * 3 * slot(128, 128)
    assert la.la_chunk_fwd_workspace(D(la.LA_GATED, T=2048)) == 0
    assert la.la_chunk_fwd_workspace(D(la.LA_GATED_DELTA, T=2048)) == 0
    # retention: the same slots, no z0 staging
    assert la.la_chunk_fwd_workspace(D(la.LA_RETENTION, B=4, H=8, T=2048)) == 32 * 9 * slot(64, 64)
    assert la.la_chunk_fwd_workspace(D(la.LA_RETENTION, B=16, H=16, T=2048)) == 0


def test_missing_workspace_is_rejected(lib):
    d = D(la.LA_NORMALIZED, B=1, H=1, T=4096)
    need = la.la_chunk_fwd_workspace(d)
    assert need > 0
    assert call_chunk(lib, d) == la.LA_EINVAL
    assert "workspace" in la.la_last_error()
    assert call_chunk(lib, d, ws=fake(8), ws_bytes=need - 1) == la.LA_EINVAL
    # overlapping an input is rejected too
    assert call_chunk(lib, d, ws=fake(0), ws_bytes=need) == la.LA_EINVAL
    assert "overlaps" in la.la_last_error()


def test_empty_problem_is_a_no_op(lib):
    # B*H == 0: valid and nothing to launch, so no HIP call happens
    assert call_chunk(lib, D(B=0), q=None, k=None, v=None, out=None, S_T=None,
                      gate=None, beta=None) == la.LA_OK
    assert call_decode(lib, D(H=0), q=None, k=None, v=None, out=None, S=None,
                       gate=None, beta=None) == la.LA_OK


def test_binding_rejects_host_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError, match="GPU memory"):
        la.la_chunk_fwd(x, x, x, variant=la.LA_NORMALIZED)
    with pytest.raises(ValueError, match="GPU memory"):
        la.la_decode_step(x[:, :, 0], x[:, :, 0], x[:, :, 0], torch.zeros(1, 1, 16, 16),
                          variant=la.LA_NORMALIZED, z=torch.zeros(1, 1, 16))


# The C library cannot see tensor sizes, so the binding checks every tensor's
# shape, dtype and device before any call; these checks run before the
# device check, so host tensors exercise them here.
def _chunk_args(variant, dtype="float32", B=2, H=3, T=10, dk=16, dv=8):
    import torch
    dt = getattr(torch, dtype)
    a = dict(q=torch.zeros(B, H, T, dk, dtype=dt), k=torch.zeros(B, H, T, dk, dtype=dt),
             v=torch.zeros(B, H, T, dv, dtype=dt))
    if variant == la.LA_GATED:
        a["gate"] = torch.ones(B, H, T, dk)
    if variant == la.LA_GATED_DELTA:
        a["gate"], a["beta"] = torch.ones(B, H, T), torch.ones(B, H, T)
    return a


CHUNK_BINDING_CASES = [
    ("k_shape", la.LA_GATED_DELTA, {"k": (2, 3, 10, 32)}, "k: shape"),
    ("v_rows", la.LA_GATED_DELTA, {"v": (2, 3, 9, 8)}, "v: shape"),
    ("k_dtype", la.LA_GATED_DELTA, {"k": "bfloat16"}, "k: dtype"),
    ("gate_shape", la.LA_GATED, {"gate": (2, 3, 10)}, "gate: shape"),
    ("gate_dtype", la.LA_GATED_DELTA, {"gate": "bfloat16"}, "gate: dtype"),
    ("beta_shape", la.LA_GATED_DELTA, {"beta": (2, 3, 11)}, "beta: shape"),
    ("S0_transposed", la.LA_GATED_DELTA, {"S0": (2, 3, 16, 8)}, "S0: shape"),
    ("S0_bf16", la.LA_GATED_DELTA, {"S0": ((2, 3, 8, 16), "bfloat16")}, "S0: dtype"),
    ("z0_shape", la.LA_NORMALIZED, {"z0": (2, 3, 8)}, "z0: shape"),
    ("out_dtype", la.LA_NORMALIZED, {"out": ((2, 3, 10, 8), "bfloat16")}, "out: dtype"),
    ("S_T_shape", la.LA_GATED, {"S_T": (2, 3, 8, 8)}, "S_T: shape"),
    ("z_T_shape", la.LA_NORMALIZED, {"z_T": (3, 16)}, "z_T: shape"),
]


@pytest.mark.parametrize("name,variant,bad,msg", CHUNK_BINDING_CASES, ids=[c[0] for c in CHUNK_BINDING_CASES])
def test_binding_rejects_mismatched_chunk_args(name, variant, bad, msg):
    import torch
    a = _chunk_args(variant)
    for key, spec in bad.items():
        if isinstance(spec, str):
            a[key] = a[key].to(getattr(torch, spec))
        else:
            shape, dt = spec if isinstance(spec[1], str) else (spec, "float32")
            a[key] = torch.zeros(shape, dtype=getattr(torch, dt))
    q, k, v = a.pop("q"), a.pop("k"), a.pop("v")
    with pytest.raises(ValueError, match=msg):
        la.la_chunk_fwd(q, k, v, variant=variant, **a)


def test_binding_rejects_mismatched_decode_args():
    import torch
    q = k = torch.zeros(2, 3, 16)
    v = torch.zeros(2, 3, 8)
    with pytest.raises(ValueError, match="S: shape"):
        la.la_decode_step(q, k, v, torch.zeros(2, 3, 16, 8), variant=la.LA_GATED_DELTA,
                          gate=torch.ones(2, 3), beta=torch.ones(2, 3))
    with pytest.raises(ValueError, match="S: dtype"):
        la.la_decode_step(q, k, v, torch.zeros(2, 3, 8, 16, dtype=torch.bfloat16), variant=la.LA_GATED_DELTA,
                          gate=torch.ones(2, 3), beta=torch.ones(2, 3))
    with pytest.raises(ValueError, match="gate: shape"):
        la.la_decode_step(q, k, v, torch.zeros(2, 3, 8, 16), variant=la.LA_GATED_DELTA,
                          gate=torch.ones(2, 3, 16), beta=torch.ones(2, 3))
    with pytest.raises(ValueError, match="v: shape"):
        la.la_decode_step(q, k, torch.zeros(2, 4, 8), torch.zeros(2, 3, 8, 16), variant=la.LA_GATED_DELTA,
                          gate=torch.ones(2, 3), beta=torch.ones(2, 3))


def test_noalloc_rejects_requests_beyond_its_scratch(lib):
    # 131072 heads of d_k = 128 in one pass would stage 64 MiB of z0, twice the
    # library's array: rejected before any HIP call
    d = D(la.LA_NORMALIZED, B=1024, H=128, T=64, d_k=128, d_v=128)
    assert la.la_chunk_fwd_workspace(d) > _lib.LA_NOALLOC_SCRATCH_BYTES
    assert lib.la_chunk_fwd_noalloc(ctypes.byref(d), fake(0), fake(1), fake(2), None, None, None, None,
                                    fake(3), None, None, None) == la.LA_EINVAL
    assert "scratch" in la.la_last_error()
    # the argument checks are those of la_chunk_fwd
    d2 = D(la.LA_GATED_DELTA)
    assert lib.la_chunk_fwd_noalloc(ctypes.byref(d2), fake(0), fake(1), fake(2), None, None, None, None,
                                    fake(3), None, None, None) == la.LA_EINVAL
    assert "gate" in la.la_last_error()


def test_noalloc_header_size_matches_binding():
    text = open(HEADER).read()
    m = re.search(r"#define LA_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.LA_NOALLOC_SCRATCH_BYTES


def call_verify(lib, desc, **kw):
    args = dict(q=fake(0), k=fake(1), v=fake(2), gate=fake(5), beta=fake(6), S=fake(4), z=None, out=fake(3))
    args.update(kw)
    return lib.la_verify(ctypes.byref(desc), args["q"], args["k"], args["v"], args["gate"], args["beta"],
                         args["S"], args["z"], args["out"], None)


def call_commit(lib, desc, **kw):
    args = dict(k=fake(1), v=fake(2), gate=fake(5), beta=fake(6), accepted=fake(8), S=fake(4), z=None)
    args.update(kw)
    return lib.la_commit(ctypes.byref(desc), args["k"], args["v"], args["gate"], args["beta"], args["accepted"],
                         args["S"], args["z"], None)


MULTI_CASES = [
    ("verify", "missing_out", D(T=4), {"out": None}, "q and out"),
    ("verify", "missing_q", D(T=4), {"q": None}, "q and out"),
    ("verify", "out_overlaps_state", D(T=4), {"out": fake(4, 256)}, "overlaps"),
    ("verify", "normalized_needs_z", D(la.LA_NORMALIZED, T=4), {"gate": None, "beta": None}, "z is required"),
    ("verify", "negative_T", D(T=-1), {}, "T="),
    ("commit", "missing_accepted", D(T=4), {"accepted": None}, "accepted"),
    ("commit", "misaligned_accepted", D(T=4), {"accepted": fake(8, 2)}, "aligned"),
    ("commit", "state_overlaps_k", D(T=4), {"S": fake(1, 64)}, "overlaps"),
    ("commit", "accepted_overlaps_state", D(T=4), {"accepted": fake(4, 16)}, "overlaps"),
    ("commit", "missing_beta", D(T=4), {"beta": None}, "beta"),
]


@pytest.mark.parametrize("which,name,desc,kw,msg", MULTI_CASES, ids=[c[0] + "-" + c[1] for c in MULTI_CASES])
def test_verify_commit_reject(lib, which, name, desc, kw, msg):
    call = call_verify if which == "verify" else call_commit
    assert call(lib, desc, **kw) != la.LA_OK
    assert msg in la.la_last_error()


def test_verify_commit_empty_is_a_no_op(lib):
    assert call_verify(lib, D(T=0), q=None, k=None, v=None, out=None, S=None, gate=None, beta=None) == la.LA_OK
    assert call_commit(lib, D(B=0, T=4), k=None, v=None, S=None, gate=None, beta=None, accepted=None) == la.LA_OK


# ------------------------------------------------------- backward (training)

def call_bwd(lib, desc, **kw):
    norm = desc.variant == la.LA_NORMALIZED
    args = dict(q=fake(0), k=fake(1), v=fake(2), gate=fake(5), S0=None, z0=None, dout=fake(7), dS_T=None,
                dz_T=None, dq=fake(10), dk=fake(11), dv=fake(12), dgate=fake(13), dS0=fake(14),
                dz0=fake(15) if norm else None, ws=fake(20), ws_bytes=1 << 30)
    args.update(kw)
    return lib.la_chunk_bwd(ctypes.byref(desc), args["q"], args["k"], args["v"], args["gate"], args["S0"],
                            args["z0"], args["dout"], args["dS_T"], args["dz_T"],
                            args["dq"], args["dk"], args["dv"], args["dgate"], args["dS0"], args["dz0"],
                            args["ws"], args["ws_bytes"], None)


BWD_CASES = [
    ("gated_unsupported", D(la.LA_GATED), {}, la.LA_EUNSUPPORTED, "LA_NORMALIZED and LA_RETENTION"),
    ("delta_unsupported", D(), {}, la.LA_EUNSUPPORTED, "LA_NORMALIZED and LA_RETENTION"),
    ("kda_unsupported", D(la.LA_KDA), {}, la.LA_EUNSUPPORTED, "LA_NORMALIZED and LA_RETENTION"),
    ("z0_on_retention", D(la.LA_RETENTION), {"z0": fake(8)}, la.LA_EINVAL, "must be NULL"),
    ("dz_T_on_retention", D(la.LA_RETENTION), {"dz_T": fake(8)}, la.LA_EINVAL, "must be NULL"),
    ("dz0_on_retention", D(la.LA_RETENTION), {"dz0": fake(15)}, la.LA_EINVAL, "must be NULL"),
    ("misaligned_gate", D(la.LA_NORMALIZED), {"gate": fake(5, 2)}, la.LA_EINVAL, "aligned"),
    ("dS0_overlaps_dS_T", D(la.LA_NORMALIZED), {"dS_T": fake(14, 256)}, la.LA_EINVAL, "overlaps"),
    ("dgate_without_gate", D(la.LA_RETENTION), {"gate": None}, la.LA_EINVAL, "dgate needs gate"),
    ("missing_dout", D(la.LA_RETENTION), {"dout": None}, la.LA_EINVAL, "required"),
    ("missing_dq", D(la.LA_NORMALIZED), {"dq": None}, la.LA_EINVAL, "required"),
    ("small_workspace", D(la.LA_RETENTION), {"ws_bytes": 1024}, la.LA_EINVAL, "workspace"),
    ("missing_workspace", D(la.LA_NORMALIZED), {"ws": None}, la.LA_EINVAL, "workspace"),
    ("misaligned_dq", D(la.LA_NORMALIZED), {"dq": fake(10, 8)}, la.LA_EINVAL, "aligned"),
    ("dq_overlaps_q", D(la.LA_RETENTION), {"dq": fake(0, 512)}, la.LA_EINVAL, "overlaps"),
    ("dv_overlaps_dk", D(la.LA_RETENTION), {"dv": fake(11, 256)}, la.LA_EINVAL, "overlaps"),
    ("dS0_overlaps_workspace", D(la.LA_RETENTION), {"dS0": fake(20, 4096)}, la.LA_EINVAL, "overlaps"),
    ("unsupported_dk", D(la.LA_RETENTION, d_k=24), {}, la.LA_EUNSUPPORTED, "head sizes"),
]


@pytest.mark.parametrize("name,desc,kw,status,msg", BWD_CASES, ids=[c[0] for c in BWD_CASES])
def test_chunk_bwd_rejects(lib, name, desc, kw, status, msg):
    assert call_bwd(lib, desc, **kw) == status
    assert msg in la.la_last_error()


def test_chunk_bwd_empty_is_a_no_op(lib):
    d = D(la.LA_RETENTION, B=0)
    assert call_bwd(lib, d, q=None, k=None, v=None, dout=None, dq=None, dk=None, dv=None, ws=None,
                    ws_bytes=0) == la.LA_OK


def test_chunk_bwd_workspace_sizes(lib):
    # states and cotangents of every chunk, float32, one float per chunk, and
    # (normalized) two floats per token
    def ws(variant, B, H, T, dk, dv, C):
        N = (T + C - 1) // C
        norm = variant == la.LA_NORMALIZED
        E = dk * dv + (dk if norm else 0)
        b = (2 * B * H * N * E + B * H * N + (2 * B * H * T if norm else 0)) * 4
        return (b + 255) // 256 * 256
    for v in (la.LA_NORMALIZED, la.LA_RETENTION):
        assert la.la_chunk_bwd_workspace(D(v, B=4, H=8, T=2048)) == ws(v, 4, 8, 2048, 64, 64, 64)
        assert la.la_chunk_bwd_workspace(D(v, B=1, H=2, T=65, d_k=16, d_v=32)) == ws(v, 1, 2, 65, 16, 32, 64)
        # float32 tiles at head size 128 run 32-token chunks
        assert la.la_chunk_bwd_workspace(D(v, dtype=la.LA_F32, B=1, H=1, T=100, d_k=128, d_v=128)) == \
            ws(v, 1, 1, 100, 128, 128, 32)
        assert la.la_chunk_bwd_workspace(D(v, T=0)) == 0
    assert la.la_chunk_bwd_workspace(D(la.LA_GATED)) == 0


def test_binding_rejects_mismatched_bwd_args():
    q = k = dout = __import__("torch").zeros((2, 3, 10, 16))
    v = __import__("torch").zeros((2, 3, 10, 8))
    with pytest.raises(ValueError, match="gate"):
        la.la_chunk_bwd(q, k, v, __import__("torch").zeros((2, 3, 10, 8)), variant=la.LA_RETENTION,
                        gate=__import__("torch").zeros((2,)))
    with pytest.raises(ValueError, match="dout"):
        la.la_chunk_bwd(q, k, v, dout, variant=la.LA_RETENTION)
    with pytest.raises(ValueError, match="dS_T"):
        la.la_chunk_bwd(q, k, v, __import__("torch").zeros((2, 3, 10, 8)), variant=la.LA_NORMALIZED,
                        dS_T=__import__("torch").zeros((2, 3, 16, 8)))
