"""la_chunk_fwd_noalloc against la_chunk_fwd, through the C ABI (GPU).

The allocation-free entry point runs the same kernels with the library's own
device scratch array in place of the caller's workspace, so its results must
equal la_chunk_fwd's bit for bit.  Two calls in a row share the array, the
second on a smaller input, and the first call on each device resolves the
array's address; the normalized variant is the one whose kernels use the
scratch (segment slots, or a staged z0 when z_T is z0).
"""
import pytest
import torch

import gated_delta_rule_causal_amd as la
import workloads as wl
from gpu_util import dev

pytestmark = pytest.mark.gpu


def _inputs(dtype, B, H, T, d, seed, z0=True):
    w = wl.variant_workload(la.LA_NORMALIZED, dtype, d, d, chunk=64, phi=la.LA_PHI_ELU1, seed=seed)
    return {k: dev(v) for k, v in wl.chunk_inputs(w, B=B, H=H, T=T, S0_std=0.1, z0=z0).items()}


def _both(d, chunk=64, in_place=False):
    ref = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=la.LA_NORMALIZED, S0=d["S0"], z0=d["z0"], chunk=chunk)
    B, H, T, dk = d["q"].shape
    dv = d["v"].shape[-1]
    out = torch.empty((B, H, T, dv), dtype=d["q"].dtype, device="cuda")
    if in_place:
        S, z = d["S0"].clone(), d["z0"].clone()
        la.la_chunk_fwd_noalloc(d["q"], d["k"], d["v"], variant=la.LA_NORMALIZED, out=out, S0=S, z0=z,
                                S_T=S, z_T=z, chunk=chunk)
    else:
        S = torch.empty((B, H, dv, dk), dtype=torch.float32, device="cuda")
        z = torch.empty((B, H, dk), dtype=torch.float32, device="cuda")
        la.la_chunk_fwd_noalloc(d["q"], d["k"], d["v"], variant=la.LA_NORMALIZED, out=out, S0=d["S0"],
                                z0=d["z0"], S_T=S, z_T=z, chunk=chunk)
    torch.cuda.synchronize()
    return ref, (out, S, z)


def _equal(ref, got):
    for r, g in zip(ref, got):
        assert torch.equal(r, g)


def test_noalloc_matches_workspace_entry_point_twice():
    # 32 heads x 2048 tokens: eight concurrent segments, 4.3 MB of scratch
    big = _inputs("bf16", 4, 8, 2048, 64, seed=91)
    assert la.la_chunk_fwd_workspace(la.make_desc(la.LA_NORMALIZED, la.LA_BF16, 4, 8, 2048, 64, 64, 64)) > 0
    _equal(*_both(big))
    # then a smaller call on the same array: 2 heads x 300 tokens (segments too)
    small = _inputs("bf16", 1, 2, 300, 64, seed=92)
    _equal(*_both(small))


def test_noalloc_in_place_one_pass_uses_staged_z0():
    # one pass, four 16-channel value blocks per head, z_T == z0: z0 is staged
    # in the scratch array
    d = _inputs("f32", 1, 2, 40, 64, seed=93)
    ref, got = _both(d, chunk=16, in_place=True)
    _equal(ref, got)


def test_noalloc_without_scratch_use():
    # the delta rule needs no scratch: the entry point runs it all the same
    w = wl.variant_workload(la.LA_GATED_DELTA, "bf16", 128, 128, seed=94)
    d = {k: dev(v) for k, v in wl.chunk_inputs(w, B=1, H=4, T=300, S0_std=0.1).items()}
    ref = la.la_chunk_fwd(d["q"], d["k"], d["v"], variant=w.variant, gate=d["gate"], beta=d["beta"], S0=d["S0"])
    out = torch.empty_like(ref[0])
    S = torch.empty_like(ref[1])
    la.la_chunk_fwd_noalloc(d["q"], d["k"], d["v"], variant=w.variant, out=out, gate=d["gate"], beta=d["beta"],
                            S0=d["S0"], S_T=S)
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(S, ref[1])
