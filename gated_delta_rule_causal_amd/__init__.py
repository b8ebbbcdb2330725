"""Causal linear attention for AMD MI355X (gfx950): Python binding of libla.so.

The entry points carry the names of the C ABI in include/la.h and only
marshal arguments: shapes become an ``la_desc``, torch tensors become device
pointers, torch's current HIP stream becomes the stream argument, and missing
outputs are allocated with torch.  Every step of the computation runs in the
library's HIP kernels; there is no other code path.

    out, S_T, z_T = la_chunk_fwd(q, k, v, variant=LA_GATED_DELTA, gate=g, beta=b)
    o = la_decode_step(q, k, v, S, variant=LA_GATED_DELTA, gate=g, beta=b)
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import (LA_BF16, LA_EHIP, LA_EINVAL, LA_EUNSUPPORTED, LA_F32, LA_GATED,  # noqa: F401
                   LA_GATED_DELTA, LA_NORMALIZED, LA_OK, LA_PHI_ELU1, LA_PHI_IDENTITY,
                   LA_RETENTION, LA_KDA, LaDesc, LaError, check, load)

__all__ = ["la_chunk_fwd", "la_chunk_fwd_noalloc", "la_chunk_bwd", "la_chunk_bwd_workspace",
           "la_decode_step", "la_verify", "la_commit", "la_chunk_fwd_workspace", "la_status_str",
           "la_last_error", "la_abi_version", "make_desc", "LaDesc", "LaError",
           "LA_NORMALIZED", "LA_GATED", "LA_GATED_DELTA", "LA_RETENTION", "LA_KDA", "LA_F32", "LA_BF16",
           "LA_PHI_IDENTITY", "LA_PHI_ELU1"]

_DTYPES = {torch.float32: LA_F32, torch.bfloat16: LA_BF16}


def _default_phi(variant: int) -> int:
    return LA_PHI_ELU1 if variant in (LA_NORMALIZED, LA_GATED) else LA_PHI_IDENTITY


def _gate_shape(variant, lead, d_k):
    """Shape of the gate argument: (H,) fixed per-head decay (normalized,
    retention); per token (delta rule); per token and key channel (gated)."""
    if variant in (LA_NORMALIZED, LA_RETENTION):
        return (lead[1],)
    if variant == LA_GATED_DELTA:
        return tuple(lead)
    return tuple(lead) + (d_k,)


def make_desc(variant: int, dtype: int, B: int, H: int, T: int, d_k: int, d_v: int,
              chunk: int = 0, phi: int | None = None) -> LaDesc:
    return LaDesc(variant, dtype, _default_phi(variant) if phi is None else phi,
                  B, H, T, d_k, d_v, chunk)


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _check(name, t, shape, dtype, device):
    """The C library cannot see tensor sizes: every tensor is checked here for
    the exact shape, element type and device include/la.h documents."""
    if t is None:
        return
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s: expected a torch.Tensor or None" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    if t.dtype != dtype:
        raise ValueError("%s: dtype %s, expected %s" % (name, t.dtype, dtype))
    if t.device != device:
        raise ValueError("%s: on %s, expected %s (q's device)" % (name, t.device, device))
    if not t.is_contiguous():
        raise ValueError("%s: must be contiguous" % name)


def _check_qkv(q, k, v, lead):
    """q, k, v: same dtype (float32 or bfloat16) and device, q on the GPU;
    returns (dtype code, d_k, d_v)."""
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError("%s: expected a torch.Tensor" % name)
    if q.dtype not in _DTYPES:
        raise TypeError("q/k/v must be float32 or bfloat16")
    if q.dim() != len(lead) + 1:
        raise ValueError("q: expected %d dimensions, got %d" % (len(lead) + 1, q.dim()))
    d_k = q.shape[-1]
    if v.dim() != q.dim():
        raise ValueError("v: expected %d dimensions, got %d" % (q.dim(), v.dim()))
    d_v = v.shape[-1]
    _check("q", q, tuple(q.shape), q.dtype, q.device)
    _check("k", k, tuple(q.shape), q.dtype, q.device)
    _check("v", v, tuple(q.shape[:-1]) + (d_v,), q.dtype, q.device)
    return _DTYPES[q.dtype], d_k, d_v


def _require_gpu(q):
    # after the shape checks, so that those are testable without a GPU
    if not q.is_cuda:
        raise ValueError("q: tensors must live in GPU memory")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def la_abi_version() -> int:
    return load().la_abi_version()


def la_status_str(status: int) -> str:
    return load().la_status_str(status).decode()


def la_last_error() -> str:
    return load().la_last_error().decode()


def la_chunk_fwd_workspace(desc: LaDesc) -> int:
    return int(load().la_chunk_fwd_workspace(ctypes.byref(desc)))


def _workspace(workspace, ws_bytes, dev):
    """The caller's workspace tensor (checked) or a new one of ws_bytes."""
    ws = workspace
    if ws is not None:
        if not isinstance(ws, torch.Tensor) or ws.device != dev or not ws.is_contiguous():
            raise ValueError("workspace: a contiguous tensor on q's device")
    if ws is None and ws_bytes:
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def la_chunk_fwd(q, k, v, *, variant, gate=None, beta=None, S0=None, z0=None, chunk=0,
                 phi=None, out=None, S_T=None, z_T=None, return_state=True, workspace=None,
                 stream=None):
    """Chunkwise-parallel forward (C: ``la_chunk_fwd``).

    q, k (B,H,T,d_k) and v (B,H,T,d_v) in float32 or bfloat16; gate / beta /
    S0 / z0 float32 as include/la.h describes.  Outputs that are not passed
    are allocated: out in q's dtype; S_T (and z_T for LA_NORMALIZED) float32
    unless return_state is False.  `workspace`: a device tensor of at least
    la_chunk_fwd_workspace() bytes, allocated here when not passed and
    needed.  Returns (out, S_T, z_T).
    """
    lib = load()
    dt, d_k, d_v = _check_qkv(q, k, v, "BHT")
    B, H, T = q.shape[:3]
    dev, f32 = q.device, torch.float32
    _check("gate", gate, _gate_shape(variant, (B, H, T), d_k), f32, dev)
    _check("beta", beta, (B, H, T), f32, dev)
    _check("S0", S0, (B, H, d_v, d_k), f32, dev)
    _check("z0", z0, (B, H, d_k), f32, dev)
    _check("out", out, (B, H, T, d_v), q.dtype, dev)
    _check("S_T", S_T, (B, H, d_v, d_k), f32, dev)
    _check("z_T", z_T, (B, H, d_k), f32, dev)
    _require_gpu(q)
    desc = make_desc(variant, dt, B, H, T, d_k, d_v, chunk, phi)
    if out is None:
        out = torch.empty((B, H, T, d_v), dtype=q.dtype, device=dev)
    if return_state and S_T is None:
        S_T = torch.empty((B, H, d_v, d_k), dtype=f32, device=dev)
    if return_state and variant == LA_NORMALIZED and z_T is None:
        z_T = torch.empty((B, H, d_k), dtype=f32, device=dev)
    ws, ws_given = _workspace(workspace, int(lib.la_chunk_fwd_workspace(ctypes.byref(desc))), dev)
    check(lib.la_chunk_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                           _ptr(S0), _ptr(z0), _ptr(out), _ptr(S_T), _ptr(z_T), _ptr(ws),
                           ws_given, _stream(stream)))
    return out, S_T, z_T


def la_chunk_bwd_workspace(desc: LaDesc) -> int:
    return int(load().la_chunk_bwd_workspace(ctypes.byref(desc)))


def la_chunk_bwd(q, k, v, dout, *, variant, gate=None, S0=None, z0=None, dS_T=None, dz_T=None, phi=None,
                 want_dgate=None, want_dS0=True, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Chunked backward pass of LA_NORMALIZED and LA_RETENTION (C:
    ``la_chunk_bwd``).  q, k, v, gate, S0, z0 as given to the forward; dout
    (B,H,T,d_v) in q's dtype; dS_T / dz_T float32 or None (zero).  Returns (dq, dk, dv, dgate,
    dS0, dz0): dgate (H,) when gate is given (and want_dgate is not False),
    dS0 / dz0 when want_dS0; None otherwise."""
    lib = load()
    dt, d_k, d_v = _check_qkv(q, k, v, "BHT")
    B, H, T = q.shape[:3]
    dev, f32 = q.device, torch.float32
    norm = variant == LA_NORMALIZED
    _check("gate", gate, (H,), f32, dev)
    _check("S0", S0, (B, H, d_v, d_k), f32, dev)
    _check("z0", z0, (B, H, d_k), f32, dev)
    _check("dout", dout, (B, H, T, d_v), q.dtype, dev)
    _check("dS_T", dS_T, (B, H, d_v, d_k), f32, dev)
    _check("dz_T", dz_T, (B, H, d_k), f32, dev)
    _check("dq", dq, (B, H, T, d_k), q.dtype, dev)
    _check("dk", dk, (B, H, T, d_k), q.dtype, dev)
    _check("dv", dv, (B, H, T, d_v), q.dtype, dev)
    if dout is None:
        raise ValueError("dout: required")
    _require_gpu(q)
    desc = make_desc(variant, dt, B, H, T, d_k, d_v, 0, phi)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    dgate = torch.empty((H,), dtype=f32, device=dev) if gate is not None and want_dgate is not False else None
    dS0 = torch.empty((B, H, d_v, d_k), dtype=f32, device=dev) if want_dS0 else None
    dz0 = torch.empty((B, H, d_k), dtype=f32, device=dev) if want_dS0 and norm else None
    ws, ws_given = _workspace(workspace, int(lib.la_chunk_bwd_workspace(ctypes.byref(desc))), dev)
    check(lib.la_chunk_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(S0), _ptr(z0),
                           _ptr(dout), _ptr(dS_T), _ptr(dz_T), _ptr(dq), _ptr(dk), _ptr(dv),
                           _ptr(dgate), _ptr(dS0), _ptr(dz0), _ptr(ws), ws_given, _stream(stream)))
    return dq, dk, dv, dgate, dS0, dz0


def la_chunk_fwd_noalloc(q, k, v, *, variant, out, gate=None, beta=None, S0=None, z0=None, chunk=0,
                         phi=None, S_T=None, z_T=None, stream=None):
    """la_chunk_fwd with the scratch from the library's own device array (C:
    ``la_chunk_fwd_noalloc``), for callers that cannot allocate: nothing is
    allocated here either, so ``out`` (and S_T / z_T when wanted) must be
    passed.  Calls on one GPU share the array and must not overlap in time.
    Returns (out, S_T, z_T)."""
    lib = load()
    dt, d_k, d_v = _check_qkv(q, k, v, "BHT")
    B, H, T = q.shape[:3]
    dev, f32 = q.device, torch.float32
    if out is None:
        raise ValueError("out: required (this entry point allocates nothing)")
    _check("gate", gate, _gate_shape(variant, (B, H, T), d_k), f32, dev)
    _check("beta", beta, (B, H, T), f32, dev)
    _check("S0", S0, (B, H, d_v, d_k), f32, dev)
    _check("z0", z0, (B, H, d_k), f32, dev)
    _check("out", out, (B, H, T, d_v), q.dtype, dev)
    _check("S_T", S_T, (B, H, d_v, d_k), f32, dev)
    _check("z_T", z_T, (B, H, d_k), f32, dev)
    _require_gpu(q)
    desc = make_desc(variant, dt, B, H, T, d_k, d_v, chunk, phi)
    check(lib.la_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta),
                                   _ptr(S0), _ptr(z0), _ptr(out), _ptr(S_T), _ptr(z_T), _stream(stream)))
    return out, S_T, z_T


def la_decode_step(q, k, v, S, *, variant, gate=None, beta=None, z=None, phi=None,
                   out=None, stream=None):
    """One recurrent step, updating S (and z) in place (C: ``la_decode_step``).

    q, k (B,H,d_k), v (B,H,d_v) in float32 or bfloat16; S (B,H,d_v,d_k)
    float32; gate / beta / z as include/la.h describes.  Returns out (B,H,d_v).
    """
    lib = load()
    dt, d_k, d_v = _check_qkv(q, k, v, "BH")
    B, H = q.shape[:2]
    dev, f32 = q.device, torch.float32
    if S is None:
        raise ValueError("S: the state is required")
    _check("gate", gate, _gate_shape(variant, (B, H), d_k), f32, dev)
    _check("beta", beta, (B, H), f32, dev)
    _check("S", S, (B, H, d_v, d_k), f32, dev)
    _check("z", z, (B, H, d_k), f32, dev)
    _check("out", out, (B, H, d_v), q.dtype, dev)
    _require_gpu(q)
    desc = make_desc(variant, dt, B, H, 1, d_k, d_v, 0, phi)
    if out is None:
        out = torch.empty((B, H, d_v), dtype=q.dtype, device=dev)
    check(lib.la_decode_step(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                             _ptr(beta), _ptr(S), _ptr(z), _ptr(out), _stream(stream)))
    return out


def la_verify(q, k, v, S, *, variant, gate=None, beta=None, z=None, phi=None, out=None, stream=None):
    """Outputs of T draft tokens from the checkpoint S (and z), which is left
    untouched (C: ``la_verify``).  q, k (B,H,T,d_k), v (B,H,T,d_v); gate and
    beta per token as in la_chunk_fwd.  Returns out (B,H,T,d_v)."""
    lib = load()
    dt, d_k, d_v = _check_qkv(q, k, v, "BHT")
    B, H, T = q.shape[:3]
    dev, f32 = q.device, torch.float32
    if S is None:
        raise ValueError("S: the checkpoint is required")
    _check("gate", gate, _gate_shape(variant, (B, H, T), d_k), f32, dev)
    _check("beta", beta, (B, H, T), f32, dev)
    _check("S", S, (B, H, d_v, d_k), f32, dev)
    _check("z", z, (B, H, d_k), f32, dev)
    _check("out", out, (B, H, T, d_v), q.dtype, dev)
    _require_gpu(q)
    desc = make_desc(variant, dt, B, H, T, d_k, d_v, 0, phi)
    if out is None:
        out = torch.empty((B, H, T, d_v), dtype=q.dtype, device=dev)
    check(lib.la_verify(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(S),
                        _ptr(z), _ptr(out), _stream(stream)))
    return out


def la_commit(k, v, S, accepted, *, variant, gate=None, beta=None, z=None, phi=None, stream=None):
    """Apply the first accepted[b] of T draft tokens to S (and z) in place
    (C: ``la_commit``).  k (B,H,T,d_k), v (B,H,T,d_v); accepted (B,) int32 on
    the device."""
    lib = load()
    dt, d_k, d_v = _check_qkv(k, k, v, "BHT")
    B, H, T = k.shape[:3]
    dev, f32 = k.device, torch.float32
    _check("gate", gate, _gate_shape(variant, (B, H, T), d_k), f32, dev)
    _check("beta", beta, (B, H, T), f32, dev)
    _check("S", S, (B, H, d_v, d_k), f32, dev)
    _check("z", z, (B, H, d_k), f32, dev)
    _check("accepted", accepted, (B,), torch.int32, dev)
    _require_gpu(k)
    desc = make_desc(variant, dt, B, H, T, d_k, d_v, 0, phi)
    check(lib.la_commit(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(gate), _ptr(beta), _ptr(accepted), _ptr(S),
                        _ptr(z), _stream(stream)))
