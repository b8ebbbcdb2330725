"""float64 CPU oracle for causal linear attention -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its binding) never touches it, and it shares no code with that path.

Two independent implementations live here:

* ``oracle.c`` (loaded through ctypes): the token-by-token recurrences of the
  three variants, in double precision, OpenMP over heads.  This is the
  oracle the GPU path is compared against.
* ``parallel_forms.py`` (numpy): the explicit T x T masked-parallel forms the
  pages state alongside the recurrences.  They exist only to pin the
  recurrence (``tests/test_oracle_pins.py``).

Variant codes: 0 normalized linear attention (optionally with a fixed
per-head decay), 1 gated linear attention, 2 gated delta rule, 3 retention
(fixed per-head decay, no normalizer), 4 gated delta rule with a per-channel
decay.  phi codes: 0 identity, 1 elu(x)+1.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

NORMALIZED, GATED, GATED_DELTA, RETENTION, KDA = 0, 1, 2, 3, 4
PHI_IDENTITY, PHI_ELU1 = 0, 1


def default_phi(variant: int) -> int:
    return PHI_ELU1 if variant in (NORMALIZED, GATED) else PHI_IDENTITY


def build(force: bool = False, src: str = _SRC, out: str = _LIB_PATH) -> str:
    """Compile an oracle C source into a shared library (plain gcc, IEEE
    double, no fused multiply-add contraction, OpenMP)."""
    if force or not os.path.exists(out):
        tmp = out + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
               "-ffp-contract=off", "-fno-fast-math", src, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, out)
    return out


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _check_gate(variant, gate, beta, lead, dk):
    """Shapes of gate / beta per variant (lead: (B, H, T) or (B, H))."""
    if variant in (GATED, KDA):
        assert gate is not None and gate.shape == lead + (dk,)
    elif variant == GATED_DELTA:
        assert gate is not None and gate.shape == lead
    else:
        assert gate is None or gate.shape == (lead[1],)
    if variant in (GATED_DELTA, KDA):
        assert beta is not None and beta.shape == lead
    else:
        assert beta is None


class OracleLib:
    """ctypes view of one compiled oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        i = ctypes.c_int
        lib.oracle_forward.argtypes = [i, i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, i]
        lib.oracle_forward.restype = i
        lib.oracle_decode_step.argtypes = [i, i, i, i, i, i, dp, dp, dp, dp, dp, dp, dp, dp, i]
        lib.oracle_decode_step.restype = i
        lib.oracle_backward.argtypes = [i, i, i, i, i, i, i] + [dp] * 15
        lib.oracle_backward.restype = i
        lib.oracle_phi.argtypes = [i, ctypes.c_double]
        lib.oracle_phi.restype = ctypes.c_double
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = i
        self._lib = lib
        self.path = path

    def num_threads(self) -> int:
        return int(self._lib.oracle_num_threads())

    def phi(self, x: float, kind: int = PHI_ELU1) -> float:
        return float(self._lib.oracle_phi(kind, float(x)))

    def forward(self, variant, q, k, v, gate=None, beta=None, S0=None, z0=None,
                phi_kind=None, nthreads=0):
        """Token-by-token forward over whole sequences.

        q, k: (B,H,T,d_k); v: (B,H,T,d_v); gate: (B,H,T,d_k) for GATED
        and KDA, (B,H,T) for GATED_DELTA, (H,) or None for NORMALIZED and
        RETENTION (a fixed per-head decay); beta: (B,H,T) for GATED_DELTA
        and KDA; S0: (B,H,d_v,d_k); z0: (B,H,d_k) (NORMALIZED only).  Returns
        (out, S_T, z_T) as float64; z_T is None unless NORMALIZED.
        """
        if phi_kind is None:
            phi_kind = default_phi(variant)
        q, k, v = _f64(q), _f64(k), _f64(v)
        gate, beta, S0, z0 = _f64(gate), _f64(beta), _f64(S0), _f64(z0)
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        assert k.shape == (B, H, T, dk) and v.shape == (B, H, T, dv)
        _check_gate(variant, gate, beta, (B, H, T), dk)
        if S0 is not None:
            assert S0.shape == (B, H, dv, dk)
        if z0 is not None:
            assert variant == NORMALIZED and z0.shape == (B, H, dk)
        out = np.empty((B, H, T, dv), np.float64)
        S_T = np.empty((B, H, dv, dk), np.float64)
        z_T = np.empty((B, H, dk), np.float64) if variant == NORMALIZED else None
        rc = self._lib.oracle_forward(variant, phi_kind, B, H, T, dk, dv, _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(gate), _ptr(beta), _ptr(S0), _ptr(z0),
                                      _ptr(out), _ptr(S_T), _ptr(z_T), int(nthreads))
        if rc != 0:
            raise RuntimeError("oracle_forward failed with code %d" % rc)
        return out, S_T, z_T

    def backward(self, variant, q, k, v, dout, gate=None, S0=None, z0=None, dS_T=None, dz_T=None,
                 phi_kind=None):
        """Gradients of forward() for NORMALIZED and RETENTION (reverse-mode
        through the token recurrence).  Returns a dict with dq, dk, dv, dS0,
        dz0 (NORMALIZED) and dgate ((H,), summed over the batch; None without
        a gate)."""
        if phi_kind is None:
            phi_kind = default_phi(variant)
        assert variant in (NORMALIZED, RETENTION)
        q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
        gate, S0, z0, dS_T, dz_T = _f64(gate), _f64(S0), _f64(z0), _f64(dS_T), _f64(dz_T)
        B, H, T, dk = q.shape
        dv = v.shape[-1]
        assert dout.shape == (B, H, T, dv)
        assert gate is None or gate.shape == (H,)
        res = {"dq": np.empty((B, H, T, dk)), "dk": np.empty((B, H, T, dk)), "dv": np.empty((B, H, T, dv)),
               "dS0": np.empty((B, H, dv, dk)), "dz0": np.empty((B, H, dk)) if variant == NORMALIZED else None,
               "dgate": np.empty(H) if gate is not None else None}
        rc = self._lib.oracle_backward(variant, phi_kind, B, H, T, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(gate),
                                       _ptr(S0), _ptr(z0), _ptr(dout), _ptr(dS_T), _ptr(dz_T), _ptr(res["dq"]),
                                       _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dgate"]), _ptr(res["dS0"]),
                                       _ptr(res["dz0"]))
        if rc != 0:
            raise RuntimeError("oracle_backward failed with code %d" % rc)
        return res

    def decode_step(self, variant, S, q, k, v, gate=None, beta=None, z=None,
                    phi_kind=None, nthreads=0):
        """One recurrent step for every head, updating S (and z) IN PLACE.

        S: (B,H,d_v,d_k) float64 C-contiguous (modified); q, k: (B,H,d_k);
        v: (B,H,d_v); gate: (B,H,d_k) GATED and KDA / (B,H) GATED_DELTA /
        (H,) or None NORMALIZED and RETENTION; beta: (B,H); z: (B,H,d_k)
        float64 (NORMALIZED, modified).  Returns out (B,H,d_v).
        """
        if phi_kind is None:
            phi_kind = default_phi(variant)
        assert S.dtype == np.float64 and S.flags.c_contiguous
        if variant == NORMALIZED:
            assert z is not None and z.dtype == np.float64 and z.flags.c_contiguous
        q, k, v, gate, beta = _f64(q), _f64(k), _f64(v), _f64(gate), _f64(beta)
        B, H, dv, dk = S.shape
        assert q.shape == (B, H, dk) and k.shape == (B, H, dk) and v.shape == (B, H, dv)
        _check_gate(variant, gate, beta, (B, H), dk)
        out = np.empty((B, H, dv), np.float64)
        rc = self._lib.oracle_decode_step(variant, phi_kind, B, H, dk, dv, _ptr(q), _ptr(k),
                                          _ptr(v), _ptr(gate), _ptr(beta), _ptr(S),
                                          _ptr(z) if variant == NORMALIZED else None,
                                          _ptr(out), int(nthreads))
        if rc != 0:
            raise RuntimeError("oracle_decode_step failed with code %d" % rc)
        return out


_default = None


def load(path: str | None = None) -> OracleLib:
    """The oracle library at ``path`` (default: the built liboracle.so)."""
    global _default
    if path is not None:
        return OracleLib(path)
    if _default is None:
        _default = OracleLib(build(force=False))
    return _default


def num_threads() -> int:
    return load().num_threads()


def phi(x: float, kind: int = PHI_ELU1) -> float:
    return load().phi(x, kind)


def forward(*args, **kwargs):
    return load().forward(*args, **kwargs)


def decode_step(*args, **kwargs):
    return load().decode_step(*args, **kwargs)


def backward(*args, **kwargs):
    return load().backward(*args, **kwargs)
