"""Seeded synthetic inputs for causal linear attention.

This module only draws random numbers and packs them into the storage types
the operator consumes (float32, or bfloat16 held as uint16 bit patterns).  It
contains none of the operator's arithmetic, so both the float64 oracle and the
GPU path can take their inputs from it.

Recipe (every workload):
  * ``rng = numpy.random.default_rng(seed)``; draws in this order: q, k, v,
    gate pre-activation, beta pre-activation, initial state.
  * Normal draws are float32 ziggurat samples, scaled in float64.
  * bfloat16 tensors are float32 values rounded to nearest-even.
  * Keys of the gated delta rule are L2-normalized in float64 before the
    cast (the rule assumes unit-length keys); after rounding to bfloat16 their
    norm is 1 only to bfloat16 precision, and both sides see the rounded keys.
  * Gates are logistic sigmoids of normal draws, stored as float32.
  * A decode sequence draws step ``s`` from ``default_rng([seed, s])`` so any
    step can be regenerated on its own.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

NORMALIZED, GATED, GATED_DELTA, RETENTION, KDA = 0, 1, 2, 3, 4
PHI_IDENTITY, PHI_ELU1 = 0, 1


# --------------------------------------------------------------------------
# storage types
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class HostTensor:
    """A host array in the operator's storage type ("f32" or "bf16")."""
    dtype: str
    data: np.ndarray          # float32 array, or uint16 bit patterns for bf16

    @property
    def shape(self):
        return self.data.shape

    def f64(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data).astype(np.float64)
        return self.data.astype(np.float64)

    def f32(self) -> np.ndarray:
        if self.dtype == "bf16":
            return bf16_bits_to_f32(self.data)
        return self.data


def _store(x, dtype) -> HostTensor:
    x = np.asarray(x)
    if dtype == "bf16":
        return HostTensor("bf16", f32_to_bf16_bits(x.astype(np.float32)))
    assert dtype == "f32"
    return HostTensor("f32", np.ascontiguousarray(x, dtype=np.float32))


def _normal(rng, shape, scale=1.0, mean=0.0):
    z = rng.standard_normal(size=shape, dtype=np.float32).astype(np.float64)
    return z * scale + mean


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _unit_rows(x):
    n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / n


# --------------------------------------------------------------------------
# workload table
# --------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    variant: int
    dtype: str            # dtype of q, k, v and out
    B: int
    H: int
    T: int                # sequence length (decode: number of steps)
    d_k: int
    d_v: int
    chunk: int            # 0 for a decode workload
    qkv_scale: float      # q, k, v ~ N(0, 1) * qkv_scale
    gate_mean: float = 0.0
    beta_mean: float = 0.0
    S0_std: float = 0.0   # 0 -> no initial state (NULL = zeros)
    decode: bool = False
    seed: int = 0
    phi: int = field(default=-1)

    @property
    def phi_kind(self) -> int:
        if self.phi >= 0:
            return self.phi
        return PHI_ELU1 if self.variant in (NORMALIZED, GATED) else PHI_IDENTITY


WORKLOADS = {
    "la_f32_b1h2t64d16": Workload(
        "la_f32_b1h2t64d16", NORMALIZED, "f32", 1, 2, 64, 16, 16, 16, 1.0, seed=1),
    "la_bf16_b4h8t2048d64": Workload(
        "la_bf16_b4h8t2048d64", NORMALIZED, "bf16", 4, 8, 2048, 64, 64, 64, 64 ** -0.5, seed=2),
    "gla_bf16_b8h16t4096d128": Workload(
        "gla_bf16_b8h16t4096d128", GATED, "bf16", 8, 16, 4096, 128, 128, 64, 128 ** -0.5,
        gate_mean=3.0, seed=3),
    "gdr_bf16_b4h16t8192d128": Workload(
        "gdr_bf16_b4h16t8192d128", GATED_DELTA, "bf16", 4, 16, 8192, 128, 128, 64, 128 ** -0.5,
        gate_mean=4.0, beta_mean=0.0, seed=4),
    "gdr_decode_b256h16d128": Workload(
        "gdr_decode_b256h16d128", GATED_DELTA, "bf16", 256, 16, 1000, 128, 128, 0, 128 ** -0.5,
        gate_mean=4.0, beta_mean=0.0, S0_std=0.1, decode=True, seed=5),
}

# Workload order of the five shapes the operator is specified on.
WORKLOAD_ORDER = list(WORKLOADS)

# Further workloads of the same recipe at the specified shapes, for the
# variants added beside the five (benchmarked, not part of the five).
EXTRA_WORKLOADS = {
    "kda_bf16_b4h16t8192d128": Workload(
        "kda_bf16_b4h16t8192d128", KDA, "bf16", 4, 16, 8192, 128, 128, 64, 128 ** -0.5,
        gate_mean=4.0, beta_mean=0.0, seed=6),
    "ret_bf16_b4h8t2048d64": Workload(
        "ret_bf16_b4h8t2048d64", RETENTION, "bf16", 4, 8, 2048, 64, 64, 64, 64 ** -0.5, gate_mean=3.0, seed=7),
}

# Training (backward-pass) workloads: the normalized configuration with a
# fixed per-head decay sigmoid(N(3, 1)) (drawn with head_decay=True), and
# retention at the delta rule's training shape; the loss gradient dout comes
# from backward_cotangents.
BWD_WORKLOADS = {
    "la_decay_bf16_b4h8t2048d64": Workload(
        "la_decay_bf16_b4h8t2048d64", NORMALIZED, "bf16", 4, 8, 2048, 64, 64, 64, 64 ** -0.5, gate_mean=3.0, seed=2),
    "ret_bf16_b4h16t8192d128": Workload(
        "ret_bf16_b4h16t8192d128", RETENTION, "bf16", 4, 16, 8192, 128, 128, 64, 128 ** -0.5, gate_mean=4.0, seed=8,
        phi=0),
}


def chunk_inputs(w: Workload, seed: int | None = None, *, T: int | None = None,
                 B: int | None = None, H: int | None = None,
                 S0_std: float | None = None, z0: bool = False, head_decay: bool = False) -> dict:
    """Inputs of one whole-sequence forward call, as HostTensors.

    Keys: q, k, v, and as the variant needs: gate, beta; S0 / z0 when an
    initial state is requested (S0_std > 0, z0=True for the normalized
    variant).  The retention variant, and the normalized one with
    head_decay, take a fixed decay per head, gate (H,) = sigmoid(N(gate_mean,
    1)), drawn in the gate slot.  Shapes may be overridden (B, H, T) for
    smaller test cases.
    """
    seed = w.seed if seed is None else seed
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    S0_std = w.S0_std if S0_std is None else S0_std
    rng = np.random.default_rng(seed)
    dk, dv = w.d_k, w.d_v
    q = _normal(rng, (B, H, T, dk), w.qkv_scale)
    k = _normal(rng, (B, H, T, dk), w.qkv_scale)
    v = _normal(rng, (B, H, T, dv), w.qkv_scale)
    out = {}
    if w.variant == GATED_DELTA:
        k = _unit_rows(k)
    out["q"], out["k"], out["v"] = _store(q, w.dtype), _store(k, w.dtype), _store(v, w.dtype)
    if w.variant in (GATED, KDA):
        out["gate"] = _store(_sigmoid(_normal(rng, (B, H, T, dk), 1.0, w.gate_mean)), "f32")
    elif w.variant == GATED_DELTA:
        out["gate"] = _store(_sigmoid(_normal(rng, (B, H, T), 1.0, w.gate_mean)), "f32")
    elif w.variant == RETENTION or (w.variant == NORMALIZED and head_decay):
        out["gate"] = _store(_sigmoid(_normal(rng, (H,), 1.0, w.gate_mean)), "f32")
    if w.variant in (GATED_DELTA, KDA):
        out["beta"] = _store(_sigmoid(_normal(rng, (B, H, T), 1.0, w.beta_mean)), "f32")
    if S0_std > 0:
        out["S0"] = _store(_normal(rng, (B, H, dv, dk), S0_std), "f32")
        if w.variant == NORMALIZED and z0:
            # a normalizer consistent with a positive history: |N(0, S0_std)| * d_k
            out["z0"] = _store(np.abs(_normal(rng, (B, H, dk), S0_std)) * dk + 1.0, "f32")
    return out


def backward_cotangents(w: Workload, seed: int | None = None, *, T: int | None = None,
                        B: int | None = None, H: int | None = None, state: bool = True) -> dict:
    """Gradients of a loss with respect to a forward call's outputs, as
    HostTensors, for the backward pass: dout (B,H,T,d_v) ~ N(0, 1) in the
    workload's dtype, and (state=True) dS_T (B,H,d_v,d_k) ~ N(0, 1) f32 and,
    for the normalized variant, dz_T (B,H,d_k) ~ N(0, 1) f32.  Drawn from
    default_rng([seed, 2**30 + 3]), independent of chunk_inputs."""
    seed = w.seed if seed is None else seed
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    rng = np.random.default_rng([seed, (1 << 30) + 3])
    out = {"dout": _store(_normal(rng, (B, H, T, w.d_v)), w.dtype)}
    if state:
        out["dS_T"] = _store(_normal(rng, (B, H, w.d_v, w.d_k)), "f32")
        if w.variant == NORMALIZED:
            out["dz_T"] = _store(_normal(rng, (B, H, w.d_k)), "f32")
    return out


def decode_state(w: Workload, seed: int | None = None, *, B=None, H=None) -> HostTensor:
    """Initial state S0 ~ N(0, S0_std) of a decode workload, (B,H,d_v,d_k) f32."""
    seed = w.seed if seed is None else seed
    B = w.B if B is None else B
    H = w.H if H is None else H
    rng = np.random.default_rng([seed, 1 << 30])
    return _store(_normal(rng, (B, H, w.d_v, w.d_k), w.S0_std), "f32")


def decode_normalizer(w: Workload, seed: int | None = None, *, B=None, H=None) -> HostTensor:
    """A positive initial normalizer z0 (B,H,d_k) f32 for the normalized variant:
    |N(0, 1)| * d_k + 1, the scale of a sum of d_k-ish positive features."""
    seed = w.seed if seed is None else seed
    B = w.B if B is None else B
    H = w.H if H is None else H
    rng = np.random.default_rng([seed, (1 << 30) + 1])
    return _store(np.abs(_normal(rng, (B, H, w.d_k))) * w.d_k + 1.0, "f32")


def decode_step_inputs(w: Workload, step: int, seed: int | None = None, *,
                       B=None, H=None) -> dict:
    """Inputs of decode step ``step``: q, k, v (B,H,d) and gate/beta per variant."""
    seed = w.seed if seed is None else seed
    B = w.B if B is None else B
    H = w.H if H is None else H
    rng = np.random.default_rng([seed, step])
    dk, dv = w.d_k, w.d_v
    q = _normal(rng, (B, H, dk), w.qkv_scale)
    k = _normal(rng, (B, H, dk), w.qkv_scale)
    v = _normal(rng, (B, H, dv), w.qkv_scale)
    out = {}
    if w.variant in (GATED_DELTA, KDA):
        k = _unit_rows(k)
    out["q"], out["k"], out["v"] = _store(q, w.dtype), _store(k, w.dtype), _store(v, w.dtype)
    if w.variant in (GATED, KDA):
        out["gate"] = _store(_sigmoid(_normal(rng, (B, H, dk), 1.0, w.gate_mean)), "f32")
    elif w.variant == GATED_DELTA:
        out["gate"] = _store(_sigmoid(_normal(rng, (B, H), 1.0, w.gate_mean)), "f32")
    if w.variant in (GATED_DELTA, KDA):
        out["beta"] = _store(_sigmoid(_normal(rng, (B, H), 1.0, w.beta_mean)), "f32")
    return out


def head_decays(w: Workload, seed: int | None = None, *, H=None) -> HostTensor:
    """A fixed decay per head, (H,) = sigmoid(N(gate_mean, 1)) f32, for decode
    sequences of the retention and (decayed) normalized variants: the same
    every step, drawn from default_rng([seed, 2**30 + 2])."""
    seed = w.seed if seed is None else seed
    H = w.H if H is None else H
    rng = np.random.default_rng([seed, (1 << 30) + 2])
    return _store(_sigmoid(_normal(rng, (H,), 1.0, w.gate_mean)), "f32")


def variant_workload(variant: int, dtype: str, d_k: int, d_v: int, chunk: int = 64,
                     seed: int = 11, S0_std: float = 0.0, phi: int = -1,
                     gate_mean: float | None = None) -> Workload:
    """An ad-hoc workload of the same recipe (used for parity sweeps); the
    gate pre-activation mean defaults to the specified workloads' (a lower
    mean gives stronger decay)."""
    if gate_mean is None:
        gate_mean = {NORMALIZED: 3.0, GATED: 3.0, GATED_DELTA: 4.0, RETENTION: 3.0, KDA: 3.0}[variant]
    return Workload("custom", variant, dtype, 1, 1, 1, d_k, d_v, chunk,
                    max(d_k, 1) ** -0.5, gate_mean=gate_mean, S0_std=S0_std, seed=seed, phi=phi)
