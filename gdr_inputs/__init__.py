"""Seeded synthetic inputs for the gated delta-rule forward pass.

This module only draws random inputs.  It holds none of the method's
arithmetic (no decay, no beta rule, no state update), so that the fp64 oracle
and the GPU library can both be fed from it without sharing any computation.

Every generator uses numpy's PCG64 bit generator.  Chunked-prefill workloads
use ``PCG64(seed)``; decode steps use ``PCG64(SeedSequence([seed, step]))`` so
that any step can be regenerated on its own.  Values are drawn in float64,
stored in float32 and, for bf16 workloads, rounded to bf16 by
round-to-nearest-even; every returned array is float32 and holds exactly the
values the GPU receives.

Workloads (the distributions follow the five benchmark configurations):

* ``gdn_tiny``   B1 H1 T256 d64, fp32, scalar decay, given beta
* ``gdn_prefill`` B4 H16 T4096 d128, bf16, scalar decay, given beta
* ``kda_prefill`` B2 H16 T8192 d128, bf16, per-channel decay, given beta
* ``kla_prefill`` B1 H16 T131072 d128, bf16, scalar decay, Kaczmarz beta
* ``decode``     256 sequences x H16 d128, 1000 single-token steps, bf16

Readings where the configurations leave a point open: the state starts at
zero for the prefill workloads; N(0, 0.02) for the decode state is a standard
deviation of 0.02; the Kaczmarz workload's unnormalised keys are a uniformly
random direction times a LogNormal(0, 0.5) norm, one draw per (b, t, h);
gates (g = log alpha, beta, eta) are float32.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np


def bf16_round(x) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) & np.uint64(0xFFFF0000)
    return r.astype(np.uint32).view(np.float32).reshape(x.shape)


def _sigmoid(x):
    return 1.0 / (1.0 + np.exp(-x))


def _softplus(x):
    return np.logaddexp(0.0, x)


def _unit_rows(z):
    """Scale the last axis of z to unit Euclidean length (in float64)."""
    z = np.asarray(z, dtype=np.float64)
    return z / np.linalg.norm(z, axis=-1, keepdims=True)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    Dk: int
    Dv: int
    dtype: str                 # "f32" or "bf16": storage type of q, k, v
    decay: str                 # "scalar" or "per_channel"
    beta_mode: str             # "given" or "kaczmarz"
    seed: int
    eps: float = 0.0
    chunk: int = 64
    gate: str = "uniform"      # how log-decays are drawn (see _draw_g)
    gate_lo: float = 0.9
    gate_hi: float = 0.999
    gate_mult: float = 0.05
    keys: str = "unit"         # "unit" or "lognormal_norm"
    steps: int = 0             # decode only
    state_std: float = 0.0     # decode only: std of the initial state
    extra: dict = field(default_factory=dict)

    @property
    def per_channel(self) -> bool:
        return self.decay == "per_channel"

    @property
    def kaczmarz(self) -> bool:
        return self.beta_mode == "kaczmarz"

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "gdn_tiny": Workload("gdn_tiny", B=1, T=256, H=1, Dk=64, Dv=64, dtype="f32",
                         decay="scalar", beta_mode="given", seed=1,
                         gate="uniform", gate_lo=0.9, gate_hi=0.999),
    "gdn_prefill": Workload("gdn_prefill", B=4, T=4096, H=16, Dk=128, Dv=128, dtype="bf16",
                            decay="scalar", beta_mode="given", seed=2,
                            gate="softplus", gate_mult=0.05),
    "kda_prefill": Workload("kda_prefill", B=2, T=8192, H=16, Dk=128, Dv=128, dtype="bf16",
                            decay="per_channel", beta_mode="given", seed=3,
                            gate="softplus", gate_mult=0.05),
    "kla_prefill": Workload("kla_prefill", B=1, T=131072, H=16, Dk=128, Dv=128, dtype="bf16",
                            decay="scalar", beta_mode="kaczmarz", seed=4, eps=1e-6,
                            gate="softplus", gate_mult=0.02, keys="lognormal_norm"),
    "decode": Workload("decode", B=256, T=1, H=16, Dk=128, Dv=128, dtype="bf16",
                       decay="scalar", beta_mode="given", seed=5,
                       gate="uniform", gate_lo=0.95, gate_hi=0.999,
                       steps=1000, state_std=0.02),
}


def _store(x, dtype: str) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    return bf16_round(x) if dtype == "bf16" else np.ascontiguousarray(x)


def _draw_g(rng, shape, w: Workload) -> np.ndarray:
    if w.gate == "uniform":
        alpha = rng.uniform(w.gate_lo, w.gate_hi, size=shape)
        return np.log(alpha).astype(np.float32)
    if w.gate == "softplus":
        return (-_softplus(rng.standard_normal(shape)) * w.gate_mult).astype(np.float32)
    raise ValueError(w.gate)


def _draw_keys(rng, shape, w: Workload) -> np.ndarray:
    z = rng.standard_normal(shape)
    if w.keys == "unit":
        return _unit_rows(z)
    if w.keys == "lognormal_norm":
        r = rng.lognormal(mean=0.0, sigma=0.5, size=shape[:-1])
        return _unit_rows(z) * r[..., None]
    raise ValueError(w.keys)


def prefill_inputs(w: Workload) -> dict:
    """Draw q, k, v, g, beta (or eta) for a chunked-prefill workload.

    Draw order: q, k (and the key-norm draw when present), v, g, beta/eta.
    Returns float32 arrays: q,k [B,T,H,Dk]; v [B,T,H,Dv]; g [B,T,H] or
    [B,T,H,Dk]; beta [B,T,H] (eta for the Kaczmarz workload); s0 None.
    """
    rng = np.random.Generator(np.random.PCG64(w.seed))
    B, T, H, Dk, Dv = w.B, w.T, w.H, w.Dk, w.Dv
    q = _store(rng.standard_normal((B, T, H, Dk)), w.dtype)
    k = _store(_draw_keys(rng, (B, T, H, Dk), w), w.dtype)
    v = _store(rng.standard_normal((B, T, H, Dv)), w.dtype)
    g = _draw_g(rng, (B, T, H, Dk) if w.per_channel else (B, T, H), w)
    if w.kaczmarz:
        beta = _sigmoid(rng.normal(1.0, 1.0, size=(B, T, H))).astype(np.float32)
    else:
        beta = _sigmoid(rng.standard_normal((B, T, H))).astype(np.float32)
    return dict(q=q, k=k, v=v, g=g, beta=beta, s0=None)


def decode_state0(w: Workload) -> np.ndarray:
    """Initial decode state [N,H,Dk,Dv] float32, N(0, state_std) entries."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 1 << 20])))
    s = rng.standard_normal((w.B, w.H, w.Dk, w.Dv)) * w.state_std
    return s.astype(np.float32)


def decode_step_inputs(w: Workload, step: int) -> dict:
    """Inputs of one decode step: q,k [N,H,Dk]; v [N,H,Dv]; g, beta [N,H]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, step])))
    N, H, Dk, Dv = w.B, w.H, w.Dk, w.Dv
    q = _store(rng.standard_normal((N, H, Dk)), w.dtype)
    k = _store(_draw_keys(rng, (N, H, Dk), w), w.dtype)
    v = _store(rng.standard_normal((N, H, Dv)), w.dtype)
    g = _draw_g(rng, (N, H, Dk) if w.per_channel else (N, H), w)
    beta = _sigmoid(rng.standard_normal((N, H))).astype(np.float32)
    return dict(q=q, k=k, v=v, g=g, beta=beta)


def decode_inputs(w: Workload, steps: int | None = None) -> dict:
    """Stack ``steps`` decode steps step-major: q [steps,N,H,Dk], ..."""
    steps = w.steps if steps is None else steps
    per = [decode_step_inputs(w, s) for s in range(steps)]
    return {key: np.stack([p[key] for p in per]) for key in per[0]}


def random_inputs(seed: int, B: int, T: int, H: int, Dk: int, Dv: int, *, dtype: str = "bf16",
                  per_channel: bool = False, kaczmarz: bool = False, gate_mult: float = 0.05,
                  key_norm: str = "unit", with_s0: bool = False, s0_std: float = 0.1) -> dict:
    """Small seeded inputs of any shape (tests use these for edge cases)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _store(rng.standard_normal((B, T, H, Dk)), dtype)
    z = rng.standard_normal((B, T, H, Dk))
    if key_norm == "unit":
        kk = _unit_rows(z)
    elif key_norm == "lognormal_norm":
        kk = _unit_rows(z) * rng.lognormal(0.0, 0.5, size=(B, T, H))[..., None]
    else:
        kk = z
    k = _store(kk, dtype)
    v = _store(rng.standard_normal((B, T, H, Dv)), dtype)
    gshape = (B, T, H, Dk) if per_channel else (B, T, H)
    g = (-_softplus(rng.standard_normal(gshape)) * gate_mult).astype(np.float32)
    if kaczmarz:
        beta = _sigmoid(rng.normal(1.0, 1.0, size=(B, T, H))).astype(np.float32)
    else:
        beta = _sigmoid(rng.standard_normal((B, T, H))).astype(np.float32)
    s0 = (rng.standard_normal((B, H, Dk, Dv)) * s0_std).astype(np.float32) if with_s0 else None
    return dict(q=q, k=k, v=v, g=g, beta=beta, s0=s0)
