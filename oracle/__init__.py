"""fp64 CPU oracle for the gated delta-rule forward pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path (the HIP library and
its Python binding) may import, load or call anything in this package.  Only
the tests, the smoke check and the CPU-baseline leg of the benchmark use it.

Two independent CPU formulations live here:

* ``oracle_fwd`` -- the token-by-token recurrence in fp64 (``gdr_oracle.c``),
  following the step order of the blog summary's Gated DeltaNet and KDA
  sections and the Kaczmarz page's update rule.  It is THE reference.
* ``chunk_form.chunk_fwd`` -- the chunked algebra of the blog summary
  ("KDA por chunks") written out in numpy fp64.  It is a second, separately
  derived algorithm and serves as one of the pins of the recurrence.

Pins that hold the oracle to the pages live in ``tests/test_oracle_pins.py``
and ``tests/test_chunk_form.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdr_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (plain C, OpenMP, no -march=native so the
    library runs on any x86-64 host)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp"
    cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra",
           "-o", tmp, _SRC, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


def bind(path: str):
    """Load an oracle shared library from ``path`` and declare its ABI."""
    lib = ctypes.CDLL(path)
    lib.gdr_oracle_fwd.restype = ctypes.c_int
    P = ctypes.c_void_p
    L = ctypes.c_long
    lib.gdr_oracle_fwd.argtypes = [L, L, L, L, L, P, P, P, P, P,
                                   ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_double,
                                   ctypes.c_int, P, P, P, P, L, ctypes.c_int]
    lib.gdr_oracle_max_threads.restype = ctypes.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = bind(_LIB)
    return _lib


def max_threads() -> int:
    return int(_load().gdr_oracle_max_threads())


def _f32(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # a torch tensor: the oracle reads host float32 copies
        a = a.detach().float().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def oracle_fwd(q, k, v, g, beta, *, per_channel: bool = False, kaczmarz: bool = False,
               eps: float = 0.0, scale: float = 1.0, delta_off: bool = False, s0=None,
               heads=None, threads: int = 0, lib=None):
    """Run the fp64 recurrence.

    q, k: [B,T,H,Dk]; v: [B,T,H,Dv]; g: [B,T,H] or [B,T,H,Dk] (log-decay);
    beta: [B,T,H] (beta, or eta when ``kaczmarz``); s0: [B,H,Dk,Dv] or None.
    ``heads`` optionally lists flattened (b*H + h) pairs to compute; the other
    pairs of the outputs are NaN.  ``lib`` selects another build of the oracle
    (the mutation tests use it).  Returns (o [B,T,H,Dv], s_final [B,H,Dk,Dv])
    as float64 arrays.
    """
    q, k, v, g = _f32(q), _f32(k), _f32(v), _f32(g)
    beta = _f32(beta) if beta is not None else None
    s0 = _f32(s0)
    B, T, H, Dk = q.shape
    Dv = v.shape[3]
    if k.shape != (B, T, H, Dk) or v.shape[:3] != (B, T, H):
        raise ValueError("q/k/v shapes disagree")
    want_g = (B, T, H, Dk) if per_channel else (B, T, H)
    if g.shape != want_g:
        raise ValueError(f"g has shape {g.shape}, expected {want_g}")
    if beta is None and not delta_off:
        raise ValueError("beta is required unless delta_off")
    if beta is not None and beta.shape != (B, T, H):
        raise ValueError("beta must be [B,T,H]")
    if s0 is not None and s0.shape != (B, H, Dk, Dv):
        raise ValueError("s0 must be [B,H,Dk,Dv]")
    o = np.full((B, T, H, Dv), np.nan, dtype=np.float64)
    s_final = np.full((B, H, Dk, Dv), np.nan, dtype=np.float64)
    if heads is None:
        bh = None
        n_bh = 0
    else:
        bh = np.ascontiguousarray(np.asarray(heads, dtype=np.int64).reshape(-1)).astype(np.int_)
        n_bh = bh.size
    rc = (lib or _load()).gdr_oracle_fwd(B, T, H, Dk, Dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                int(per_channel), int(kaczmarz), float(eps), float(scale),
                                int(delta_off), _ptr(s0), _ptr(o), _ptr(s_final),
                                _ptr(bh), n_bh, int(threads))
    if rc != 0:
        raise RuntimeError(f"gdr_oracle_fwd failed with code {rc}")
    return o, s_final


def oracle_decode(q, k, v, g, beta, state0, **kw):
    """A run of single-token decode steps is the recurrence over the step axis.

    Step-major inputs: q,k [steps,N,H,Dk]; v [steps,N,H,Dv]; g [steps,N,H] or
    [steps,N,H,Dk]; beta [steps,N,H]; state0 [N,H,Dk,Dv].  Returns
    (o [steps,N,H,Dv], final state [N,H,Dk,Dv]).
    """
    def tr(a):
        a = _f32(a)
        return np.ascontiguousarray(np.swapaxes(a, 0, 1))
    o, s = oracle_fwd(tr(q), tr(k), tr(v), tr(g), tr(beta), s0=state0, **kw)
    return np.ascontiguousarray(np.swapaxes(o, 0, 1)), s
