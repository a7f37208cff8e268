"""Python binding of libgdr, the MI355X gated delta-rule forward pass.

Argument marshalling only: this module checks tensor devices, dtypes, shapes
and contiguity, allocates outputs and workspace with torch (device memory is
the only thing torch is used for, with the current stream), and calls the
C ABI declared in ``include/gdr.h``.  Every step of the computation runs in
the HIP kernels of ``libgdr.so``; there is no fallback.  If the library is not
built, importing works but every call raises ``GdrNotBuilt``.

Entry points (same names as the C ABI):
  chunk_fwd(q, k, v, g, beta, ...)        -> (o, s_final)   chunked prefill
  recurrent_step(q, k, v, g, beta, state) -> o              one decode step (state in place)
  recurrent_fwd(q, k, v, g, beta, state)  -> o              T tokens, recurrent (state in place)
  chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, ...) -> (o, s_final)   packed batch of sequences
  chunk_bwd(q, k, v, g, beta, d_o, ...)   -> dict of gradients  backward pass (training)
  chunk_fwd_noalloc(q, k, v, g, beta, o, ...) -> o         chunked prefill, no device allocation
  chunk_fwd_workspace_size(...)           -> bytes
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_varlen", "chunk_bwd", "chunk_bwd_workspace_size", "recurrent_step", "recurrent_fwd", "chunk_fwd_workspace_size",
           "chunk_fwd_varlen_workspace_size", "GdrError", "GdrNotBuilt",
           "library_path", "abi_version", "load_library", "Desc"]

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libgdr.so")

F32, BF16 = 0, 1
DECAY_SCALAR, DECAY_PER_CHANNEL = 0, 1
BETA_GIVEN, BETA_KACZMARZ = 0, 1
DELTA_RULE, DELTA_OFF = 0, 1
ALGOS = {"auto": 0, "vector": 1, "matrix": 2}
STATUS = {0: "GDR_OK", -1: "GDR_E_NULL", -2: "GDR_E_SHAPE", -3: "GDR_E_UNSUPPORTED", -4: "GDR_E_ALIGN",
          -5: "GDR_E_WORKSPACE", -6: "GDR_E_HIP", -7: "GDR_E_ALIAS", -8: "GDR_E_MODE"}


class GdrError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status})")


class GdrNotBuilt(RuntimeError):
    pass


class Desc(ctypes.Structure):
    """Mirror of ``gdr_desc`` in include/gdr.h."""
    _fields_ = [("B", ctypes.c_int32), ("T", ctypes.c_int32), ("H", ctypes.c_int32),
                ("Dk", ctypes.c_int32), ("Dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("qkv_dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32),
                ("decay_mode", ctypes.c_int32), ("beta_mode", ctypes.c_int32),
                ("algo", ctypes.c_int32), ("delta_mode", ctypes.c_int32),
                ("eps", ctypes.c_float), ("scale", ctypes.c_float)]


_lib = None


def load_library(path: str | None = None):
    """Load libgdr.so (once) and declare its ABI."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or library_path
    if not os.path.exists(p):
        raise GdrNotBuilt(f"{p} is missing: build it with __graft_entry__.build() "
                          f"(or python gated_delta_rule_26_amd/build.py)")
    lib = ctypes.CDLL(p)
    V = ctypes.c_void_p
    D = ctypes.POINTER(Desc)
    lib.gdr_abi_version.restype = ctypes.c_int
    lib.gdr_status_string.restype = ctypes.c_char_p
    lib.gdr_status_string.argtypes = [ctypes.c_int]
    lib.gdr_chunk_fwd_workspace_size.restype = ctypes.c_int
    lib.gdr_chunk_fwd_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_fwd.restype = ctypes.c_int
    lib.gdr_chunk_fwd.argtypes = [D, V, V, V, V, V, V, V, V, V, ctypes.c_size_t, V]
    lib.gdr_chunk_fwd_varlen_workspace_size.restype = ctypes.c_int
    lib.gdr_chunk_fwd_varlen_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_fwd_varlen.restype = ctypes.c_int
    lib.gdr_chunk_fwd_varlen.argtypes = [D, V, V, V, V, V, V, V, V, V, V, ctypes.c_size_t, V]
    lib.gdr_chunk_bwd_workspace_size.restype = ctypes.c_int
    lib.gdr_chunk_bwd_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_bwd.restype = ctypes.c_int
    lib.gdr_chunk_bwd.argtypes = [D] + [V] * 15 + [ctypes.c_size_t, V]
    lib.gdr_chunk_bwd_varlen_workspace_size.restype = ctypes.c_int
    lib.gdr_chunk_bwd_varlen_workspace_size.argtypes = [D, ctypes.POINTER(ctypes.c_size_t)]
    lib.gdr_chunk_bwd_varlen.restype = ctypes.c_int
    lib.gdr_chunk_bwd_varlen.argtypes = [D] + [V] * 16 + [ctypes.c_size_t, V]
    lib.gdr_chunk_fwd_stage.restype = ctypes.c_int
    lib.gdr_chunk_fwd_stage.argtypes = [ctypes.c_int, D, V, V, V, V, V, V, V, V, V, ctypes.c_size_t, V]
    lib.gdr_chunk_fwd_stage_timed.restype = ctypes.c_int
    lib.gdr_chunk_fwd_stage_timed.argtypes = [ctypes.c_int, D, V, V, V, V, V, V, V, V, V, ctypes.c_size_t, V, V, V]
    lib.gdr_recurrent_step.restype = ctypes.c_int
    lib.gdr_recurrent_step.argtypes = [D, V, V, V, V, V, V, V, V]
    lib.gdr_recurrent_step_timed.restype = ctypes.c_int
    lib.gdr_recurrent_step_timed.argtypes = [D, V, V, V, V, V, V, V, V, V, V]
    lib.gdr_recurrent_fwd.restype = ctypes.c_int
    lib.gdr_recurrent_fwd.argtypes = [D, V, V, V, V, V, V, V, V]
    lib.gdr_recurrent_fwd_varlen.restype = ctypes.c_int
    lib.gdr_recurrent_fwd_varlen.argtypes = [D, V, V, V, V, V, V, V, V, V]
    lib.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
    lib.gdr_chunk_fwd_noalloc.argtypes = [D, V, V, V, V, V, V, V, V, V]
    if path is None:
        _lib = lib
    return lib


def abi_version() -> int:
    return int(load_library().gdr_abi_version())


def _dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return F32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t}; use float32 or bfloat16")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check_dev(name, t, device, dtype=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _stream(stream, dev):
    """The stream the work is enqueued on: ``stream``, or torch's current stream of ``dev``."""
    return stream if stream is not None else torch.cuda.current_stream(dev)


def _used_on(st, dev, *tensors):
    """Tensors allocated here come from the caching allocator's pool of the
    current stream.  When the work runs on another stream, record that stream
    on them, so that their memory is not handed out again (and overwritten)
    before the work queued there has finished with it."""
    if st.cuda_stream == torch.cuda.current_stream(dev).cuda_stream:
        return
    for t in tensors:
        if t is not None:
            t.record_stream(st)


def make_desc(B, T, H, Dk, Dv, *, qkv_dtype, o_dtype, per_channel=False, kaczmarz=False, eps=0.0,
              scale=1.0, algo="auto", chunk=64, delta_off=False) -> Desc:
    return Desc(B=B, T=T, H=H, Dk=Dk, Dv=Dv, chunk=chunk, qkv_dtype=_dtype_code(qkv_dtype),
                o_dtype=_dtype_code(o_dtype), decay_mode=DECAY_PER_CHANNEL if per_channel else DECAY_SCALAR,
                beta_mode=BETA_KACZMARZ if kaczmarz else BETA_GIVEN, algo=ALGOS[algo],
                delta_mode=DELTA_OFF if delta_off else DELTA_RULE, eps=float(eps), scale=float(scale))


def chunk_fwd_workspace_size(desc: Desc) -> int:
    out = ctypes.c_size_t(0)
    rc = load_library().gdr_chunk_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(out))
    if rc != 0:
        raise GdrError(rc, "gdr_chunk_fwd_workspace_size")
    return int(out.value)


def chunk_fwd(q, k, v, g, beta, *, per_channel: bool = False, kaczmarz: bool = False, eps: float = 0.0,
              scale: float = 1.0, s0=None, output_final_state: bool = True, s_final=None, o=None,
              o_dtype=None, algo: str = "auto", workspace=None, stream=None, stage=None,
              delta_off: bool = False, events=None):
    """Chunked forward pass (prefill) through ``gdr_chunk_fwd``.

    q, k [B,T,H,Dk] and v [B,T,H,Dv] in float32 or bfloat16; g float32
    [B,T,H] (scalar decay) or [B,T,H,Dk] (``per_channel``); beta float32
    [B,T,H] (eta when ``kaczmarz``; None with ``delta_off``, the additive
    write S = D S + k v^T); s0 float32 [B,H,Dk,Dv] or None.
    ``s_final`` may be ``s0`` itself for an in-place state update.
    Returns (o [B,T,H,Dv], s_final [B,H,Dk,Dv] or None).  The work is enqueued
    on ``stream`` (default: torch's current stream of q's device).  ``stage``
    (0 = intra kernel, 1 = state kernel) runs one kernel of the pipeline
    through ``gdr_chunk_fwd_stage``; both stages must then share ``workspace``.
    ``events`` (with ``stage``): a pair of torch.cuda.Event(enable_timing=True)
    that have been recorded once (so that they exist); the stage's kernels
    record them when they begin and end (``gdr_chunk_fwd_stage_timed``).
    """
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (B, T, H, Dk))
    _check_dev("v", v, dev, q.dtype, (B, T, H, Dv))
    _check_dev("g", g, dev, torch.float32, (B, T, H, Dk) if per_channel else (B, T, H))
    if delta_off:
        beta = None
    else:
        _check_dev("beta", beta, dev, torch.float32, (B, T, H))
    if s0 is not None:
        _check_dev("s0", s0, dev, torch.float32, (B, H, Dk, Dv))
    if stage is not None and workspace is None:
        raise ValueError("stage= runs one kernel of the pipeline: pass the workspace both stages share")
    o_dtype = o_dtype or q.dtype
    fresh = []
    if o is None:
        o = torch.empty((B, T, H, Dv), dtype=o_dtype, device=dev)
        fresh.append(o)
    else:
        _check_dev("o", o, dev, o_dtype, (B, T, H, Dv))
    if s_final is None and output_final_state:
        s_final = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
        fresh.append(s_final)
    elif s_final is not None:
        _check_dev("s_final", s_final, dev, torch.float32, (B, H, Dk, Dv))
    desc = make_desc(B, T, H, Dk, Dv, qkv_dtype=q.dtype, o_dtype=o_dtype, per_channel=per_channel,
                     kaczmarz=kaczmarz, eps=eps, scale=scale, algo=algo, delta_off=delta_off)
    need = chunk_fwd_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
        fresh.append(workspace)
    else:
        _check_dev("workspace", workspace, dev, torch.uint8)
    st = _stream(stream, dev)
    _used_on(st, dev, *fresh)
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(o),
            _ptr(s_final), _ptr(workspace), workspace.numel(), ctypes.c_void_p(st.cuda_stream))
    if stage is None:
        if events is not None:
            raise ValueError("events time one stage: pass stage=0 or 1")
        rc, name = lib.gdr_chunk_fwd(*args), "gdr_chunk_fwd"
    elif events is None:
        rc, name = lib.gdr_chunk_fwd_stage(int(stage), *args), "gdr_chunk_fwd_stage"
    else:
        e0, e1 = (ctypes.c_void_p(e.cuda_event) for e in events)
        if not e0.value or not e1.value:
            raise ValueError("record each event once before passing it")
        rc, name = lib.gdr_chunk_fwd_stage_timed(int(stage), *args, e0, e1), "gdr_chunk_fwd_stage_timed"
    if rc != 0:
        raise GdrError(rc, name)
    return o, s_final


def recurrent_step(q, k, v, g, beta, state, *, per_channel: bool = False, kaczmarz: bool = False,
                   eps: float = 0.0, scale: float = 1.0, o=None, o_dtype=None, stream=None,
                   delta_off: bool = False, events=None):
    """One fused decode step through ``gdr_recurrent_step``.

    q, k [N,H,Dk], v [N,H,Dv] (float32 or bfloat16); g float32 [N,H] or
    [N,H,Dk]; beta float32 [N,H] (None with ``delta_off``); state float32
    [N,H,Dk,Dv], updated in place.  Returns o [N,H,Dv].  ``events``: a pair of
    recorded torch.cuda.Event(enable_timing=True) that the step's kernel
    records when it begins and ends (``gdr_recurrent_step_timed``).
    """
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    N, H, Dk = q.shape
    Dv = v.shape[-1]
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (N, H, Dk))
    _check_dev("v", v, dev, q.dtype, (N, H, Dv))
    _check_dev("g", g, dev, torch.float32, (N, H, Dk) if per_channel else (N, H))
    if delta_off:
        beta = None
    else:
        _check_dev("beta", beta, dev, torch.float32, (N, H))
    _check_dev("state", state, dev, torch.float32, (N, H, Dk, Dv))
    o_dtype = o_dtype or q.dtype
    fresh_o = o is None
    if fresh_o:
        o = torch.empty((N, H, Dv), dtype=o_dtype, device=dev)
    else:
        _check_dev("o", o, dev, o_dtype, (N, H, Dv))
    desc = make_desc(N, 1, H, Dk, Dv, qkv_dtype=q.dtype, o_dtype=o_dtype, per_channel=per_channel,
                     kaczmarz=kaczmarz, eps=eps, scale=scale, delta_off=delta_off)
    st = _stream(stream, dev)
    _used_on(st, dev, o if fresh_o else None)
    args = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
            ctypes.c_void_p(st.cuda_stream))
    if events is None:
        rc, name = lib.gdr_recurrent_step(*args), "gdr_recurrent_step"
    else:
        e0, e1 = (ctypes.c_void_p(e.cuda_event) for e in events)
        if not e0.value or not e1.value:
            raise ValueError("record each event once before passing it")
        rc, name = lib.gdr_recurrent_step_timed(*args, e0, e1), "gdr_recurrent_step_timed"
    if rc != 0:
        raise GdrError(rc, name)
    return o


def recurrent_fwd(q, k, v, g, beta, state, *, per_channel: bool = False, kaczmarz: bool = False,
                  eps: float = 0.0, scale: float = 1.0, o=None, o_dtype=None, stream=None,
                  delta_off: bool = False):
    """T recurrent tokens per sequence through ``gdr_recurrent_fwd``.

    q, k [B,T,H,Dk], v [B,T,H,Dv] (float32 or bfloat16); g float32 [B,T,H]
    or [B,T,H,Dk]; beta float32 [B,T,H] (None with ``delta_off``); state
    float32 [B,H,Dk,Dv], updated in place.  Returns o [B,T,H,Dv].
    """
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (B, T, H, Dk))
    _check_dev("v", v, dev, q.dtype, (B, T, H, Dv))
    _check_dev("g", g, dev, torch.float32, (B, T, H, Dk) if per_channel else (B, T, H))
    if delta_off:
        beta = None
    else:
        _check_dev("beta", beta, dev, torch.float32, (B, T, H))
    _check_dev("state", state, dev, torch.float32, (B, H, Dk, Dv))
    o_dtype = o_dtype or q.dtype
    fresh_o = o is None
    if fresh_o:
        o = torch.empty((B, T, H, Dv), dtype=o_dtype, device=dev)
    else:
        _check_dev("o", o, dev, o_dtype, (B, T, H, Dv))
    desc = make_desc(B, T, H, Dk, Dv, qkv_dtype=q.dtype, o_dtype=o_dtype, per_channel=per_channel,
                     kaczmarz=kaczmarz, eps=eps, scale=scale, delta_off=delta_off)
    st = _stream(stream, dev)
    _used_on(st, dev, o if fresh_o else None)
    rc = lib.gdr_recurrent_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                               _ptr(state), _ptr(o), ctypes.c_void_p(st.cuda_stream))
    if rc != 0:
        raise GdrError(rc, "gdr_recurrent_fwd")
    return o


def chunk_fwd_varlen_workspace_size(desc: Desc) -> int:
    out = ctypes.c_size_t(0)
    rc = load_library().gdr_chunk_fwd_varlen_workspace_size(ctypes.byref(desc), ctypes.byref(out))
    if rc != 0:
        raise GdrError(rc, "gdr_chunk_fwd_varlen_workspace_size")
    return int(out.value)


def chunk_fwd_varlen(q, k, v, g, beta, cu_seqlens, *, per_channel: bool = False, kaczmarz: bool = False,
                     eps: float = 0.0, scale: float = 1.0, s0=None, output_final_state: bool = True,
                     s_final=None, o=None, o_dtype=None, algo: str = "auto", workspace=None, stream=None,
                     delta_off: bool = False):
    """Chunked forward pass over a packed batch through ``gdr_chunk_fwd_varlen``.

    q, k [T,H,Dk], v [T,H,Dv] hold the tokens of N sequences back to back;
    sequence n is tokens cu_seqlens[n] .. cu_seqlens[n+1]-1 (cu_seqlens: int32
    [N+1] on the device).  g float32 [T,H] or [T,H,Dk]; beta float32 [T,H]
    (None with ``delta_off``); s0 float32 [N,H,Dk,Dv] or None.  Returns
    (o [T,H,Dv], s_final [N,H,Dk,Dv] or None).
    """
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    T, H, Dk = q.shape
    Dv = v.shape[-1]
    _check_dev("cu_seqlens", cu_seqlens, dev, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d int32 tensor of N + 1 entries")
    N = cu_seqlens.numel() - 1
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (T, H, Dk))
    _check_dev("v", v, dev, q.dtype, (T, H, Dv))
    _check_dev("g", g, dev, torch.float32, (T, H, Dk) if per_channel else (T, H))
    if delta_off:
        beta = None
    else:
        _check_dev("beta", beta, dev, torch.float32, (T, H))
    if s0 is not None:
        _check_dev("s0", s0, dev, torch.float32, (N, H, Dk, Dv))
    o_dtype = o_dtype or q.dtype
    fresh_o = o is None
    if fresh_o:
        o = torch.empty((T, H, Dv), dtype=o_dtype, device=dev)
    else:
        _check_dev("o", o, dev, o_dtype, (T, H, Dv))
    fresh_s = s_final is None and output_final_state
    if fresh_s:
        s_final = torch.empty((N, H, Dk, Dv), dtype=torch.float32, device=dev)
    elif s_final is not None:
        _check_dev("s_final", s_final, dev, torch.float32, (N, H, Dk, Dv))
    desc = make_desc(N, T, H, Dk, Dv, qkv_dtype=q.dtype, o_dtype=o_dtype, per_channel=per_channel,
                     kaczmarz=kaczmarz, eps=eps, scale=scale, algo=algo, delta_off=delta_off)
    need = chunk_fwd_varlen_workspace_size(desc)
    fresh_ws = workspace is None
    if fresh_ws:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _check_dev("workspace", workspace, dev, torch.uint8)
    st = _stream(stream, dev)
    _used_on(st, dev, o if fresh_o else None, s_final if fresh_s else None, workspace if fresh_ws else None)
    rc = lib.gdr_chunk_fwd_varlen(ctypes.byref(desc), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                  _ptr(beta), _ptr(s0), _ptr(o), _ptr(s_final), _ptr(workspace),
                                  workspace.numel(), ctypes.c_void_p(st.cuda_stream))
    if rc != 0:
        raise GdrError(rc, "gdr_chunk_fwd_varlen")
    return o, s_final


def chunk_bwd_workspace_size(desc: Desc) -> int:
    out = ctypes.c_size_t(0)
    rc = load_library().gdr_chunk_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(out))
    if rc != 0:
        raise GdrError(rc, "gdr_chunk_bwd_workspace_size")
    return int(out.value)


def chunk_bwd(q, k, v, g, beta, d_o, *, per_channel: bool = False, kaczmarz: bool = False, eps: float = 0.0,
              scale: float = 1.0, s0=None, ds_final=None, need_ds0: bool = True, workspace=None, stream=None,
              delta_off: bool = False):
    """Backward pass of ``chunk_fwd`` through ``gdr_chunk_bwd``.

    Inputs as for chunk_fwd, plus d_o float32 [B,T,H,Dv] (dL/do) and
    ds_final float32 [B,H,Dk,Dv] or None (dL/ds_final).  Returns a dict of
    float32 tensors: dq, dk, dv, dg, dbeta (dL/deta with ``kaczmarz``; None
    with ``delta_off``) and ds0 (None unless ``need_ds0``).
    """
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (B, T, H, Dk))
    _check_dev("v", v, dev, q.dtype, (B, T, H, Dv))
    gshape = (B, T, H, Dk) if per_channel else (B, T, H)
    _check_dev("g", g, dev, torch.float32, gshape)
    if delta_off:
        beta = None
    else:
        _check_dev("beta", beta, dev, torch.float32, (B, T, H))
    _check_dev("d_o", d_o, dev, torch.float32, (B, T, H, Dv))
    if s0 is not None:
        _check_dev("s0", s0, dev, torch.float32, (B, H, Dk, Dv))
    if ds_final is not None:
        _check_dev("ds_final", ds_final, dev, torch.float32, (B, H, Dk, Dv))
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.empty((B, T, H, Dk), **f32), "dk": torch.empty((B, T, H, Dk), **f32),
           "dv": torch.empty((B, T, H, Dv), **f32), "dg": torch.empty(gshape, **f32),
           "dbeta": None if delta_off else torch.empty((B, T, H), **f32),
           "ds0": torch.empty((B, H, Dk, Dv), **f32) if need_ds0 else None}
    desc = make_desc(B, T, H, Dk, Dv, qkv_dtype=q.dtype, o_dtype=torch.float32, per_channel=per_channel,
                     kaczmarz=kaczmarz, eps=eps, scale=scale, delta_off=delta_off)
    need = chunk_bwd_workspace_size(desc)
    fresh_ws = workspace is None
    if fresh_ws:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _check_dev("workspace", workspace, dev, torch.uint8)
    st = _stream(stream, dev)
    _used_on(st, dev, *out.values(), workspace if fresh_ws else None)
    rc = lib.gdr_chunk_bwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                           _ptr(d_o), _ptr(ds_final), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                           _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["ds0"]), _ptr(workspace),
                           workspace.numel(), ctypes.c_void_p(st.cuda_stream))
    if rc != 0:
        raise GdrError(rc, "gdr_chunk_bwd")
    return out


def chunk_bwd_varlen_workspace_size(desc: Desc) -> int:
    out = ctypes.c_size_t(0)
    rc = load_library().gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(desc), ctypes.byref(out))
    if rc != 0:
        raise GdrError(rc, "gdr_chunk_bwd_varlen_workspace_size")
    return int(out.value)


def chunk_bwd_varlen(q, k, v, g, beta, d_o, cu_seqlens, *, per_channel: bool = False, kaczmarz: bool = False,
                     eps: float = 0.0, scale: float = 1.0, s0=None, ds_final=None, need_ds0: bool = True,
                     workspace=None, stream=None, delta_off: bool = False):
    """Backward pass of ``chunk_fwd_varlen`` through ``gdr_chunk_bwd_varlen``.

    Token tensors [T,H,..] of N packed sequences (cu_seqlens int32 [N+1] on
    the device) as for chunk_fwd_varlen, d_o float32 [T,H,Dv]; s0, ds_final
    float32 [N,H,Dk,Dv] or None.  Returns a dict of float32 tensors dq, dk, dv,
    dg, dbeta (None with ``delta_off``) and ds0 (None unless ``need_ds0``);
    gradients of tokens outside every sequence are left unwritten.
    """
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    T, H, Dk = q.shape
    Dv = v.shape[-1]
    _check_dev("cu_seqlens", cu_seqlens, dev, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d int32 tensor of N + 1 entries")
    N = cu_seqlens.numel() - 1
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (T, H, Dk))
    _check_dev("v", v, dev, q.dtype, (T, H, Dv))
    gshape = (T, H, Dk) if per_channel else (T, H)
    _check_dev("g", g, dev, torch.float32, gshape)
    if delta_off:
        beta = None
    else:
        _check_dev("beta", beta, dev, torch.float32, (T, H))
    _check_dev("d_o", d_o, dev, torch.float32, (T, H, Dv))
    if s0 is not None:
        _check_dev("s0", s0, dev, torch.float32, (N, H, Dk, Dv))
    if ds_final is not None:
        _check_dev("ds_final", ds_final, dev, torch.float32, (N, H, Dk, Dv))
    f32 = dict(dtype=torch.float32, device=dev)
    out = {"dq": torch.zeros((T, H, Dk), **f32), "dk": torch.zeros((T, H, Dk), **f32),
           "dv": torch.zeros((T, H, Dv), **f32), "dg": torch.zeros(gshape, **f32),
           "dbeta": None if delta_off else torch.zeros((T, H), **f32),
           "ds0": torch.empty((N, H, Dk, Dv), **f32) if need_ds0 else None}
    desc = make_desc(N, T, H, Dk, Dv, qkv_dtype=q.dtype, o_dtype=torch.float32, per_channel=per_channel,
                     kaczmarz=kaczmarz, eps=eps, scale=scale, delta_off=delta_off)
    need = chunk_bwd_varlen_workspace_size(desc)
    fresh_ws = workspace is None
    if fresh_ws:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    else:
        _check_dev("workspace", workspace, dev, torch.uint8)
    st = _stream(stream, dev)
    _used_on(st, dev, *out.values(), workspace if fresh_ws else None)
    rc = lib.gdr_chunk_bwd_varlen(ctypes.byref(desc), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                  _ptr(beta), _ptr(s0), _ptr(d_o), _ptr(ds_final), _ptr(out["dq"]),
                                  _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]), _ptr(out["dbeta"]),
                                  _ptr(out["ds0"]), _ptr(workspace), workspace.numel(),
                                  ctypes.c_void_p(st.cuda_stream))
    if rc != 0:
        raise GdrError(rc, "gdr_chunk_bwd_varlen")
    return out


def recurrent_fwd_varlen(q, k, v, g, beta, state, cu_seqlens, *, per_channel: bool = False,
                         kaczmarz: bool = False, eps: float = 0.0, scale: float = 1.0, o=None, o_dtype=None,
                         stream=None, delta_off: bool = False):
    """Recurrent tokens of N packed sequences through ``gdr_recurrent_fwd_varlen``.

    q, k [T,H,Dk], v [T,H,Dv] hold the tokens of N sequences back to back
    (cu_seqlens int32 [N+1] on the device); g float32 [T,H] or [T,H,Dk]; beta
    float32 [T,H] (None with ``delta_off``); state float32 [N,H,Dk,Dv],
    updated in place.  Returns o [T,H,Dv] (tokens outside every sequence are
    left unwritten).
    """
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    T, H, Dk = q.shape
    Dv = v.shape[-1]
    _check_dev("cu_seqlens", cu_seqlens, dev, torch.int32)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d int32 tensor of N + 1 entries")
    N = cu_seqlens.numel() - 1
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (T, H, Dk))
    _check_dev("v", v, dev, q.dtype, (T, H, Dv))
    _check_dev("g", g, dev, torch.float32, (T, H, Dk) if per_channel else (T, H))
    if delta_off:
        beta = None
    else:
        _check_dev("beta", beta, dev, torch.float32, (T, H))
    _check_dev("state", state, dev, torch.float32, (N, H, Dk, Dv))
    o_dtype = o_dtype or q.dtype
    fresh_o = o is None
    if fresh_o:
        o = torch.empty((T, H, Dv), dtype=o_dtype, device=dev)
    else:
        _check_dev("o", o, dev, o_dtype, (T, H, Dv))
    desc = make_desc(N, T, H, Dk, Dv, qkv_dtype=q.dtype, o_dtype=o_dtype, per_channel=per_channel,
                     kaczmarz=kaczmarz, eps=eps, scale=scale, delta_off=delta_off)
    st = _stream(stream, dev)
    _used_on(st, dev, o if fresh_o else None)
    rc = lib.gdr_recurrent_fwd_varlen(ctypes.byref(desc), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                      _ptr(beta), _ptr(state), _ptr(o), ctypes.c_void_p(st.cuda_stream))
    if rc != 0:
        raise GdrError(rc, "gdr_recurrent_fwd_varlen")
    return o



NOALLOC_SCRATCH_BYTES = 128 << 20   # GDR_NOALLOC_SCRATCH_BYTES


def chunk_fwd_noalloc(q, k, v, g, beta, o, *, s0=None, s_final=None, per_channel: bool = False,
                      kaczmarz: bool = False, eps: float = 0.0, scale: float = 1.0, algo: str = "auto",
                      stream=None, delta_off: bool = False):
    """The chunked forward pass through ``gdr_chunk_fwd_noalloc``: the
    workspace is the library's fixed device array, and nothing is allocated
    here either, so the caller passes the output ``o`` [B,T,H,Dv] (its dtype
    is the output dtype) and, if wanted, ``s_final`` (may be ``s0``).  Calls
    on one GPU share that array: overlapping calls race.  Returns (o,
    s_final)."""
    lib = load_library()
    dev = q.device
    if dev.type != "cuda":
        raise ValueError("q must be a GPU tensor")
    B, T, H, Dk = q.shape
    Dv = v.shape[-1]
    _check_dev("q", q, dev)
    _check_dev("k", k, dev, q.dtype, (B, T, H, Dk))
    _check_dev("v", v, dev, q.dtype, (B, T, H, Dv))
    _check_dev("g", g, dev, torch.float32, (B, T, H, Dk) if per_channel else (B, T, H))
    if delta_off:
        beta = None
    else:
        _check_dev("beta", beta, dev, torch.float32, (B, T, H))
    if s0 is not None:
        _check_dev("s0", s0, dev, torch.float32, (B, H, Dk, Dv))
    _check_dev("o", o, dev, None, (B, T, H, Dv))
    if s_final is not None:
        _check_dev("s_final", s_final, dev, torch.float32, (B, H, Dk, Dv))
    desc = make_desc(B, T, H, Dk, Dv, qkv_dtype=q.dtype, o_dtype=o.dtype, per_channel=per_channel,
                     kaczmarz=kaczmarz, eps=eps, scale=scale, algo=algo, delta_off=delta_off)
    st = _stream(stream, dev)
    rc = lib.gdr_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0),
                                   _ptr(o), _ptr(s_final), ctypes.c_void_p(st.cuda_stream))
    if rc != 0:
        raise GdrError(rc, "gdr_chunk_fwd_noalloc")
    return o, s_final
