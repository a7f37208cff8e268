"""gdr_chunk_fwd_noalloc, the chunked pass whose workspace is the library's
fixed device array, against gdr_chunk_fwd with a caller-provided workspace,
both called through the C ABI.  Two calls in a row, the second on a smaller
input, so the second call runs on the array the first one left behind; each
result equals the workspace entry point's bit for bit (the same kernels and
arithmetic), and therefore meets the oracle's bar wherever gdr_chunk_fwd does.
The last case asks for more scratch than the array holds."""
import ctypes

import pytest
import torch

import gated_delta_rule_26_amd as gdr
from gdr_inputs import random_inputs
from tests.gpu_util import DEV, to_dev

pytestmark = pytest.mark.gpu

CASES = {
    # name: (per_channel, kaczmarz, dtype, algo, D, first (B, T, H), second (B, T, H))
    "gdn_matrix": (False, False, "bf16", "matrix", 128, (2, 700, 4), (1, 130, 2)),
    "kda_matrix": (True, False, "bf16", "matrix", 128, (1, 300, 3), (2, 65, 1)),
    "kla_vector_f32": (False, True, "f32", "vector", 64, (2, 257, 2), (1, 64, 1)),
}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _call(lib, entry, x, shape, pc, kz, dtype, algo, D):
    B, T, H = shape
    d = to_dev(x, dtype)
    qdt = d["q"].dtype
    desc = gdr.make_desc(B, T, H, D, D, qkv_dtype=qdt, o_dtype=torch.float32, per_channel=pc, kaczmarz=kz,
                         eps=1e-6 if kz else 0.0, algo=algo)
    o = torch.full((B, T, H, D), float("nan"), dtype=torch.float32, device=DEV)
    s = torch.full((B, H, D, D), float("nan"), dtype=torch.float32, device=DEV)
    args = [ctypes.byref(desc), _ptr(d["q"]), _ptr(d["k"]), _ptr(d["v"]), _ptr(d["g"]), _ptr(d["beta"]),
            _ptr(d["s0"]), _ptr(o), _ptr(s)]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if entry == "noalloc":
        rc = lib.gdr_chunk_fwd_noalloc(*args, stream)
    else:
        ws = torch.empty(max(1, gdr.chunk_fwd_workspace_size(desc)), dtype=torch.uint8, device=DEV)
        rc = lib.gdr_chunk_fwd(*args, _ptr(ws), ws.numel(), stream)
    assert rc == 0, gdr.STATUS.get(rc, rc)
    torch.cuda.synchronize()
    return o, s


@pytest.mark.parametrize("name", list(CASES))
def test_noalloc_equals_workspace_entry_point_twice(name):
    pc, kz, dtype, algo, D, first, second = CASES[name]
    lib = gdr.load_library()
    for i, shape in enumerate((first, second)):
        B, T, H = shape
        x = random_inputs(9100 + 10 * i + len(name), B, T, H, D, D, dtype=dtype, per_channel=pc, kaczmarz=kz,
                          key_norm="lognormal_norm" if kz else "unit", with_s0=True)
        o_ref, s_ref = _call(lib, "workspace", x, shape, pc, kz, dtype, algo, D)
        o, s = _call(lib, "noalloc", x, shape, pc, kz, dtype, algo, D)
        print(f"noalloc {name} call {i} {shape}: max |diff| o {float((o - o_ref).abs().max()):.3e} "
              f"S {float((s - s_ref).abs().max()):.3e}", flush=True)
        assert torch.isfinite(o).all() and torch.isfinite(s).all()
        assert torch.equal(o, o_ref) and torch.equal(s, s_ref)


def test_noalloc_refuses_work_beyond_its_scratch():
    lib = gdr.load_library()
    B, T, H = 8, 8192, 16
    desc = gdr.make_desc(B, T, H, 128, 128, qkv_dtype=torch.bfloat16, o_dtype=torch.float32, algo="matrix")
    assert gdr.chunk_fwd_workspace_size(desc) > gdr.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, T, H, 128), dtype=torch.bfloat16, device=DEV)
    g = torch.zeros((B, T, H), dtype=torch.float32, device=DEV)
    o = torch.zeros((B, T, H, 128), dtype=torch.float32, device=DEV)
    rc = lib.gdr_chunk_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(q), _ptr(q), _ptr(g), _ptr(g), None,
                                   _ptr(o), None, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == -5   # GDR_E_WORKSPACE, nothing enqueued
    torch.cuda.synchronize()
    assert not o.any()


def test_noalloc_binding_matches_chunk_fwd():
    x = random_inputs(9200, 2, 190, 2, 128, 128, dtype="bf16", with_s0=True)
    d = to_dev(x, "bf16")
    o_ref, s_ref = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=d["s0"], o_dtype=torch.bfloat16)
    o = torch.empty_like(o_ref)
    state = d["s0"].clone()
    gdr.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], o, s0=state, s_final=state)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(state, s_ref)
