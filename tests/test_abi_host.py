"""libgdr on a host without a GPU: the library loads, exports every function
include/gdr.h declares, and its host-side validation rejects bad arguments
with the documented status codes before any HIP call.  No call here passes
validation, so nothing is ever launched."""
import ctypes
import os
import re

import pytest

import gated_delta_rule_26_amd as gdr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")

pytestmark = pytest.mark.skipif(not os.path.exists(gdr.library_path), reason="libgdr.so not built")

E = {name: code for code, name in gdr.STATUS.items()}


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gdr_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = gdr.load_library()
    names = declared_functions()
    assert names == sorted(["gdr_abi_version", "gdr_status_string", "gdr_chunk_fwd_workspace_size",
                            "gdr_chunk_fwd", "gdr_chunk_fwd_stage", "gdr_chunk_fwd_stage_timed", "gdr_recurrent_step",
                            "gdr_recurrent_step_timed",
                            "gdr_recurrent_fwd", "gdr_chunk_fwd_varlen", "gdr_chunk_fwd_varlen_workspace_size",
                            "gdr_chunk_bwd", "gdr_chunk_bwd_workspace_size", "gdr_chunk_bwd_varlen",
                            "gdr_chunk_bwd_varlen_workspace_size", "gdr_recurrent_fwd_varlen",
                            "gdr_chunk_fwd_noalloc"])
    for n in names:
        assert hasattr(lib, n), n


def test_desc_layout_matches_header():
    text = open(HEADER).read()
    body = text[text.index("typedef struct gdr_desc"):text.index("} gdr_desc;")]
    fields = re.findall(r"(int32_t|float)\s+(\w+);", body)
    assert [f for _, f in fields] == [f for f, _ in gdr.Desc._fields_]
    assert ctypes.sizeof(gdr.Desc) == 4 * len(fields)


def test_version_and_strings():
    lib = gdr.load_library()
    assert lib.gdr_abi_version() == 2
    for code in gdr.STATUS:
        assert lib.gdr_status_string(code).decode().startswith(gdr.STATUS[code])


def _desc(**kw):
    # The vector path needs a workspace, so a missing workspace fails validation;
    # no call in this file may pass validation (it would launch a kernel).
    base = dict(B=2, T=100, H=3, Dk=128, Dv=128, qkv_dtype=__import__("torch").bfloat16,
                o_dtype=__import__("torch").float32, algo="vector")
    base.update(kw)
    return gdr.make_desc(**base)


def _ws(desc):
    n = ctypes.c_size_t(0)
    rc = gdr.load_library().gdr_chunk_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    return rc, n.value


def test_workspace_size_query():
    rc, n = _ws(_desc())
    assert rc == 0 and n > 0
    rc2, n2 = _ws(_desc(T=200))
    assert rc2 == 0 and n2 > n
    assert _ws(_desc(Dk=96))[0] == E["GDR_E_UNSUPPORTED"]
    assert _ws(_desc(chunk=32))[0] == E["GDR_E_UNSUPPORTED"]
    assert _ws(_desc(B=-1))[0] == E["GDR_E_SHAPE"]
    d = _desc()
    d.delta_mode = 2
    assert _ws(d)[0] == E["GDR_E_MODE"]
    d = _desc()
    d.decay_mode = 7
    assert _ws(d)[0] == E["GDR_E_MODE"]
    d = _desc(kaczmarz=True, eps=-1.0)
    assert _ws(d)[0] == E["GDR_E_MODE"]
    d = _desc(scale=float("inf"))
    assert _ws(d)[0] == E["GDR_E_MODE"]
    # huge problems are rejected, not overflowed
    assert _ws(_desc(B=2 ** 30, T=2 ** 30, H=2 ** 10))[0] == E["GDR_E_SHAPE"]
    lib = gdr.load_library()
    assert lib.gdr_chunk_fwd_workspace_size(None, ctypes.byref(ctypes.c_size_t())) == E["GDR_E_NULL"]


# Fake, well-separated "device" addresses: these calls never reach a launch.
BASE = 1 << 40
def P(i, off=0):
    return ctypes.c_void_p(BASE + i * (1 << 32) + off)


def _call_chunk(desc, q=P(1), k=P(2), v=P(3), g=P(4), b=P(5), s0=None, o=P(6), sf=P(7), ws=P(8), wsb=None):
    if wsb is None:
        wsb = _ws(desc)[1]
    return gdr.load_library().gdr_chunk_fwd(ctypes.byref(desc), q, k, v, g, b, s0, o, sf, ws, wsb, None)


def test_chunk_validation_errors():
    d = _desc()
    assert _call_chunk(d, q=None) == E["GDR_E_NULL"]
    assert _call_chunk(d, o=None) == E["GDR_E_NULL"]
    assert _call_chunk(d, ws=None) == E["GDR_E_WORKSPACE"]
    assert _call_chunk(d, wsb=_ws(d)[1] - 1) == E["GDR_E_WORKSPACE"]
    assert _call_chunk(d, q=P(1, 8)) == E["GDR_E_ALIGN"]
    assert _call_chunk(d, g=P(4, 2)) == E["GDR_E_ALIGN"]
    assert _call_chunk(_desc(per_channel=True), g=P(4, 4)) == E["GDR_E_ALIGN"]
    assert _call_chunk(d, o=P(1)) == E["GDR_E_ALIAS"]            # o on top of q
    assert _call_chunk(d, sf=P(6, 1024)) == E["GDR_E_ALIAS"]    # s_final inside o
    assert _call_chunk(d, ws=P(2, 4096)) == E["GDR_E_ALIAS"]    # workspace inside k
    assert _call_chunk(d, s0=P(9), sf=P(9, 16)) == E["GDR_E_ALIAS"]  # partial s0/s_final overlap
    assert _call_chunk(_desc(Dv=80)) == E["GDR_E_UNSUPPORTED"]
    assert gdr.load_library().gdr_chunk_fwd(None, P(1), P(2), P(3), P(4), P(5), None, P(6), P(7), P(8), 0,
                                            None) == E["GDR_E_NULL"]
    lib = gdr.load_library()
    wsb = _ws(d)[1]
    assert lib.gdr_chunk_fwd_stage(2, ctypes.byref(d), P(1), P(2), P(3), P(4), P(5), None, P(6), P(7), P(8),
                                   wsb, None) == E["GDR_E_MODE"]
    assert lib.gdr_chunk_fwd_stage(0, ctypes.byref(d), None, P(2), P(3), P(4), P(5), None, P(6), P(7), P(8),
                                   wsb, None) == E["GDR_E_NULL"]
    # the timed stage: the same checks, and both events are required
    assert lib.gdr_chunk_fwd_stage_timed(2, ctypes.byref(d), P(1), P(2), P(3), P(4), P(5), None, P(6), P(7),
                                         P(8), wsb, None, P(10), P(11)) == E["GDR_E_MODE"]
    assert lib.gdr_chunk_fwd_stage_timed(1, ctypes.byref(d), P(1), P(2), P(3), P(4), P(5), None, P(6), P(7),
                                         P(8), wsb, None, None, P(11)) == E["GDR_E_NULL"]
    assert lib.gdr_chunk_fwd_stage_timed(1, ctypes.byref(d), P(1), P(2), P(3), P(4), P(5), None, P(6), P(7),
                                         P(8), wsb, None, P(10), None) == E["GDR_E_NULL"]
    assert lib.gdr_chunk_fwd_stage_timed(0, ctypes.byref(d), None, P(2), P(3), P(4), P(5), None, P(6), P(7),
                                         P(8), wsb, None, P(10), P(11)) == E["GDR_E_NULL"]


def test_delta_off_ignores_beta_and_its_mode():
    """Without the delta rule beta_or_eta is not read (it may be NULL) and
    beta_mode and eps are ignored; everything else is validated as before."""
    d = _desc(delta_off=True)
    d.beta_mode = 9
    d.eps = -1.0
    assert _ws(d) == _ws(_desc())
    # beta NULL passes the pointer checks: the call fails later, on the workspace
    assert _call_chunk(d, b=None, ws=None) == E["GDR_E_WORKSPACE"]
    assert _call_chunk(_desc(), b=None, ws=None) == E["GDR_E_NULL"]
    # a beta pointer given anyway is ignored, even one that would alias o
    assert _call_chunk(d, b=P(6), ws=None) == E["GDR_E_WORKSPACE"]
    assert _call_chunk(d, q=None) == E["GDR_E_NULL"]
    lib = gdr.load_library()
    ds = _desc(T=1, delta_off=True)
    call = lambda b, s: lib.gdr_recurrent_step(ctypes.byref(ds), P(1), P(2), P(3), P(4), b, s, P(7), None)
    assert call(None, P(6, 4)) == E["GDR_E_ALIGN"]
    assert call(None, None) == E["GDR_E_NULL"]
    dr = _desc(T=1)
    assert lib.gdr_recurrent_step(ctypes.byref(dr), P(1), P(2), P(3), P(4), None, P(6, 4), P(7),
                                  None) == E["GDR_E_NULL"]


def test_matrix_algo_support_and_workspace():
    torch = __import__("torch")
    nc = (100 + 63) // 64
    # fp32 q/k/v or a width of 64: the fp32-tile kernels, whose workspace per chunk and head is the
    # backward's prep part: T, A, M (C x C), G (C, or C x Dk per channel), beta (C), K~, K^, Q~ (C x Dk)
    def tile(Dk, pc):
        return 4 * (3 * 64 * 64 + 64 * (Dk if pc else 1) + 64 + 3 * 64 * Dk)
    for kw, Dk in ((dict(qkv_dtype=torch.float32), 128), (dict(Dk=64, Dv=64), 64), (dict(Dk=64, Dv=128), 64),
                   (dict(Dk=128, Dv=64, qkv_dtype=torch.float32), 128)):
        for pc in (False, True):
            assert _ws(_desc(per_channel=pc, algo="matrix", **kw)) == (0, 2 * 3 * nc * tile(Dk, pc))
            assert _ws(_desc(per_channel=pc, algo="auto", **kw)) == _ws(_desc(per_channel=pc, algo="matrix", **kw))
    # scalar decay, per chunk: T'' and A, each hi and lo, as six 1 KiB MFMA
    # operand fragments, then two fp32 decay factors per token
    assert _ws(_desc(algo="matrix")) == (0, 2 * 3 * nc * (4 * 6 * 1024 + 2 * 64 * 4))
    assert _ws(_desc(algo="auto")) == _ws(_desc(algo="matrix"))
    # per-channel decay: the same head, then the decayed K, Q (for K S, Q S) and
    # K (for the update), each hi and lo as sixteen 1 KiB fragments, and one
    # fp32 chunk-end decay per key channel
    pc = 4 * 6 * 1024 + 6 * 16 * 1024 + 128 * 4
    assert _ws(_desc(per_channel=True, algo="matrix")) == (0, 2 * 3 * nc * pc)
    assert _ws(_desc(per_channel=True, algo="auto")) == _ws(_desc(per_channel=True, algo="matrix"))
    # the vector kernels stay available on request, with their own workspace
    rc, n = _ws(_desc(Dk=64, Dv=64, per_channel=True, algo="vector"))
    assert rc == 0 and n > 0 and (rc, n) != _ws(_desc(Dk=64, Dv=64, per_channel=True, algo="auto"))


def test_long_sequence_workspace_includes_segment_states():
    """A few long sequences are walked in time segments: the workspace adds,
    per (sequence, head) and segment, the chunk map (two d_k x d_v fp32
    matrices) and the entering state (one)."""
    rec = 4 * 6 * 1024 + 2 * 64 * 4
    # 16 heads x 2048 chunks: 4 segments
    rc, n = _ws(_desc(B=1, T=131072, H=16, algo="matrix"))
    assert rc == 0 and n == 16 * 2048 * rec + 16 * 4 * 3 * 128 * 128 * 4
    # many heads or short sequences: a single walk
    assert _ws(_desc(B=4, T=4096, H=16, algo="matrix")) == (0, 64 * 64 * rec)
    assert _ws(_desc(B=1, T=64 * 127, H=1, algo="matrix")) == (0, 127 * rec)
    assert _ws(_desc(B=1, T=64 * 128, H=1, algo="matrix")) == (0, 128 * rec + 1 * 4 * 3 * 128 * 128 * 4)


def test_step_validation_errors():
    lib = gdr.load_library()
    d = _desc(T=1)

    def call(q=P(1), k=P(2), v=P(3), g=P(4), b=P(5), s=P(6), o=P(7), desc=d):
        return lib.gdr_recurrent_step(ctypes.byref(desc), q, k, v, g, b, s, o, None)

    assert call(q=None) == E["GDR_E_NULL"]
    assert call(s=None) == E["GDR_E_NULL"]
    assert call(s=P(6, 4)) == E["GDR_E_ALIGN"]
    assert call(o=P(6, 64)) == E["GDR_E_ALIAS"]
    assert call(s=P(2)) == E["GDR_E_ALIAS"]
    assert call(desc=_desc(Dk=32)) == E["GDR_E_UNSUPPORTED"]
    bad = _desc()
    bad.o_dtype = 5
    assert call(desc=bad) == E["GDR_E_MODE"]


def test_recurrent_fwd_validation_errors():
    """T tokens per sequence: T is validated (the single step ignores it) and
    the chunk length is not."""
    lib = gdr.load_library()

    def call(desc, q=P(1), k=P(2), v=P(3), g=P(4), b=P(5), s=P(6), o=P(7)):
        return lib.gdr_recurrent_fwd(ctypes.byref(desc), q, k, v, g, b, s, o, None)

    d = _desc(T=40, chunk=7)
    assert call(d, q=None) == E["GDR_E_NULL"]
    assert call(d, s=P(6, 4)) == E["GDR_E_ALIGN"]
    assert call(d, o=P(2, 256)) == E["GDR_E_ALIAS"]
    assert call(_desc(T=-1)) == E["GDR_E_SHAPE"]
    assert call(_desc(T=5, Dk=96)) == E["GDR_E_UNSUPPORTED"]
    # T = 0 (and B = 0) are no-ops that touch no pointer
    assert call(_desc(T=0), q=None, s=None, o=None) == E["GDR_OK"]
    assert call(_desc(B=0), q=None, s=None, o=None) == E["GDR_OK"]
    # the single step ignores T
    assert lib.gdr_recurrent_step(ctypes.byref(_desc(T=-5)), P(1), P(2), P(3), P(4), P(5), P(6, 4), P(7),
                                  None) == E["GDR_E_ALIGN"]


def _ws_varlen(desc):
    n = ctypes.c_size_t(0)
    rc = gdr.load_library().gdr_chunk_fwd_varlen_workspace_size(ctypes.byref(desc), ctypes.byref(n))
    return rc, n.value


def test_varlen_workspace_and_validation():
    """A packed batch of N sequences, T tokens in all: at most
    floor((T + 63 N) / 64) chunks, each with one record per head, after a
    table of 2 (N + 1) + 2 x chunks + N int32 rounded up to 256 bytes."""
    N, T, H = 5, 1000, 3
    nc = (T + 63 * N) // 64
    table = -(-4 * (2 * (N + 1) + 2 * nc + N) // 256) * 256
    rec = 4 * 6 * 1024 + 2 * 64 * 4
    assert _ws_varlen(_desc(B=N, T=T, H=H, algo="matrix")) == (0, table + nc * H * rec)
    pc = 4 * 6 * 1024 + 6 * 16 * 1024 + 128 * 4
    assert _ws_varlen(_desc(B=N, T=T, H=H, per_channel=True, algo="matrix")) == (0, table + nc * H * pc)
    # no time segments for packed batches, however long the sequence
    assert _ws_varlen(_desc(B=1, T=131072, H=16, algo="matrix")) == (0, 256 * -(-4 * (4 + 2 * 2048) // 256)
                                                                     + 2048 * 16 * rec)
    lib = gdr.load_library()
    d = _desc(B=N, T=T, H=H, algo="matrix")
    wsb = _ws_varlen(d)[1]

    def call(cu=P(10), q=P(1), ws=P(8), sf=P(7), desc=d):
        return lib.gdr_chunk_fwd_varlen(ctypes.byref(desc), cu, q, P(2), P(3), P(4), P(5), None, P(6), sf, ws,
                                        wsb, None)

    assert call(cu=None) == E["GDR_E_NULL"]
    assert call(cu=P(10, 2)) == E["GDR_E_ALIGN"]
    assert call(cu=P(6, 64)) == E["GDR_E_ALIAS"]      # cu_seqlens inside o
    assert call(cu=P(8, 64)) == E["GDR_E_ALIAS"]      # cu_seqlens inside the workspace
    assert call(q=None) == E["GDR_E_NULL"]
    assert call(ws=None) == E["GDR_E_WORKSPACE"]
    # the packed token count is T (not B x T): q may be as small as T*H*Dk elements
    assert call(desc=_desc(B=N, T=T, H=H, Dk=96, algo="matrix")) == E["GDR_E_UNSUPPORTED"]


def test_backward_workspace_and_validation():
    """Per chunk slot: T, A, M, dA, dT'' (64 x 64 fp32 each), G and dG (64 x
    GK), GK, beta (64), the entering state and its gradient (Dk x Dv each),
    and the decayed K~, K^, Q~ (64 x Dk each) unless the decay is scalar and
    q, k are bf16 (then the kernels form them from k, q and the token factors).
    With bf16 q, k at d = 128 and scalar decay: no A, M, dA, dT'', dG, dG63
    (one kernel forms and uses them), and the chunk records of the bf16 walks: the
    forward walk's (25,088 bytes: T'' and A as bf16 hi/lo fragments, two
    decay rows) and the reverse walk's (24,576 bytes: the transposes of T''
    and A as bf16 hi/lo fragments)."""
    lib = gdr.load_library()
    n = ctypes.c_size_t(0)

    def ws(desc):
        rc = lib.gdr_chunk_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n))
        return rc, n.value

    slots = 2 * 3 * 2
    assert ws(_desc()) == (0, slots * (4 * (4096 + 64 + 64 + 2 * 128 * 128) + 25088 + 24576))
    assert ws(_desc(Dv=64)) == (0, slots * 4 * (5 * 4096 + 2 * 64 + 1 + 64 + 2 * 128 * 64))
    # one 8,192-token sequence on two heads walks in four time segments: the forward chunk maps (two per
    # segment) and entering states, then the reverse walk's N' and entering gradients, 128 x 128 fp32 each
    long_slots = 1 * 2 * 128
    assert ws(_desc(B=1, T=8192, H=2)) == (0, long_slots * (4 * (4096 + 64 + 64 + 2 * 128 * 128) + 25088 + 24576)
                                           + 2 * 4 * 5 * 128 * 128 * 4)
    assert ws(_desc(qkv_dtype=__import__("torch").float32)) == (
        0, slots * 4 * (5 * 4096 + 2 * 64 + 1 + 64 + 2 * 128 * 128 + 3 * 64 * 128))
    assert ws(_desc(per_channel=True)) == (0, slots * 4 * (5 * 4096 + 2 * 64 * 128 + 128 + 64 + 2 * 128 * 128
                                                           + 3 * 64 * 128))
    assert ws(_desc(delta_off=True)) == ws(_desc())
    d = _desc()
    wsb = ws(d)[1]

    def call(q=P(1), b=P(5), do=P(9), dq=P(10), dk=P(11), dv=P(12), dg=P(13), db=P(14), ds0=None, w=P(8)):
        return lib.gdr_chunk_bwd(ctypes.byref(d), q, P(2), P(3), P(4), b, None, do, None, dq, dk, dv, dg, db, ds0,
                                 w, wsb, None)

    assert call(q=None) == E["GDR_E_NULL"]
    assert call(b=None) == E["GDR_E_NULL"]
    assert call(db=None) == E["GDR_E_NULL"]
    assert call(do=None) == E["GDR_E_NULL"]
    assert call(w=None) == E["GDR_E_WORKSPACE"]
    assert call(dq=P(10, 4)) == E["GDR_E_ALIGN"]
    assert call(dk=P(10, 64)) == E["GDR_E_ALIAS"]    # dk inside dq
    assert call(dv=P(3)) == E["GDR_E_ALIAS"]         # dv on top of v


def test_backward_without_delta_rule_needs_no_beta():
    lib = gdr.load_library()
    d = _desc(delta_off=True)
    n = ctypes.c_size_t(0)
    assert lib.gdr_chunk_bwd_workspace_size(ctypes.byref(d), ctypes.byref(n)) == 0
    # beta and dbeta NULL pass the pointer checks: the call fails later, on the workspace
    rc = lib.gdr_chunk_bwd(ctypes.byref(d), P(1), P(2), P(3), P(4), None, None, P(9), None, P(10), P(11), P(12),
                           P(13), None, None, None, n.value, None)
    assert rc == E["GDR_E_WORKSPACE"]


def test_backward_varlen_workspace_and_validation():
    """A packed batch for the backward: the sequence table, then one backward
    slot per head for each of the floor((T + 63 N) / 64) chunks."""
    lib = gdr.load_library()
    n = ctypes.c_size_t(0)

    def ws(desc):
        rc = lib.gdr_chunk_bwd_varlen_workspace_size(ctypes.byref(desc), ctypes.byref(n))
        return rc, n.value

    N, T, H = 5, 1000, 3
    nc = (T + 63 * N) // 64
    table = -(-4 * (2 * (N + 1) + 2 * nc + N) // 256) * 256
    slot = 4 * (4096 + 64 + 64 + 2 * 128 * 128) + 25088 + 24576  # bf16, scalar: T, G, beta, states, records
    assert ws(_desc(B=N, T=T, H=H)) == (0, table + nc * H * slot)
    d = _desc(B=N, T=T, H=H)
    wsb = ws(d)[1]

    def call(cu=P(20), q=P(1), w=P(8), dq=P(10)):
        return lib.gdr_chunk_bwd_varlen(ctypes.byref(d), cu, q, P(2), P(3), P(4), P(5), None, P(9), None, dq,
                                        P(11), P(12), P(13), P(14), None, w, wsb, None)

    assert call(cu=None) == E["GDR_E_NULL"]
    assert call(cu=P(20, 2)) == E["GDR_E_ALIGN"]
    assert call(cu=P(10, 64)) == E["GDR_E_ALIAS"]    # cu_seqlens inside dq
    assert call(q=None) == E["GDR_E_NULL"]
    assert call(w=None) == E["GDR_E_WORKSPACE"]


def test_recurrent_fwd_varlen_validation():
    lib = gdr.load_library()
    d = _desc(B=4, T=37, H=2)

    def call(cu=P(20), q=P(1), st=P(7), o=P(6)):
        return lib.gdr_recurrent_fwd_varlen(ctypes.byref(d), cu, q, P(2), P(3), P(4), P(5), st, o, None)

    assert call(cu=None) == E["GDR_E_NULL"]
    assert call(cu=P(20, 2)) == E["GDR_E_ALIGN"]
    assert call(cu=P(7, 64)) == E["GDR_E_ALIAS"]     # cu_seqlens inside the state
    assert call(q=None) == E["GDR_E_NULL"]
    assert call(o=P(7)) == E["GDR_E_ALIAS"]          # o on top of the state



@pytest.mark.parametrize("D,h_max", [(128, 65535), (64, 131071)])
def test_head_count_limit_of_the_chunk_kernels(D, h_max):
    """The chunk kernels address the 64 token rows of a chunk ([64, H, D],
    up to 4-byte elements) with 32-bit byte offsets: 64 H max(Dk, Dv) 4 must
    stay below 2^31, else GDR_E_SHAPE (the recurrent entry points use 64-bit
    offsets and have no such limit)."""
    for algo in ("auto", "vector") + (("matrix",) if D == 128 else ()):   # the matrix path takes d128
        assert _ws(_desc(B=1, T=64, H=h_max, Dk=D, Dv=D, algo=algo))[0] == 0
        assert _ws(_desc(B=1, T=64, H=h_max + 1, Dk=D, Dv=D, algo=algo))[0] == E["GDR_E_SHAPE"]
    n = ctypes.c_size_t(0)
    bwd = gdr.load_library().gdr_chunk_bwd_workspace_size
    assert bwd(ctypes.byref(_desc(B=1, T=64, H=h_max + 1, Dk=D, Dv=D)), ctypes.byref(n)) == E["GDR_E_SHAPE"]
    # mixed widths: the wider one counts
    assert _ws(_desc(B=1, T=64, H=65536, Dk=64, Dv=128))[0] == E["GDR_E_SHAPE"]
    assert _ws(_desc(B=1, T=64, H=65535, Dk=64, Dv=128))[0] == 0


def test_noalloc_rejects_work_beyond_its_scratch_before_any_hip_call():
    """gdr_chunk_fwd_noalloc checks the workspace the call needs against its
    fixed scratch array (GDR_NOALLOC_SCRATCH_BYTES) before any HIP call: too
    large returns GDR_E_WORKSPACE with nothing enqueued; a bad descriptor
    returns the same status as gdr_chunk_fwd."""
    import torch
    lib = gdr.load_library()
    text = open(HEADER).read()
    assert "#define GDR_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)" in text
    assert gdr.NOALLOC_SCRATCH_BYTES == 128 << 20
    big = _desc(B=4, T=8192, H=16, algo="matrix")
    rc, need = _ws(big)
    assert rc == 0 and need > gdr.NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(16)
    assert lib.gdr_chunk_fwd_noalloc(ctypes.byref(big), p, p, p, p, p, None, p, None, None) == E["GDR_E_WORKSPACE"]
    bad = _desc(Dk=96)
    assert lib.gdr_chunk_fwd_noalloc(ctypes.byref(bad), p, p, p, p, p, None, p, None, None) == E["GDR_E_UNSUPPORTED"]
    assert lib.gdr_chunk_fwd_noalloc(None, p, p, p, p, p, None, p, None, None) == E["GDR_E_NULL"]
    # the GDN prefill workload (B4 H16 T4096, scalar decay) fits
    rc, need = _ws(_desc(B=4, T=4096, H=16, algo="matrix", qkv_dtype=torch.bfloat16))
    assert rc == 0 and need <= gdr.NOALLOC_SCRATCH_BYTES
