"""Chunked prefill on the GPU against the fp64 oracle: modes, dtypes, widths,
ragged tails and edge cases (the full benchmark workloads, every head, are in
test_gpu_full_workloads.py)."""
import numpy as np
import pytest
import torch

import gated_delta_rule_26_amd as gdr
import oracle
from gdr_inputs import random_inputs
from tests.gpu_util import DEV, TOL, host, rel, to_dev

pytestmark = pytest.mark.gpu

MODES = {"gdn": dict(per_channel=False, kaczmarz=False),
         "kda": dict(per_channel=True, kaczmarz=False),
         "kla": dict(per_channel=False, kaczmarz=True)}
ALGOS = ["vector", "matrix"]


def _skip_unsupported(algo, mode, dtype, D):
    """Every combination runs on both paths: the matrix-core path takes bf16
    inputs at d_k = d_v = 128 on its bf16 kernels and everything else on its
    fp32-tile kernels."""


def _inputs(seed, B, T, H, Dk, Dv, mode, dtype, with_s0=True, **kw):
    m = MODES[mode]
    return random_inputs(seed, B, T, H, Dk, Dv, dtype=dtype, per_channel=m["per_channel"],
                         kaczmarz=m["kaczmarz"], key_norm="lognormal_norm" if m["kaczmarz"] else "unit",
                         with_s0=with_s0, **kw)


def _gpu(x, mode, dtype, *, algo="vector", o_dtype=torch.float32, scale=1.0, eps=1e-6, s_final=None):
    m = MODES[mode]
    d = to_dev(x, dtype)
    o, s = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=d["s0"], o_dtype=o_dtype,
                         scale=scale, eps=eps if m["kaczmarz"] else 0.0, algo=algo, s_final=s_final, **m)
    torch.cuda.synchronize()
    return o, s


def _ref(x, mode, scale=1.0, eps=1e-6, heads=None):
    m = MODES[mode]
    return oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s0=x["s0"], scale=scale,
                             eps=eps if m["kaczmarz"] else 0.0, heads=heads, **m)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("T", [1, 63, 64, 200])
@pytest.mark.parametrize("mode", ["gdn", "kda", "kla"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("D", [(128, 128), (64, 64)])
def test_chunk_parity(algo, T, mode, dtype, D):
    _skip_unsupported(algo, mode, dtype, D)
    x = _inputs(1000 + T, 2, T, 3, D[0], D[1], mode, dtype, with_s0=(T % 2 == 0))
    o, s = _gpu(x, mode, dtype, algo=algo)
    o_ref, s_ref = _ref(x, mode)
    eo, es = rel(host(o), o_ref), rel(host(s), s_ref)
    print(f"chunk {algo} {mode} {dtype} T={T} D={D}: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL[dtype] and es < TOL[dtype]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("D", [(128, 64), (64, 128)])
def test_chunk_mixed_widths(algo, D):
    _skip_unsupported(algo, "kda", "bf16", D)
    x = _inputs(7, 1, 150, 2, D[0], D[1], "kda", "bf16")
    o, s = _gpu(x, "kda", "bf16", algo=algo)
    o_ref, s_ref = _ref(x, "kda")
    assert rel(host(o), o_ref) < TOL["bf16"] and rel(host(s), s_ref) < TOL["bf16"]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("mode", ["gdn", "kda"])
def test_bf16_output_and_scale(algo, mode):
    x = _inputs(8, 2, 130, 2, 128, 128, mode, "bf16")
    sc = 128 ** -0.5
    o, s = _gpu(x, mode, "bf16", algo=algo, o_dtype=torch.bfloat16, scale=sc)
    o_ref, s_ref = _ref(x, mode, scale=sc)
    eo = rel(host(o), o_ref)
    print(f"bf16 output {mode} {algo}: rel o {eo:.2e}")
    assert eo < TOL["bf16"] and rel(host(s), s_ref) < TOL["bf16"]


@pytest.mark.parametrize("mode,D", [("gdn", 64), ("gdn", 128), ("kda", 128)])
def test_empty_and_zero_length(mode, D):
    x = _inputs(9, 2, 0, 2, D, D, mode, "bf16")
    o, s = _gpu(x, mode, "bf16", algo="auto")
    assert o.shape == (2, 0, 2, D)
    np.testing.assert_array_equal(host(s), x["s0"])
    x["s0"] = None
    o, s = _gpu(x, mode, "bf16", algo="auto")
    assert not host(s).any()
    # B = 0 is a no-op
    x = _inputs(9, 1, 10, 1, 64, 64, "gdn", "bf16")
    d = to_dev(x, "bf16")
    o, s = gdr.chunk_fwd(d["q"][:0], d["k"][:0], d["v"][:0], d["g"][:0], d["beta"][:0])
    assert o.shape[0] == 0 and s.shape[0] == 0


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("mode", ["kla", "kda"])
def test_in_place_state_and_resume(algo, mode):
    x = _inputs(10, 2, 200, 2, 128, 128, mode, "bf16")
    o_full, s_full = _gpu(x, mode, "bf16", algo=algo)
    d = to_dev(x, "bf16")
    state = d["s0"].clone()
    outs = []
    for t0, t1 in [(0, 130), (130, 131), (131, 200)]:   # split mid-chunk, and a single token
        sl = {key: (d[key][:, t0:t1].contiguous() if key != "s0" else None) for key in d}
        o, _ = gdr.chunk_fwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], s0=state, s_final=state,
                             o_dtype=torch.float32, eps=1e-6 if MODES[mode]["kaczmarz"] else 0.0,
                             algo=algo, **MODES[mode])
        outs.append(o)
    torch.cuda.synchronize()
    o_split = torch.cat(outs, dim=1)
    o_ref, s_ref = _ref(x, mode)
    # both schedules meet the bar against the oracle; the vector path (fp32
    # throughout) also agrees with itself across chunk boundaries to 1e-5
    assert rel(host(o_split), o_ref) < TOL["bf16"] and rel(host(state), s_ref) < TOL["bf16"]
    assert rel(host(o_full), o_ref) < TOL["bf16"] and rel(host(s_full), s_ref) < TOL["bf16"]
    if algo == "vector":
        assert rel(host(o_split), host(o_full)) < 1e-5
        assert rel(host(state), host(s_full)) < 1e-5


@pytest.mark.parametrize("algo", ALGOS)
def test_prefill_then_decode_step(algo):
    x = _inputs(11, 2, 129, 3, 128, 128, "gdn", "bf16")
    d = to_dev(x, "bf16")
    T = 129
    cut = {key: (d[key][:, :T - 1].contiguous() if key != "s0" else d[key]) for key in d}
    _, s = gdr.chunk_fwd(cut["q"], cut["k"], cut["v"], cut["g"], cut["beta"], s0=cut["s0"],
                         o_dtype=torch.float32, algo=algo)
    last = {key: d[key][:, T - 1].contiguous() for key in ("q", "k", "v", "g", "beta")}
    o_last = gdr.recurrent_step(last["q"], last["k"], last["v"], last["g"], last["beta"], s,
                                o_dtype=torch.float32)
    o_full, s_full = _gpu(x, "gdn", "bf16", algo=algo)
    tol = 1e-5 if algo == "vector" else 2e-4
    assert rel(host(o_last), host(o_full[:, T - 1])) < tol
    assert rel(host(s), host(s_full)) < tol


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("mode", ["gdn", "kda"])
def test_beta_zero_and_one(mode, algo):
    D = 128 if algo == "matrix" else 64
    _skip_unsupported(algo, mode, "bf16", (D, D))
    x = _inputs(12, 1, 100, 2, D, D, mode, "bf16")
    x["beta"] = np.zeros_like(x["beta"])
    o, s = _gpu(x, mode, "bf16", algo=algo)
    o_ref, s_ref = _ref(x, mode)
    assert rel(host(s), s_ref) < 1e-5 and rel(host(o), o_ref) < 1e-5
    x["beta"] = np.ones_like(x["beta"])
    o, s = _gpu(x, mode, "bf16", algo=algo)
    o_ref, s_ref = _ref(x, mode)
    assert rel(host(s), s_ref) < TOL["bf16"] and rel(host(o), o_ref) < TOL["bf16"]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("mode", ["gdn", "kda"])
def test_strong_decay(mode, algo):
    _skip_unsupported(algo, mode, "bf16", (128, 128))
    x = _inputs(13, 1, 150, 2, 128, 128, mode, "bf16")
    x["g"] = np.full_like(x["g"], -5.0)
    o, s = _gpu(x, mode, "bf16", algo=algo)
    o_ref, s_ref = _ref(x, mode)
    assert np.isfinite(host(o)).all()
    assert rel(host(o), o_ref) < TOL["bf16"] and rel(host(s), s_ref) < TOL["bf16"]


@pytest.mark.parametrize("algo", ALGOS)
def test_per_channel_with_uniform_gate_equals_scalar(algo):
    x = _inputs(14, 1, 150, 2, 128, 128, "gdn", "bf16")
    o1, s1 = _gpu(x, "gdn", "bf16", algo=algo)
    xp = dict(x)
    xp["g"] = np.repeat(x["g"][..., None], 128, axis=-1)
    o2, s2 = _gpu(xp, "kda", "bf16", algo=algo)
    tol = 1e-5 if algo == "vector" else 2e-5
    assert rel(host(o2), host(o1)) < tol and rel(host(s2), host(s1)) < tol


@pytest.mark.parametrize("algo", ALGOS)
def test_deterministic_and_workspace_poison_does_not_leak(algo):
    x = _inputs(15, 2, 190, 2, 128, 128, "kda", "bf16")
    d = to_dev(x, "bf16")
    desc = gdr.make_desc(2, 190, 2, 128, 128, qkv_dtype=torch.bfloat16, o_dtype=torch.float32,
                         per_channel=True, algo=algo)
    ws = torch.empty(gdr.chunk_fwd_workspace_size(desc), dtype=torch.uint8, device=DEV)
    runs = []
    for fill in (0.0, float("nan")):
        ws.view(torch.float32)[: ws.numel() // 4].fill_(fill) if ws.numel() >= 4 else None
        o, s = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=d["s0"], per_channel=True,
                             o_dtype=torch.float32, workspace=ws, algo=algo)
        torch.cuda.synchronize()
        runs.append((o.clone(), s.clone()))
    assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1])


@pytest.mark.parametrize("algo", ALGOS)
def test_per_channel_decay_with_kaczmarz_step(algo):
    """Per-channel decay and the Kaczmarz step size together (a combination
    none of the benchmark workloads uses), unnormalised keys, partial chunk."""
    _skip_unsupported(algo, "kda", "bf16", (128, 128))
    x = random_inputs(21, 2, 170, 2, 128, 128, dtype="bf16", per_channel=True, kaczmarz=True,
                      key_norm="lognormal_norm", with_s0=True)
    d = to_dev(x, "bf16")
    o, s = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=d["s0"], o_dtype=torch.float32,
                         per_channel=True, kaczmarz=True, eps=1e-6, algo=algo)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s0=x["s0"], eps=1e-6,
                                     per_channel=True, kaczmarz=True)
    eo, es = rel(host(o), o_ref), rel(host(s), s_ref)
    print(f"kda+kaczmarz {algo}: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("span", ["mixed", "near_limit"])
def test_per_channel_strong_decay_in_some_channels(algo, span):
    """Per-channel gates where a few key channels decay very fast: "mixed"
    puts a block span of 75 in some 16-token blocks (beyond what the matrix
    kernels take in factored form) and weak decay elsewhere; "near_limit"
    gives every block a span just under that bound (63)."""
    _skip_unsupported(algo, "kda", "bf16", (128, 128))
    x = _inputs(22, 1, 200, 2, 128, 128, "kda", "bf16")
    g = x["g"].copy()
    if span == "mixed":
        g[:, 40:90, :, 5:9] = -5.0
        g[:, 150:160, 1, 100] = -8.0
    else:
        g[..., 77] = -4.2
    x["g"] = g
    o, s = _gpu(x, "kda", "bf16", algo=algo)
    o_ref, s_ref = _ref(x, "kda")
    eo, es = rel(host(o), o_ref), rel(host(s), s_ref)
    print(f"kda strong decay {span} {algo}: rel o {eo:.2e} S {es:.2e}")
    assert np.isfinite(host(o)).all() and np.isfinite(host(s)).all()
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("mode", ["gdn", "kla", "kda"])
def test_matrix_path_deterministic_and_close_to_vector_path(mode):
    x = _inputs(16, 2, 333, 3, 128, 128, mode, "bf16")
    o1, s1 = _gpu(x, mode, "bf16", algo="matrix")
    o2, s2 = _gpu(x, mode, "bf16", algo="matrix")
    assert torch.equal(o1, o2) and torch.equal(s1, s2)
    ov, sv = _gpu(x, mode, "bf16", algo="vector")
    eo, es = rel(host(o1), host(ov)), rel(host(s1), host(sv))
    print(f"matrix vs vector {mode}: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("mode", ["gdn", "kda"])
@pytest.mark.parametrize("B,H,T", [(1, 8, 130), (3, 8, 70), (1, 2, 65), (2, 1, 129), (1, 2, 64 * 40 + 5),
                                   (5, 8, 130), (3, 11, 100)])
def test_matrix_chunk_counts_and_workgroup_mapping(B, H, T, mode):
    """Matrix path: chunk counts that exercise the doubled LDS buffers and the
    loop tails (2, 3 and 41 chunks), and (sequence, head) counts that do and
    do not divide by 8 (the XCD-aware workgroup mapping and its fallback),
    and more walks (160, 132) than compute units."""
    x = _inputs(2000 + T + 7 * H + B, B, T, H, 128, 128, mode, "bf16", with_s0=True)
    o, s = _gpu(x, mode, "bf16", algo="matrix")
    o_ref, s_ref = _ref(x, mode)
    eo, es = rel(host(o), o_ref), rel(host(s), s_ref)
    print(f"matrix {mode} B{B} H{H} T{T}: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("mode", ["gdn", "kla"])
def test_matrix_walk_in_time_segments(mode):
    """Few heads and long sequences: the walk runs as chunk maps per time
    segment, their composition, and one walk per segment (4 segments of 33,
    33, 33 and 30 chunks here, the last one partial).  Checked against the
    oracle with an initial state updated in place."""
    x = _inputs(3100, 1, 64 * 128 + 37, 2, 128, 128, mode, "bf16", with_s0=True)
    d = to_dev(x, "bf16")
    state = d["s0"].clone()
    m = MODES[mode]
    o, _ = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=state, s_final=state,
                         o_dtype=torch.float32, eps=1e-6 if m["kaczmarz"] else 0.0, algo="matrix", **m)
    torch.cuda.synchronize()
    o_ref, s_ref = _ref(x, mode)
    eo, es = rel(host(o), o_ref), rel(host(state), s_ref)
    print(f"segmented walk {mode}: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("algo", ALGOS)
def test_kaczmarz_eps_zero_with_partial_chunk(algo):
    """KLA with eps = 0 and a partial last chunk: the padded rows (zero keys)
    must not turn 0 / |0|^2 into NaN; valid rows match the oracle."""
    x = _inputs(2100, 2, 100, 2, 128, 128, "kla", "bf16", with_s0=False)
    o, s = _gpu(x, "kla", "bf16", algo=algo, eps=0.0)
    o_ref, s_ref = _ref(x, "kla", eps=0.0)
    assert torch.isfinite(o).all() and torch.isfinite(s).all()
    eo, es = rel(host(o), o_ref), rel(host(s), s_ref)
    print(f"kla eps=0 {algo}: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


# ------------------------------------------------------------ without the delta rule
# The additive write S = D S + k v^T (no prediction, no beta): linear attention
# (D = I), RetNet / Mamba-2 (scalar decay) and GLA (per-channel decay).
NO_DELTA = {"linear": dict(per_channel=False), "retnet": dict(per_channel=False),
            "gla": dict(per_channel=True)}


def _no_delta_inputs(seed, B, T, H, D, variant, dtype, with_s0=True):
    x = random_inputs(seed, B, T, H, D, D, dtype=dtype, per_channel=NO_DELTA[variant]["per_channel"],
                      with_s0=with_s0)
    if variant == "linear":
        x["g"] = np.zeros_like(x["g"])
    return x


def _no_delta_run(x, variant, dtype, *, algo, o_dtype=torch.float32, scale=1.0, state=None):
    d = to_dev(x, dtype)
    s0 = d["s0"] if state is None else state
    o, s = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], None, s0=s0, s_final=state, o_dtype=o_dtype,
                         scale=scale, algo=algo, delta_off=True, **NO_DELTA[variant])
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], None, s0=x["s0"], scale=scale,
                                     delta_off=True, **NO_DELTA[variant])
    return o, s, o_ref, s_ref


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("variant", list(NO_DELTA))
@pytest.mark.parametrize("T", [1, 64, 200])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_no_delta_parity(algo, variant, T, dtype, D):
    _skip_unsupported(algo, "gdn", dtype, (D, D))
    x = _no_delta_inputs(4000 + T, 2, T, 3, D, variant, dtype, with_s0=(T != 64))
    o, s, o_ref, s_ref = _no_delta_run(x, variant, dtype, algo=algo)
    eo, es = rel(host(o), o_ref), rel(host(s), s_ref)
    print(f"no delta {variant} {algo} {dtype} T={T}: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL[dtype] and es < TOL[dtype]


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("variant", ["retnet", "gla"])
def test_no_delta_bf16_output_scale_and_beta_ignored(algo, variant):
    """bf16 output with KDA's read scale; a beta tensor passed anyway (here
    full of NaN) is not read."""
    x = _no_delta_inputs(4100, 2, 150, 2, 128, variant, "bf16")
    sc = 128 ** -0.5
    o, s, o_ref, s_ref = _no_delta_run(x, variant, "bf16", algo=algo, o_dtype=torch.bfloat16, scale=sc)
    assert rel(host(o), o_ref) < TOL["bf16"] and rel(host(s), s_ref) < TOL["bf16"]
    d = to_dev(x, "bf16")
    nan_beta = torch.full_like(d["beta"], float("nan"))
    desc = gdr.make_desc(2, 150, 2, 128, 128, qkv_dtype=torch.bfloat16, o_dtype=torch.bfloat16,
                         per_channel=NO_DELTA[variant]["per_channel"], scale=sc, algo=algo, delta_off=True)
    ws = torch.empty(gdr.chunk_fwd_workspace_size(desc), dtype=torch.uint8, device=DEV)
    o2 = torch.empty_like(o)
    s2 = torch.empty_like(s)
    lib = gdr.load_library()
    import ctypes
    rc = lib.gdr_chunk_fwd(ctypes.byref(desc), *[ctypes.c_void_p(t.data_ptr()) for t in
                                                 (d["q"], d["k"], d["v"], d["g"], nan_beta, d["s0"], o2, s2, ws)],
                           ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(o2, o) and torch.equal(s2, s)


@pytest.mark.parametrize("variant", ["linear", "retnet"])
def test_no_delta_walk_in_time_segments(variant):
    """The time-segmented walk without the delta rule (the chunk map's M is
    then the product of the chunk decays times I), state updated in place."""
    x = _no_delta_inputs(4200, 1, 64 * 128 + 37, 2, 128, variant, "bf16")
    if variant == "linear":  # keep the undecayed sums of 8229 writes moderate (a power of two: bf16 stays exact)
        x["v"] = (x["v"] * 0.0625).astype(np.float32)
    state = torch.from_numpy(x["s0"]).to(DEV)
    o, _, o_ref, s_ref = _no_delta_run(x, variant, "bf16", algo="matrix", state=state)
    eo, es = rel(host(o), o_ref), rel(host(state), s_ref)
    print(f"segmented walk, no delta, {variant}: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("variant", list(NO_DELTA))
def test_no_delta_matrix_close_to_vector_and_chunk_counts(variant):
    x = _no_delta_inputs(4300, 3, 64 * 5 + 11, 3, 128, variant, "bf16")
    om, sm, o_ref, s_ref = _no_delta_run(x, variant, "bf16", algo="matrix")
    ov, sv, _, _ = _no_delta_run(x, variant, "bf16", algo="vector")
    assert rel(host(om), host(ov)) < TOL["bf16"] and rel(host(sm), host(sv)) < TOL["bf16"]
    assert rel(host(om), o_ref) < TOL["bf16"] and rel(host(sm), s_ref) < TOL["bf16"]


def test_side_stream_call_and_binding_allocations():
    """Work enqueued on a caller's stream that is not torch's current stream.
    The binding allocates o, the final state and the workspace from the
    current stream's pool and releases the workspace on return; it records the
    caller's stream on them, so memory the current stream allocates and fills
    right after the call is not memory the kernels still use.  Results equal
    the same call on the current stream, bit for bit."""
    x = _inputs(17, 2, 900, 4, 128, 128, "gdn", "bf16")
    d = to_dev(x, "bf16")
    kw = dict(s0=d["s0"], o_dtype=torch.float32)
    o_ref, s_ref = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], **kw)
    st_ref = d["s0"].clone()
    o1_ref = gdr.recurrent_step(d["q"][:, 0].contiguous(), d["k"][:, 0].contiguous(), d["v"][:, 0].contiguous(),
                                d["g"][:, 0].contiguous(), d["beta"][:, 0].contiguous(), st_ref,
                                o_dtype=torch.float32)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    args1 = [d[key][:, 0].contiguous() for key in ("q", "k", "v", "g", "beta")]
    st = d["s0"].clone()
    torch.cuda.synchronize()
    o, s = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], stream=side, **kw)
    o1 = gdr.recurrent_step(*args1, st, o_dtype=torch.float32, stream=side)
    scribble = [torch.full((1 << 22,), float("nan"), device=DEV) for _ in range(16)]
    side.synchronize()
    torch.cuda.synchronize()
    del scribble
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
    assert torch.equal(o1, o1_ref) and torch.equal(st, st_ref)


def test_one_stage_needs_the_shared_workspace():
    x = _inputs(18, 1, 64, 1, 128, 128, "gdn", "bf16")
    d = to_dev(x, "bf16")
    with pytest.raises(ValueError):
        gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], stage=1)
