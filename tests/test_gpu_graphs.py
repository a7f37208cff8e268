"""The library under HIP graph capture (torch.cuda.CUDAGraph), the way a
serving loop or a training step that cannot afford one launch per kernel runs
it.  A call enqueues only kernel launches on the caller's stream (no memory
sets, copies, allocations or host synchronisation), so capturing it records
every kernel, and each replay reads the current contents of the input tensors
and rewrites the outputs.

Each test captures calls on tensors allocated beforehand.  Then, three times
over with new values: it copies the values into the captured inputs (and
resets any state the calls update in place), runs the same calls eagerly on
copies of those values, synchronises, replays the graph, and requires the
replay's results to equal the eager ones bit for bit (the same kernels and
launch configuration on the same values).  The eager results of the first set
of values are checked against the fp64 oracle, so the replays meet the
oracle's bar as well."""
import numpy as np
import pytest
import torch

import gated_delta_rule_26_amd as gdr
import oracle
from gdr_inputs import random_inputs
from oracle.backward import oracle_bwd
from tests.gpu_util import DEV, TOL, host, rel, to_dev

pytestmark = pytest.mark.gpu

ROUNDS = 3


def _fill(dst: dict, src: dict):
    """Copy new values into the captured input tensors (eager work between replays)."""
    for key, t in dst.items():
        if t is not None and src.get(key) is not None:
            t.copy_(src[key])


def _assert_same(name, got, want):
    assert got.shape == want.shape and got.dtype == want.dtype, name
    assert torch.equal(got, want), f"{name}: replay differs from the eager call (max |diff| " \
                                   f"{(got.float() - want.float()).abs().max().item():.3e})"


def _capture(fn):
    """Warm up eagerly (library load, one-time look-ups), then capture fn's calls."""
    fn()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = fn()
    torch.cuda.synchronize()
    return graph, out


def test_decode_steps_replay_like_eager_calls():
    N, H, D, steps = 3, 2, 128, 4

    def values(seed):
        rng = np.random.default_rng(seed)
        v = {}
        q = rng.standard_normal((steps, N, H, D))
        z = rng.standard_normal((steps, N, H, D))
        v["q"] = torch.from_numpy(q).to(DEV, torch.bfloat16)
        v["k"] = torch.from_numpy(z / np.linalg.norm(z, axis=-1, keepdims=True)).to(DEV, torch.bfloat16)
        v["v"] = torch.from_numpy(rng.standard_normal((steps, N, H, D))).to(DEV, torch.bfloat16)
        v["g"] = torch.from_numpy(np.log(rng.uniform(0.95, 0.999, (steps, N, H)))).to(DEV, torch.float32)
        v["beta"] = torch.from_numpy(1.0 / (1.0 + np.exp(-rng.standard_normal((steps, N, H))))).to(DEV, torch.float32)
        v["s_init"] = torch.from_numpy(rng.standard_normal((N, H, D, D)) * 0.02).to(DEV, torch.float32)
        return v

    x = {key: torch.empty_like(t) for key, t in values(0).items()}
    state = torch.empty((N, H, D, D), dtype=torch.float32, device=DEV)
    o = torch.empty((steps, N, H, D), dtype=torch.float32, device=DEV)

    def calls(inp, st, out):
        for i in range(steps):
            gdr.recurrent_step(inp["q"][i], inp["k"][i], inp["v"][i], inp["g"][i], inp["beta"][i], st, o=out[i],
                               o_dtype=torch.float32)

    _fill(x, values(0))
    state.copy_(x["s_init"])
    graph, _ = _capture(lambda: calls(x, state, o))
    for r in range(ROUNDS):
        vals = values(100 + r)
        st_e, o_e = vals["s_init"].clone(), torch.empty_like(o)
        calls(vals, st_e, o_e)
        _fill(x, vals)
        state.copy_(vals["s_init"])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _assert_same(f"decode o, replay {r}", o, o_e)
        _assert_same(f"decode state, replay {r}", state, st_e)
        if r == 0:
            o_ref, s_ref = oracle.oracle_decode(host(vals["q"]), host(vals["k"]), host(vals["v"]), host(vals["g"]),
                                                host(vals["beta"]), host(vals["s_init"]))
            assert rel(host(o_e), o_ref) < TOL["f32"] and rel(host(st_e), s_ref) < TOL["f32"]


# name: (mode kwargs, dtype, B, T, H, D); the KLA case is long enough for its walk to run in time segments
# (transfer walk, segment combine, segment walks), every other case is one walk per (sequence, head)
FWD_CASES = {
    "gdn_bf16": (dict(), "bf16", 2, 200, 2, 128),
    "kda_bf16": (dict(per_channel=True), "bf16", 1, 130, 2, 128),
    "kla_bf16_segments": (dict(kaczmarz=True, eps=1e-6), "bf16", 1, 8192, 2, 128),
    "gdn_f32_d64": (dict(), "f32", 1, 100, 2, 64),
}


@pytest.mark.parametrize("name", list(FWD_CASES))
def test_chunked_forward_replays_like_eager_calls(name):
    m, dtype, B, T, H, D = FWD_CASES[name]
    kz, pc = m.get("kaczmarz", False), m.get("per_channel", False)

    def values(seed):
        x = random_inputs(seed, B, T, H, D, D, dtype=dtype, per_channel=pc, kaczmarz=kz,
                          key_norm="lognormal_norm" if kz else "unit", with_s0=True)
        return x, to_dev(x, dtype)

    _, first = values(7000)
    x = {key: torch.empty_like(t) for key, t in first.items()}
    _fill(x, first)
    o = torch.empty((B, T, H, D), dtype=torch.float32, device=DEV)
    s = torch.empty((B, H, D, D), dtype=torch.float32, device=DEV)
    desc = gdr.make_desc(B, T, H, D, D, qkv_dtype=x["q"].dtype, o_dtype=torch.float32, per_channel=pc,
                         kaczmarz=kz, eps=m.get("eps", 0.0))
    ws = torch.empty(max(1, gdr.chunk_fwd_workspace_size(desc)), dtype=torch.uint8, device=DEV)

    def call(inp, out, sf, w):
        gdr.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], s0=inp["s0"], o=out, s_final=sf,
                      o_dtype=torch.float32, workspace=w, **m)

    graph, _ = _capture(lambda: call(x, o, s, ws))
    for r in range(ROUNDS):
        xn, vals = values(7100 + r)
        o_e, s_e, ws_e = torch.empty_like(o), torch.empty_like(s), torch.empty_like(ws)
        call(vals, o_e, s_e, ws_e)
        _fill(x, vals)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _assert_same(f"{name} o, replay {r}", o, o_e)
        _assert_same(f"{name} s_final, replay {r}", s, s_e)
        if r == 0:
            o_ref, s_ref = oracle.oracle_fwd(xn["q"], xn["k"], xn["v"], xn["g"], xn["beta"], s0=xn["s0"],
                                             per_channel=pc, kaczmarz=kz, eps=m.get("eps", 0.0))
            eo, es = rel(host(o_e), o_ref), rel(host(s_e), s_ref)
            print(f"{name}: eager vs oracle o {eo:.2e} s {es:.2e}")
            assert eo < TOL[dtype] and es < TOL[dtype]


def test_packed_batch_replays_like_eager_calls():
    H, D = 2, 128
    lens = [70, 1, 129]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    T, N = int(sum(lens)), len(lens)

    def values(seed):
        x = random_inputs(seed, 1, T, H, D, D, dtype="bf16")
        x["s0"] = (np.random.default_rng(seed).standard_normal((N, H, D, D)) * 0.1).astype(np.float32)
        d = to_dev(x, "bf16")
        return x, {key: (t[0] if key != "s0" else t) for key, t in d.items()}

    _, first = values(7200)
    x = {key: torch.empty_like(t) for key, t in first.items()}
    _fill(x, first)
    o = torch.empty((T, H, D), dtype=torch.float32, device=DEV)
    s = torch.empty((N, H, D, D), dtype=torch.float32, device=DEV)
    desc = gdr.make_desc(N, T, H, D, D, qkv_dtype=torch.bfloat16, o_dtype=torch.float32)
    ws = torch.empty(max(1, gdr.chunk_fwd_varlen_workspace_size(desc)), dtype=torch.uint8, device=DEV)

    def call(inp, out, sf, w):
        gdr.chunk_fwd_varlen(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], cu, s0=inp["s0"], o=out,
                             s_final=sf, o_dtype=torch.float32, workspace=w)

    graph, _ = _capture(lambda: call(x, o, s, ws))
    for r in range(ROUNDS):
        xn, vals = values(7300 + r)
        o_e, s_e, ws_e = torch.empty_like(o), torch.empty_like(s), torch.empty_like(ws)
        call(vals, o_e, s_e, ws_e)
        _fill(x, vals)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _assert_same(f"packed o, replay {r}", o, o_e)
        _assert_same(f"packed s_final, replay {r}", s, s_e)
        if r == 0:
            a = 0
            for n, ln in enumerate(lens):
                sl = {key: xn[key][:, a:a + ln] for key in ("q", "k", "v", "g", "beta")}
                o_ref, s_ref = oracle.oracle_fwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"],
                                                 s0=xn["s0"][n:n + 1])
                assert rel(host(o_e[a:a + ln]), o_ref[0]) < TOL["bf16"]
                assert rel(host(s_e[n]), s_ref[0]) < TOL["bf16"]
                a += ln


def test_noalloc_entry_point_replays_like_the_workspace_entry_point():
    B, T, H, D = 1, 200, 2, 128

    def values(seed):
        return to_dev(random_inputs(seed, B, T, H, D, D, dtype="bf16", with_s0=True), "bf16")

    x = {key: torch.empty_like(t) for key, t in values(7400).items()}
    _fill(x, values(7400))
    o = torch.empty((B, T, H, D), dtype=torch.float32, device=DEV)
    s = torch.empty((B, H, D, D), dtype=torch.float32, device=DEV)
    graph, _ = _capture(lambda: gdr.chunk_fwd_noalloc(x["q"], x["k"], x["v"], x["g"], x["beta"], o, s0=x["s0"],
                                                      s_final=s))
    for r in range(ROUNDS):
        vals = values(7500 + r)
        o_e, s_e = gdr.chunk_fwd(vals["q"], vals["k"], vals["v"], vals["g"], vals["beta"], s0=vals["s0"],
                                 o_dtype=torch.float32)
        _fill(x, vals)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _assert_same(f"noalloc o, replay {r}", o, o_e)
        _assert_same(f"noalloc s_final, replay {r}", s, s_e)


# name: (mode kwargs, B, T, H, relative-L2 bar of the eager gradients against the oracle: bf16 tiles for
# scalar decay at d128 with bf16 inputs, fp32 tiles for per-channel decay)
BWD_CASES = {
    "gdn_bf16_tiles": (dict(), 1, 130, 2, 1e-4),
    "kda_fp32_tiles": (dict(per_channel=True), 1, 100, 2, 1e-5),
}


@pytest.mark.parametrize("name", list(BWD_CASES))
def test_backward_replays_like_eager_calls(name):
    m, B, T, H, bar = BWD_CASES[name]
    D = 128
    pc = m.get("per_channel", False)

    def values(seed):
        x = random_inputs(seed, B, T, H, D, D, dtype="bf16", per_channel=pc, with_s0=True)
        rng = np.random.default_rng(seed + 1)
        x["do"] = rng.standard_normal((B, T, H, D)).astype(np.float32)
        x["ds"] = rng.standard_normal((B, H, D, D)).astype(np.float32)
        return x, to_dev(x, "bf16")

    _, first = values(7600)
    x = {key: torch.empty_like(t) for key, t in first.items()}
    _fill(x, first)
    desc = gdr.make_desc(B, T, H, D, D, qkv_dtype=torch.bfloat16, o_dtype=torch.float32, per_channel=pc)
    ws = torch.empty(gdr.chunk_bwd_workspace_size(desc), dtype=torch.uint8, device=DEV)

    def call(inp, w):
        return gdr.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["do"], s0=inp["s0"],
                             ds_final=inp["ds"], workspace=w, **m)

    graph, out = _capture(lambda: call(x, ws))  # the outputs live in the graph's memory pool
    for r in range(ROUNDS):
        xn, vals = values(7700 + r)
        ref_e = call(vals, torch.empty_like(ws))
        _fill(x, vals)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key in ("dq", "dk", "dv", "dg", "dbeta", "ds0"):
            _assert_same(f"{name} {key}, replay {r}", out[key], ref_e[key])
        if r == 0:
            ref = oracle_bwd(xn["q"], xn["k"], xn["v"], xn["g"], xn["beta"], xn["do"], ds_final=xn["ds"],
                             s0=xn["s0"], **m)
            errs = {key: rel(host(ref_e[key]), ref[key]) for key in ("dq", "dk", "dv", "dg", "dbeta", "ds0")}
            print(f"{name}: eager vs oracle " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
            assert all(v < bar for v in errs.values()), errs
