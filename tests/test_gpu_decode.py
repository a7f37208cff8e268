"""Fused recurrent decode step on the GPU against the fp64 oracle."""
import numpy as np
import pytest
import torch

import gated_delta_rule_26_amd as gdr
import oracle
from gdr_inputs import WORKLOADS, decode_state0, decode_step_inputs, random_inputs
from tests.gpu_util import DEV, TOL, host, rel, to_dev

pytestmark = pytest.mark.gpu


def _run(w, steps, *, o_dtype=torch.float32, scale=1.0, kaczmarz=False, delta_off=False, zero_gate=False):
    s0 = decode_state0(w)
    state = torch.from_numpy(s0).to(DEV)
    inputs, outs = [], []
    for t in range(steps):
        x = decode_step_inputs(w, t)
        if kaczmarz:
            x["beta"] = (x["beta"] * 1.5).astype(np.float32)   # eta
        if zero_gate:
            x["g"] = np.zeros_like(x["g"])
        inputs.append(x)
        d = to_dev(x, w.dtype)
        o = gdr.recurrent_step(d["q"], d["k"], d["v"], d["g"], None if delta_off else d["beta"], state,
                               per_channel=w.per_channel, kaczmarz=kaczmarz, eps=1e-6 if kaczmarz else 0.0,
                               scale=scale, o_dtype=o_dtype, delta_off=delta_off)
        outs.append(host(o))
    torch.cuda.synchronize()
    st = {key: np.stack([x[key] for x in inputs]) for key in inputs[0]}
    o_ref, s_ref = oracle.oracle_decode(st["q"], st["k"], st["v"], st["g"], st["beta"], s0,
                                        per_channel=w.per_channel, kaczmarz=kaczmarz,
                                        eps=1e-6 if kaczmarz else 0.0, scale=scale, delta_off=delta_off)
    return np.stack(outs), host(state), o_ref, s_ref


@pytest.mark.parametrize("D", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("mode", ["gdn", "kda", "kla"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_parity(D, mode, dtype):
    w = WORKLOADS["decode"].scaled(B=5, H=3, Dk=D[0], Dv=D[1], dtype=dtype,
                                   decay="per_channel" if mode == "kda" else "scalar")
    o, s, o_ref, s_ref = _run(w, 12, kaczmarz=mode == "kla")
    eo, es = rel(o, o_ref), rel(s, s_ref)
    print(f"decode {mode} {dtype} D={D}: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL[dtype] and es < TOL[dtype]
    assert eo < 1e-5 and es < 1e-5          # fp32 arithmetic on exact inputs


@pytest.mark.parametrize("variant", ["linear", "retnet", "gla"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_without_delta_rule(variant, dtype):
    """The additive write S = D S + k v^T (no prediction, no beta) per step."""
    w = WORKLOADS["decode"].scaled(B=5, H=3, dtype=dtype, decay="per_channel" if variant == "gla" else "scalar")
    o, s, o_ref, s_ref = _run(w, 12, delta_off=True, zero_gate=variant == "linear", scale=0.5)
    eo, es = rel(o, o_ref), rel(s, s_ref)
    print(f"decode no delta {variant} {dtype}: rel o {eo:.2e} S {es:.2e}")
    assert eo < 1e-5 and es < 1e-5


def test_decode_bf16_output_and_scale():
    w = WORKLOADS["decode"].scaled(B=4, H=2)
    o, s, o_ref, s_ref = _run(w, 6, o_dtype=torch.bfloat16, scale=128 ** -0.5)
    assert rel(o, o_ref) < TOL["bf16"] and rel(s, s_ref) < 1e-5


# ------------------------------------------------------------ T tokens per call
from gdr_inputs import random_inputs  # noqa: E402

RMODES = {"gdn": dict(per_channel=False, kaczmarz=False),
          "kda": dict(per_channel=True, kaczmarz=False),
          "kla": dict(per_channel=False, kaczmarz=True)}


def _recurrent_fwd(x, dtype, mode, *, delta_off=False, scale=1.0, o_dtype=torch.float32):
    m = RMODES[mode]
    d = to_dev(x, dtype)
    state = d["s0"].clone()
    o = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], None if delta_off else d["beta"], state,
                          eps=1e-6 if m["kaczmarz"] else 0.0, scale=scale, o_dtype=o_dtype,
                          delta_off=delta_off, **m)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s0=x["s0"], scale=scale,
                                     eps=1e-6 if m["kaczmarz"] else 0.0, delta_off=delta_off, **m)
    return o, state, o_ref, s_ref


@pytest.mark.parametrize("T", [1, 7, 40])
@pytest.mark.parametrize("mode", ["gdn", "kda", "kla"])
@pytest.mark.parametrize("dtype,D", [("bf16", (128, 128)), ("f32", (64, 128)), ("bf16", (128, 64))])
def test_recurrent_fwd_parity(T, mode, dtype, D):
    x = random_inputs(500 + T, 3, T, 2, D[0], D[1], dtype=dtype, per_channel=RMODES[mode]["per_channel"],
                      kaczmarz=RMODES[mode]["kaczmarz"],
                      key_norm="lognormal_norm" if mode == "kla" else "unit", with_s0=True)
    o, s, o_ref, s_ref = _recurrent_fwd(x, dtype, mode)
    eo, es = rel(host(o), o_ref), rel(host(s), s_ref)
    print(f"recurrent fwd {mode} {dtype} D={D} T={T}: rel o {eo:.2e} S {es:.2e}")
    assert eo < 1e-5 and es < 1e-5          # fp32 arithmetic on exact inputs


@pytest.mark.parametrize("variant", ["retnet", "gla"])
def test_recurrent_fwd_without_delta_rule_and_bf16_output(variant):
    mode = "kda" if variant == "gla" else "gdn"
    x = random_inputs(600, 2, 33, 3, 128, 128, dtype="bf16", per_channel=variant == "gla", with_s0=True)
    o, s, o_ref, s_ref = _recurrent_fwd(x, "bf16", mode, delta_off=True, scale=128 ** -0.5,
                                        o_dtype=torch.bfloat16)
    assert rel(host(o), o_ref) < TOL["bf16"] and rel(host(s), s_ref) < 1e-5


@pytest.mark.parametrize("mode", ["gdn", "kda"])
def test_recurrent_fwd_equals_chunked_and_steps(mode):
    """The same recurrence three ways: T = 100 tokens in one recurrent call,
    one chunked call, and 100 single decode steps."""
    T = 100
    x = random_inputs(700, 2, T, 2, 128, 128, dtype="bf16", per_channel=RMODES[mode]["per_channel"],
                      with_s0=True)
    o_r, s_r, o_ref, s_ref = _recurrent_fwd(x, "bf16", mode)
    d = to_dev(x, "bf16")
    o_c, s_c = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=d["s0"], o_dtype=torch.float32,
                             algo="vector", **RMODES[mode])
    state = d["s0"].clone()
    o_s = torch.stack([gdr.recurrent_step(d["q"][:, t].contiguous(), d["k"][:, t].contiguous(),
                                          d["v"][:, t].contiguous(), d["g"][:, t].contiguous(),
                                          d["beta"][:, t].contiguous(), state, o_dtype=torch.float32,
                                          **RMODES[mode]) for t in range(T)], dim=1)
    torch.cuda.synchronize()
    assert rel(host(o_r), host(o_c)) < 1e-5 and rel(host(s_r), host(s_c)) < 1e-5
    assert torch.equal(o_r, o_s) and torch.equal(s_r, state)   # the same arithmetic, token by token
    assert rel(host(o_r), o_ref) < 1e-5


def test_recurrent_fwd_zero_tokens_is_a_no_op():
    x = random_inputs(800, 2, 0, 2, 64, 64, dtype="bf16", with_s0=True)
    d = to_dev(x, "bf16")
    state = d["s0"].clone()
    o = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], state)
    torch.cuda.synchronize()
    assert o.shape == (2, 0, 2, 64) and torch.equal(state, d["s0"])


@pytest.mark.parametrize("mode", ["gdn", "kda", "kla"])
def test_recurrent_fwd_varlen_matches_each_sequence_alone(mode):
    """Packed requests of different lengths (an empty one included) on the
    recurrent schedule: each sequence's outputs and final state equal the
    oracle's for that sequence alone."""
    m = dict(per_channel=mode == "kda", kaczmarz=mode == "kla")
    lens = [3, 0, 1, 17, 64, 5]
    T, H, D = sum(lens), 2, 128
    x = random_inputs(7400 + len(mode), 1, T, H, D, D, dtype="bf16",
                      key_norm="lognormal_norm" if mode == "kla" else "unit", with_s0=False, **m)
    x = {key: (val[0] if val is not None else None) for key, val in x.items()}
    rng = np.random.default_rng(7401)
    s0 = (rng.standard_normal((len(lens), H, D, D)) * 0.1).astype(np.float32)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    d = to_dev(x, "bf16")
    state = torch.from_numpy(s0).to(DEV)
    eps = 1e-6 if m["kaczmarz"] else 0.0
    o = gdr.recurrent_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], state, torch.from_numpy(cu).to(DEV),
                                 o_dtype=torch.float32, eps=eps, **m)
    torch.cuda.synchronize()
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = {key: x[key][None, a:b] for key in ("q", "k", "v", "g", "beta")}
        o_ref, s_ref = oracle.oracle_fwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], s0=s0[n:n + 1], eps=eps,
                                         **m)
        es = rel(host(state[n]), s_ref[0])
        eo = rel(host(o[a:b]), o_ref[0]) if b > a else 0.0
        print(f"recurrent varlen {mode} sequence {n} (length {b - a}): rel o {eo:.2e} S {es:.2e}")
        assert eo < TOL["bf16"] and es < TOL["bf16"], (n, eo, es)
