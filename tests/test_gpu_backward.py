"""Backward pass on the GPU (gdr_chunk_bwd) against the backward oracle
(reverse mode over the float64 token recurrence), every gradient."""
import numpy as np
import pytest
import torch

import gated_delta_rule_26_amd as gdr
from gdr_inputs import random_inputs
from oracle.backward import oracle_bwd
from tests.gpu_util import DEV, host, rel, to_dev

pytestmark = pytest.mark.gpu

MODES = {"gdn": dict(per_channel=False, kaczmarz=False),
         "kda": dict(per_channel=True, kaczmarz=False),
         "kla": dict(per_channel=False, kaczmarz=True)}
# fp32 arithmetic on inputs that are exact in fp32 (fp32 inputs, per-channel
# decay, d = 64): the bar of the fp32 forward path (measured: 1e-7 .. 5e-7
# relative L2 on these cases)
TOL_BWD = 1e-5
# bf16 inputs with scalar decay at d_k = d_v = 128 run on bf16 tiles, as the
# forward pass's matrix path does: a product of fp32 values taken as bf16
# hi/lo pairs (hi*hi + hi*lo + lo*hi) keeps about 16 significant bits, so each
# is exact to about 2^-16 = 1.5e-5 relative at worst.  The bar for bf16
# inputs is the forward pass's, 2e-3; this is a 1e-4 sentinel under it
# (measured: 2e-6 .. 3e-5, the largest on a one-token sequence's dg).
TOL_BWD16 = 1e-4


def _tol(mode, dtype, D=(128, 128)):
    tile16 = dtype == "bf16" and D == (128, 128) and mode not in ("kda", "gla")
    return TOL_BWD16 if tile16 else TOL_BWD


def _case(seed, B, T, H, D, mode, dtype, *, with_ds=True):
    m = MODES[mode]
    x = random_inputs(seed, B, T, H, D[0], D[1], dtype=dtype, per_channel=m["per_channel"], kaczmarz=m["kaczmarz"],
                      key_norm="lognormal_norm" if m["kaczmarz"] else "unit", with_s0=True)
    rng = np.random.default_rng(seed + 7)
    x["do"] = rng.standard_normal((B, T, H, D[1])).astype(np.float32)
    x["ds"] = rng.standard_normal((B, H, D[0], D[1])).astype(np.float32) if with_ds else None
    return x


def _run(x, mode, dtype, *, scale=1.0, eps=1e-6):
    m = MODES[mode]
    d = to_dev(x, dtype)
    g = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], s0=d["s0"], ds_final=d["ds"],
                      scale=scale, eps=eps if m["kaczmarz"] else 0.0, **m)
    torch.cuda.synchronize()
    ref = oracle_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], ds_final=x["ds"], s0=x["s0"], scale=scale,
                     eps=eps if m["kaczmarz"] else 0.0, **m)
    errs = {key: rel(host(g[key]), ref[key]) for key in ("dq", "dk", "dv", "dg", "dbeta", "ds0")}
    return errs


@pytest.mark.parametrize("T", [1, 64, 100, 200])
@pytest.mark.parametrize("mode", ["gdn", "kda", "kla"])
def test_backward_parity(T, mode):
    x = _case(6000 + T, 2, T, 2, (128, 128), mode, "bf16")
    errs = _run(x, mode, "bf16")
    print(f"backward {mode} T={T}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v < _tol(mode, "bf16") for v in errs.values()), errs


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [(64, 64), (64, 128), (128, 64)])
@pytest.mark.parametrize("mode", ["gdn", "kda"])
def test_backward_widths_input_dtypes_and_scale(D, mode, dtype):
    """Widths of 64 (fp32 tiles); with bf16 inputs and scalar decay the
    kernels that form the decayed operands from k and q themselves."""
    x = _case(6100, 1, 90, 3, D, mode, dtype)
    errs = _run(x, mode, dtype, scale=D[0] ** -0.5)
    print(f"backward {mode} D={D} {dtype}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v < _tol(mode, dtype, D) for v in errs.values()), errs


@pytest.mark.parametrize("mode", ["gdn", "kda"])
def test_backward_strong_decay_and_no_final_gradient(mode):
    x = _case(6200, 1, 130, 2, (128, 128), mode, "bf16", with_ds=False)
    g = x["g"].copy()
    if mode == "kda":
        g[:, 20:90, :, 3:7] = -6.0
    else:
        g[:, 40:70] = -4.0
    x["g"] = g
    errs = _run(x, mode, "bf16")
    print(f"backward strong decay {mode}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v < _tol(mode, "bf16") for v in errs.values()), errs


def test_backward_deterministic_and_zero_length():
    x = _case(6300, 2, 150, 2, (128, 128), "kla", "bf16")
    d = to_dev(x, "bf16")
    kw = dict(s0=d["s0"], ds_final=d["ds"], kaczmarz=True, eps=1e-6)
    a = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], **kw)
    b = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], **kw)
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key
    # T = 0: only ds0 (= ds_final)
    z = {key: (val[:, :0].contiguous() if key not in ("s0", "ds") else val) for key, val in d.items()}
    r = gdr.chunk_bwd(z["q"], z["k"], z["v"], z["g"], z["beta"], z["do"], s0=z["s0"], ds_final=z["ds"])
    torch.cuda.synchronize()
    assert torch.equal(r["ds0"], d["ds"])


@pytest.mark.parametrize("variant", ["linear", "retnet", "gla"])
@pytest.mark.parametrize("T", [64, 150])
def test_backward_without_delta_rule(variant, T):
    """The additive write S = D S + k v^T (linear attention with g = 0,
    RetNet / Mamba-2, GLA): every gradient but beta's."""
    pc = variant == "gla"
    x = random_inputs(6400 + T, 2, T, 2, 128, 128, dtype="bf16", per_channel=pc, with_s0=True)
    if variant == "linear":
        x["g"] = np.zeros_like(x["g"])
    rng = np.random.default_rng(6401)
    x["do"] = rng.standard_normal((2, T, 2, 128)).astype(np.float32)
    x["ds"] = rng.standard_normal((2, 2, 128, 128)).astype(np.float32)
    d = to_dev(x, "bf16")
    g = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], None, d["do"], s0=d["s0"], ds_final=d["ds"],
                      per_channel=pc, scale=0.5, delta_off=True)
    torch.cuda.synchronize()
    ref = oracle_bwd(x["q"], x["k"], x["v"], x["g"], None, x["do"], ds_final=x["ds"], s0=x["s0"], scale=0.5,
                     per_channel=pc, delta_off=True)
    assert g["dbeta"] is None
    errs = {key: rel(host(g[key]), ref[key]) for key in ("dq", "dk", "dv", "dg", "ds0")}
    print(f"backward no delta {variant} T={T}: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v < _tol(variant, "bf16") for v in errs.values()), errs


@pytest.mark.parametrize("mode", ["gdn", "kda"])
def test_backward_more_walks_than_compute_units(mode):
    """fp32 inputs on 80 heads: the fp32-tile path launches its forward and
    reverse walks together, 320 of each (640 workgroups for 256 compute
    units), so most of them wait for a free unit; every gradient of every
    head against the oracle."""
    x = _case(6200, 4, 70, 20, (128, 128), mode, "f32")
    errs = _run(x, mode, "f32")
    print(f"backward {mode} 80 heads: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v < _tol(mode, "f32") for v in errs.values()), errs


@pytest.mark.parametrize("name,nheads", [("gdn_prefill", 2), ("kda_prefill", 1)])
def test_backward_full_workload_sampled(name, nheads):
    """The backward pass at the full size of a prefill workload (as the
    benchmark runs it: zero initial state, a standard-normal dL/do), every
    gradient of sampled (batch, head) pairs against the oracle run on that
    pair alone."""
    from gdr_inputs import WORKLOADS, prefill_inputs
    w = WORKLOADS[name]
    print(f"backward full workload {name}: inputs", flush=True)
    x = prefill_inputs(w)
    d = to_dev(x, w.dtype)
    rng = np.random.default_rng(12345)
    do = rng.standard_normal((w.B, w.T, w.H, w.Dv), dtype=np.float32)
    m = dict(per_channel=w.per_channel, kaczmarz=w.kaczmarz, eps=w.eps)
    g = gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], torch.from_numpy(do).to(DEV), need_ds0=False, **m)
    torch.cuda.synchronize()
    pairs = np.random.default_rng(7).choice(w.B * w.H, nheads, replace=False)
    for bh in pairs:
        b, h = divmod(int(bh), w.H)
        print(f"backward full workload {name}: oracle on (b={b}, h={h})", flush=True)
        sl = {key: x[key][b:b + 1, :, h:h + 1] for key in ("q", "k", "v", "g", "beta")}
        ref = oracle_bwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], do[b:b + 1, :, h:h + 1], **m)
        errs = {key: rel(host(g[key][b:b + 1, :, h:h + 1]), ref[key]) for key in ("dq", "dk", "dv", "dg", "dbeta")}
        print(f"backward full workload {name} (b={b}, h={h}): " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
        assert all(v < _tol("kda" if w.per_channel else "gdn", w.dtype) for v in errs.values()), errs


def test_backward_long_sequence_in_time_segments():
    """One 8,192-token sequence on two heads (128 chunks for two walks): the
    entering states are walked in four time segments, as the forward pass
    does for long sequences (chunk maps, entering states, then the segments);
    with an initial state and a final-state gradient, every gradient against
    the oracle."""
    x = _case(6600, 1, 8192, 2, (128, 128), "kla", "bf16")
    print("backward long sequence: GPU", flush=True)
    errs = _run(x, "kla", "bf16")
    print("backward long sequence: " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    assert all(v < _tol("kla", "bf16") for v in errs.values()), errs


def _packed_case(seed, lens, H, D, mode):
    m = MODES.get(mode, dict(per_channel=mode == "gla", kaczmarz=False))
    T = int(sum(lens))
    x = random_inputs(seed, 1, T, H, D, D, dtype="bf16", per_channel=m["per_channel"], kaczmarz=m["kaczmarz"],
                      key_norm="lognormal_norm" if m["kaczmarz"] else "unit", with_s0=False)
    x = {key: (val[0] if val is not None else None) for key, val in x.items()}
    rng = np.random.default_rng(seed + 3)
    N = len(lens)
    x["s0"] = (rng.standard_normal((N, H, D, D)) * 0.1).astype(np.float32)
    x["do"] = rng.standard_normal((T, H, D)).astype(np.float32)
    x["ds"] = rng.standard_normal((N, H, D, D)).astype(np.float32)
    return x, np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)


@pytest.mark.parametrize("mode", ["gdn", "kda", "kla", "retnet"])
def test_backward_varlen_matches_each_sequence_alone(mode):
    """A packed batch with an empty sequence, a one-token one, a full chunk
    and ragged tails: every gradient of every sequence equals the oracle's
    for that sequence alone."""
    delta_off = mode == "retnet"
    m = MODES.get(mode, dict(per_channel=False, kaczmarz=False))
    lens = [0, 1, 64, 100, 200, 130]
    x, cu = _packed_case(6500 + len(mode), lens, 2, 128, mode)
    d = to_dev({key: val for key, val in x.items()}, "bf16")
    eps = 1e-6 if m["kaczmarz"] else 0.0
    g = gdr.chunk_bwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], d["do"], torch.from_numpy(cu).to(DEV),
                             s0=d["s0"], ds_final=d["ds"], eps=eps, scale=0.75, delta_off=delta_off, **m)
    torch.cuda.synchronize()
    keys = ("dq", "dk", "dv", "dg") + (() if delta_off else ("dbeta",))
    for n in range(len(lens)):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:  # nothing to differentiate: dL/ds0 = dL/ds_final
            assert torch.equal(g["ds0"][n], d["ds"][n]), n
            continue
        sl = {key: x[key][None, a:b] for key in ("q", "k", "v", "g", "beta")}
        ref = oracle_bwd(sl["q"], sl["k"], sl["v"], sl["g"], None if delta_off else sl["beta"],
                         x["do"][None, a:b], ds_final=x["ds"][n:n + 1], s0=x["s0"][n:n + 1], scale=0.75, eps=eps,
                         delta_off=delta_off, **m)
        errs = {key: rel(host(g[key][a:b]), ref[key][0]) for key in keys}
        errs["ds0"] = rel(host(g["ds0"][n]), ref["ds0"][0])
        print(f"backward varlen {mode} sequence {n} (length {b - a}): "
              + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
        assert all(v < _tol(mode, "bf16") for v in errs.values()), (n, errs)
