"""Seeded input generators: reproducible, bf16-exact, and shaped like the
five workloads."""
import numpy as np
import torch

from gdr_inputs import WORKLOADS, bf16_round, decode_step_inputs, decode_state0, prefill_inputs


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, -3.0e38], np.float32)]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(bf16_round(x), want)


def test_prefill_reproducible_and_bf16_exact():
    w = WORKLOADS["gdn_prefill"].scaled(B=1, T=130, H=2)
    a = prefill_inputs(w)
    b = prefill_inputs(w)
    for key in ("q", "k", "v", "g", "beta"):
        np.testing.assert_array_equal(a[key], b[key])
        assert a[key].dtype == np.float32
    for key in ("q", "k", "v"):
        np.testing.assert_array_equal(bf16_round(a[key]), a[key])
    # keys are unit vectors up to bf16 rounding
    nrm = np.linalg.norm(a["k"].astype(np.float64), axis=-1)
    assert np.all(np.abs(nrm - 1.0) < 1e-2)
    assert np.all(a["g"] <= 0) and a["g"].shape == (1, 130, 2)
    assert np.all((a["beta"] > 0) & (a["beta"] < 1))


def test_workload_shapes():
    w = WORKLOADS["kda_prefill"].scaled(B=1, T=70, H=1)
    x = prefill_inputs(w)
    assert x["g"].shape == (1, 70, 1, 128)
    w = WORKLOADS["kla_prefill"].scaled(T=300, H=2)
    x = prefill_inputs(w)
    nrm = np.linalg.norm(x["k"].astype(np.float64), axis=-1)
    assert nrm.std() > 0.2                 # lognormal key norms, not unit
    assert np.all((x["beta"] > 0) & (x["beta"] < 1))   # eta = sigmoid(N(1,1))
    w = WORKLOADS["gdn_tiny"]
    x = prefill_inputs(w)
    assert x["q"].shape == (1, 256, 1, 64)
    alpha = np.exp(x["g"].astype(np.float64))
    assert alpha.min() >= 0.9 - 1e-6 and alpha.max() <= 0.999 + 1e-6


def test_decode_steps_independent_and_reproducible():
    w = WORKLOADS["decode"].scaled(B=4, H=2)
    s3 = decode_step_inputs(w, 3)
    np.testing.assert_array_equal(s3["q"], decode_step_inputs(w, 3)["q"])
    assert not np.array_equal(s3["q"], decode_step_inputs(w, 4)["q"])
    s0 = decode_state0(w)
    assert s0.shape == (4, 2, 128, 128)
    assert abs(s0.std() - 0.02) < 1e-3
