"""The fp64 oracle against what the pages fix (worked numbers, closed forms,
invariants, brute force).  CPU only."""
import numpy as np
import pytest

import oracle
from tests import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin, golden):
    if pins.needs_golden(pin):
        pin(oracle.oracle_fwd, golden)
    else:
        pin(oracle.oracle_fwd)


def test_threads_and_head_subsets_agree():
    from gdr_inputs import random_inputs
    x = random_inputs(3, 2, 70, 3, 16, 8, dtype="bf16", with_s0=True)
    o1, s1 = oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s0=x["s0"], threads=1)
    o4, s4 = oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s0=x["s0"], threads=4)
    np.testing.assert_array_equal(o1, o4)
    np.testing.assert_array_equal(s1, s4)
    heads = [4, 1]
    o2, s2 = oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s0=x["s0"], heads=heads)
    for bh in heads:
        b, h = divmod(bh, 3)
        np.testing.assert_array_equal(o2[b, :, h], o1[b, :, h])
        np.testing.assert_array_equal(s2[b, h], s1[b, h])
    assert np.isnan(o2[0, :, 0]).all()


def test_decode_is_recurrence_over_steps():
    from gdr_inputs import WORKLOADS, decode_inputs, decode_state0
    w = WORKLOADS["decode"].scaled(B=3, H=2, Dk=16, Dv=8)
    x = decode_inputs(w, steps=5)
    s0 = decode_state0(w)
    o, s = oracle.oracle_decode(x["q"], x["k"], x["v"], x["g"], x["beta"], s0)
    st = s0.astype(np.float64)
    for t in range(5):
        # one step at a time through the prefill entry with T = 1
        ot, st = oracle.oracle_fwd(x["q"][t][:, None], x["k"][t][:, None], x["v"][t][:, None],
                                   x["g"][t][:, None], x["beta"][t][:, None], s0=st)
        np.testing.assert_allclose(o[t], ot[:, 0], rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(s, st, rtol=1e-6, atol=1e-7)
