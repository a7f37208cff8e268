"""The blog summary's chunked algebra (numpy fp64) against the token recurrence
(the C oracle).  The page states the chunked schedule gives exactly the state
and outputs of the token-by-token one, so the two must agree to rounding."""
import numpy as np
import pytest

import oracle
from oracle.chunk_form import chunk_fwd
from gdr_inputs import random_inputs


def _rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


@pytest.mark.parametrize("mode", ["gdn", "kda", "kla"])
@pytest.mark.parametrize("chunk,T", [(16, 100), (64, 150), (64, 64), (64, 1), (8, 37)])
def test_chunk_form_equals_recurrence(mode, chunk, T):
    per_channel = mode == "kda"
    kaczmarz = mode == "kla"
    x = random_inputs(100 + T + chunk, 2, T, 2, 16, 12, dtype="bf16", per_channel=per_channel,
                      kaczmarz=kaczmarz, key_norm="lognormal_norm" if kaczmarz else "unit",
                      with_s0=True, gate_mult=0.3)
    kw = dict(per_channel=per_channel, kaczmarz=kaczmarz, eps=1e-6 if kaczmarz else 0.0,
              scale=0.7, s0=x["s0"])
    o_r, s_r = oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], **kw)
    o_c, s_c = chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], chunk=chunk, **kw)
    assert _rel(o_c, o_r) < 1e-12
    assert _rel(s_c, s_r) < 1e-12


def test_chunk_form_strong_decay():
    """g = -5 per token per channel: every in-chunk decay factor stays <= 1."""
    x = random_inputs(7, 1, 40, 1, 8, 8, dtype="f32", per_channel=True)
    g = np.full_like(x["g"], -5.0)
    o_r, s_r = oracle.oracle_fwd(x["q"], x["k"], x["v"], g, x["beta"], per_channel=True)
    o_c, s_c = chunk_fwd(x["q"], x["k"], x["v"], g, x["beta"], chunk=16, per_channel=True)
    assert np.all(np.isfinite(o_c))
    np.testing.assert_allclose(o_c, o_r, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s_c, s_r, rtol=1e-10, atol=1e-12)
