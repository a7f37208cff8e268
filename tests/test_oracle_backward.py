"""The backward oracle (reverse mode over a float64 torch copy of the token
recurrence) against what fixes a gradient without it: central finite
differences of the C oracle (an independent forward implementation), and a
closed form.  CPU only."""
import numpy as np
import pytest

import oracle
from oracle.backward import oracle_bwd


def _dyadic(rng, shape, scale=1.0, bits=6):
    """Values with few significant bits, so x +- 2^-8 is exact in float32
    (the C oracle reads float32 inputs)."""
    return (np.round(rng.standard_normal(shape) * scale * 2 ** bits) / 2 ** bits).astype(np.float64)


def _inputs(mode, seed=3):
    rng = np.random.default_rng(seed)
    B, T, H, Dk, Dv = 1, 7, 2, 4, 3
    x = dict(q=_dyadic(rng, (B, T, H, Dk)), k=_dyadic(rng, (B, T, H, Dk), 0.5), v=_dyadic(rng, (B, T, H, Dv)),
             s0=_dyadic(rng, (B, H, Dk, Dv), 0.3))
    gshape = (B, T, H, Dk) if mode in ("kda", "gla") else (B, T, H)
    x["g"] = -np.abs(_dyadic(rng, gshape, 0.3)) - 2.0 ** -5
    x["beta"] = np.abs(_dyadic(rng, (B, T, H), 0.4)) + 0.25
    x["do"] = _dyadic(rng, (B, T, H, Dv))
    x["ds"] = _dyadic(rng, (B, H, Dk, Dv))
    return x


MODES = {"gdn": dict(per_channel=False, kaczmarz=False),
         "kda": dict(per_channel=True, kaczmarz=False),
         "kla": dict(per_channel=False, kaczmarz=True, eps=0.125),
         "retnet": dict(per_channel=False, delta_off=True),
         "gla": dict(per_channel=True, delta_off=True)}


def _loss(x, m, scale):
    o, s = oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], s0=x["s0"], scale=scale, **m)
    return float(np.sum(o * x["do"]) + np.sum(s * x["ds"]))


@pytest.mark.parametrize("mode", list(MODES))
def test_gradients_match_finite_differences_of_the_c_oracle(mode):
    """Every element of every input: Richardson-extrapolated central
    differences (steps 2^-7 and 2^-8, exact in float32) of
    L = sum(o do) + sum(S_T dS) through the C oracle."""
    m = MODES[mode]
    scale = 0.75
    x = _inputs(mode)
    grads = oracle_bwd(x["q"], x["k"], x["v"], x["g"], x["beta"], x["do"], ds_final=x["ds"], s0=x["s0"],
                       scale=scale, **m)
    names = {"q": "dq", "k": "dk", "v": "dv", "g": "dg", "beta": "dbeta", "s0": "ds0"}
    if m.get("delta_off"):
        del names["beta"]
    for key, gname in names.items():
        fd = np.zeros_like(x[key])
        for idx in np.ndindex(x[key].shape):
            def central(h):
                xp = {kk: vv.copy() for kk, vv in x.items()}
                xm = {kk: vv.copy() for kk, vv in x.items()}
                xp[key][idx] += h
                xm[key][idx] -= h
                return (_loss(xp, m, scale) - _loss(xm, m, scale)) / (2 * h)
            d1, d2 = central(2.0 ** -7), central(2.0 ** -8)
            fd[idx] = (4 * d2 - d1) / 3
        got = grads[gname]
        err = np.linalg.norm(got - fd) / max(np.linalg.norm(fd), 1e-30)
        assert err < 1e-7, (mode, key, err)


def test_gradients_without_writes_closed_form():
    """beta = 0: no write, S_t = exp(G_t) s0 with G_t = g_0 + ... + g_t, and
    o_t = scale exp(G_t) s0^T q_t, so dq_t = scale exp(G_t) s0 do_t,
    ds0 = scale sum_t exp(G_t) q_t do_t^T, dg_m = sum_{t >= m} scale exp(G_t)
    q_t^T s0 do_t, and dk = dv = 0."""
    rng = np.random.default_rng(11)
    B, T, H, Dk, Dv = 1, 9, 1, 5, 3
    q = rng.standard_normal((B, T, H, Dk))
    k = rng.standard_normal((B, T, H, Dk))
    v = rng.standard_normal((B, T, H, Dv))
    g = -rng.uniform(0.01, 0.3, (B, T, H))
    s0 = rng.standard_normal((B, H, Dk, Dv))
    do = rng.standard_normal((B, T, H, Dv))
    scale = 1.5
    r = oracle_bwd(q, k, v, g, np.zeros((B, T, H)), do, s0=s0, scale=scale)
    G = np.cumsum(g[0, :, 0])
    S0 = s0[0, 0]
    dq = np.stack([scale * np.exp(G[t]) * S0 @ do[0, t, 0] for t in range(T)])
    ds0 = sum(scale * np.exp(G[t]) * np.outer(q[0, t, 0], do[0, t, 0]) for t in range(T))
    per_t = np.array([scale * np.exp(G[t]) * q[0, t, 0] @ S0 @ do[0, t, 0] for t in range(T)])
    dg = np.cumsum(per_t[::-1])[::-1]
    np.testing.assert_allclose(r["dq"][0, :, 0], dq, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["ds0"][0, 0], ds0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(r["dg"][0, :, 0], dg, rtol=1e-12, atol=1e-12)
    assert not r["dk"].any() and not r["dv"].any()
