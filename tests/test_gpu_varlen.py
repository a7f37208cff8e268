"""Packed batches of sequences of different lengths (gdr_chunk_fwd_varlen)
against the fp64 oracle run on each sequence alone."""
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


def _packed(seed, lens, H, D, mode, dtype, with_s0=True):
    """Inputs of len(lens) sequences packed along one token axis, and cu_seqlens."""
    m = MODES[mode]
    T = int(sum(lens))
    x = random_inputs(seed, 1, T, H, D, D, dtype=dtype, per_channel=m["per_channel"], kaczmarz=m["kaczmarz"],
                      key_norm="lognormal_norm" if m["kaczmarz"] else "unit", with_s0=False)
    x = {key: (val[0] if val is not None else None) for key, val in x.items()}
    rng = np.random.default_rng(seed + 1)
    x["s0"] = (rng.standard_normal((len(lens), H, D, D)) * 0.1).astype(np.float32) if with_s0 else None
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return x, cu


def _run(x, cu, mode, dtype, *, algo="auto", o_dtype=torch.float32, delta_off=False, scale=1.0, eps=1e-6):
    m = MODES[mode]
    d = to_dev(x, dtype)
    cu_d = torch.from_numpy(cu).to(DEV)
    o, s = gdr.chunk_fwd_varlen(d["q"], d["k"], d["v"], d["g"], d["beta"], cu_d, s0=d["s0"], o_dtype=o_dtype,
                                algo=algo, eps=eps if m["kaczmarz"] else 0.0, delta_off=delta_off, scale=scale,
                                **m)
    torch.cuda.synchronize()
    return o, s


def _ref(x, cu, mode, *, delta_off=False, scale=1.0, eps=1e-6):
    """The oracle on each sequence alone (a batch of one)."""
    m = MODES[mode]
    N = len(cu) - 1
    T, H = x["q"].shape[:2]
    o = np.zeros((T, H, x["v"].shape[2]))
    s = []
    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        sl = {key: x[key][None, a:b] for key in ("q", "k", "v", "g", "beta")}
        s0 = x["s0"][n:n + 1] if x["s0"] is not None else None
        on, sn = oracle.oracle_fwd(sl["q"], sl["k"], sl["v"], sl["g"], sl["beta"], s0=s0, scale=scale,
                                   eps=eps if m["kaczmarz"] else 0.0, delta_off=delta_off, **m)
        o[a:b] = on[0]
        s.append(sn[0])
    return o, np.stack(s)


@pytest.mark.parametrize("algo", ["vector", "matrix"])
@pytest.mark.parametrize("mode", ["gdn", "kda", "kla"])
def test_varlen_parity(algo, mode):
    """Lengths with an empty sequence, a single token, a partial chunk, exact
    chunks and several chunks with a ragged tail."""
    lens = [130, 0, 1, 64, 63, 200, 5]
    x, cu = _packed(5000, lens, 3, 128, mode, "bf16")
    o, s = _run(x, cu, mode, "bf16", algo=algo)
    o_ref, s_ref = _ref(x, cu, mode)
    eo, es = rel(host(o), o_ref), rel(host(s), s_ref)
    print(f"varlen {algo} {mode}: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]
    # the empty sequence keeps its initial state
    np.testing.assert_array_equal(host(s)[1], x["s0"][1])


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("bf16", 64)])
def test_varlen_vector_path_other_widths(dtype, D):
    lens = [70, 3, 129]
    x, cu = _packed(5100, lens, 2, D, "gdn", dtype)
    o, s = _run(x, cu, "gdn", dtype, algo="auto")
    o_ref, s_ref = _ref(x, cu, "gdn")
    assert rel(host(o), o_ref) < TOL[dtype] and rel(host(s), s_ref) < TOL[dtype]


@pytest.mark.parametrize("algo", ["vector", "matrix"])
@pytest.mark.parametrize("mode", ["gdn", "kda"])
def test_varlen_equal_lengths_match_fixed_batch(algo, mode):
    """B sequences of one length packed are the fixed-length batch: the same
    arithmetic per chunk, so the same bits."""
    B, T, H = 3, 150, 2
    x = random_inputs(5200, B, T, H, 128, 128, dtype="bf16", per_channel=MODES[mode]["per_channel"],
                      with_s0=True)
    d = to_dev(x, "bf16")
    o_f, s_f = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], s0=d["s0"], o_dtype=torch.float32,
                             algo=algo, **MODES[mode])
    cu = torch.arange(0, B * T + 1, T, dtype=torch.int32, device=DEV)
    flat = {key: d[key].reshape((B * T,) + tuple(d[key].shape[2:])) for key in ("q", "k", "v", "g", "beta")}
    o_p, s_p = gdr.chunk_fwd_varlen(flat["q"], flat["k"], flat["v"], flat["g"], flat["beta"], cu, s0=d["s0"],
                                    o_dtype=torch.float32, algo=algo, **MODES[mode])
    torch.cuda.synchronize()
    assert torch.equal(o_p.reshape(o_f.shape), o_f) and torch.equal(s_p, s_f)


@pytest.mark.parametrize("variant", ["retnet", "gla"])
def test_varlen_without_delta_rule_bf16_output(variant):
    mode = "kda" if variant == "gla" else "gdn"
    lens = [100, 17, 0, 64]
    x, cu = _packed(5300, lens, 2, 128, mode, "bf16")
    sc = 128 ** -0.5
    o, s = _run(x, cu, mode, "bf16", algo="matrix", o_dtype=torch.bfloat16, delta_off=True, scale=sc)
    o_ref, s_ref = _ref(x, cu, mode, delta_off=True, scale=sc)
    assert rel(host(o), o_ref) < TOL["bf16"] and rel(host(s), s_ref) < TOL["bf16"]


def test_varlen_many_short_sequences_and_zero_start():
    """Serving-shaped batch: 40 requests of 1..90 tokens, no initial state."""
    rng = np.random.default_rng(5400)
    lens = [int(v) for v in rng.integers(1, 91, 40)]
    x, cu = _packed(5400, lens, 4, 128, "gdn", "bf16", with_s0=False)
    o, s = _run(x, cu, "gdn", "bf16", algo="matrix")
    o_ref, s_ref = _ref(x, cu, "gdn")
    eo, es = rel(host(o), o_ref), rel(host(s), s_ref)
    print(f"varlen 40 short sequences: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]


@pytest.mark.parametrize("algo", ["vector", "matrix"])
def test_varlen_malformed_offsets_are_clamped(algo):
    """Offsets out of order or out of range are read as their clamped form
    (each entry in [0, T], at least the one before it): the call gives exactly
    the results of those offsets and never touches memory out of bounds."""
    lens = [50, 80, 30]
    x, _ = _packed(5500, lens, 2, 128, "gdn", "bf16", with_s0=False)
    T = sum(lens)
    bad = np.array([-7, 50, 20, 130, 10 ** 6], dtype=np.int32)   # decreasing, then past the end
    clamped = np.maximum.accumulate(np.clip(bad, 0, T)).astype(np.int32)
    assert list(clamped) == [0, 50, 50, 130, 160]
    o_bad, s_bad = _run(x, bad, "gdn", "bf16", algo=algo)
    o_ok, s_ok = _run(x, clamped, "gdn", "bf16", algo=algo)
    assert torch.equal(s_bad, s_ok) and torch.equal(o_bad, o_ok)


@pytest.mark.parametrize("mode", list(MODES))
def test_varlen_results_do_not_depend_on_the_walk_order(mode):
    """The walks of a packed batch run longest sequence first.  A sequence's
    outputs and final state are the same bits wherever it sits in the batch:
    the batch and a permutation of it agree sequence by sequence."""
    lens = [5, 300, 64, 0, 130, 1, 257, 64]
    perm = [3, 1, 6, 0, 7, 5, 2, 4]
    x, cu = _packed(5600 + len(mode), lens, 2, 128, mode, "bf16")
    y = {key: np.concatenate([x[key][cu[n]:cu[n + 1]] for n in perm]) for key in ("q", "k", "v", "g", "beta")}
    y["s0"] = x["s0"][perm]
    cu_p = np.concatenate([[0], np.cumsum([lens[n] for n in perm])]).astype(np.int32)
    o, s = _run(x, cu, mode, "bf16", algo="matrix")
    o_p, s_p = _run(y, cu_p, mode, "bf16", algo="matrix")
    for i, n in enumerate(perm):
        assert torch.equal(s_p[i], s[n]), (mode, n)
        assert torch.equal(o_p[cu_p[i]:cu_p[i + 1]], o[cu[n]:cu[n + 1]]), (mode, n)
    o_ref, s_ref = _ref(x, cu, mode)
    assert rel(host(o), o_ref) < TOL["bf16"] and rel(host(s), s_ref) < TOL["bf16"]


@pytest.mark.parametrize("algo", ["vector", "matrix"])
def test_varlen_more_sequences_than_the_sorted_order(algo):
    """1100 sequences: more than the table sorts into its longest-first order
    (1024), so the walks run in sequence order; the results are the same."""
    rng = np.random.default_rng(5700)
    lens = [int(v) for v in rng.integers(0, 40, 1100)]
    lens[17], lens[1099] = 200, 130
    x, cu = _packed(5700, lens, 1, 128, "gdn", "bf16")
    o, s = _run(x, cu, "gdn", "bf16", algo=algo)
    o_ref, s_ref = _ref(x, cu, "gdn")
    eo, es = rel(host(o), o_ref), rel(host(s), s_ref)
    print(f"varlen 1100 sequences {algo}: rel o {eo:.2e} S {es:.2e}")
    assert eo < TOL["bf16"] and es < TOL["bf16"]
