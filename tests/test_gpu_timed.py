"""The measurement entry points (gdr_chunk_fwd_stage_timed,
gdr_recurrent_step_timed): results identical to the untimed calls, and the
events the kernels record give a positive duration.  The results are pinned to
the oracle through the untimed calls' own tests."""
import pytest
import torch

import gated_delta_rule_26_amd as gdr
from gdr_inputs import random_inputs
from tests.gpu_util import DEV, to_dev

pytestmark = pytest.mark.gpu


def _events(n):
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()  # create it
    torch.cuda.synchronize()
    return evs


@pytest.mark.parametrize("mode,T,algo", [("gdn", 200, "matrix"), ("kda", 130, "matrix"), ("kla", 8200, "matrix"),
                                         ("gdn", 100, "vector")])
def test_timed_stages_match_the_untimed_pass(mode, T, algo):
    """Both stages through the timed entry point equal gdr_chunk_fwd bit for
    bit; the long sequence takes the time-segmented walk (transfer, combine,
    walk), whose first and last launches record the events."""
    pc, kz = mode == "kda", mode == "kla"
    x = random_inputs(7100 + T, 1, T, 4, 128, 128, dtype="bf16", per_channel=pc, kaczmarz=kz,
                      key_norm="lognormal_norm" if kz else "unit", with_s0=True)
    d = to_dev(x, "bf16")
    kw = dict(per_channel=pc, kaczmarz=kz, eps=1e-6 if kz else 0.0, o_dtype=torch.float32, algo=algo, s0=d["s0"])
    o_ref, s_ref = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], **kw)
    desc = gdr.make_desc(1, T, 4, 128, 128, qkv_dtype=torch.bfloat16, o_dtype=torch.float32, per_channel=pc,
                         kaczmarz=kz, eps=kw["eps"], algo=algo)
    ws = torch.empty(gdr.chunk_fwd_workspace_size(desc), dtype=torch.uint8, device=DEV)
    o = torch.empty_like(o_ref)
    s = torch.empty_like(s_ref)
    ev = _events(4)
    gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], stage=0, events=(ev[0], ev[1]), workspace=ws, o=o,
                  s_final=s, **kw)
    gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], stage=1, events=(ev[2], ev[3]), workspace=ws, o=o,
                  s_final=s, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
    assert ev[0].elapsed_time(ev[1]) > 0 and ev[2].elapsed_time(ev[3]) > 0
    assert ev[0].elapsed_time(ev[3]) >= ev[2].elapsed_time(ev[3])


def test_timed_decode_step_matches_the_untimed_step():
    x = random_inputs(7200, 8, 1, 4, 128, 128, dtype="bf16", with_s0=True)
    d = to_dev(x, "bf16")
    args = [d[key][:, 0].contiguous() for key in ("q", "k", "v", "g", "beta")]
    s_ref = d["s0"].clone()
    s = d["s0"].clone()
    o_ref = gdr.recurrent_step(*args, s_ref, o_dtype=torch.float32)
    ev = _events(2)
    o = gdr.recurrent_step(*args, s, o_dtype=torch.float32, events=(ev[0], ev[1]))
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(s, s_ref)
    assert ev[0].elapsed_time(ev[1]) > 0


def test_events_must_exist():
    x = random_inputs(7300, 2, 1, 2, 128, 128, dtype="bf16", with_s0=True)
    d = to_dev(x, "bf16")
    args = [d[key][:, 0].contiguous() for key in ("q", "k", "v", "g", "beta")]
    fresh = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))  # never recorded
    with pytest.raises(ValueError):
        gdr.recurrent_step(*args, d["s0"].clone(), events=fresh)
