#!/usr/bin/env python3
"""Benchmark of the gated delta-rule forward pass on one MI355X.

A step is one chunked prefill over the Gated DeltaNet workload (B4 H16 T4096,
d_k = d_v = 128, bf16 q/k/v, fp32 state, bf16 output, chunk 64): the
intra-chunk kernel then the state/output kernel, with the inputs resident in
HBM and the 256 MB last-level (Infinity) cache flushed before each timed step
by writing a 512 MiB buffer, so the step reads its inputs from HBM.  Kernel
times come from HIP events the kernels record themselves
(gdr_chunk_fwd_stage_timed: the first kernel records its begin, the last its
end), on the stream they are launched on.  The same steps with warm caches,
the fp32-output configuration, the other prefill workloads (tiny fp32, KDA
per-channel decay, KLA long sequence), the fused decode step (256 sequences,
and 512 sequences whose state is twice the last-level cache), the backward
pass and the serving entry points are timed beside it, and the fp64 oracle on
the host cores.

Prints ONE JSON line.  ``--gpus`` above 1 is refused: the benchmark runs on
one GPU (the path shards over (sequence, head) pairs with no communication).
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

C = 64
PEAK_BF16_MFMA = 2500.0      # TFLOP/s, MI355X dense bf16
PEAK_FP32_VALU = 157.3       # TFLOP/s, MI355X fp32 vector
PEAK_HBM = 8000.0            # GB/s, MI355X HBM3E
FLUSH_BYTES = 512 << 20      # twice the 256 MB last-level cache


# HBM bytes per launch from rocprofv3 FETCH_SIZE (x2.0) + WRITE_SIZE (x1.0), scaled by a 1 GiB device
# copy read in the same runs, by (algorithm, kernel, workload, output dtype).  Each figure holds only for
# the sources it was measured on: when the sha256 of those files (concatenated in order) differs, it is
# reported as null.
# The build script is part of each group: it holds the compiler options the kernels are built with.
_BUILD = "gated_delta_rule_26_amd/build.py"
_SCALAR = ("gated_delta_rule_26_amd/csrc/chunk_matrix.hip", "gated_delta_rule_26_amd/csrc/matrix_common.h", _BUILD)
_PER_CHANNEL = ("gated_delta_rule_26_amd/csrc/chunk_matrix_pc.hip", "gated_delta_rule_26_amd/csrc/matrix_common.h",
                _BUILD)
_DECODE = ("gated_delta_rule_26_amd/csrc/recurrent_step.hip", _BUILD)
_SHA_SCALAR = "56ddce87d2e9f9048edeb14b17576298c1243a1b1d50385eeb534ea256465355"
_SHA_PC = "33b1131f292acb6a99b56ad42a44c5b921576f955b5af34734db1d36c37f9f00"
_SHA_DECODE = "32418c0ee1020b20d96212e92a32fa306ea808bb4ec78f7b7f401d35e5af79d4"
MEASURED_TRAFFIC = {
    ("matrix", "state", "gdn_prefill", "bf16"): (_SCALAR, _SHA_SCALAR, (148662.5 * 2.0 + 69642.4) * 1024),
    ("matrix", "intra", "gdn_prefill", "bf16"): (_SCALAR, _SHA_SCALAR, (66989.6 * 2.0 + 100352.0) * 1024),
    ("matrix", "state", "gdn_prefill", "f32"): (_SCALAR, _SHA_SCALAR, (148655.4 * 2.0 + 135233.3) * 1024),
    ("matrix", "intra", "gdn_prefill", "f32"): (_SCALAR, _SHA_SCALAR, (66988.1 * 2.0 + 100352.0) * 1024),
    ("matrix", "state", "kda_prefill", "bf16"): (_PER_CHANNEL, _SHA_PC, (279781.7 * 2.0 + 93798.4) * 1024),
    ("matrix", "intra", "kda_prefill", "bf16"): (_PER_CHANNEL, _SHA_PC, (134521.8 * 2.0 + 493568.2) * 1024),
    # the state phase of the long sequence is three launches: the segment transfer walk, the
    # combine of the entering states and the per-segment walk
    ("matrix", "state", "kla_prefill", "bf16"): (_SCALAR, _SHA_SCALAR,
                                                 (729447.8 * 2.0 + 8192.0 + 15394.5 * 2.0 + 4096.0
                                                  + 1190059.2 * 2.0 + 525320.5) * 1024),
    ("matrix", "intra", "kla_prefill", "bf16"): (_SCALAR, _SHA_SCALAR, (656379.1 * 2.0 + 802816.0) * 1024),
    ("decode", "step", "decode", "f32"): (_DECODE, _SHA_DECODE, (132913.0 * 2.0 + 264729.0) * 1024),
    ("decode", "step", "decode_512", "f32"): (_DECODE, _SHA_DECODE, (265782.2 * 2.0 + 529423.2) * 1024),
}


# Matrix-core use of the dominant kernel from rocprofv3 counters: SQ_VALU_MFMA_BUSY_CYCLES over the kernel's
# duration x 1024 SIMDs x the shader clock from GRBM_GUI_ACTIVE (per XCD), and the MFMA flops it issued
# (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512) per second.  The issued flops count every bf16 hi/lo product, so they
# exceed the algorithmic flops.  (files, sha, busy fraction, issued TFLOP/s), as for the traffic.
MEASURED_MFMA = {
    ("matrix", "state", "gdn_prefill", "bf16"): (_SCALAR, _SHA_SCALAR, 0.206, 497.0),
    ("matrix", "state", "kda_prefill", "bf16"): (_PER_CHANNEL, _SHA_PC, 0.080, 200.4),
    # the long sequence: transfer + combine + walk, weighted by duration
    ("matrix", "state", "kla_prefill", "bf16"): (_SCALAR, _SHA_SCALAR, 0.255, 573.4),
}


def sources_sha(files) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def _current(entry):
    if entry is None:
        return None
    files, sha = entry[0], entry[1]
    try:
        return entry if sources_sha(files) == sha else None
    except OSError:
        return None


def measured_mfma(path_kind: str, kernel: str, workload: str, o_dtype: str = "f32"):
    """Counter-measured matrix-core busy fraction and issued TFLOP/s, or None if not measured on the current
    sources."""
    entry = _current(MEASURED_MFMA.get((path_kind, kernel, workload, o_dtype)))
    return None if entry is None else {"counter_busy_frac": entry[2], "issued_tflops": entry[3]}


def measured_traffic(path_kind: str, kernel: str, workload: str, o_dtype: str = "f32"):
    """Counter-measured HBM bytes per launch, or None if not measured on the current sources."""
    entry = _current(MEASURED_TRAFFIC.get((path_kind, kernel, workload, o_dtype)))
    return None if entry is None else entry[2]


def alg_flops_per_token_head(dk: int, dv: int) -> dict:
    """Algorithmic (triangle-aware) flops per token and head, by kernel.

    intra: R = beta.decay-weighted K K^T strictly below the diagonal
    ((C-1) dk), the causal read matrix A (diagonal kept, (C+1) dk), the
    triangular inverse (C^2/3) and W, U ((C+1)(dk + dv)).
    state: E = U - W S, the read (decayed Q) S and the update K^T E
    (2 dk dv each) plus the in-chunk read A E ((C+1) dv).
    """
    intra = (C - 1) * dk + (C + 1) * dk + C * C / 3.0 + (C + 1) * dk + (C + 1) * dv
    state = 6.0 * dk * dv + (C + 1) * dv
    return {"intra": intra, "state": state, "total": intra + state}


def alg_bytes_prefill(B, T, H, dk, dv, in_bytes=2, out_bytes=4, per_channel=False) -> float:
    """Minimal HBM bytes of one chunked pass: read q, k, v, g, beta once,
    write o and the final state once."""
    tok = B * T * H
    g_bytes = 4 * (dk if per_channel else 1)
    return tok * ((2 * dk + dv) * in_bytes + g_bytes + 4 + dv * out_bytes) + B * H * dk * dv * 4


def alg_bytes_state_kernel(B, T, H, dk, dv, in_bytes=2, out_bytes=4) -> float:
    """The state kernel's share of the pass's minimal bytes: q, k, v read once,
    o and the final state written once (the gates belong to the intra
    kernel; its second read of q and k, and the chunk records, are not
    algorithmic and appear only in the measured traffic)."""
    tok = B * T * H
    return tok * ((2 * dk + dv) * in_bytes + dv * out_bytes) + B * H * dk * dv * 4


def decode_bytes_per_step(N, H, dk, dv, in_bytes=2, out_bytes=4) -> float:
    """Minimal HBM bytes of one decode step: the state in and out, plus the
    token's q, k, v, g, beta and the output."""
    return N * H * (2 * dk * dv * 4 + (2 * dk + dv) * in_bytes + 8 + dv * out_bytes)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def median(xs):
    ys = sorted(xs)
    return ys[len(ys) // 2] if ys else float("nan")


def mean(xs):
    return sum(xs) / len(xs) if xs else float("nan")


def quantile(xs, f):
    """Nearest-rank quantile: the smallest value with at least a fraction f of the values at or below it."""
    ys = sorted(xs)
    if not ys:
        return float("nan")
    return ys[min(len(ys) - 1, max(0, int(-(-f * len(ys) // 1)) - 1))]


def _to_device(x, w, dev):
    import torch
    d = {}
    for key, val in x.items():
        if val is None:
            continue
        t = torch.from_numpy(val).to(dev)
        d[key] = t.to(torch.bfloat16) if key in ("q", "k", "v") and w.dtype == "bf16" else t
    return d


def bench_prefill(w, x, steps, warmup, algo, o_dtype):
    """Timed chunked passes of workload w on inputs x (numpy): `steps` with warm caches (wall clock
    around them, and per-step events), then `steps` each after a cache flush (per-step events; the
    flush is not inside the events).  Returns the per-step times and the last pass's o and final
    state (on the device)."""
    import torch
    import gated_delta_rule_26_amd as gdr

    dev = torch.device("cuda:0")
    d = _to_device(x, w, dev)
    B, T, H, Dk, Dv = w.B, w.T, w.H, w.Dk, w.Dv
    odt = torch.float32 if o_dtype == "f32" else torch.bfloat16
    qdt = d["q"].dtype
    o = torch.empty((B, T, H, Dv), dtype=odt, device=dev)
    s = torch.empty((B, H, Dk, Dv), dtype=torch.float32, device=dev)
    desc = gdr.make_desc(B, T, H, Dk, Dv, qkv_dtype=qdt, o_dtype=odt, per_channel=w.per_channel,
                         kaczmarz=w.kaczmarz, eps=w.eps, algo=algo)
    ws = torch.empty(max(1, gdr.chunk_fwd_workspace_size(desc)), dtype=torch.uint8, device=dev)
    kw = dict(per_channel=w.per_channel, kaczmarz=w.kaczmarz, eps=w.eps, o=o, s_final=s, o_dtype=odt,
              algo=algo, workspace=ws)

    def step(ev=None):
        gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], stage=0, events=ev and (ev[0], ev[1]), **kw)
        gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], stage=1, events=ev and (ev[2], ev[3]), **kw)

    def new_events(n):
        # per step: the intra kernel's begin and end, the state phase's begin and end, recorded by the
        # kernels themselves (gdr_chunk_fwd_stage_timed); each is recorded once here so that it exists
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n)]
        for e in evs:
            for ev in e:
                ev.record()
        return evs

    def times(evs):
        return {"intra": [e[0].elapsed_time(e[1]) for e in evs], "state": [e[2].elapsed_time(e[3]) for e in evs],
                "step": [e[0].elapsed_time(e[3]) for e in evs]}

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = new_events(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    warm = times(evs)
    scratch = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
    cev = new_events(steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        scratch.fill_(i & 0xff)
        step(cev[i])
    torch.cuda.synchronize()
    cold_wall = time.perf_counter() - t0
    del scratch
    return {"warm": warm, "warm_wall_s": wall, "cold": times(cev), "cold_wall_s": cold_wall, "o": o, "s": s,
            "o_bytes": 4 if odt == torch.float32 else 2, "in_bytes": 2 if qdt == torch.bfloat16 else 4,
            "workspace_bytes": ws.numel()}


def resolve_algo(w, algo):
    """The path `algo` selects: auto takes the matrix-core kernels (bf16 MFMA for bf16 q/k/v at d128,
    fp32 MFMA tiles otherwise)."""
    return "matrix" if algo == "auto" else algo


def prefill_block(w, pre, algo, o_dtype):
    """Throughput, per-kernel times and the roofline of the dominant kernel for one prefill
    configuration, with the cold-cache step as the headline figure."""
    tok_heads = w.B * w.T * w.H
    fl = alg_flops_per_token_head(w.Dk, w.Dv)
    cold, warm = pre["cold"], pre["warm"]
    step_ms = mean(cold["step"])
    intra_ms, state_ms = mean(cold["intra"]), mean(cold["state"])
    dom = "state" if state_ms >= intra_ms else "intra"
    dom_ms = state_ms if dom == "state" else intra_ms
    dom_flops = fl[dom] * tok_heads
    mfma_tflops = dom_flops / (dom_ms * 1e-3) / 1e12
    # bf16 inputs at d128 run on bf16 MFMA; every other input on fp32 MFMA tiles, whose peak equals the
    # fp32 vector peak on MI355X (157.3 TFLOP/s)
    bf16_kernels = pre["in_bytes"] == 2 and w.Dk == 128 and w.Dv == 128
    mfma_peak = PEAK_BF16_MFMA if bf16_kernels else PEAK_FP32_VALU
    # The bf16 pass's algorithmic intensity (~110 flop/B at d128 with fp32 o, ~135 with bf16 o) is below
    # MI355X's ridge (2.5 PFLOP/s / 8 TB/s = 312 flop/B), so the roof that bounds the bf16 matrix path is
    # HBM: the state kernel against its algorithmic bytes, with its MFMA fraction beside it.  The vector
    # path (fp32 ALU) is bounded by its ALU peak.
    if algo == "matrix" and not bf16_kernels:
        # the fp32-tile kernels: 103 flop/B on fp32 data, above the fp32 matrix ridge (157.3 / 8 = 20 flop/B)
        roof = {"bound": "mfma", "achieved": mfma_tflops, "peak": PEAK_FP32_VALU, "unit": "TFLOP/s",
                "frac": mfma_tflops / PEAK_FP32_VALU, "alg_bytes_per_launch": None}
    elif algo == "matrix" and dom == "state":
        dom_bytes = alg_bytes_state_kernel(w.B, w.T, w.H, w.Dk, w.Dv, pre["in_bytes"], pre["o_bytes"])
        achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM, "unit": "GB/s", "frac": achieved / PEAK_HBM,
                "alg_bytes_per_launch": dom_bytes}
    elif algo == "matrix":
        roof = {"bound": "mfma", "achieved": mfma_tflops, "peak": PEAK_BF16_MFMA, "unit": "TFLOP/s",
                "frac": mfma_tflops / PEAK_BF16_MFMA, "alg_bytes_per_launch": None}
    else:
        roof = {"bound": "alu", "achieved": mfma_tflops, "peak": PEAK_FP32_VALU, "unit": "TFLOP/s",
                "frac": mfma_tflops / PEAK_FP32_VALU, "alg_bytes_per_launch": None}
    roof.update({"kernel": f"{dom} ({algo} path)", "traffic": measured_traffic(algo, dom, w.name, o_dtype),
                 "alg_flops_per_launch": dom_flops, "avg_launch_ms": dom_ms,
                 "mfma_view": {"achieved_tflops": mfma_tflops, "peak_tflops": mfma_peak,
                               "frac": mfma_tflops / mfma_peak,
                               "counters": measured_mfma(algo, dom, w.name, o_dtype)}})
    total_tflops = fl["total"] * tok_heads / (step_ms * 1e-3) / 1e12
    abytes = alg_bytes_prefill(w.B, w.T, w.H, w.Dk, w.Dv, pre["in_bytes"], pre["o_bytes"], w.per_channel)
    warm_ms = pre["warm_wall_s"] / len(warm["step"]) * 1e3
    return {
        "workload": f"{w.name}: chunked prefill B{w.B} H{w.H} T{w.T} d_k={w.Dk} d_v={w.Dv}, {w.dtype} q/k/v, "
                    f"fp32 state, {o_dtype} output, chunk {C}, {w.decay} decay, {w.beta_mode} beta",
        "algo": algo, "o_dtype": o_dtype,
        "tokens_per_s": w.B * w.T / (step_ms * 1e-3), "ms_per_step": step_ms,
        "ms_per_step_median": median(cold["step"]),
        "ms_per_step_p10": quantile(cold["step"], 0.1), "ms_per_step_p90": quantile(cold["step"], 0.9),
        "intra_ms": intra_ms, "state_ms": state_ms,
        "timing": "cold caches: 512 MiB written before each step (outside the events); events recorded by the "
                  "first and last kernels of each stage",
        "warm": {"ms_per_step_wall": warm_ms, "tokens_per_s_wall": w.B * w.T / (warm_ms * 1e-3),
                 "event_step_ms": mean(warm["step"]), "intra_ms": mean(warm["intra"]),
                 "state_ms": mean(warm["state"])},
        "roofline": roof,
        "alg_tflops": total_tflops, "frac_bf16_mfma_peak": total_tflops / PEAK_BF16_MFMA,
        "alg_bytes": abytes, "alg_gbps": abytes / (step_ms * 1e-3) / 1e9,
        "frac_hbm_peak": abytes / (step_ms * 1e-3) / 1e9 / PEAK_HBM,
        "alg_flops_per_token_head": fl, "workspace_bytes": pre["workspace_bytes"],
    }


def backward_label(w) -> str:
    tiles = ("fp32 tiles" if w.per_channel or w.dtype != "bf16" or w.Dk != 128 or w.Dv != 128
             else "bf16 tiles with hi/lo split fp32 operands")
    return f"{w.name}: gdr_chunk_bwd on the same inputs, standard-normal dL/do, fp32 gradients ({tiles})"


def bench_backward(w, x, steps, warmup):
    """The backward pass (gdr_chunk_bwd) on the prefill workload's inputs
    with a seeded standard-normal dL/do; events around each call."""
    import numpy as np
    import torch
    import gated_delta_rule_26_amd as gdr

    dev = torch.device("cuda:0")
    d = _to_device({key: x[key] for key in ("q", "k", "v", "g", "beta")}, w, dev)
    rng = np.random.default_rng(12345)
    d_o = torch.from_numpy(rng.standard_normal((w.B, w.T, w.H, w.Dv), dtype=np.float32)).to(dev)
    desc = gdr.make_desc(w.B, w.T, w.H, w.Dk, w.Dv, qkv_dtype=d["q"].dtype, o_dtype=torch.float32,
                         per_channel=w.per_channel, kaczmarz=w.kaczmarz, eps=w.eps)
    ws = torch.empty(gdr.chunk_bwd_workspace_size(desc), dtype=torch.uint8, device=dev)
    kw = dict(per_channel=w.per_channel, kaczmarz=w.kaczmarz, eps=w.eps, workspace=ws, need_ds0=False)
    for _ in range(warmup):
        gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d_o, **kw)
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        gdr.chunk_bwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d_o, **kw)
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return {"ms_per_step_median": median(per), "ms_per_step": mean(per),
            "workspace_bytes": ws.numel(), "steps": steps}


def bench_decode(w, steps, distinct, warmup=10):
    """`steps` fused decode steps on the state of w (updated in place), cycling `distinct` resident
    inputs after `warmup` untimed steps.  Returns per-step kernel and begin-to-begin times, the
    initial state, the inputs used in order and the final state and last output (device)."""
    import torch
    import gated_delta_rule_26_amd as gdr
    from gdr_inputs import decode_state0, decode_step_inputs

    dev = torch.device("cuda:0")
    s0 = decode_state0(w)
    state = torch.from_numpy(s0).to(dev)
    host_inputs = [decode_step_inputs(w, i) for i in range(distinct)]
    inputs = []
    for x in host_inputs:
        dd = {key: torch.from_numpy(val).to(dev) for key, val in x.items()}
        for key in ("q", "k", "v"):
            dd[key] = dd[key].to(torch.bfloat16)
        inputs.append(dd)
    o = torch.empty((w.B, w.H, w.Dv), dtype=torch.float32, device=dev)
    kw = dict(per_channel=w.per_channel, kaczmarz=w.kaczmarz, eps=w.eps, o=o, o_dtype=torch.float32)
    for i in range(warmup):
        dd = inputs[i % distinct]
        gdr.recurrent_step(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], state, **kw)
    # per step the kernel's begin and end, recorded by the kernel (gdr_recurrent_step_timed); each
    # event is recorded once first so that it exists
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e in evs:
        e[0].record()
        e[1].record()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        dd = inputs[i % distinct]
        gdr.recurrent_step(dd["q"], dd["k"], dd["v"], dd["g"], dd["beta"], state, events=evs[i], **kw)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern = [e[0].elapsed_time(e[1]) for e in evs]
    step = [evs[i][0].elapsed_time(evs[i + 1][0]) for i in range(steps - 1)]  # begin to begin
    order = [i % distinct for i in range(warmup)] + [i % distinct for i in range(steps)]
    return {"wall_s": wall, "kernel_ms": kern, "step_ms": step, "s0": s0, "host_inputs": host_inputs,
            "order": order, "state": state, "o": o}


def decode_block(w, dec, steps, distinct, note):
    dms = mean(dec["step_ms"])        # per-step latency: kernel begin to kernel begin
    kms = mean(dec["kernel_ms"])      # the kernel alone
    dbytes = decode_bytes_per_step(w.B, w.H, w.Dk, w.Dv)
    gbps = dbytes / (kms * 1e-3) / 1e9
    state_mib = w.B * w.H * w.Dk * w.Dv * 4 / 2 ** 20
    return {
        "workload": f"decode: {w.B} sequences x H{w.H}, d_k=d_v={w.Dk}, bf16 q/k/v, fp32 state in place "
                    f"({state_mib:.0f} MiB{note}), scalar decay, given beta, fp32 output; {steps} steps cycling "
                    f"{distinct} resident inputs",
        "ms_per_step": dms, "ms_per_step_median": median(dec["step_ms"]), "tokens_per_s": w.B / (dms * 1e-3),
        "state_gbps_per_step": dbytes / (dms * 1e-3) / 1e9,
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": PEAK_HBM, "unit": "GB/s", "frac": gbps / PEAK_HBM,
                     "traffic": measured_traffic("decode", "step", w.name, "f32"),
                     "alg_bytes_per_launch": dbytes, "avg_launch_ms": kms},
    }


def serving_lengths(total, seed=2026, lo=64, hi=2048):
    """A seeded serving mix: lengths log-uniform in [lo, hi] tokens, drawn until they cover `total`
    tokens (the last one cut to fit)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    lens = []
    while sum(lens) < total:
        lens.append(min(int(round(float(np.exp(rng.uniform(np.log(lo), np.log(hi)))))), total - sum(lens)))
    return lens


def _timed_calls(fn, steps, warmup):
    """Mean and median ms per call over `steps` calls (events on torch's current stream, on which
    the binding launches), after `warmup` calls."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        fn()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return mean(per), median(per)


def bench_next_rows(w, x, steps, warmup, recurrent_tokens=8):
    """The serving and variant entry points on the prefill workload's tokens (whole calls, both
    stages): a packed batch of a serving mix of lengths (gdr_chunk_fwd_varlen), the same batch
    without the delta rule (gdr_chunk_fwd with delta_off), and T tokens per call on the recurrent
    schedule for the decode workload's sequences (gdr_recurrent_fwd)."""
    import itertools
    import torch
    import gated_delta_rule_26_amd as gdr
    from gdr_inputs import WORKLOADS, random_inputs

    dev = torch.device("cuda:0")
    d = _to_device({key: x[key] for key in ("q", "k", "v", "g", "beta")}, w, dev)
    ntok = w.B * w.T
    res = {}

    # packed batch: the B*T tokens as one token axis, sequences of a serving mix
    lens = serving_lengths(ntok)
    cu = torch.tensor([0] + list(itertools.accumulate(lens)), dtype=torch.int32, device=dev)
    pk = {key: val.reshape((ntok,) + tuple(val.shape[2:])) for key, val in d.items()}
    N = len(lens)
    desc = gdr.make_desc(N, ntok, w.H, w.Dk, w.Dv, qkv_dtype=pk["q"].dtype, o_dtype=torch.float32,
                         per_channel=w.per_channel, kaczmarz=w.kaczmarz, eps=w.eps)
    ws = torch.empty(max(1, gdr.chunk_fwd_varlen_workspace_size(desc)), dtype=torch.uint8, device=dev)
    o = torch.empty((ntok, w.H, w.Dv), dtype=torch.float32, device=dev)
    sf = torch.empty((N, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    kw = dict(per_channel=w.per_channel, kaczmarz=w.kaczmarz, eps=w.eps, o=o, s_final=sf, workspace=ws,
              o_dtype=torch.float32)
    ms, med = _timed_calls(lambda: gdr.chunk_fwd_varlen(pk["q"], pk["k"], pk["v"], pk["g"], pk["beta"], cu,
                                                        **kw), steps, warmup)
    res["packed_batch"] = {
        "entry": "gdr_chunk_fwd_varlen",
        "workload": f"{w.name} tokens ({ntok} x H{w.H}) packed as {N} sequences, lengths log-uniform in "
                    f"[64, 2048] (seed 2026; {min(lens)}..{max(lens)} tokens), fp32 output",
        "sequences": N, "ms_per_call": ms, "ms_per_call_median": med, "tokens_per_s": ntok / (ms * 1e-3)}

    # without the delta rule (the additive write, scalar decay: RetNet / Mamba-2 style), fixed length
    o2 = torch.empty((w.B, w.T, w.H, w.Dv), dtype=torch.float32, device=dev)
    s2 = torch.empty((w.B, w.H, w.Dk, w.Dv), dtype=torch.float32, device=dev)
    desc2 = gdr.make_desc(w.B, w.T, w.H, w.Dk, w.Dv, qkv_dtype=d["q"].dtype, o_dtype=torch.float32,
                          per_channel=w.per_channel, delta_off=True)
    ws2 = torch.empty(max(1, gdr.chunk_fwd_workspace_size(desc2)), dtype=torch.uint8, device=dev)
    ms, med = _timed_calls(lambda: gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], None, per_channel=w.per_channel,
                                                 delta_off=True, o=o2, o_dtype=torch.float32, s_final=s2,
                                                 workspace=ws2),
                           steps, warmup)
    res["no_delta"] = {
        "entry": "gdr_chunk_fwd (delta_off)",
        "workload": f"{w.name} inputs, additive write S = D S + k v^T ({w.decay} decay), fp32 output",
        "ms_per_call": ms, "ms_per_call_median": med, "tokens_per_s": ntok / (ms * 1e-3)}

    # T tokens per call on the recurrent schedule (short prefills, several decode tokens)
    wd = WORKLOADS["decode"]
    T = recurrent_tokens
    xr = random_inputs(77, wd.B, T, wd.H, wd.Dk, wd.Dv, dtype="bf16")
    r = {key: torch.from_numpy(xr[key]).to(dev) for key in ("q", "k", "v", "g", "beta")}
    for key in ("q", "k", "v"):
        r[key] = r[key].to(torch.bfloat16)
    gen = torch.Generator(device=dev).manual_seed(5)
    state = torch.empty((wd.B, wd.H, wd.Dk, wd.Dv), dtype=torch.float32, device=dev).normal_(0.0, 0.02,
                                                                                             generator=gen)
    o3 = torch.empty((wd.B, T, wd.H, wd.Dv), dtype=torch.float32, device=dev)
    ms, med = _timed_calls(lambda: gdr.recurrent_fwd(r["q"], r["k"], r["v"], r["g"], r["beta"], state, o=o3,
                                                    o_dtype=torch.float32),
                           steps, warmup)
    nb = wd.B * wd.H * (2 * wd.Dk * wd.Dv * 4 + T * ((2 * wd.Dk + wd.Dv) * 2 + 8 + wd.Dv * 4))
    fl_rec = wd.B * wd.H * T * 6 * wd.Dk * wd.Dv
    res["recurrent_tokens"] = {
        "entry": "gdr_recurrent_fwd",
        "workload": f"{wd.B} sequences x H{wd.H}, {T} tokens per call, d_k=d_v={wd.Dk}, bf16 q/k/v, fp32 "
                    f"state in place, scalar decay, given beta, fp32 output",
        "ms_per_call": ms, "ms_per_call_median": med, "tokens_per_s": wd.B * T / (ms * 1e-3),
        "roofline": {"bound": "hbm", "achieved": nb / (ms * 1e-3) / 1e9, "peak": PEAK_HBM, "unit": "GB/s",
                     "frac": nb / (ms * 1e-3) / 1e9 / PEAK_HBM, "alg_bytes_per_call": nb,
                     # per token and head three passes over the state (S~^T k, S~^T q, the rank-1
                     # write), 2 flops per element each, on the fp32 vector ALUs
                     "alu_view": {"alg_flops_per_call": fl_rec,
                                  "achieved_tflops": fl_rec / (ms * 1e-3) / 1e12, "peak_tflops": PEAK_FP32_VALU,
                                  "frac": fl_rec / (ms * 1e-3) / 1e12 / PEAK_FP32_VALU}}}
    return res


def measured_peaks(reps=10):
    """What this GPU reaches on plain library work, beside the spec peaks: a 1 GiB device-to-device
    copy (bytes read + written per second) and a bf16 GEMM of 8192^3 through torch.matmul
    (hipBLASLt), both timed with events after a warm-up."""
    import torch
    dev = torch.device("cuda:0")
    n = 1 << 30
    a = torch.empty(n // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    ms_copy, _ = _timed_calls(lambda: b.copy_(a), reps, 3)
    del a, b
    m = 8192
    gen = torch.Generator(device=dev).manual_seed(3)
    x = torch.randn((m, m), dtype=torch.bfloat16, device=dev, generator=gen)
    y = torch.randn((m, m), dtype=torch.bfloat16, device=dev, generator=gen)
    ms_mm, _ = _timed_calls(lambda: torch.matmul(x, y), reps, 3)
    del x, y
    torch.cuda.empty_cache()
    copy_gbps = 2 * n / (ms_copy * 1e-3) / 1e9
    gemm_tflops = 2 * m ** 3 / (ms_mm * 1e-3) / 1e12
    return {"copy_gbps": copy_gbps, "copy_frac_of_spec": copy_gbps / PEAK_HBM,
            "bf16_gemm_tflops": gemm_tflops, "bf16_gemm_frac_of_spec": gemm_tflops / PEAK_BF16_MFMA,
            "how": "1 GiB torch copy_ (2 GiB moved per call); torch.matmul bf16 8192x8192x8192 (hipBLASLt); "
                   f"mean of {reps} calls timed with events after 3 warm-up calls"}


def calibrate_copy(nbytes=1 << 30, reps=3):
    """A plain device copy of known size, so that rocprofv3 byte counters of
    the same command can be scaled (FETCH_SIZE / WRITE_SIZE per dispatch)."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    return nbytes


def _rel_heads(gpu_o, ref_o, gpu_s, ref_s):
    """Aggregate and largest per-(batch, head) relative L2 of o [B,T,H,Dv] and S [B,H,Dk,Dv]."""
    import numpy as np
    B, _, H = ref_o.shape[:3]
    acc = np.zeros(4)
    worst = [0.0, 0.0]
    for b in range(B):
        for h in range(H):
            for i, (g, r) in enumerate(((gpu_o[b, :, h], ref_o[b, :, h]), (gpu_s[b, h], ref_s[b, h]))):
                dd = np.asarray(g, dtype=np.float64) - r
                d2, r2 = float(np.sum(dd * dd)), float(np.sum(r * r))
                acc[2 * i] += d2
                acc[2 * i + 1] += r2
                worst[i] = max(worst[i], (d2 / r2) ** 0.5 if r2 > 0 else d2 ** 0.5)
    return {"rel_l2_o": float((acc[0] / acc[1]) ** 0.5), "rel_l2_s": float((acc[2] / acc[3]) ** 0.5),
            "worst_head_rel_l2_o": worst[0], "worst_head_rel_l2_s": worst[1]}


def cpu_baseline(w, x, gpu_runs, decode_runs, min_seconds=8.0, max_passes=64):
    """The fp64 oracle, as it stands, on the host cores.

    * The headline figure: whole passes over every (batch, head) pair of the prefill workload w,
      repeated until about min_seconds of wall time have passed; and one pass over a single pair on
      one thread (the per-core rate).
    * The same oracle on the other configurations timed in this run (one pass over every pair each,
      a bounded sample of the decode workload's steps), whose results double as the parity of the
      GPU outputs of this run: relative L2 over all heads and the worst single head.
    """
    import oracle
    threads = oracle.max_threads()
    nbh = w.B * w.H
    heads = list(range(nbh))
    passes = 0
    t0 = time.perf_counter()
    while True:
        ref_w = oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], per_channel=w.per_channel,
                                  kaczmarz=w.kaczmarz, eps=w.eps, heads=heads, threads=threads)
        passes += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or passes >= max_passes:
            break
    t1 = time.perf_counter()
    oracle.oracle_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], per_channel=w.per_channel, kaczmarz=w.kaczmarz,
                      eps=w.eps, heads=[0], threads=1)
    dt1 = time.perf_counter() - t1
    out = {"value": passes * nbh * w.T / w.H / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{w.name}: {nbh} of {nbh} (batch, head) pairs, all {w.T} tokens each, fp64 token "
                     f"recurrence, {passes} passes; {dt:.2f} s wall x {threads} threads; tokens/s counts all "
                     f"{w.H} heads of a token",
           "seconds": dt, "passes": passes, "cpu": cpu_model(),
           "single_thread": {"token_heads_per_s": w.T / dt1, "seconds": dt1,
                             "sample": f"{w.name}: (batch, head) pair 0, {w.T} tokens, 1 thread"},
           "per_config": {}}
    for name, (wc, xc, runs) in gpu_runs.items():
        if wc is w:  # the timed passes above
            ref, dt2 = ref_w, dt / passes
        else:
            t2 = time.perf_counter()
            ref = oracle.oracle_fwd(xc["q"], xc["k"], xc["v"], xc["g"], xc["beta"], per_channel=wc.per_channel,
                                    kaczmarz=wc.kaczmarz, eps=wc.eps, threads=threads)
            dt2 = time.perf_counter() - t2
        entry = {"oracle_seconds": dt2, "oracle_tokens_per_s": wc.B * wc.T / dt2}
        for o_dtype, (o, s) in runs.items():
            entry[f"parity_{o_dtype}_o"] = _rel_heads(o, ref[0], s, ref[1])
        out["per_config"][name] = entry
    if decode_runs:
        import numpy as np
        wd, dec = decode_runs
        xs = [dec["host_inputs"][i] for i in dec["order"]]
        st = {key: np.stack([xi[key] for xi in xs]) for key in xs[0]}
        t2 = time.perf_counter()
        o_ref, s_ref = oracle.oracle_decode(st["q"], st["k"], st["v"], st["g"], st["beta"], dec["s0"],
                                            threads=threads)
        dt2 = time.perf_counter() - t2
        o_last = dec["o"].cpu().numpy()
        s_gpu = dec["state"].cpu().numpy()
        d_o = o_last - o_ref[-1]
        d_s = s_gpu - s_ref
        out["per_config"]["decode"] = {
            "oracle_seconds": dt2, "oracle_tokens_per_s": wd.B * len(xs) / dt2,
            "parity_f32_o": {"rel_l2_o_last_step": float(np.linalg.norm(d_o) / np.linalg.norm(o_ref[-1])),
                             "rel_l2_s": float(np.linalg.norm(d_s) / np.linalg.norm(s_ref)),
                             "steps": len(xs)}}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gdn_prefill",
                    choices=["gdn_prefill", "kda_prefill", "kla_prefill", "gdn_tiny"])
    ap.add_argument("--qkv-dtype", default=None, choices=["f32", "bf16"],
                    help="store q, k, v of the headline workload in this dtype instead of its own")
    ap.add_argument("--algo", default="auto", choices=["auto", "vector", "matrix"])
    ap.add_argument("--o-dtype", default="bf16", choices=["f32", "bf16"])
    ap.add_argument("--other-configs", default="gdn_tiny,kda_prefill,kla_prefill",
                    help="comma-separated prefill workloads timed beside the headline ('' for none)")
    ap.add_argument("--other-steps", type=int, default=10, help="timed steps of each other configuration")
    ap.add_argument("--decode-steps", type=int, default=200)
    ap.add_argument("--decode-distinct", type=int, default=16,
                    help="distinct decode-step inputs kept resident and cycled through")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the copy and GEMM peak measurements")
    ap.add_argument("--backward-steps", type=int, default=5,
                    help="timed calls of the backward pass on each prefill workload (0: skip)")
    ap.add_argument("--next-rows-steps", type=int, default=5,
                    help="timed calls of the packed-batch, no-delta and multi-token recurrent entry points (0: skip)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device copy (for rocprofv3 counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: bench.py measures one MI355X; the path "
              f"shards over independent (sequence, head) pairs, so N GPUs run N independent shares.",
              file=sys.stderr)
        sys.exit(2)
    rank = int(os.environ.get("RANK", "0"))

    import torch
    import gated_delta_rule_26_amd as gdr
    from gdr_inputs import WORKLOADS, prefill_inputs

    gdr.load_library()  # fail loudly if the HIP library is missing
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(3)

    def host(t):
        return t.float().cpu().numpy()

    w = WORKLOADS[args.workload]
    if args.qkv_dtype and args.qkv_dtype != w.dtype:
        w = w.scaled(name=f"{w.name}_{args.qkv_dtype}", dtype=args.qkv_dtype)
    x = prefill_inputs(w)
    algo = resolve_algo(w, args.algo)
    pre = bench_prefill(w, x, args.steps, args.warmup, algo, args.o_dtype)
    head = prefill_block(w, pre, algo, args.o_dtype)
    gpu_runs = {w.name: (w, x, {args.o_dtype: (host(pre["o"]), host(pre["s"]))})}
    del pre
    other_o = "f32" if args.o_dtype == "bf16" else "bf16"
    pre2 = bench_prefill(w, x, args.other_steps, 2, algo, other_o)
    gpu_runs[w.name][2][other_o] = (host(pre2["o"]), host(pre2["s"]))
    beside = prefill_block(w, pre2, algo, other_o)
    del pre2
    torch.cuda.empty_cache()

    out = {
        "metric": "prefill tokens/s (chunkwise GDN, H16 d128, % MFMA peak) + decode HBM GB/s",
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if algo == "matrix" and w.dtype == "bf16" and w.Dk == 128 and w.Dv == 128 else "f32",
        "data": "synthetic",
        "config": {"workload": head["workload"], "B": w.B, "T": w.T, "H": w.H, "Dk": w.Dk, "Dv": w.Dv,
                   "chunk": C, "algo": algo, "o_dtype": args.o_dtype, "timing": head["timing"]},
        "mfma_peak_frac": head["frac_bf16_mfma_peak"],
        "roofline": head["roofline"],
        "prefill": {key: head[key] for key in ("tokens_per_s", "ms_per_step", "ms_per_step_median",
                                               "ms_per_step_p10", "ms_per_step_p90", "intra_ms",
                                               "state_ms", "warm", "alg_tflops", "frac_bf16_mfma_peak",
                                               "alg_bytes", "alg_gbps", "frac_hbm_peak",
                                               "alg_flops_per_token_head", "workspace_bytes")},
        "prefill_other_output": beside,
        "configs": {},
    }

    for name in [n for n in args.other_configs.split(",") if n and n != w.name]:
        wc = WORKLOADS[name]
        xc = prefill_inputs(wc)
        ac = resolve_algo(wc, args.algo)
        od = "f32" if wc.dtype == "f32" else args.o_dtype
        pc = bench_prefill(wc, xc, args.other_steps, 2, ac, od)
        out["configs"][name] = prefill_block(wc, pc, ac, od)
        gpu_runs[name] = (wc, xc, {od: (host(pc["o"]), host(pc["s"]))})
        del pc
        torch.cuda.empty_cache()
        if args.backward_steps > 0:
            out["configs"][name]["backward"] = {"workload": backward_label(wc),
                                                **bench_backward(wc, xc, args.backward_steps, 1)}
            torch.cuda.empty_cache()

    decode_runs = None
    if not args.no_decode:
        wd = WORKLOADS["decode"]
        dec = bench_decode(wd, args.decode_steps, args.decode_distinct)
        out["decode"] = decode_block(wd, dec, args.decode_steps, args.decode_distinct,
                                     ", the size of the 256 MB last-level cache")
        decode_runs = (wd, dec)
        # twice the sequences: a 512 MiB state the last-level cache cannot hold
        wb = wd.scaled(name="decode_512", B=2 * wd.B)
        decb = bench_decode(wb, args.decode_steps, args.decode_distinct)
        out["decode_beyond_cache"] = decode_block(wb, decb, args.decode_steps, args.decode_distinct,
                                                  ", twice the 256 MB last-level cache")
        del decb
        torch.cuda.empty_cache()

    if not args.no_peaks:
        pk = measured_peaks()
        # the headline figures against what this GPU measurably reaches, beside their fractions of the spec
        pk["vs_measured"] = {
            "state_kernel_gbps_frac_of_copy": head["roofline"]["achieved"] / pk["copy_gbps"]
            if head["roofline"]["unit"] == "GB/s" else None,
            "pass_alg_tflops_frac_of_gemm": head["alg_tflops"] / pk["bf16_gemm_tflops"],
        }
        if "decode" in out:
            pk["vs_measured"]["decode_gbps_frac_of_copy"] = out["decode"]["roofline"]["achieved"] / pk["copy_gbps"]
        out["peaks_measured"] = pk

    if args.backward_steps > 0:
        bwd = bench_backward(w, x, args.backward_steps, 1)
        out["backward"] = {
            "workload": backward_label(w),
            **bwd,
            "train_step_tokens_per_s": w.B * w.T / ((head["warm"]["event_step_ms"] + bwd["ms_per_step"]) * 1e-3),
        }

    if args.next_rows_steps > 0 and not w.per_channel:
        out["next_rows"] = bench_next_rows(w, x, args.next_rows_steps, 2)

    if args.calibrate_copy:
        out["calibration_copy_bytes"] = calibrate_copy()

    if not args.no_cpu_baseline and rank == 0:
        out["cpu_baseline"] = cpu_baseline(w, x, gpu_runs, decode_runs)

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
