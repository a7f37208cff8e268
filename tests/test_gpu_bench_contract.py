"""bench.py end to end on the GPU, shortened: it prints exactly one JSON line
on stdout, and that line carries the fields its readers rely on (the metric,
the whole-job value and its unit, the step counts, the roofline of the
dominant kernel, the CPU baseline of the oracle, the backward and serving
blocks) with values of the right kind; the oracle comparison it makes on the
passes it timed meets the parity bar."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_one_complete_json_line():
    args = [sys.executable, "-u", os.path.join(ROOT, "bench.py"), "--steps", "2", "--warmup", "1",
            "--other-steps", "1", "--other-configs=", "--no-decode", "--no-peaks", "--backward-steps", "1",
            "--next-rows-steps", "1"]
    r = subprocess.run(args, capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, r.stdout[-2000:]
    d = json.loads(lines[0])

    assert isinstance(d["metric"], str) and d["metric"]
    assert d["unit"] == "tokens/s" and d["value"] > 0 and d["higher_is_better"] is True
    assert (d["n_gpus"], d["steps"], d["warmup"]) == (1, 2, 1)
    assert d["ms_per_step"] > 0 and d["scaling"] in ("weak", "strong")
    assert d["vs_baseline"] is None and d["data"] == "synthetic" and d["dtype"] == "bf16"
    assert "gdn_prefill" in d["config"]["workload"]
    # whole-job throughput: tokens of the timed pass over its time
    assert abs(d["value"] - d["config"]["B"] * d["config"]["T"] / (d["ms_per_step"] * 1e-3)) < 1e-6 * d["value"]

    roof = d["roofline"]
    assert roof["bound"] in ("hbm", "mfma", "alu") and roof["unit"] in ("GB/s", "TFLOP/s")
    assert roof["achieved"] > 0 and roof["peak"] > 0
    assert abs(roof["frac"] - roof["achieved"] / roof["peak"]) < 1e-9
    assert roof["traffic"] is None or roof["traffic"] > 0

    cpu = d["cpu_baseline"]
    assert cpu["kind"] == "oracle" and cpu["value"] > 0 and cpu["cores"] >= 1 and cpu["sample"]
    par = cpu["per_config"]["gdn_prefill"]["parity_bf16_o"]
    assert par["rel_l2_o"] < 2e-3 and par["rel_l2_s"] < 2e-3

    assert d["backward"]["ms_per_step"] > 0
    assert set(d["next_rows"]) >= {"packed_batch", "no_delta", "recurrent_tokens"}
