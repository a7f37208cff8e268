"""Host-side pieces of bench.py (no GPU): the refusal of several GPUs, the
serving length mix, the algorithmic byte and flop counts, the step-time quantiles and the guard that
drops counter figures measured on other kernel sources."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_several_gpus_are_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60, cwd=ROOT)
    assert r.returncode == 2 and "--gpus 2 is not supported" in r.stderr and r.stdout == ""


def test_serving_lengths_cover_the_tokens_exactly_and_are_seeded():
    for total in (1, 63, 16384, 131072):
        lens = bench.serving_lengths(total)
        assert sum(lens) == total and all(n >= 1 for n in lens)
        assert all(n <= 2048 for n in lens)
        assert lens == bench.serving_lengths(total)          # the same mix every run
    assert bench.serving_lengths(16384) != bench.serving_lengths(16384, seed=1)


def test_algorithmic_counts_at_d128():
    # per token and head q, k, v in bf16 (768 B) and the fp32 output (512 B); per head the final state
    assert bench.alg_bytes_state_kernel(4, 4096, 16, 128, 128, 2, 4) == 4 * 4096 * 16 * 1280 + 4 * 16 * 65536
    assert bench.alg_bytes_state_kernel(4, 4096, 16, 128, 128, 2, 4) == 339_738_624
    # decode: the state in and out plus one token's inputs and output, per (sequence, head)
    assert bench.decode_bytes_per_step(256, 16, 128, 128) == 4096 * 132_360
    fl = bench.alg_flops_per_token_head(128, 128)
    assert fl["state"] == 6 * 128 * 128 + 65 * 128 and fl["total"] == fl["state"] + fl["intra"]


def test_counter_figures_follow_their_sources():
    # each recorded figure names the files it was measured on; a figure whose files changed is dropped
    for key, (files, sha, *_value) in list(bench.MEASURED_TRAFFIC.items()) + list(bench.MEASURED_MFMA.items()):
        assert all(os.path.exists(os.path.join(ROOT, f)) for f in files), key
        fn = bench.measured_traffic if key in bench.MEASURED_TRAFFIC else bench.measured_mfma
        assert (fn(*key) is not None) == (bench.sources_sha(files) == sha), key


def test_cpu_model_is_named():
    name = bench.cpu_model()
    assert isinstance(name, str) and name and name != "x86_64"


def test_step_time_quantiles_are_nearest_rank():
    xs = [float(x) for x in range(20, 0, -1)]      # unsorted on purpose
    assert (bench.quantile(xs, 0.1), bench.median(xs), bench.quantile(xs, 0.9)) == (2.0, 11.0, 18.0)
    assert bench.quantile([3.5], 0.1) == bench.quantile([3.5], 0.9) == 3.5
    assert bench.quantile(list(range(1, 11)), 0.9) == 9     # ceil(0.9 * 10) = the 9th value
    assert bench.quantile([], 0.5) != bench.quantile([], 0.5)  # nan for no samples
