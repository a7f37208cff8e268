"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* The fp64 oracle (plain C) is rebuilt with gcc's -fsanitize=address,undefined
  and every pin runs on that build, in a child process that loads the
  sanitizer runtimes first.  A copy of the oracle with an out-of-bounds read
  planted in it must make that child fail with an AddressSanitizer report, so
  the check is known to be live.
* The C ABI's host validation (gdr_api.cpp: descriptor, pointer-range,
  overflow and alias checks) is rebuilt with the host half of hipcc's
  -fsanitize=address,undefined and linked with the library's other objects
  as built by the package's build step; the ABI host tests
  (test_abi_host.py) then run against it in a child process under clang's
  AddressSanitizer runtime.  No GPU is involved: none of those calls passes
  validation.
"""
import glob
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_SRC = os.path.join(ROOT, "oracle", "gdr_oracle.c")
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]

PIN_RUNNER = r"""
import functools, json, sys
sys.path.insert(0, {root!r})
import oracle
from tests import pins
fwd = functools.partial(oracle.oracle_fwd, lib=oracle.bind(sys.argv[1]), threads=2)
golden = json.load(open({golden!r}))
for pin in pins.ALL_PINS:
    pin(fwd, golden) if pins.needs_golden(pin) else pin(fwd)
print("pins passed:", len(pins.ALL_PINS))
"""


def _gcc_runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


def _build_oracle(src_text, out):
    src = out + ".c"
    with open(src, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", *SAN, "-std=c99", "-fPIC", "-shared", "-fopenmp", "-o", out, src, "-lm"], check=True)
    return out


def _run_pins(lib, tmp_path):
    runner = tmp_path / "run_pins.py"
    runner.write_text(PIN_RUNNER.format(root=ROOT, golden=os.path.join(ROOT, "tests", "golden",
                                                                      "pages_worked_examples.json")))
    env = dict(os.environ, LD_PRELOAD=f"{_gcc_runtime('libasan.so')}:{_gcc_runtime('libubsan.so')}",
               ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1")
    return subprocess.run([sys.executable, str(runner), lib], capture_output=True, text=True, env=env,
                          timeout=300, cwd=ROOT)


@pytest.mark.skipif(shutil.which("gcc") is None or _gcc_runtime("libasan.so") is None
                    or _gcc_runtime("libubsan.so") is None, reason="gcc sanitizer runtimes not installed")
def test_oracle_pins_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    text = open(ORACLE_SRC).read()
    lib = _build_oracle(text, str(tmp_path / "liboracle_san.so"))
    r = _run_pins(lib, tmp_path)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "pins passed" in r.stdout and "ERROR: AddressSanitizer" not in r.stderr
    assert "runtime error" not in r.stderr
    # the same check must catch a planted out-of-bounds read: the final-state copy reads one
    # element past the end of its head's state
    planted, n = re.subn(r"(s_final\[[^\]]*\]\s*=\s*)S\[([^\]]+)\]", r"\1S[(\2) + 1]", text, count=1)
    assert n == 1, "no final-state copy found to plant the read in"
    bad = _build_oracle(planted, str(tmp_path / "liboracle_oob.so"))
    r = _run_pins(bad, tmp_path)
    assert r.returncode != 0 and "AddressSanitizer" in r.stderr, r.stdout + r.stderr[-2000:]


def _clang_asan_runtime():
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    return found[-1] if found else None


def test_abi_host_validation_under_sanitizers(tmp_path):
    from gated_delta_rule_26_amd import build as b
    objdir = b.OBJDIR
    others = [o for o in sorted(glob.glob(os.path.join(objdir, "*.o"))) if not o.endswith("gdr_api.cpp.o")]
    runtime = _clang_asan_runtime()
    if not others or runtime is None:
        pytest.skip("library objects not built (run __graft_entry__.build()) or no clang sanitizer runtime")
    host = []
    for flag in SAN + ["-shared-libsan"]:
        host += ["-Xarch_host", flag]
    obj = str(tmp_path / "gdr_api_san.o")
    subprocess.run([b.hipcc(), *b.compile_flags(), *host, "-c", os.path.join(b.CSRC, "gdr_api.cpp"), "-o", obj],
                   check=True, capture_output=True)
    lib = str(tmp_path / "libgdr_san.so")
    subprocess.run([b.hipcc(), f"--offload-arch={b.ARCH}", "-shared", "-fPIC", "-fsanitize=address,undefined",
                    "-shared-libsan", "-o", lib, *others, obj], check=True, capture_output=True)
    code = ("import sys; sys.path.insert(0, {root!r}); import pytest, gated_delta_rule_26_amd as gdr; "
            "gdr._lib = gdr.load_library({lib!r}); "
            "sys.exit(pytest.main([{test!r}, '-q', '-p', 'no:cacheprovider', '-m', 'not gpu']))").format(
        root=ROOT, lib=lib, test=os.path.join(ROOT, "tests", "test_abi_host.py"))
    env = dict(os.environ, LD_PRELOAD=runtime, ASAN_OPTIONS="detect_leaks=0:alloc_dealloc_mismatch=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=600, cwd=ROOT)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "passed" in r.stdout and "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr
