"""The C ABI without Python in the loop: tests/c_abi/parity (built by
__graft_entry__.build()) allocates device memory with the HIP runtime, calls
libgdr through include/gdr.h and compares with the fp64 oracle."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi", "parity")


def test_c_abi_program_matches_the_oracle():
    assert os.path.exists(BIN), f"{BIN} is missing: build it with __graft_entry__.build()"
    r = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(r.stdout + r.stderr)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.count("rel-L2") == 3 + 2 * 4 and "c-abi: ok" in r.stdout
