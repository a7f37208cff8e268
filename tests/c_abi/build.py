"""Build the C ABI check program (tests/c_abi/parity.cpp): host code only,
g++ against the HIP runtime, libgdr.so and the oracle's liboracle.so, with
run paths relative to the program so that it runs from any copy of the tree."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "parity.cpp")
BIN = os.path.join(HERE, "parity")


def build() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = BIN + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__", f"-I{rocm}/include",
           f"-I{os.path.join(ROOT, 'include')}", SRC, "-o", tmp,
           f"-L{os.path.join(ROOT, 'gated_delta_rule_26_amd')}", "-lgdr",
           f"-L{os.path.join(ROOT, 'oracle')}", "-loracle", f"-L{rocm}/lib", "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../../gated_delta_rule_26_amd:$ORIGIN/../../oracle:" + f"{rocm}/lib"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build())
