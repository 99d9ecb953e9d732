"""Build tests/c/decode_step, a host-only C++ program that runs one decode
step of one layer through the C ABI (include/orthrus.h) and liborthrus.so,
with no Python in the call path.  Host code only: g++ and the HIP runtime.

    python tests/c/build_example.py
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
SRC = os.path.join(HERE, "decode_step.cpp")
BIN = os.path.join(HERE, "decode_step")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def command(out: str = BIN) -> list:
    return ["g++", "-O2", "-std=c++17", "-Wall", "-D__HIP_PLATFORM_AMD__",
            "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"), SRC, "-o", out,
            "-L", os.path.join(ROOT, "dual_view_block_amd"), "-lorthrus",
            "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
            "-Wl,-rpath,$ORIGIN/../../dual_view_block_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib")]


def build(verbose: bool = False) -> str:
    tmp = BIN + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"g++ failed ({res.returncode}):\n{res.stderr}")
    os.replace(tmp, BIN)
    return BIN


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
