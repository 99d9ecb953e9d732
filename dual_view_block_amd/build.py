"""Build liborthrus.so (gfx950 only) in-tree with hipcc.

    python -m dual_view_block_amd.build
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "liborthrus.so")
# the same library with AddressSanitizer and UndefinedBehaviorSanitizer in its
# host code (argument checks, planning, launch set-up); device code is built
# as usual.  Loaded only by the CPU tests, with the ASan runtime preloaded.
SAN_LIB = os.path.join(HERE, "liborthrus_hostsan.so")
SOURCES = ("api.hip", "attention.hip", "consensus.hip", "commit.hip", "kl.hip", "train_bwd.hip", "tree.hip")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


def command(out: str = LIB, host_sanitizers: bool = False) -> list:
    # sanitizers apply to the host side only: each -fsanitize= follows -Xarch_host
    san = ["-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-omit-frame-pointer", "-shared-libasan"] if host_sanitizers else []
    return [
        hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
        # keep the compiler from emitting packed fp32 arithmetic
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", os.path.join(ROOT, "include"),
    ] + san + ["-o", out] + [os.path.join(CSRC, s) for s in SOURCES]


def asan_runtime() -> str:
    """Path of the compiler's shared AddressSanitizer runtime (to preload)."""
    res = subprocess.run([hipcc(), "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip()
    if res.returncode != 0 or not os.path.isabs(path) or not os.path.exists(path):
        raise RuntimeError("the AddressSanitizer runtime of hipcc's clang was not found")
    return path


def build(verbose: bool = False, host_sanitizers: bool = False) -> str:
    out = SAN_LIB if host_sanitizers else LIB
    tmp = out + ".tmp"
    cmd = command(tmp, host_sanitizers)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
