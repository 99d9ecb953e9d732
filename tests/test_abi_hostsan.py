"""The C ABI's host side under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only, no GPU call): tests/test_abi.py runs again in a child process
against the host-sanitised build of the library (device code unchanged), with
the compiler's ASan runtime preloaded.  Any sanitizer report fails the test."""
import os
import subprocess
import sys

import pytest

from dual_view_block_amd import build as B

pytestmark = pytest.mark.nogpu  # it runs tests/test_abi.py, whose calls carry made-up device pointers

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _stale() -> bool:
    if not os.path.exists(B.SAN_LIB):
        return True
    built = os.path.getmtime(B.SAN_LIB)
    srcs = [os.path.join(B.CSRC, f) for f in os.listdir(B.CSRC)] + [os.path.join(ROOT, "include", "orthrus.h")]
    return any(os.path.getmtime(s) > built for s in srcs)


def test_abi_checks_are_clean_under_host_sanitizers():
    if _stale():
        B.build(host_sanitizers=True)
    env = dict(os.environ)
    rt = B.asan_runtime()
    env["LD_PRELOAD"] = rt + (":" + env["LD_PRELOAD"] if env.get("LD_PRELOAD") else "")
    env["ORTHRUS_LIBRARY"] = B.SAN_LIB
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    out = res.stdout + res.stderr
    assert res.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert " passed" in out, out[-2000:]
    print(out.strip().splitlines()[-1])
