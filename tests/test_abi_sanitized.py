"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer
(runs without a GPU).

Builds every library source with both sanitizers on the host side only
(`-Xarch_host`; device code is compiled as usual) into an executable together
with tests/abi_sanitize/abi_check.cpp, which drives every entry point's
argument validation and the workspace-size queries over a spread of shapes,
and runs it: any sanitizer report, or an unexpected status, fails the test.
"""
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

from long_context_hybrid_amd import build as B

HIPCC = B.HIPCC
DRIVER = os.path.join(os.path.dirname(os.path.abspath(__file__)), "abi_sanitize", "abi_check.cpp")
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not found")


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"


def test_abi_host_code_sanitized(tmp_path):
    common = ["-O1", "-g", "-std=c++17", f"--offload-arch={B.ARCH}", "-I", B.INCLUDE, "-I", B.CSRC, *SAN]
    objs = []

    def compile_one(src):
        obj = str(tmp_path / (os.path.splitext(src)[0] + ".o"))
        _run([HIPCC, *common, *B.DEVICE_FLAGS, "-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(max_workers=min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(compile_one, B.SOURCES))
    main = str(tmp_path / "abi_check.o")
    _run([HIPCC, "-O1", "-g", "-std=c++17", "-I", B.INCLUDE, *SAN, "-c", DRIVER, "-o", main])
    exe = str(tmp_path / "abi_check")
    _run([HIPCC, "--hip-link", f"--offload-arch={B.ARCH}", *SAN, *objs, main, "-o", exe])
    env = dict(os.environ)
    # the HIP runtime keeps allocations for the process lifetime: leak reports are not about this code
    env["ASAN_OPTIONS"] = "detect_leaks=0:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error" not in out, out
    assert r.returncode == 0 and "OK: 0 unexpected" in r.stdout, out
