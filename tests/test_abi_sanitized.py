"""The C ABI's host validation (csrc/api.hip) under
AddressSanitizer and UndefinedBehaviorSanitizer: tests/c/abi_validation.cpp calls every
entry point with refused arguments and the pure host queries, and any out-of-bounds
access, leak-free misuse or undefined behaviour in the validation aborts the run. No GPU:
the kernel launchers are stubs that abort if a refused call ever reached one."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    pytest.skip("hipcc not found")


def test_abi_validation_under_asan_ubsan(tmp_path):
    hipcc = _hipcc()
    exe = str(tmp_path / "abi_validation")
    # the sanitizer flags apply to the host pass only (api.hip's device half -- its scratch
    # array -- is compiled plainly)
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
    cmd = [hipcc, "-std=c++17", "-O1", "-g", "--offload-arch=gfx950", *san,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "fp8_w8a8_linear_amd", "csrc", "api.hip"),
           os.path.join(ROOT, "tests", "c", "abi_validation.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stdout + r.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0 and "abi validation ok" in r.stdout, r.stdout + r.stderr
