"""The quant kernels' division-free quotient equals the IEEE quotient x / s.

The HIP quantizer (a1 and a9) computes E4M3(x / s) from one correctly rounded reciprocal
r = 1/s and one correction by the exact residual (two fused multiply-adds) instead of an
IEEE division per element. `tests/c/recip_div_check.c` proves the identity on the host's
IEEE f32 arithmetic: bit for bit over every (bf16 significand, f32 scale significand)
pair, and on all bf16 patterns across the scale range [2^-80, 2^100] that the kernels use it
for. A negative control (the uncorrected product) must fail the same check.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


def _has_fma():
    try:
        with open("/proc/cpuinfo") as f:
            return " fma " in f.read()
    except OSError:
        return False


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    if shutil.which("gcc") is None or not _has_fma():
        pytest.skip("needs gcc and a host with f32 fused multiply-add")
    exe = str(tmp_path_factory.mktemp("recip") / "recip_div_check")
    subprocess.run(["gcc", "-O2", "-mfma", "-ffp-contract=off", "-o", exe,
                    os.path.join(HERE, "c", "recip_div_check.c"), "-lm"], check=True)
    return exe


def test_reciprocal_form_equals_ieee_quotient(checker):
    r = subprocess.run([checker], capture_output=True, text=True, timeout=600)
    print(r.stdout)
    assert r.returncode == 0, r.stdout
    assert "mismatches 0;" in r.stdout and r.stdout.strip().endswith("mismatches 0")


def test_negative_control_fails(checker):
    r = subprocess.run([checker, "neg"], capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, r.stdout
