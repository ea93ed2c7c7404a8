"""The quantizer kernels compute fl32(x / s) from the reciprocal of the block
scale and two FMA correction steps (Markstein's theorem) instead of a
division.  This checks that identity on the host, independently of both the
oracle and the GPU: every bf16 value against a set of scales, every scale
mantissa in one binade, and random pairs over the whole exponent range."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def checker(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("quotient") / "quotient_check")
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-o", exe,
                           os.path.join(HERE, "native", "quotient_check.c"), "-lm"])
    return exe


def test_fma_quotient_equals_ieee_division(checker):
    out = subprocess.run([checker, "20000000"], capture_output=True, text=True)
    assert out.returncode == 0, out.stdout + out.stderr
    assert " 0 disagree" in out.stdout, out.stdout
