"""Runs tests/gpu_arith_check (built by tests/build_checks.py): exhaustive
on-GPU checks of the arithmetic identities the kernels rely on -- the
corrected division by each integer codec's qmax, the one-step reciprocal of
binary16 scales, rounding by the 1.5*2^23 addition, and gfx950's fp8 encode
and decode and bf16 conversion against their definitions."""
import os
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "gpu_arith_check")


@pytest.mark.gpu
def test_arithmetic_identities_exhaustive():
    assert os.path.exists(EXE), "build it first: python tests/build_checks.py"
    print("running", EXE, flush=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=100)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ALL OK" in res.stdout
