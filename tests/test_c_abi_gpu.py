"""The C ABI from a plain C program (tests/c_abi_check.c, built by gcc with
no C++ and no torch): every entry point it calls gives the oracle's outputs
bit for bit, and a rejected call writes nothing."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_abi_check")


def test_c_program_against_oracle():
    assert os.path.exists(EXE), "build it first: python tests/build_checks.py"
    print("running", EXE, flush=True)
    res = subprocess.run([EXE], capture_output=True, text=True, timeout=100)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "ALL OK" in res.stdout
