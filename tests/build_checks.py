"""Build the GPU check programs of tests/ (hipcc, gfx950), with the same
numerics flags as libqr.so.  Called by __graft_entry__.build()."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
from quantized_two_stage_amd import build as qbuild  # noqa: E402

CHECKS = {"gpu_arith_check": os.path.join(HERE, "gpu_arith_check.hip")}


def build():
    flags = [f for f in qbuild.FLAGS if f not in ("-shared", "-fPIC")]
    out = []
    for name, src in CHECKS.items():
        exe = os.path.join(HERE, name)
        tmp = exe + ".tmp%d" % os.getpid()
        subprocess.run(["hipcc", *flags, src, "-o", tmp], check=True)
        os.replace(tmp, exe)
        out.append(exe)
    return out


if __name__ == "__main__":
    print(build())
