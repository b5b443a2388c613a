"""Build the GPU check programs of tests/: gpu_arith_check (hipcc, gfx950,
with the same numerics flags as libqr.so) and c_abi_check (gcc, plain C
against the library's C ABI).  Called by __graft_entry__.build(), after
libqr.so and the oracle library are built."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
sys.path.insert(0, ROOT)
from quantized_two_stage_amd import build as qbuild  # noqa: E402

CHECKS = {"gpu_arith_check": os.path.join(HERE, "gpu_arith_check.hip")}
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build_c_abi_check():
    """tests/c_abi_check: plain C (gcc) against include/qr.h, libqr.so, the
    oracle library and the HIP runtime's C API; both libraries are found next
    to the program's own tree at run time.  The HIP headers need the
    platform named when a plain C compiler reads them."""
    exe = os.path.join(HERE, "c_abi_check")
    tmp = exe + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROOT, "include"), "-I", os.path.join(ROCM, "include"),
                    os.path.join(HERE, "c_abi_check.c"), "-o", tmp,
                    "-L", os.path.join(ROOT, "quantized_two_stage_amd"), "-l:libqr.so",
                    "-L", os.path.join(ROOT, "oracle"), "-l:libqr_oracle.so",
                    "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
                    "-Wl,-rpath,$ORIGIN/../quantized_two_stage_amd:$ORIGIN/../oracle:" +
                    os.path.join(ROCM, "lib")], check=True)
    os.replace(tmp, exe)
    return exe


def build():
    flags = [f for f in qbuild.FLAGS if f not in ("-shared", "-fPIC")]
    out = []
    for name, src in CHECKS.items():
        exe = os.path.join(HERE, name)
        tmp = exe + ".tmp%d" % os.getpid()
        subprocess.run(["hipcc", *flags, src, "-o", tmp], check=True)
        os.replace(tmp, exe)
        out.append(exe)
    out.append(build_c_abi_check())
    return out


if __name__ == "__main__":
    print(build())
