"""Build the CPU oracle (test infrastructure) into oracle/libqr_oracle.so.

Compiled with gcc at -O2 with floating-point contraction off, no fast-math and
SSE arithmetic, so every binary32 operation in qr_oracle.c is rounded on its
own as the C source states.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "qr_oracle.c")
LIB = os.path.join(HERE, "libqr_oracle.so")

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math",
          "-fno-finite-math-only", "-frounding-math", "-fPIC", "-shared",
          "-Wall", "-Wextra"]


def build(out=LIB, src=SRC, extra=()):
    """Compile `src` into the shared library `out` (returns its path)."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
