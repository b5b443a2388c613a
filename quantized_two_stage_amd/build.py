"""Build libqr.so (the HIP kernels and the C ABI of include/qr.h) for gfx950,
and libqr_pattern.so, the benchmark's access-pattern reference (not part of
the library's ABI).

Flags that matter for the numerics: -ffp-contract=off (no fused multiply-add
the source does not ask for), no fast-math (IEEE division and denormals);
packed fp32 instructions are disabled for the device code.
"""
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqr.so")
SOURCES = [os.path.join(CSRC, "qr_kernels.hip"), os.path.join(CSRC, "qr_api.cpp")]
PATTERN_LIB = os.path.join(PKG, "libqr_pattern.so")
PATTERN_SOURCES = [os.path.join(CSRC, "qr_pattern.hip")]
ARCH = os.environ.get("QR_OFFLOAD_ARCH", "gfx950")

FLAGS = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-shared",
         "-ffp-contract=off", "-fno-fast-math",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-I", os.path.join(ROOT, "include"), "-I", CSRC]


def build(out=LIB, extra=(), verbose=False, sources=SOURCES):
    """Compile the library into `out`; returns its path."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["hipcc", *FLAGS, *extra, *sources, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed (%d)" % res.returncode)
    os.replace(tmp, out)
    return out


def build_pattern(verbose=False):
    """the benchmark's access-pattern reference library"""
    return build(out=PATTERN_LIB, verbose=verbose, sources=PATTERN_SOURCES)


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_pattern(verbose=True))
