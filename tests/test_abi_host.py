"""The C ABI's host code without a GPU: tests/abi_host_check.cpp links
qr_api.cpp with recording stubs in place of the kernel launchers and checks
what every entry point would launch (fused vs staged sim, workspace layout,
owner block ranges, no launch on a rejected call, QR_ERR_HIP on a failed
launch).  Built with g++ under AddressSanitizer and
UndefinedBehaviorSanitizer (host code only; no HIP device code is built)."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "quantized_two_stage_amd", "csrc")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_abi_host_code(tmp_path):
    exe = str(tmp_path / "abi_host_check")
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", "-Wall", "-Wextra",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__",
                    "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"),
                    "-I", CSRC, os.path.join(HERE, "abi_host_check.cpp"),
                    os.path.join(CSRC, "qr_api.cpp"), "-o", exe], check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1", UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, res.stdout + res.stderr[-4000:]
    assert ", 0 failed" in res.stdout, res.stdout
