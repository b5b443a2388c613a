"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer:
tests/oracle_sanitize.c drives every oracle entry point over ragged sizes,
owner chunks, every codec, buffer type and code, with buffers allocated at
exactly their stated sizes.  Built with gcc (CPU only; the oracle shares
nothing with the HIP path) and run in a subprocess, so that the sanitizer
runtimes load first."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer",
                    os.path.join(HERE, "oracle_sanitize.c"),
                    os.path.join(ROOT, "oracle", "qr_oracle.c"), "-lm", "-o", exe],
                   check=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    assert res.returncode == 0, res.stdout + res.stderr[-4000:]
    assert "no report" in res.stdout
