"""Host-side logic of bench.py, on the CPU: the one-GPU rule, the algorithmic
byte counts the roofline divides by, and the kernel-source hash that decides
whether the recorded HBM traffic counters still apply."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 2
    assert "one GPU" in res.stderr and res.stdout == ""


def test_algorithmic_bytes_of_the_64MB_workload():
    # W=2, n = 32 Mi elements; a Q4 symmetric wire image is 16 B of codes and
    # 2 B of scale per 32-element block: 1 Mi blocks -> 18,874,368 bytes
    n, wb = 1 << 25, 18874368
    assert bench.algorithmic_bytes("quantize", 2, n, wb) == 2 * (2 * n) + 2 * wb
    assert bench.algorithmic_bytes("stage1", 2, n, wb) == 56623104      # 2 read + 1 written
    assert bench.algorithmic_bytes("stage2", 2, n, wb) == 2 * wb + 2 * (2 * n)
    # FP: the wire is the buffer itself
    assert bench.algorithmic_bytes("stage1", 8, n, 2 * n) == 9 * 2 * n


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    src = tmp_path / "k.hip"
    body = "int f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n"
    src.write_text(body)
    monkeypatch.setattr(bench, "KERNEL_SOURCES", [str(src)])
    h0 = bench.kernel_source_sha()
    src.write_text(body.replace("// one", "// a different comment").replace(
        "/* block\n comment */", "/* other */") + "\n\n")
    assert bench.kernel_source_sha() == h0
    src.write_text(body.replace("x + 1", "x + 2"))
    assert bench.kernel_source_sha() != h0


def test_min_sizes_takes_the_size_from_which_the_lead_holds():
    def pt(one, q4, q8, spread=0.0):
        return {"1stage": {"us": one, "spread": spread}, "q4": {"us": q4, "spread": spread},
                "q8": {"us": q8, "spread": spread}}
    sweep = {"W2": {"4096": pt(5.0, 5.1, 5.2),
                    "8388608": pt(12.0, 9.0, 13.0),      # q4 ahead, q8 behind
                    "16777216": pt(20.0, 21.0, 15.0),    # q4 behind again, q8 ahead
                    "33554432": pt(40.0, 30.0, 30.0),
                    "67108864": pt(80.0, 60.0, 60.0)}}
    got, _ = bench.min_sizes(sweep, margin=0.2)
    assert got["W2"] == {"q4": 33554432, "q8": 16777216}
    sweep["W2"]["67108864"]["q8"]["us"] = 90.0          # behind at the largest size
    assert bench.min_sizes(sweep, margin=0.2)[0]["W2"]["q8"] is None


def test_min_sizes_counts_only_leads_beyond_the_spread():
    def pt(one, q4, s1, s4):
        return {"1stage": {"us": one, "spread": s1}, "q4": {"us": q4, "spread": s4}}
    sweep = {"W8": {"2097152": pt(10.0, 9.0, 0.4, 0.4),   # 9.4 < 9.6: a lead
                    "4194304": pt(20.0, 19.0, 0.6, 0.5),  # 19.5 < 19.4 fails: a tie
                    "8388608": pt(40.0, 30.0, 1.0, 1.0),
                    "16777216": pt(80.0, 60.0, 1.0, 1.0)}}
    assert bench.min_sizes(sweep, margin=0.0)[0]["W8"]["q4"] == 8388608
    sweep["W8"]["4194304"]["1stage"]["spread"] = 0.2      # 19.5 < 19.8: a lead
    assert bench.min_sizes(sweep, margin=0.0)[0]["W8"]["q4"] == 2097152


def test_min_sizes_needs_the_margin_and_reports_points_near_it():
    def pt(one, q4):
        return {"1stage": {"us": one, "spread": 0.0}, "q4": {"us": q4, "spread": 0.0}}
    sweep = {"W4": {"4194304": pt(10.0, 8.5),      # 15 % ahead: short of a 20 % margin
                    "8388608": pt(20.0, 16.05),    # 19.75 % ahead: short, and marginal
                    "16777216": pt(40.0, 30.0)}}   # 25 % ahead
    tab, marginal = bench.min_sizes(sweep, margin=0.2)
    assert tab["W4"]["q4"] == 16777216
    assert [m["bytes"] for m in marginal] == [8388608]
    assert bench.min_sizes(sweep, margin=0.1)[0]["W4"]["q4"] == 4194304
    # the benchmark's own margin, 30 %: only the 25 % lead at 16 MB falls short
    assert bench.MIN_SIZE_MARGIN == 0.30
    assert bench.min_sizes(sweep)[0]["W4"]["q4"] is None
    assert bench.min_sizes(sweep, margin=0.3) == bench.min_sizes(sweep)


def test_stage2_hbm_bytes_read_the_reduced_image_once():
    n, wb = 1 << 25, 18874368
    assert bench.hbm_bytes_stage2(8, n, wb) == wb + 8 * 2 * n
    assert bench.hbm_bytes_stage2(8, n, wb) < bench.algorithmic_bytes("stage2", 8, n, wb)

