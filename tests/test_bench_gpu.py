"""bench.py's output contract, on the GPU: a short run prints one short JSON
line with every field the benchmark driver reads (metric, value, unit, steps,
timing, config, the roofline of the stage-1 kernel and the CPU oracle
baseline), with values of the right kind."""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_bench_prints_the_contract_line():
    print("running bench.py --steps 2 --warmup 1 --cold-reps 1", flush=True)
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--steps", "2",
                          "--warmup", "1", "--cold-reps", "1", "--cpu-sample", "65536"],
                         capture_output=True, text=True, timeout=240, cwd=ROOT)
    assert res.returncode == 0, res.stderr[-3000:]
    lines = [ln for ln in res.stdout.splitlines() if ln.strip()]
    assert len(lines) == 1, res.stdout[-2000:]
    assert len(lines[0]) < 6000, len(lines[0])       # the driver keeps a few KB of stdout
    d = json.loads(lines[0])
    for key, kind in (("metric", str), ("value", float), ("unit", str), ("n_gpus", int),
                      ("steps", int), ("warmup", int), ("ms_per_step", float),
                      ("higher_is_better", bool), ("scaling", str), ("dtype", str),
                      ("data", str), ("config", dict), ("roofline", dict),
                      ("cpu_baseline", dict)):
        assert isinstance(d[key], kind), (key, d.get(key))
    assert d["n_gpus"] == 1 and d["steps"] == 2 and d["warmup"] == 1
    assert d["unit"] == "GB/s" and d["value"] > 0 and d["higher_is_better"] is True
    assert d["vs_baseline"] is None and d["data"] == "synthetic"
    assert "workload" in d["config"]
    r = d["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert 0 < r["achieved"] and abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    assert r["traffic"] is None or r["traffic"] > 0
    assert r["frac"] == min(r["per_codec_frac"].values()) or \
        abs(r["frac"] - min(r["per_codec_frac"].values())) < 1e-4
    assert set(r["per_codec_frac"]) == set(r["pattern_frac"]) == set(r["copy_frac"]) == \
        set(r["in_pipeline_frac"])
    # traffic: the calibrated stage-1 counters under profiles/, reported only
    # while the kernel sources are those the counters were taken on
    with open(os.path.join(ROOT, "profiles",
                           "bench_w8_fp16_64MB_stage1_traffic.json")) as f:
        tj = json.load(f)
    codec = r["kernel"].split(",")[-2].strip()          # "<kernel> (...), <codec>, cold"
    if tj["source_sha"] == d["kernel_source_sha"]:
        assert r["traffic"] == tj["kernels"]["stage1/" + codec]["bytes"]
    else:
        assert r["traffic"] is None
    c = d["cpu_baseline"]
    assert c["kind"] == "oracle" and c["value"] > 0 and c["cores"] >= 1
    assert isinstance(c["unit"], str) and isinstance(c["sample"], str)


def test_stage1_scan_and_stream_probes_run():
    """bench.py's stage-1 size scan and plain-stream legs, at small sizes:
    every kernel timed at every size, fractions of 8 TB/s in a plausible
    range, and the plateau taken over the sizes from 64 MB per rank up"""
    import torch

    import bench
    from quantized_two_stage_amd import inputs as I
    from quantized_two_stage_amd import qr

    torch.cuda.set_device(0)
    st = torch.cuda.current_stream()
    sizes = (1 << 20, 1 << 25)                      # 2 MB and 64 MB per rank
    print("stage-1 scan at", sizes, flush=True)
    sc = bench.measure_stage1_scan(qr, I, torch, st, lambda m: None, sizes=sizes, reps=2)
    assert sc["sizes_bytes_per_rank"] == [2 * n for n in sizes]
    assert set(sc["per_codec"]) == {I.CODEC_NAMES[c] for c in I.CONFIGS[5]["codecs"]}
    for c, r in sc["per_codec"].items():
        assert len(r["bytes"]) == len(sizes)
        for k in ("stage1", "pattern", "copy"):
            assert len(r[k]["us"]) == len(sizes) and all(u > 0 for u in r[k]["us"]), (c, k)
            assert all(0.0 < f < 1.2 for f in r[k]["frac"]), (c, k, r[k]["frac"])
            assert r[k]["plateau_frac"] == r[k]["frac"][-1], (c, k)     # only 64 MB counts
    print("plain streams", flush=True)
    ps = bench.measure_streams(torch, st, lambda m: None, sizes_mib=(256,), reps=2)
    row = ps["per_size"]["256 MiB"]
    assert len(row) == len(bench.STREAM_PROBES)
    assert all(v["us"] > 0 and 0.0 < v["frac"] < 1.5 for v in row.values()), row
