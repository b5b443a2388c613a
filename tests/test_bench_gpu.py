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
