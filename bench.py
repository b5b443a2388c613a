"""Benchmark of the simulated two-stage quantized allreduce on one MI355X.

One step = one simulated allreduce per codec of the 64 MB workload (W=2
ranks, fp16, 32Mi elements per rank, N(0,1) with 0.1% x50 outliers; codecs
FP, fp8, Q8, Q6, Q4 symmetric), each as its three launches: quantize all
ranks, fused stage 1, stage 2 -- exactly the launches qr_allreduce_sim makes.
Inputs are resident in HBM before the timed region starts.

Two passes of the same K steps:
  1. the timed region: each allreduce is one qr_allreduce_sim call (its
     three launches), nothing else on the stream; `value` and `ms_per_step`
     come from this pass.
  2. the instrumented pass: each allreduce as the three staged calls with a
     HIP event recorded on the launch stream before and after every launch;
     the per-kernel durations and the roofline come from this pass (an event
     record between two launches costs the GPU about 2 us, which is why it
     is kept out of pass 1).

Prints one JSON line: effective GB/s = per-rank payload bytes (2n per
allreduce) / time, per step over all codecs; per-codec microseconds and
GB/s; per-kernel durations; the roofline of the kernel that takes the most
time; a cold-cache measurement of stage 1; beside every kernel figure, a
plain device copy that moves the same number of bytes (`copy_us`, and
`vs_copy` = copy time / kernel time), the achievable reference at that size;
and the CPU oracle timed on a bounded sample.  Unless --no-extra: the other workloads (W=8, the bf16
workload with and without the cast option, and size sweeps from 4 KB to
64 MB per rank buffer).
"""
import argparse
import hashlib
import json
import os
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "effective GB/s and μs per simulated allreduce, 4KB–64MB, W=2/4/8, per codec"
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_two_stage_amd", "csrc", f)
                  for f in ("qr_kernels.hip", "qr_device.h")]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=2)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=1 << 25,
                   help="elements per rank of the oracle's sample")
    p.add_argument("--no-cold", action="store_true")
    p.add_argument("--no-extra", action="store_true",
                   help="skip the other workloads (size sweeps, W=8)")
    return p.parse_args()


def kernel_source_sha():
    """hash of the kernel sources with comments and blank lines removed: a
    change to a comment leaves recorded counters valid, any change to the
    code does not"""
    import re
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        src = re.sub(r"/\*.*?\*/", "", open(f).read(), flags=re.S)
        src = re.sub(r"//[^\n]*", "", src)
        lines = [ln.rstrip() for ln in src.splitlines()]
        h.update("\n".join(ln for ln in lines if ln).encode())
    return h.hexdigest()[:16]


def algorithmic_bytes(stage, W, n, wb):
    """bytes the method must move per launch (W ranks, n elements each, wire
    image wb bytes): quantize reads 2n and writes wb per rank; stage 1 reads
    W wire images and writes one; stage 2 reads the reduced image and writes
    2n per rank."""
    if stage == "quantize":
        return W * (2 * n + wb)
    if stage == "stage1":
        return (W + 1) * wb
    return W * (wb + 2 * n)


class HipEvents:
    """HIP events recorded directly on the launch stream.  Created with
    hipEventDisableSystemFence: an event record then adds no system-scope
    release (no L2 write-back) between the kernels it brackets, so the time
    between two records is the kernel's own, as a profiler sees it."""
    FLAGS = 0x20000000          # hipEventDisableSystemFence

    def __init__(self, count):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p),
                                                     ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float),
                                                 ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(count):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.FLAGS)
            if rc != 0:
                raise RuntimeError("hipEventCreateWithFlags failed (%d)" % rc)
            self.ev.append(e)

    def record(self, i, stream):
        rc = self.hip.hipEventRecord(self.ev[i], self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("hipEventRecord failed (%d)" % rc)

    def ms(self, i, j):
        out = self.ct.c_float()
        rc = self.hip.hipEventElapsedTime(self.ct.byref(out), self.ev[i], self.ev[j])
        if rc != 0:
            raise RuntimeError("hipEventElapsedTime failed (%d)" % rc)
        return out.value

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)


_COPY_US = {}


def copy_same_bytes_us(torch, stream, nbytes, flush=None):
    """Median microseconds of a plain device-to-device copy (torch's copy_)
    that moves `nbytes` in all: nbytes/2 read and nbytes/2 written.  The
    achievable reference for a kernel whose algorithmic bytes are nbytes.
    With `flush` (a 1 GiB tensor), L2 and the Infinity Cache are flushed
    before each copy, as before a cold kernel."""
    key = (nbytes, flush is not None)
    if key not in _COPY_US:
        half = (nbytes // 2 + 15) // 16 * 16
        src = torch.ones(half, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        ev = HipEvents(2)
        ts = []
        for _ in range(7):
            if flush is not None:
                flush.sum()
            ev.record(0, stream)
            dst.copy_(src)
            ev.record(1, stream)
            torch.cuda.synchronize()
            ts.append(ev.ms(0, 1) * 1e3)
        ev.close()
        del src, dst
        _COPY_US[key] = float(np.median(ts))
    return _COPY_US[key]


SPIN_CYCLES = 400000      # ~0.2 ms of GPU clock: longer than the host needs to enqueue a call


def time_each(fn, iters, stream):
    """Microseconds of each of `iters` calls of fn(), from a pair of HIP
    events recorded on the launch stream around each call.  Before each call
    the stream runs a short spin kernel, so that the events and the call's
    launches are all enqueued while the GPU is busy: the time between the
    events is then the device's own (launch processing included), not the
    host's submission of a call that takes only a few microseconds."""
    import torch
    ev = HipEvents(2 * iters)
    for i in range(iters):
        torch.cuda._sleep(SPIN_CYCLES)
        ev.record(2 * i, stream)
        fn()
        ev.record(2 * i + 1, stream)
    torch.cuda.synchronize()
    us = [ev.ms(2 * i, 2 * i + 1) * 1e3 for i in range(iters)]
    ev.close()
    return us


def measure_workload(qr, I, torch, stream, config, n=None, codecs=None, iters=20,
                     kernels=True, cold=True, oneshot=True, dtype=None):
    """One workload of inputs.CONFIGS: per codec, the simulated allreduce
    (qr_allreduce_sim) timed call by call (median and min us, effective GB/s
    = 2n bytes / time); optionally the three kernels timed one by one through
    the staged calls (us, algorithmic GB/s, fraction of HBM peak) and stage 1
    after a cache flush; and the one-stage allreduce (qr_allreduce_oneshot,
    key "1stage"), whose algorithmic bytes are W*(W+1)*2n: every rank reads
    the W buffers and writes its own."""
    cfg = I.CONFIGS[config]
    W = cfg["W"]
    dtype = cfg["dtype"] if dtype is None else dtype
    n = cfg["n"] if n is None else n
    codecs = cfg["codecs"] if codecs is None else codecs
    xs = [torch.from_numpy(x.view(np.int16)).to("cuda") for x in I.make(config, n=n)]
    ys = [torch.empty_like(xs[0]) for _ in range(W)]
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda") if cold else None
    out = {}
    for c in codecs:
        wb = qr.qr_wire_bytes(c, n)
        ws = qr.alloc_workspace(W, c, n)
        for _ in range(3):
            qr.qr_allreduce_sim(c, xs, ys, ws, dtype=dtype)
        us = time_each(lambda: qr.qr_allreduce_sim(c, xs, ys, ws, dtype=dtype), iters, stream)
        med = float(np.median(us))
        r = {"us_median": med, "us_min": float(min(us)),
             "effective_gbps": 2 * n / (med * 1e-6) / 1e9}
        if kernels or cold:
            wires = [qr.alloc_wire(c, n) for _ in range(W)]
            red = qr.alloc_wire(c, n)
            launches = {
                "quantize": lambda: qr.qr_quantize_ranks(c, xs, wires, dtype=dtype),
                "stage1": lambda: qr.qr_reduce_stage1(c, wires, n, red, dtype),
                "stage2": lambda: qr.qr_gather_stage2(c, red, ys, dtype=dtype)}
            for f in launches.values():
                f()
        if kernels:
            r["kernels"] = {}
            for st, f in launches.items():
                t = float(np.median(time_each(f, iters, stream)))
                ab = algorithmic_bytes(st, W, n, wb)
                cu = copy_same_bytes_us(torch, stream, ab)
                r["kernels"][st] = {"us": t, "gbps": ab / (t * 1e-6) / 1e9,
                                    "frac": ab / (t * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                    "copy_us": cu, "vs_copy": cu / t}
        if cold:
            ts = []
            launches["quantize"]()
            for _ in range(5):
                flush.sum()
                ts += time_each(launches["stage1"], 1, stream)
            t = float(np.median(ts))
            ab = algorithmic_bytes("stage1", W, n, wb)
            cu = copy_same_bytes_us(torch, stream, ab, flush)
            r["stage1_cold"] = {"us": t, "gbps": ab / (t * 1e-6) / 1e9,
                                "frac": ab / (t * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                "copy_us": cu, "vs_copy": cu / t}
        if kernels or cold:
            del wires, red
        del ws
        out[I.CODEC_NAMES[c]] = r
    if oneshot:
        # the one-stage allreduce: one launch; every simulated rank reads all
        # W buffers and writes its own output
        for _ in range(3):
            qr.qr_allreduce_oneshot(xs, ys, dtype=dtype)
        us = time_each(lambda: qr.qr_allreduce_oneshot(xs, ys, dtype=dtype), iters, stream)
        med = float(np.median(us))
        ab = W * (W + 1) * 2 * n
        out["1stage"] = {"us_median": med, "us_min": float(min(us)),
                         "effective_gbps": 2 * n / (med * 1e-6) / 1e9,
                         "kernels": {"oneshot": {"us": med, "gbps": ab / (med * 1e-6) / 1e9,
                                                 "frac": ab / (med * 1e-6) / 1e9 /
                                                 HBM_PEAK_GBPS}}}
    del xs, ys, flush
    torch.cuda.empty_cache()
    return out


def measure_stage1_sizes(qr, I, torch, stream, sizes=(1 << 25, 1 << 27, 1 << 29), reps=5):
    """Stage 1 alone, cold, at W=2 and fp16 for growing rank buffers (64 MB,
    256 MB and 1 GiB per rank), every codec of the W=2 workload: the kernel's
    fraction of HBM peak once the transfer is large enough that launch ramp
    and drain no longer dominate.  Rank buffers larger than the workload's
    64 MB repeat its seeded buffers; stage 1's time does not depend on the
    values.  Beside each figure, a cold device copy of the same bytes."""
    cfg = I.CONFIGS[2]
    W, codecs = cfg["W"], cfg["codecs"]
    base = [torch.from_numpy(x.view(np.int16)).to("cuda") for x in I.make(2)]
    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    out = {}
    for n in sizes:
        xs = [b.repeat((n + b.numel() - 1) // b.numel())[:n].contiguous() for b in base]
        per = {}
        for c in codecs:
            wb = qr.qr_wire_bytes(c, n)
            wires = [qr.alloc_wire(c, n) for _ in range(W)]
            red = qr.alloc_wire(c, n)
            qr.qr_quantize_ranks(c, xs, wires, dtype=I.FP16)
            qr.qr_reduce_stage1(c, wires, n, red, I.FP16)
            ev = HipEvents(2)
            ts = []
            for _ in range(reps):
                flush.sum()
                ev.record(0, stream)
                qr.qr_reduce_stage1(c, wires, n, red, I.FP16)
                ev.record(1, stream)
                torch.cuda.synchronize()
                ts.append(ev.ms(0, 1) * 1e3)
            ev.close()
            t = float(np.median(ts))
            ab = algorithmic_bytes("stage1", W, n, wb)
            cu = copy_same_bytes_us(torch, stream, ab, flush)
            per[I.CODEC_NAMES[c]] = {"us": t, "algorithmic_bytes": ab,
                                     "gbps": ab / (t * 1e-6) / 1e9,
                                     "frac": ab / (t * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                     "copy_us": cu, "vs_copy": cu / t}
            del wires, red
            torch.cuda.empty_cache()
        out["%d" % (2 * n)] = per
        del xs
    del base, flush
    torch.cuda.empty_cache()
    return out


SWEEP_SIZES = tuple(2 ** k for k in range(11, 26))      # elements: 4 KB .. 64 MB per rank


def min_sizes(sweep):
    """From a sweep (measure_sweep's result): for every W and codec, the
    smallest rank buffer (bytes) from which the two-stage allreduce with that
    codec is faster than the one-stage allreduce at that size and at every
    larger size of the sweep; None where it is not faster at the largest size.
    The analogue of the minimum sizes below which the pages' wrapper keeps the
    one-stage kernel, for this single-GPU simulation (no link time)."""
    out = {}
    for Wk, per_size in sweep.items():
        sizes = sorted(per_size, key=int)
        row = {}
        for c in per_size[sizes[0]]:
            if c == "1stage":
                continue
            best = None
            for sz in reversed(sizes):
                if per_size[sz][c]["us"] < per_size[sz]["1stage"]["us"]:
                    best = int(sz)
                else:
                    break
            row[c] = best
        out[Wk] = row
    return out


def measure_sweep(qr, I, torch, stream, Ws=(2, 4, 8), sizes=SWEEP_SIZES, dtype=0):
    """The simulated allreduce (qr_allreduce_sim) of every codec, and the
    one-stage allreduce (key "1stage"), at every size from 4 KB to 64 MB per
    rank buffer and W = 2, 4, 8.  Buffers drawn as in the W=2 64 MB workload
    and rounded to the buffer type (`dtype`: 0 fp16, 1 bf16, 2 bf16 buffers
    through binary16, the cast option); rank r's buffer is the same at every
    W, and a smaller size is the leading part of the largest.  Per point:
    median and minimum us per call, timed call by call as in
    measure_workload."""
    Wmax, nmax = max(Ws), max(sizes)
    xs_all = [torch.from_numpy(x.view(np.int16)).to("cuda")
              for x in I.make(2, W=Wmax, n=nmax, dtype=I.BF16 if dtype else I.FP16)]
    ys_all = [torch.empty_like(x) for x in xs_all]
    res = {}
    for W in Ws:
        per_size = {}
        for n in sizes:
            xs = [x[:n] for x in xs_all[:W]]
            ys = [y[:n] for y in ys_all[:W]]
            iters = 100 if 2 * n <= (1 << 20) else 20
            r = {}
            for c in I.ALL_CODECS:
                ws = qr.alloc_workspace(W, c, n)
                for _ in range(3):
                    qr.qr_allreduce_sim(c, xs, ys, ws, dtype=dtype)
                us = time_each(lambda: qr.qr_allreduce_sim(c, xs, ys, ws, dtype=dtype),
                               iters, stream)
                r[I.CODEC_NAMES[c]] = {"us": float(np.median(us)), "us_min": float(min(us))}
                del ws
            for _ in range(3):
                qr.qr_allreduce_oneshot(xs, ys, dtype=dtype)
            us = time_each(lambda: qr.qr_allreduce_oneshot(xs, ys, dtype=dtype), iters, stream)
            r["1stage"] = {"us": float(np.median(us)), "us_min": float(min(us))}
            per_size["%d" % (2 * n)] = r
        res["W%d" % W] = per_size
    del xs_all, ys_all
    torch.cuda.empty_cache()
    return res


def cpu_baseline(codecs, dtype, xs_np, sample, threads):
    """The oracle as it stands, on blocks [0, sample/32) of every rank (the
    same computation as the full buffers restricted to those blocks), split
    over `threads` host threads by block range."""
    import oracle
    n = xs_np[0].size
    nb = min(sample, n) // 32
    bounds = np.linspace(0, nb, threads + 1).astype(int)
    ys = [np.zeros(n, np.uint16) for _ in xs_np]

    def work(lo, hi, codec):
        oracle.allreduce(codec, dtype, xs_np, int(lo), int(hi), ys=ys)

    t0 = time.perf_counter()
    for codec in codecs:
        ts = [threading.Thread(target=work, args=(bounds[i], bounds[i + 1], codec))
              for i in range(threads)]
        for t in ts:
            t.start()
        for t in ts:
            t.join()
    dt = time.perf_counter() - t0
    payload = len(codecs) * nb * 32 * 2
    # the same scalar code on one thread, on a sixteenth of the sample
    nb1 = max(1, nb // 16)
    t1 = time.perf_counter()
    for codec in codecs:
        work(0, nb1, codec)
    dt1 = time.perf_counter() - t1
    return {"value": payload / dt / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "blocks 0..%d (%d elements = %.1f MB per rank) of each of the %d "
                      "ranks, all %d codecs, full pipeline; %.2f s wall" % (
                          nb, nb * 32, nb * 64 / 2 ** 20, len(xs_np), len(codecs), dt),
            "seconds": dt,
            "single_thread": {"value": len(codecs) * nb1 * 64 / dt1 / 1e9, "unit": "GB/s",
                              "sample": "blocks 0..%d, %.2f s" % (nb1, dt1)},
            "host": host_info()}


def host_info():
    """core count and CPU model of the host the oracle ran on"""
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"cpu_count": os.cpu_count(), "usable_cores": len(os.sched_getaffinity(0)),
            "model": model}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU: the W ranks of the allreduce are simulated "
              "as W buffers on that GPU; --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    from quantized_two_stage_amd import inputs as I
    from quantized_two_stage_amd import qr

    torch.cuda.set_device(0)
    cfg = I.CONFIGS[args.config]
    W, n, dtype, codecs = cfg["W"], cfg["n"], cfg["dtype"], cfg["codecs"]
    print("bench: config %d (%s), generating inputs" % (args.config, cfg["desc"]),
          file=sys.stderr, flush=True)
    xs_np = I.make(args.config)
    xs = [torch.from_numpy(x.view(np.int16)).to("cuda") for x in xs_np]
    ys = [torch.empty_like(xs[0]) for _ in range(W)]
    bufs = {}
    for c in codecs:
        wb = qr.qr_wire_bytes(c, n)
        bufs[c] = ([qr.alloc_wire(c, n) for _ in range(W)], qr.alloc_wire(c, n), wb)
    stream = torch.cuda.current_stream()

    def one_allreduce(c, ev=None, base=0):
        wires, red, _ = bufs[c]
        if ev is not None:
            ev.record(base, stream)
        qr.qr_quantize_ranks(c, xs, wires, dtype=dtype)
        if ev is not None:
            ev.record(base + 1, stream)
        qr.qr_reduce_stage1(c, wires, n, red, dtype)
        if ev is not None:
            ev.record(base + 2, stream)
        qr.qr_gather_stage2(c, red, ys, dtype=dtype)
        if ev is not None:
            ev.record(base + 3, stream)

    # one workspace per codec for the one-call entry point
    wss = {c: qr.alloc_workspace(W, c, n) for c in codecs}

    # check once: the staged calls give what the one-call entry point gives
    ys_ref = [torch.empty_like(xs[0]) for _ in range(W)]
    qr.qr_allreduce_sim(codecs[0], xs, ys_ref, wss[codecs[0]], dtype=dtype)
    one_allreduce(codecs[0])
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip(ys, ys_ref)), "staged != one-call"
    del ys_ref

    for _ in range(args.warmup):
        for c in codecs:
            qr.qr_allreduce_sim(c, xs, ys, wss[c], dtype=dtype)
            one_allreduce(c)
    torch.cuda.synchronize()

    # pass 1: the timed region
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        for c in codecs:
            qr.qr_allreduce_sim(c, xs, ys, wss[c], dtype=dtype)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / args.steps

    # pass 2: the same steps, staged, with events around every launch
    nc = len(codecs)
    evs = HipEvents(4 * nc * args.steps)
    print("bench: instrumented pass, %d steps" % args.steps, file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(args.steps):
        for ci, c in enumerate(codecs):
            one_allreduce(c, evs, 4 * (s * nc + ci))
    torch.cuda.synchronize()
    ms_per_step_instr = (time.perf_counter() - t1) * 1e3 / args.steps

    stages = ("quantize", "stage1", "stage2")
    kernels, per_codec = [], {}
    for ci, c in enumerate(codecs):
        d = np.array([[evs.ms(4 * (s * nc + ci) + k, 4 * (s * nc + ci) + k + 1)
                       for k in range(3)] for s in range(args.steps)])            # ms
        avg = d.mean(axis=0)
        wb = bufs[c][2]
        us = float(avg.sum() * 1e3)
        per_codec[I.CODEC_NAMES[c]] = {
            "us": us, "us_median": float(np.median(d.sum(axis=1)) * 1e3),
            "effective_gbps": 2 * n / (us * 1e-6) / 1e9}
        for k, st in enumerate(stages):
            ab = algorithmic_bytes(st, W, n, wb)
            cu = copy_same_bytes_us(torch, stream, ab)
            kernels.append({"kernel": "%s/%s" % (st, I.CODEC_NAMES[c]),
                            "us": float(avg[k] * 1e3),
                            "algorithmic_bytes": ab,
                            "gbps": ab / (avg[k] * 1e-3) / 1e9,
                            "copy_us": cu, "vs_copy": cu / float(avg[k] * 1e3)})
    evs.close()
    total_payload = len(codecs) * 2 * n
    value = total_payload / (ms_per_step * 1e-3) / 1e9
    dom = max(kernels, key=lambda k: k["us"])
    traffic = None
    if os.path.exists(PROFILE_TRAFFIC) and args.config == 2:    # the profiled workload
        tr = json.load(open(PROFILE_TRAFFIC))
        ent = tr.get("kernels", {}).get(dom["kernel"])
        if ent and tr.get("source_sha") == kernel_source_sha():
            traffic = ent["bytes"]
    roofline = {"bound": "hbm", "kernel": dom["kernel"], "achieved": dom["gbps"],
                "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": dom["gbps"] / HBM_PEAK_GBPS,
                "traffic": traffic, "algorithmic_bytes_per_launch": dom["algorithmic_bytes"],
                "avg_launch_us": dom["us"], "copy_same_bytes_us": dom["copy_us"],
                "vs_copy": dom["vs_copy"]}

    # plain device copies: 64 MB (fits the 256 MB Infinity Cache, like the
    # workload's own buffers) and 1 GiB (streams from HBM)
    copy_gbps = {}
    for size in (64 << 20, 1 << 30):
        src = torch.empty(size, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20 if size < (1 << 30) else 5
        e0.record(stream)
        for _ in range(reps):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_gbps["%dMiB" % (size >> 20)] = 2 * size * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
        del src, dst

    # the floor of a call's time as time_each measures it: one launch of a
    # kernel that writes a single element
    tiny = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        tiny.zero_()
    launch_floor_us = float(np.median(time_each(lambda: tiny.zero_(), 100, stream)))
    del tiny

    cold = None
    if not args.no_cold:
        # stage 1 with L2 and the 256 MB Infinity Cache flushed before each
        # timed launch by reading 1 GiB of other data (a read leaves no dirty
        # lines to write back during the timed kernel)
        flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        cold = {}
        for c in codecs:
            wires, red, wb = bufs[c]
            qr.qr_quantize_ranks(c, xs, wires, dtype=dtype)
            ts = []
            ce = HipEvents(2)
            for _ in range(5):
                flush.sum()
                ce.record(0, stream)
                qr.qr_reduce_stage1(c, wires, n, red, dtype)
                ce.record(1, stream)
                torch.cuda.synchronize()
                ts.append(ce.ms(0, 1))
            ce.close()
            us = float(np.median(ts) * 1e3)
            ab = algorithmic_bytes("stage1", W, n, wb)
            cu = copy_same_bytes_us(torch, stream, ab, flush)
            cold["stage1/" + I.CODEC_NAMES[c]] = {"us": us, "gbps": ab / (us * 1e-6) / 1e9,
                                                  "frac": ab / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS,
                                                  "copy_us": cu, "vs_copy": cu / us}
        del flush

    extra = None
    if not args.no_extra:
        extra = {}
        for cid in (2, 5, 4):
            c = I.CONFIGS[cid]
            print("bench: config %d (%s)" % (cid, c["desc"]), file=sys.stderr, flush=True)
            extra["config%d" % cid] = {
                "workload": c["desc"], "W": c["W"], "elements_per_rank": c["n"],
                "per_codec": measure_workload(qr, I, torch, stream, cid, cold=not args.no_cold)}
        # the bf16 -> fp16 cast option (buffer type 2) on the bf16 workload
        c = I.CONFIGS[4]
        print("bench: config 4 with the bf16->fp16 cast", file=sys.stderr, flush=True)
        extra["config4_cast"] = {
            "workload": c["desc"] + "; bf16 buffers through binary16 (cast option)",
            "W": c["W"], "elements_per_rank": c["n"],
            "per_codec": measure_workload(qr, I, torch, stream, 4, cold=False,
                                          dtype=qr.QR_BF16_VIA_FP16)}
        print("bench: stage 1 alone, cold, W=2, 64 MB .. 1 GiB per rank", file=sys.stderr,
              flush=True)
        extra["stage1_sizes"] = {
            "workload": "stage 1 alone, cold caches, W=2 fp16, codecs of the W=2 64 MB workload; "
                        "rank buffers beyond 64 MB repeat its seeded buffers",
            "key": "bytes per rank buffer",
            "results": measure_stage1_sizes(qr, I, torch, stream)}
        c = I.CONFIGS[3]
        print("bench: config 3 size sweep (%s)" % c["desc"], file=sys.stderr, flush=True)
        sweep = {}
        for size in c["sizes"]:
            iters = 100 if 2 * size <= (1 << 20) else 20
            r = measure_workload(qr, I, torch, stream, 3, n=size, iters=iters,
                                 kernels=False, cold=False)
            sweep["%d" % (2 * size)] = r
        extra["config3_sweep"] = {"workload": c["desc"], "W": c["W"],
                                  "key": "bytes per rank buffer", "per_size": sweep}
        print("bench: size sweep, W=2/4/8, every codec, fp16", file=sys.stderr, flush=True)
        extra["sweep_fp16"] = {
            "workload": "fp16 buffers drawn as the W=2 64 MB workload, 4 KB..64 MB per rank, "
                        "W=2/4/8, every codec and the one-stage allreduce; us per call "
                        "(median, min)",
            "key": "W, then bytes per rank buffer",
            "results": measure_sweep(qr, I, torch, stream)}
        print("bench: size sweep, bf16 and bf16 through fp16", file=sys.stderr, flush=True)
        for key, dt, what in (("sweep_bf16", I.BF16, "bf16 buffers"),
                              ("sweep_bf16_via_fp16", 2, "bf16 buffers through binary16 "
                                                         "(the cast option)")):
            extra[key] = {
                "workload": "%s drawn as the W=2 64 MB workload, 4 KB..64 MB per rank, "
                            "W=2/4/8, every codec and the one-stage allreduce; us per call "
                            "(median, min)" % what,
                "key": "W, then bytes per rank buffer",
                "results": measure_sweep(qr, I, torch, stream, dtype=dt)}
        extra["min_sizes"] = {
            "what": "per buffer type, W and codec: the smallest rank buffer (bytes) from which "
                    "the two-stage allreduce is faster than the one-stage allreduce at every "
                    "larger size of the sweep (null: not faster at 64 MB)",
            "fp16": min_sizes(extra["sweep_fp16"]["results"]),
            "bf16": min_sizes(extra["sweep_bf16"]["results"]),
            "bf16_via_fp16": min_sizes(extra["sweep_bf16_via_fp16"]["results"])}

    cpu = None
    if not args.no_cpu_baseline:
        threads = min(16, os.cpu_count() or 1)
        print("bench: CPU oracle on a sample, %d threads" % threads, file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(codecs, dtype, xs_np, args.cpu_sample, threads)

    out = {
        "metric": METRIC, "value": value, "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "ms_per_step_instrumented": ms_per_step_instr,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "W=%d simulated ranks, %s, %d elements (%d MB) per rank, "
                               "codecs %s, 32-element blocks; %s" % (
                                   W, "fp16" if dtype == 0 else "bf16", n, 2 * n >> 20,
                                   "/".join(I.CODEC_NAMES[c] for c in codecs), cfg["desc"]),
                   "W": W, "elements_per_rank": n, "buffer_dtype": "fp16" if dtype == 0
                   else "bf16", "codecs": [I.CODEC_NAMES[c] for c in codecs],
                   "allreduces_per_step": len(codecs)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_codec": per_codec,
        "kernels": kernels,
        "stage1_cold": cold,
        "other_workloads": extra,
        "device_copy_gbps": copy_gbps,
        "launch_floor_us": launch_floor_us,
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
