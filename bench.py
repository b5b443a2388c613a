"""Benchmark of the simulated two-stage quantized allreduce on one MI355X.

Workload (default): W=8 simulated ranks, fp16, 64 MB (32 Mi elements) per
rank buffer, every codec (FP, fp8, Q8, Q6, Q4 symmetric, Q8, Q6, Q4
asymmetric); 32-element blocks cycling N(0,1) with all-zero, constant,
single-spike and +-max-finite blocks.  One step = one simulated allreduce per
codec (qr_allreduce_sim: quantize into the receive buffer, fused stage 1,
stage 2), eight allreduces.  Inputs are resident in HBM before the timed
region starts.

Passes, in order:
  1. the timed region: K steps, nothing but the qr_allreduce_sim calls on the
     stream; `value` (per-rank payload bytes 2n per allreduce, over the step
     time) and `ms_per_step` come from it;
  2. the instrumented pass: the same K steps as the three staged calls with a
     HIP event on the launch stream before and after every launch: the
     in-pipeline duration of every kernel;
  3. cold launches: each stage of each codec alone after reading 1 GiB of
     other data (L2 and the 256 MB Infinity Cache hold none of its bytes),
     beside the same-bytes references: the stage-1 access pattern without
     the arithmetic (libqr_pattern.so) and a plain device copy.

`roofline` is stage 1 (the fused dequantize-sum-requantize kernel), cold: its
algorithmic bytes per launch, (W+1) * wire bytes, over its event-timed
duration; `frac` is the lowest over the eight codecs, each codec's figure and
its access-pattern ceiling beside it.  `cpu_baseline` times the CPU oracle on
a bounded sample of the same workload.  The one JSON line on stdout carries
the contract fields and compact per-codec figures; --extra PATH writes the
other workloads, the size sweeps and the minimum-size table to a file, and
--stage1-scan PATH stage 1 at 8 to 256 MB per rank beside its access pattern
and a copy of the same bytes, and --stream-probes PATH plain reads, writes and
copies of the memory system.
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
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "bench_w8_fp16_64MB_stage1_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "quantized_two_stage_amd", "csrc", f)
                  for f in ("qr_kernels.hip", "qr_device.h", "qr_stage_io.h")]
STAGES = ("quantize", "stage1", "stage2")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--config", type=int, default=5)
    p.add_argument("--cold-reps", type=int, default=15)
    p.add_argument("--no-cold", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=1 << 21,
                   help="elements per rank of the oracle's sample")
    p.add_argument("--extra", metavar="PATH",
                   help="also measure the other workloads, the size sweeps and the "
                        "minimum-size table, written as JSON to PATH")
    p.add_argument("--sweep-repeats", type=int, default=3)
    p.add_argument("--stream-probes", metavar="PATH",
                   help="also time plain reads, writes and copies (one or four 16-byte "
                        "accesses per lane, cached or non-temporal) cold at 192 MiB-1.1 GiB, "
                        "written as JSON to PATH")
    p.add_argument("--stage1-scan", metavar="PATH",
                   help="also time stage 1 cold at 8-256 MB per rank (W=8) beside its "
                        "access pattern and a copy of the same bytes, written as JSON to PATH")
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
    W wire images and writes one; stage 2 reads the reduced image once per
    rank and writes 2n per rank."""
    if stage == "quantize":
        return W * (2 * n + wb)
    if stage == "stage1":
        return (W + 1) * wb
    return W * (wb + 2 * n)


def hbm_bytes_stage2(W, n, wb):
    """stage 2's HBM floor in this simulation: the one reduced image is read
    once from HBM (the W simulated ranks' re-reads hit the caches) and the W
    outputs are written"""
    return wb + W * 2 * n


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


class Pattern:
    """libqr_pattern.so: stage 1's loads and stores without the arithmetic"""

    def __init__(self):
        import ctypes
        from quantized_two_stage_amd import build as qbuild
        if not os.path.exists(qbuild.PATTERN_LIB):
            raise ImportError("libqr_pattern.so is not built (%s)" % qbuild.PATTERN_LIB)
        self.L = ctypes.CDLL(qbuild.PATTERN_LIB)
        P, i32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        self.L.qrp_stage1_pattern.argtypes = [i32, i32, P, sz, P, P]
        self.L.qrp_stage1_pattern.restype = i32
        self.L.qrp_stream.argtypes = [i32, i32, i32, P, P, sz, P]
        self.L.qrp_stream.restype = i32
        self.ct = ctypes

    def stream(self, kind, per_lane, nt, src, dst, nbytes, stream):
        """qrp_stream: kind 0 read, 1 write, 2 copy of nbytes (src, dst: device
        tensors of at least nbytes)"""
        rc = self.L.qrp_stream(kind, per_lane, nt, self.ct.c_void_p(src.data_ptr()),
                               self.ct.c_void_p(dst.data_ptr()), nbytes,
                               self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("qrp_stream failed (%d)" % rc)

    def stage1(self, codec, W, recv, n, red, stream):
        rc = self.L.qrp_stage1_pattern(codec, W, self.ct.c_void_p(recv.data_ptr()), n,
                                       self.ct.c_void_p(red.data_ptr()),
                                       self.ct.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError("qrp_stage1_pattern failed (%d)" % rc)


class Cold:
    """Cold launches: before each, a read of 1 GiB of other data evicts L2 and
    the Infinity Cache without leaving dirty lines; the launch alone is
    bracketed by HIP events; the median of `reps` launches."""

    def __init__(self, torch, stream, reps):
        self.torch, self.stream, self.reps = torch, stream, reps
        # binary32, so that sum() is one reduction reading the 1 GiB (an
        # integer sum would first write a widened copy: dirty lines)
        self.flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        self.ev = HipEvents(2)

    def us(self, fn, reps=None):
        ts = []
        for _ in range(reps or self.reps):
            self.flush.sum()
            self.ev.record(0, self.stream)
            fn()
            self.ev.record(1, self.stream)
            self.torch.cuda.synchronize()
            ts.append(self.ev.ms(0, 1) * 1e3)
        return float(np.median(ts))

    def us_interleaved(self, fns, reps=None):
        """{name: median us} of cold launches of several functions taken in
        turn, one launch of each per round, so that they see the same drift of
        the machine's state"""
        ts = {k: [] for k in fns}
        for _ in range(reps or self.reps):
            for k, fn in fns.items():
                ts[k].append(self.us(fn, 1))
        return {k: float(np.median(v)) for k, v in ts.items()}

    def copy_fn(self, nbytes):
        """a plain device copy moving nbytes in all (half read, half written),
        as a function to time, and the buffers to free afterwards"""
        half = (nbytes // 2 + 15) // 16 * 16
        src = self.torch.ones(half, dtype=self.torch.uint8, device="cuda")
        dst = self.torch.empty_like(src)
        dst.copy_(src)
        return (lambda: dst.copy_(src)), (src, dst)

    def close(self):
        self.ev.close()
        del self.flush


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


def frac(nbytes, us):
    return nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS


# ---------------------------------------------------------------------------
# the headline workload

def measure_headline(args, qr, I, torch, stream, log):
    cfg = I.CONFIGS[args.config]
    W, n, dtype, codecs = cfg["W"], cfg["n"], cfg["dtype"], cfg["codecs"]
    log("bench: config %d (%s), generating inputs" % (args.config, cfg["desc"]))
    xs_np = I.make(args.config)
    xs = [torch.from_numpy(x.view(np.int16)).to("cuda") for x in xs_np]
    ys = [torch.empty_like(xs[0]) for _ in range(W)]
    bufs = {}
    for c in codecs:
        bufs[c] = dict(ws=qr.alloc_workspace(W, c, n), recv=qr.alloc_recv(W, c, n),
                       red=qr.alloc_wire(c, n), wb=qr.qr_wire_bytes(c, n))

    def staged(c, ev=None, base=0):
        b = bufs[c]
        if ev is not None:
            ev.record(base, stream)
        qr.qr_quantize_recv(c, xs, b["recv"], dtype=dtype)
        if ev is not None:
            ev.record(base + 1, stream)
        qr.qr_reduce_recv(c, W, b["recv"], n, b["red"], dtype)
        if ev is not None:
            ev.record(base + 2, stream)
        qr.qr_gather_stage2(c, b["red"], ys, dtype=dtype)
        if ev is not None:
            ev.record(base + 3, stream)

    # the staged calls give what the one-call entry point gives
    ys_ref = [torch.empty_like(xs[0]) for _ in range(W)]
    for c in codecs:
        qr.qr_allreduce_sim(c, xs, ys_ref, bufs[c]["ws"], dtype=dtype)
        staged(c)
        torch.cuda.synchronize()
        assert all(torch.equal(a, b) for a, b in zip(ys, ys_ref)), ("staged != one call", c)
    del ys_ref

    for _ in range(args.warmup):
        for c in codecs:
            qr.qr_allreduce_sim(c, xs, ys, bufs[c]["ws"], dtype=dtype)
    torch.cuda.synchronize()

    # pass 1: the timed region
    log("bench: timing %d steps" % args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        for c in codecs:
            qr.qr_allreduce_sim(c, xs, ys, bufs[c]["ws"], dtype=dtype)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps

    # pass 2: the same steps, staged, with events around every launch
    nc = len(codecs)
    evs = HipEvents(4 * nc * args.steps)
    log("bench: instrumented pass, %d steps" % args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for s in range(args.steps):
        for ci, c in enumerate(codecs):
            staged(c, evs, 4 * (s * nc + ci))
    torch.cuda.synchronize()
    ms_instr = (time.perf_counter() - t1) * 1e3 / args.steps
    per = {}
    for ci, c in enumerate(codecs):
        d = np.array([[evs.ms(4 * (s * nc + ci) + k, 4 * (s * nc + ci) + k + 1)
                       for k in range(3)] for s in range(args.steps)]) * 1e3     # us
        wb = bufs[c]["wb"]
        per[c] = {"us_per_allreduce": float(d.sum(axis=1).mean()),
                  "kernels": {st: {"us": float(d[:, k].mean()),
                                   "frac": frac(algorithmic_bytes(st, W, n, wb), d[:, k].mean())}
                              for k, st in enumerate(STAGES)}}
        per[c]["kernels"]["stage2"]["frac_hbm"] = frac(hbm_bytes_stage2(W, n, wb),
                                                       d[:, 2].mean())
    evs.close()

    cold = None
    if not args.no_cold:
        log("bench: cold launches, references")
        pat = Pattern()
        cl = Cold(torch, stream, args.cold_reps)
        cold = {}
        for c in codecs:
            b = bufs[c]
            wb = b["wb"]
            staged(c)
            torch.cuda.synchronize()
            r = {}
            r["quantize"] = cl.us(lambda: qr.qr_quantize_recv(c, xs, b["recv"], dtype=dtype))
            r["stage2"] = cl.us(lambda: qr.qr_gather_stage2(c, b["red"], ys, dtype=dtype))
            # stage 1 and its references, in turn: the access pattern alone,
            # a plain copy of the same bytes, and the same stage 1 from W
            # separate wire images (W streams instead of the receive
            # buffer's one)
            ab1 = algorithmic_bytes("stage1", W, n, wb)
            copy, keep = cl.copy_fn(ab1)
            wires = [qr.alloc_wire(c, n) for _ in range(W)]
            qr.qr_quantize_ranks(c, xs, wires, dtype=dtype)
            red2 = qr.alloc_wire(c, n)
            t = cl.us_interleaved({
                "stage1": lambda: qr.qr_reduce_recv(c, W, b["recv"], n, b["red"], dtype),
                "stage1_pattern": lambda: pat.stage1(c, W, b["recv"], n, red2, stream),
                "stage1_copy": copy,
                "stage1_planar": lambda: qr.qr_reduce_stage1(c, wires, n, red2, dtype)})
            r.update(t)
            del wires, keep, red2
            staged(c)           # leave the reduced image the kernels wrote
            cold[c] = r
        cl.close()
    return dict(cfg=cfg, W=W, n=n, dtype=dtype, codecs=codecs, bufs=bufs, xs_np=xs_np,
                ms_per_step=ms_per_step, ms_per_step_instrumented=ms_instr, per=per,
                cold=cold)


def roofline(h, I):
    """stage 1 cold, lowest codec; each codec beside it with its access-pattern
    ceiling; the kernel that takes the most time in the pipeline as a
    secondary field"""
    W, n, cold, per = h["W"], h["n"], h["cold"], h["per"]
    src = cold if cold is not None else {c: {"stage1": per[c]["kernels"]["stage1"]["us"]}
                                         for c in h["codecs"]}
    fr = {}
    for c in h["codecs"]:
        wb = h["bufs"][c]["wb"]
        fr[c] = frac(algorithmic_bytes("stage1", W, n, wb), src[c]["stage1"])
    worst = min(fr, key=fr.get)
    wb = h["bufs"][worst]["wb"]
    ab = algorithmic_bytes("stage1", W, n, wb)
    us = src[worst]["stage1"]
    kname = "k_sum_fp" if worst == I.FP else "k_stage1"
    traffic = None
    if os.path.exists(PROFILE_TRAFFIC):
        tr = json.load(open(PROFILE_TRAFFIC))
        ent = tr.get("kernels", {}).get("stage1/" + I.CODEC_NAMES[worst])
        if ent and tr.get("source_sha") == kernel_source_sha() and \
                tr.get("workload") == h["cfg"]["desc"]:
            traffic = ent["bytes"]
    dom_c, dom_st = max(((c, st) for c in h["codecs"] for st in STAGES),
                        key=lambda k: per[k[0]]["kernels"][k[1]]["us"])
    out = {"bound": "hbm", "kernel": "%s (stage 1, receive buffer), %s, %s" % (
               kname, I.CODEC_NAMES[worst], "cold" if cold is not None else "in pipeline"),
           "achieved": ab / (us * 1e-6) / 1e9, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
           "frac": fr[worst], "traffic": traffic, "algorithmic_bytes_per_launch": ab,
           "avg_launch_us": us,
           "per_codec_frac": {I.CODEC_NAMES[c]: round(fr[c], 4) for c in h["codecs"]}}
    if cold is not None:
        out["pattern_frac"] = {I.CODEC_NAMES[c]: round(frac(algorithmic_bytes(
            "stage1", W, n, h["bufs"][c]["wb"]), cold[c]["stage1_pattern"]), 4)
            for c in h["codecs"]}
        out["copy_frac"] = {I.CODEC_NAMES[c]: round(frac(algorithmic_bytes(
            "stage1", W, n, h["bufs"][c]["wb"]), cold[c]["stage1_copy"]), 4)
            for c in h["codecs"]}
        out["in_pipeline_frac"] = {I.CODEC_NAMES[c]: round(
            per[c]["kernels"]["stage1"]["frac"], 4) for c in h["codecs"]}
    out["dominant_kernel"] = {"kernel": "%s/%s" % (dom_st, I.CODEC_NAMES[dom_c]),
                              "us": per[dom_c]["kernels"][dom_st]["us"],
                              "frac": per[dom_c]["kernels"][dom_st]["frac"]}
    return out


# ---------------------------------------------------------------------------
# the CPU oracle

def cpu_baseline(codecs, dtype, xs_np, sample, threads):
    """The oracle as it stands, the full pipeline of every codec on blocks
    [0, sample/32) of every rank (the computation of the whole buffers
    restricted to those blocks): once on `threads` host threads split by block
    range (ctypes releases the GIL), best of 3, and once on one thread."""
    import oracle
    n = xs_np[0].size
    nb = min(sample, n) // 32
    bounds = np.linspace(0, nb, threads + 1).astype(int)
    ys = [np.zeros(n, np.uint16) for _ in xs_np]

    def work(lo, hi, codec):
        oracle.allreduce(codec, dtype, xs_np, int(lo), int(hi), ys=ys)

    def run_threads():
        t0 = time.perf_counter()
        for codec in codecs:
            ts = [threading.Thread(target=work, args=(bounds[i], bounds[i + 1], codec))
                  for i in range(threads)]
            for t in ts:
                t.start()
            for t in ts:
                t.join()
        return time.perf_counter() - t0

    dt = min(run_threads() for _ in range(3))
    t1 = time.perf_counter()
    for codec in codecs:
        work(0, nb, codec)
    dt1 = time.perf_counter() - t1
    payload = len(codecs) * nb * 32 * 2
    return {"value": payload / dt / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": "blocks 0..%d (%d elements = %.1f MiB) of each of the %d ranks, all %d "
                      "codecs, full pipeline; best of 3 on %d threads %.2f s" % (
                          nb, nb * 32, nb * 64 / 2 ** 20, len(xs_np), len(codecs), threads, dt),
            "single_thread": {"value": payload / dt1 / 1e9, "unit": "GB/s",
                              "seconds": round(dt1, 2)},
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


# ---------------------------------------------------------------------------
# other workloads (--extra)

def measure_workload(qr, I, torch, stream, config, n=None, iters=20, cold=True, dtype=None,
                     oneshot=True):
    """One workload of inputs.CONFIGS: per codec, qr_allreduce_sim timed call
    by call (median and min us, effective GB/s = 2n / time), and cold stage 1
    through the receive buffer beside the cold access pattern of the same
    launch (its loads and stores alone); the one-stage allreduce (key
    "1stage")."""
    cfg = I.CONFIGS[config]
    W = cfg["W"]
    dtype = cfg["dtype"] if dtype is None else dtype
    n = cfg["n"] if n is None else n
    xs = [torch.from_numpy(x.view(np.int16)).to("cuda") for x in I.make(config, n=n)]
    ys = [torch.empty_like(xs[0]) for _ in range(W)]
    cl = Cold(torch, stream, 11) if cold else None
    pat = Pattern() if cold else None
    out = {}
    for c in cfg["codecs"]:
        ws = qr.alloc_workspace(W, c, n)
        for _ in range(3):
            qr.qr_allreduce_sim(c, xs, ys, ws, dtype=dtype)
        us = time_each(lambda: qr.qr_allreduce_sim(c, xs, ys, ws, dtype=dtype), iters, stream)
        med = float(np.median(us))
        r = {"us_median": med, "us_min": float(min(us)),
             "effective_gbps": 2 * n / (med * 1e-6) / 1e9}
        if cold:
            recv, red = qr.alloc_recv(W, c, n), qr.alloc_wire(c, n)
            qr.qr_quantize_recv(c, xs, recv, dtype=dtype)
            red2 = qr.alloc_wire(c, n)
            tt = cl.us_interleaved({
                "k": lambda: qr.qr_reduce_recv(c, W, recv, n, red, dtype),
                "p": lambda: pat.stage1(c, W, recv, n, red2, stream)})
            t, tp = tt["k"], tt["p"]
            del red2
            r["stage1_cold_us"] = t
            ab = algorithmic_bytes("stage1", W, n, qr.qr_wire_bytes(c, n))
            r["stage1_cold_frac"] = frac(ab, t)
            r["pattern_cold_us"] = tp
            r["pattern_cold_frac"] = frac(ab, tp)
            r["stage1_vs_pattern"] = tp / t
            del recv, red
        del ws
        out[I.CODEC_NAMES[c]] = r
    if oneshot:
        for _ in range(3):
            qr.qr_allreduce_oneshot(xs, ys, dtype=dtype)
        us = time_each(lambda: qr.qr_allreduce_oneshot(xs, ys, dtype=dtype), iters, stream)
        med = float(np.median(us))
        out["1stage"] = {"us_median": med, "us_min": float(min(us)),
                         "frac": frac(W * (W + 1) * 2 * n, med)}
    if cl is not None:
        cl.close()
    del xs, ys
    torch.cuda.empty_cache()
    return out


SWEEP_SIZES = tuple(2 ** k for k in range(11, 26))      # elements: 4 KB .. 64 MB per rank


def measure_sweep(qr, I, torch, stream, repeats, Ws=(2, 4, 8), sizes=SWEEP_SIZES, dtype=0):
    """qr_allreduce_sim of every codec and the one-stage allreduce ("1stage")
    at every size from 4 KB to 64 MB per rank buffer and W = 2, 4, 8; buffers
    drawn as in the W=2 64 MB workload, rounded to the buffer type (0 fp16,
    1 bf16, 2 bf16 through binary16); a smaller size is the leading part of
    the largest.  Every point is measured `repeats` times, each time the
    median of a run of calls (100 calls up to 1 MB, 20 above); the point
    keeps the median of those medians and their spread (max - min)."""
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
            calls = {I.CODEC_NAMES[c]: (lambda c=c, ws=qr.alloc_workspace(W, c, n):
                                        qr.qr_allreduce_sim(c, xs, ys, ws, dtype=dtype))
                     for c in I.ALL_CODECS}
            calls["1stage"] = lambda: qr.qr_allreduce_oneshot(xs, ys, dtype=dtype)
            meds = {k: [] for k in calls}
            for _ in range(repeats):
                for k, f in calls.items():
                    for _ in range(3):
                        f()
                    meds[k].append(float(np.median(time_each(f, iters, stream))))
            per_size["%d" % (2 * n)] = {k: {"us": float(np.median(v)),
                                            "spread": float(max(v) - min(v))}
                                        for k, v in meds.items()}
            del calls
        res["W%d" % W] = per_size
    del xs_all, ys_all
    torch.cuda.empty_cache()
    return res


MIN_SIZE_MARGIN = 0.30


def min_sizes(sweep, margin=MIN_SIZE_MARGIN):
    """For every W and codec: the smallest rank buffer (bytes) from which the
    two-stage allreduce beats the one-stage allreduce at that size and at
    every larger size of the sweep; None where it does not win at the
    largest size.  A win needs both: the two-stage median at most
    (1 - margin) times the one-stage median, and the gap wider than both
    points' spread (two-stage median + spread below one-stage median -
    spread).  The analogue of the minimum sizes below which the pages'
    wrapper keeps another allreduce, for this single-GPU simulation (no link
    time).  Also returns the deciding points (every point the rule looked
    at) whose time ratio lies within 1% of 1 - margin, where a repeat run
    may decide the other way."""
    out, marginal = {}, []
    for Wk, per_size in sweep.items():
        sizes = sorted(per_size, key=int)
        row = {}
        for c in per_size[sizes[0]]:
            if c == "1stage":
                continue
            best = None
            for sz in reversed(sizes):
                a, b = per_size[sz][c], per_size[sz]["1stage"]
                ratio = a["us"] / b["us"]
                if abs(ratio - (1 - margin)) < 0.01:
                    marginal.append({"W": Wk, "codec": c, "bytes": int(sz),
                                     "ratio": round(ratio, 4)})
                if a["us"] + a["spread"] < b["us"] - b["spread"] and ratio <= 1 - margin:
                    best = int(sz)
                else:
                    break
            row[c] = best
        out[Wk] = row
    return out, marginal


def launch_floor(torch, stream, iters=100, repeats=3):
    """the device time of one launch of a kernel that does nothing (torch's
    spin kernel asked for zero cycles), timed as every sweep point is: the
    floor under any one-launch call"""
    meds = []
    for _ in range(repeats):
        for _ in range(3):
            torch.cuda._sleep(0)
        meds.append(float(np.median(time_each(lambda: torch.cuda._sleep(0), iters, stream))))
    return {"us": float(np.median(meds)), "spread": float(max(meds) - min(meds))}


SCAN_SIZES = tuple(2 ** k for k in range(22, 28))        # elements: 8 .. 256 MB per rank


def measure_stage1_scan(qr, I, torch, stream, log, sizes=SCAN_SIZES, reps=11):
    """Stage 1 of the W=8 fp16 workload (same generator, a smaller size being
    the leading part of the largest) at 8 to 256 MB per rank, cold, each
    codec's launch in turn with its access pattern and a plain copy of the
    same bytes: whether a larger launch streams faster than the 64 MB one.
    Per codec and kernel: us and fraction of 8 TB/s at every size, and the
    plateau, the median fraction over the sizes from 64 MB per rank up."""
    cfg = I.CONFIGS[5]
    W, dtype, nmax = cfg["W"], cfg["dtype"], max(sizes)
    log("bench: stage-1 size scan, generating %d MB per rank" % (2 * nmax >> 20))
    xs_all = [torch.from_numpy(x.view(np.int16)).to("cuda") for x in I.make(5, n=nmax)]
    cl, pat = Cold(torch, stream, reps), Pattern()
    out = {"workload": cfg["desc"], "W": W, "sizes_bytes_per_rank": [2 * n for n in sizes],
           "reps": reps, "plateau_from_bytes_per_rank": 64 << 20, "per_codec": {}}
    for c in cfg["codecs"]:
        pts = {"stage1": [], "pattern": [], "copy": []}
        abs_ = []
        for n in sizes:
            xs = [x[:n] for x in xs_all]
            recv, red, red2 = qr.alloc_recv(W, c, n), qr.alloc_wire(c, n), qr.alloc_wire(c, n)
            qr.qr_quantize_recv(c, xs, recv, dtype=dtype)
            ab = algorithmic_bytes("stage1", W, n, qr.qr_wire_bytes(c, n))
            copy, keep = cl.copy_fn(ab)
            t = cl.us_interleaved({
                "stage1": lambda: qr.qr_reduce_recv(c, W, recv, n, red, dtype),
                "pattern": lambda: pat.stage1(c, W, recv, n, red2, stream),
                "copy": copy})
            for k in pts:
                pts[k].append(t[k])
            abs_.append(ab)
            del recv, red, red2, keep, copy
        r = {"bytes": abs_}
        big = [i for i, n in enumerate(sizes) if 2 * n >= out["plateau_from_bytes_per_rank"]]
        for k, ts in pts.items():
            fr = [frac(x, y) for x, y in zip(abs_, ts)]
            r[k] = {"us": [round(y, 2) for y in ts], "frac": [round(f, 4) for f in fr],
                    "plateau_frac": round(float(np.median([fr[i] for i in big])), 4)}
        r["stage1_vs_pattern"] = [round(p / s, 4) for p, s in zip(pts["pattern"], pts["stage1"])]
        out["per_codec"][I.CODEC_NAMES[c]] = r
        log("  %-4s plateau: stage 1 %.3f, pattern %.3f, copy %.3f" % (
            I.CODEC_NAMES[c], r["stage1"]["plateau_frac"], r["pattern"]["plateau_frac"],
            r["copy"]["plateau_frac"]))
    cl.close()
    del xs_all
    torch.cuda.empty_cache()
    return out


STREAM_PROBES = (("read", 0, 1, 0), ("read", 0, 4, 0), ("read, non-temporal", 0, 4, 1),
                 ("write", 1, 1, 0), ("write", 1, 4, 0), ("write, non-temporal", 1, 1, 1),
                 ("write, non-temporal", 1, 4, 1), ("copy", 2, 1, 0), ("copy", 2, 4, 0),
                 ("copy, non-temporal loads", 2, 4, 1))


def measure_streams(torch, stream, log, sizes_mib=(192, 576, 1152), reps=11):
    """Plain reads, writes and copies of 16-byte accesses (libqr_pattern.so's
    qrp_stream), cold, taken in turn launch by launch: the memory system's
    own rates for one or four accesses per lane, through the caches or not.
    A write's cold time ends with the launch, so the last lines it wrote may
    still sit dirty in the Infinity Cache (up to 256 MB) and are not in it."""
    pat, cl = Pattern(), Cold(torch, stream, reps)
    out = {"reps": reps, "per_size": {}}
    for mib in sizes_mib:
        nbytes = mib << 20
        a = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        b = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
        fns = {"%s, %d per lane" % (name, k): (lambda kind=kind, k=k, nt=nt:
                                               pat.stream(kind, k, nt, a, b, nbytes, stream))
               for name, kind, k, nt in STREAM_PROBES}
        t = cl.us_interleaved(fns)
        out["per_size"]["%d MiB" % mib] = {k: {"us": round(v, 2), "frac": round(frac(nbytes, v), 4)}
                                          for k, v in t.items()}
        log("  %d MiB: " % mib + ", ".join("%s %.3f" % (k, frac(nbytes, v)) for k, v in t.items()))
        del a, b
    cl.close()
    torch.cuda.empty_cache()
    return out


def measure_extra(args, qr, I, torch, stream, log):
    extra = {}
    log("bench: launch floor (an empty kernel, timed as the sweeps are)")
    extra["launch_floor"] = launch_floor(torch, stream)
    for cid in (2, 4):
        c = I.CONFIGS[cid]
        log("bench: config %d (%s)" % (cid, c["desc"]))
        extra["config%d" % cid] = {"workload": c["desc"], "W": c["W"],
                                   "elements_per_rank": c["n"],
                                   "per_codec": measure_workload(qr, I, torch, stream, cid)}
    c = I.CONFIGS[4]
    log("bench: config 4 with the bf16->fp16 cast")
    extra["config4_cast"] = {"workload": c["desc"] + "; bf16 buffers through binary16",
                             "per_codec": measure_workload(qr, I, torch, stream, 4, cold=False,
                                                           dtype=qr.QR_BF16_VIA_FP16)}
    c = I.CONFIGS[3]
    log("bench: config 3 size sweep")
    sweep = {}
    for size in c["sizes"]:
        sweep["%d" % (2 * size)] = measure_workload(
            qr, I, torch, stream, 3, n=size, iters=100 if 2 * size <= (1 << 20) else 20,
            cold=2 * size >= (16 << 20))
    extra["config3_sweep"] = {"workload": c["desc"], "key": "bytes per rank buffer",
                              "per_size": sweep}
    for key, dt in (("sweep_fp16", 0), ("sweep_bf16", 1), ("sweep_bf16_via_fp16", 2)):
        log("bench: size sweep %s, %d repeats" % (key, args.sweep_repeats))
        extra[key] = {"key": "W, then bytes per rank buffer; us = median of %d medians, "
                             "spread = max - min of them" % args.sweep_repeats,
                      "results": measure_sweep(qr, I, torch, stream, args.sweep_repeats,
                                               dtype=dt)}
    extra["min_sizes_rule"] = ("two-stage at most %.2f x the one-stage median and ahead "
                               "by more than both spreads, at the size and every larger one"
                               % (1 - MIN_SIZE_MARGIN))
    extra["min_sizes"], extra["min_sizes_marginal"] = {}, {}
    for k in ("fp16", "bf16", "bf16_via_fp16"):
        extra["min_sizes"][k], extra["min_sizes_marginal"][k] = min_sizes(
            extra["sweep_" + k]["results"])
    return extra


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py runs on one GPU: the W ranks of the allreduce are simulated "
              "as W buffers on that GPU; --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    import torch
    from quantized_two_stage_amd import inputs as I
    from quantized_two_stage_amd import qr

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    h = measure_headline(args, qr, I, torch, stream, log)
    W, n, codecs = h["W"], h["n"], h["codecs"]
    value = len(codecs) * 2 * n / (h["ms_per_step"] * 1e-3) / 1e9
    roof = roofline(h, I)

    cpu = None
    if not args.no_cpu_baseline:
        threads = min(16, len(os.sched_getaffinity(0)))
        log("bench: CPU oracle on a sample, %d threads" % threads)
        cpu = cpu_baseline(codecs, h["dtype"], h["xs_np"], args.cpu_sample, threads)

    stages = {}
    for c in codecs:
        k = h["per"][c]["kernels"]
        e = {"us_per_allreduce": round(h["per"][c]["us_per_allreduce"], 2)}
        for st in STAGES:
            e[st] = {"us": round(k[st]["us"], 2), "frac": round(k[st]["frac"], 4)}
        e["stage2"]["frac_hbm"] = round(k["stage2"]["frac_hbm"], 4)
        if h["cold"] is not None:
            cd = h["cold"][c]
            wb = h["bufs"][c]["wb"]
            for st in STAGES:
                e[st]["cold_us"] = round(cd[st], 2)
                e[st]["cold_frac"] = round(frac(algorithmic_bytes(st, W, n, wb), cd[st]), 4)
            e["stage2"]["cold_frac_hbm"] = round(frac(hbm_bytes_stage2(W, n, wb),
                                                      cd["stage2"]), 4)
            ab1 = algorithmic_bytes("stage1", W, n, wb)
            for key in ("pattern", "copy", "planar"):
                e["stage1"][key + "_cold_us"] = round(cd["stage1_" + key], 2)
                e["stage1"][key + "_cold_frac"] = round(frac(ab1, cd["stage1_" + key]), 4)
        stages[I.CODEC_NAMES[c]] = e

    extra = None
    if args.extra:
        extra = measure_extra(args, qr, I, torch, stream, log)
        extra["headline_stages"] = stages
        with open(args.extra, "w") as f:
            json.dump(extra, f, indent=1)
        log("bench: other workloads written to %s" % args.extra)

    if args.stage1_scan:
        scan = measure_stage1_scan(qr, I, torch, stream, log)
        with open(args.stage1_scan, "w") as f:
            json.dump(scan, f, indent=1)
        log("bench: stage-1 size scan written to %s" % args.stage1_scan)

    if args.stream_probes:
        log("bench: plain streams, cold")
        with open(args.stream_probes, "w") as f:
            json.dump(measure_streams(torch, stream, log), f, indent=1)

    for name, e in stages.items():
        log("  %-4s %8.1f us/allreduce  stage0 %.3f  stage1 %.3f (cold %s, pattern %s, "
            "W wire images %s)  stage2 %.3f" % (
                name, e["us_per_allreduce"], e["quantize"]["frac"], e["stage1"]["frac"],
                e["stage1"].get("cold_frac"), e["stage1"].get("pattern_cold_frac"),
                e["stage1"].get("planar_cold_frac"), e["stage2"]["frac"]))

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(h["ms_per_step"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": "W=%d simulated ranks, %s, %d elements (%d MB) per rank, all "
                               "%d codecs, 32-element blocks: %s" % (
                                   W, "fp16" if h["dtype"] == 0 else "bf16", n, 2 * n >> 20,
                                   len(codecs), h["cfg"]["desc"]),
                   "W": W, "elements_per_rank": n,
                   "buffer_dtype": "fp16" if h["dtype"] == 0 else "bf16",
                   "allreduces_per_step": len(codecs)},
        "roofline": roof,
        "cpu_baseline": cpu,
        "us_per_allreduce": {I.CODEC_NAMES[c]: round(h["per"][c]["us_per_allreduce"], 1)
                             for c in codecs},
        "ms_per_step_instrumented": round(h["ms_per_step_instrumented"], 4),
        "kernel_source_sha": kernel_source_sha(),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
