"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (one qr_allreduce_sim call per codec), checked against the
oracle on sampled block windows (first, last and random blocks; the oracle
computes those blocks alone), and by properties that hold at any size: every
rank's output is identical, inputs are untouched, and the staged entry points
give the same wire planes and outputs as the one-call pipeline."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (assert_within_ulp, assert_wire_blocks, dev16, host16, hostu8,
                      sample_windows, say)
from quantized_two_stage_amd import inputs as I

pytestmark = pytest.mark.gpu

_cache = {}


@pytest.fixture(scope="module")
def qr():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_two_stage_amd import qr as q
    return q


def _data(cfg, n=None):
    key = (cfg, n)
    if key not in _cache:
        _cache.clear()
        c = I.CONFIGS[cfg]
        n_ = n or c["n"]
        xs_np = []
        for r in range(c["W"]):
            say("generating config", cfg, "n", n_, "rank", r)
            xs_np.append(I.to_bits(I.draw(cfg, r, n_), c["dtype"]))
        _cache[key] = (xs_np, [dev16(x) for x in xs_np])
    return _cache[key]


def _check_full(qr, cfg, codec, n=None, windows=12, staged=True, dtype=None):
    c = I.CONFIGS[cfg]
    W = c["W"]
    dtype = c["dtype"] if dtype is None else dtype
    xs_np, xs = _data(cfg, n)
    n = xs_np[0].size
    nb = (n + 31) // 32
    label = "cfg%d %s W%d n%d dtype%d" % (cfg, I.CODEC_NAMES[codec], W, n, dtype)
    say("full", label)
    ys = [torch.empty_like(xs[0]) for _ in range(W)]
    ws = qr.alloc_workspace(W, codec, n)
    ws.fill_(0xA7)           # no reliance on what an earlier call left there
    qr.qr_allreduce_sim(codec, xs, ys, ws, dtype=dtype)
    torch.cuda.synchronize()
    y0 = host16(ys[0])
    for r in range(1, W):
        assert torch.equal(ys[r], ys[0]), (label, "rank outputs differ", r)
    for (lo, hi) in sample_windows(nb, count=windows, seed=cfg * 100 + codec):
        want = O.allreduce(codec, dtype, xs_np, lo, hi)[0]
        e0, e1 = 32 * lo, min(32 * hi, n)
        assert_within_ulp(y0[e0:e1], want[e0:e1], dtype, "%s y blocks %d..%d" % (label, lo, hi))
    if staged:
        wires = [qr.alloc_wire(codec, n) for _ in range(W)]
        qr.qr_quantize_ranks(codec, xs, wires, dtype=dtype)
        red = qr.alloc_wire(codec, n)
        qr.qr_reduce_stage1(codec, wires, n, red, dtype)
        ys2 = [torch.empty_like(xs[0]) for _ in range(W)]
        qr.qr_gather_stage2(codec, red, ys2, dtype=dtype)
        torch.cuda.synchronize()
        for r in range(W):
            assert torch.equal(ys2[r], ys[0]), (label, "staged != one call")
        gw = [hostu8(w) for w in wires]
        gr = hostu8(red)
        for (lo, hi) in sample_windows(nb, count=4, seed=cfg * 100 + codec + 1):
            rw = [O.quantize(codec, dtype, x, lo, hi) for x in xs_np]
            for r in range(W):
                assert_wire_blocks(gw[r], rw[r], codec, n, lo, hi, "%s wire[%d]" % (label, r))
            rr = O.stage1(codec, dtype, rw, n, lo, hi)
            assert_wire_blocks(gr, rr, codec, n, lo, hi, label + " reduced")
        del wires, red, ys2
    for r in range(W):
        assert torch.equal(xs[r], dev16(xs_np[r])), (label, "input modified")


def test_config1_full(qr):
    """4 KB per rank, W=2, Q8: small enough to compare everything."""
    xs_np, xs = _data(1)
    n = xs_np[0].size
    ys = [torch.empty_like(xs[0]) for _ in range(2)]
    ws = qr.alloc_workspace(2, O.Q8, n)
    say("cfg1")
    qr.qr_allreduce_sim(O.Q8, xs, ys, ws, dtype=O.FP16)
    torch.cuda.synchronize()
    want = O.allreduce(O.Q8, O.FP16, xs_np)
    for r in range(2):
        assert_within_ulp(host16(ys[r]), want[r], O.FP16, "cfg1 y")


@pytest.mark.parametrize("codec", I.CONFIGS[2]["codecs"],
                         ids=[I.CODEC_NAMES[c] for c in I.CONFIGS[2]["codecs"]])
def test_config2_full(qr, codec):
    _check_full(qr, 2, codec)


@pytest.mark.parametrize("n", I.CONFIGS[3]["sizes"])
def test_config3_sweep(qr, n):
    if n <= 1 << 16:                       # whole-buffer comparison
        xs_np, xs = _data(3, n)
        ys = [torch.empty_like(xs[0]) for _ in range(4)]
        ws = qr.alloc_workspace(4, O.Q4A, n)
        say("cfg3 full compare n", n)
        qr.qr_allreduce_sim(O.Q4A, xs, ys, ws, dtype=O.BF16)
        torch.cuda.synchronize()
        want = O.allreduce(O.Q4A, O.BF16, xs_np)
        for r in range(4):
            assert_within_ulp(host16(ys[r]), want[r], O.BF16, "cfg3 n%d y" % n)
    else:
        _check_full(qr, 3, O.Q4A, n=n, windows=6, staged=(n == 1 << 25))


def test_config4_full(qr):
    _check_full(qr, 4, O.Q6)


@pytest.mark.parametrize("codec", I.CONFIGS[5]["codecs"],
                         ids=[I.CODEC_NAMES[c] for c in I.CONFIGS[5]["codecs"]])
def test_config5_full(qr, codec):
    _check_full(qr, 5, codec)


@pytest.mark.parametrize("codec", (O.Q4, O.FP8, O.FP))
def test_max_size(qr, codec):
    """n = 2^30 elements (QR_MAX_BYTES = 2 GiB per rank), W = 2: the largest
    byte offsets the kernels compute.  Inputs are drawn on the GPU from a
    seeded torch generator; the oracle sees host copies of the sampled
    windows only (window-local inputs give the same blocks)."""
    n, W, dtype = 1 << 30, 2, O.FP16
    say("max size", codec)
    g = torch.Generator(device="cuda")
    g.manual_seed(4242 + codec)
    xs = [torch.randn(n, generator=g, device="cuda", dtype=torch.float32)
          .to(torch.float16).view(torch.int16) for _ in range(W)]
    ys = [torch.empty_like(xs[0]) for _ in range(W)]
    ws = qr.alloc_workspace(W, codec, n)
    qr.qr_allreduce_sim(codec, xs, ys, ws, dtype=dtype)
    torch.cuda.synchronize()
    nb = n // 32
    for (lo, hi) in sample_windows(nb, count=6, seed=codec):
        e0, e1 = 32 * lo, 32 * hi
        loc = [host16(x[e0:e1]) for x in xs]
        want = O.allreduce(codec, dtype, loc)[0]
        assert_within_ulp(host16(ys[0][e0:e1]), want, dtype, "max y %d..%d" % (lo, hi))
        assert torch.equal(ys[1][e0:e1], ys[0][e0:e1])
    del xs, ys, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg,codec", [(4, O.Q6), (3, O.Q4A), (4, O.FP), (3, O.Q8)],
                         ids=("cfg4-q6", "cfg3-q4a", "cfg4-fp", "cfg3-q8"))
def test_cast_option_full(qr, cfg, codec):
    """the bf16 workloads with the bf16 -> fp16 cast option (buffer type 2):
    64 MB (configuration 3's largest size) and 16 MB W=8"""
    _check_full(qr, cfg, codec, n=(1 << 25) if cfg == 3 else None, windows=8,
                dtype=O.BF16_VIA_FP16)


FUSED_EDGE = 2 * 1024 * 1024          # elements: 4 MiB per rank, the single-launch limit


@pytest.mark.parametrize("n", (FUSED_EDGE, FUSED_EDGE + 8), ids=("4MiB-one-launch", "above"))
@pytest.mark.parametrize("codec", (O.FP, O.FP8, O.Q8, O.Q6, O.Q4, O.Q8A, O.Q6A, O.Q4A),
                         ids=[I.CODEC_NAMES[c] for c in (O.FP, O.FP8, O.Q8, O.Q6, O.Q4, O.Q8A,
                                                           O.Q6A, O.Q4A)])
def test_sim_launch_paths(qr, codec, n):
    """qr_allreduce_sim at the size where it switches from one launch to
    three, W=2 fp16, W=4 bf16 and W=8 bf16: every element equals the staged
    calls', sampled blocks equal the oracle's"""
    _check_full(qr, 2, codec, n=n, windows=6)
    _check_full(qr, 3, codec, n=n, windows=6)
    _check_full(qr, 4, codec, n=n, windows=6)
