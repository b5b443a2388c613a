"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (one qr_allreduce_sim call per codec), against the oracle run
over the whole buffers (threaded by block range): every output element of
every rank, every byte of the receive buffer and of the reduced image in the
call's workspace, and the planar staged calls' wire images, all bit-exact.
Inputs are untouched.  At the largest rank buffer the library takes (2 GiB),
sampled block windows instead."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import (assert_bytes_equal, assert_recv_equal, assert_within_ulp, block_ranges,
                      dev16, host16, hostu8, oracle_whole, plane_slices, recv_tile_bytes,
                      sample_windows, say)
from quantized_two_stage_amd import inputs as I

pytestmark = pytest.mark.gpu

_cache = {}


@pytest.fixture(scope="module")
def qr():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_two_stage_amd import qr as q
    return q


def _data(cfg, n=None, W=None):
    key = (cfg, n, W)
    if key not in _cache:
        _cache.clear()
        c = I.CONFIGS[cfg]
        n_ = n or c["n"]
        xs_np = []
        for r in range(W or c["W"]):
            say("generating config", cfg, "n", n_, "rank", r)
            xs_np.append(I.to_bits(I.draw(cfg, r, n_), c["dtype"]))
        _cache[key] = (xs_np, [dev16(x) for x in xs_np])
    return _cache[key]


def _planes_equal(got, want, codec, n, what):
    for name, (a, e) in plane_slices(codec, n).items():
        assert_bytes_equal(got[a:e], want[a:e], "%s %s" % (what, name))


def _check_full(qr, cfg, codec, n=None, staged=True, dtype=None, W=None):
    """one qr_allreduce_sim call against the oracle over the whole buffers
    (W: the workload's recipe for another number of ranks)"""
    c = I.CONFIGS[cfg]
    W = W or c["W"]
    dtype = c["dtype"] if dtype is None else dtype
    xs_np, xs = _data(cfg, n, W)
    n = xs_np[0].size
    label = "cfg%d %s W%d n%d dtype%d" % (cfg, I.CODEC_NAMES[codec], W, n, dtype)
    say("full", label)
    ys = [torch.empty_like(xs[0]) for _ in range(W)]
    ws = qr.alloc_workspace(W, codec, n)
    ws.fill_(0xA7)           # no reliance on what an earlier call left there
    qr.qr_allreduce_sim(codec, xs, ys, ws, dtype=dtype)
    torch.cuda.synchronize()
    say("full", label, "oracle")
    r_wires, r_red, r_y = oracle_whole(codec, dtype, xs_np)
    say("full", label, "compare")
    for r in range(W):
        assert_within_ulp(host16(ys[r]), r_y, dtype, "%s y[%d]" % (label, r))
    wsh = hostu8(ws)
    rb = qr.qr_recv_bytes(W, codec, n)
    red_at = (rb + 255) // 256 * 256
    assert_recv_equal(wsh[:rb], r_wires, codec, n, label + " receive buffer", fill=0xA7)
    _planes_equal(wsh[red_at:red_at + qr.qr_wire_bytes(codec, n)], r_red, codec, n,
                  label + " reduced")
    del ws, wsh
    if staged:
        # the planar staged calls: W separate wire images
        wires = [qr.alloc_wire(codec, n) for _ in range(W)]
        qr.qr_quantize_ranks(codec, xs, wires, dtype=dtype)
        red = qr.alloc_wire(codec, n)
        qr.qr_reduce_stage1(codec, wires, n, red, dtype)
        torch.cuda.synchronize()
        for r in range(W):
            _planes_equal(hostu8(wires[r]), r_wires[r], codec, n, "%s wire[%d]" % (label, r))
        _planes_equal(hostu8(red), r_red, codec, n, label + " planar reduced")
        del wires, red
    for r in range(W):
        assert torch.equal(xs[r], dev16(xs_np[r])), (label, "input modified")
    del ys
    torch.cuda.empty_cache()


def test_config1_full(qr):
    """4 KB per rank, W=2, Q8"""
    _check_full(qr, 1, O.Q8)


@pytest.mark.parametrize("codec", I.CONFIGS[2]["codecs"],
                         ids=[I.CODEC_NAMES[c] for c in I.CONFIGS[2]["codecs"]])
def test_config2_full(qr, codec):
    _check_full(qr, 2, codec)


@pytest.mark.parametrize("n", I.CONFIGS[3]["sizes"])
def test_config3_sweep(qr, n):
    _check_full(qr, 3, O.Q4A, n=n, staged=(n in (1 << 11, 1 << 25)))


def test_config4_full(qr):
    _check_full(qr, 4, O.Q6)


# W=4 at 64 MB per rank in fp16, every codec (the W=2 64 MB workload's recipe
# for four ranks): the stage-1 kernels that stream their wire data
# non-temporally from W=4 up, at the size the W=2 and W=8 workloads run
@pytest.mark.parametrize("codec", I.ALL_CODECS, ids=[I.CODEC_NAMES[c] for c in I.ALL_CODECS])
def test_w4_64MB_full(qr, codec):
    _check_full(qr, 2, codec, W=4, staged=codec in (O.Q8, O.Q6A))


@pytest.mark.parametrize("codec", I.CONFIGS[5]["codecs"],
                         ids=[I.CODEC_NAMES[c] for c in I.CONFIGS[5]["codecs"]])
def test_config5_full(qr, codec):
    _check_full(qr, 5, codec)


# Sizes just past the workloads' own, with ragged tails, so that the launch
# shapes the library picks for large grids (stage 0 with two quarters per lane
# from W*n >= 2^28, stage 2 with one from W*n >= 2^26, stage 1 at W=2 with
# 128-lane workgroups from 2^20 blocks) run their range-checked paths: at W=8
# the last tile holds 6 blocks, the last of them 8 elements, so whole stage-0
# and stage-2 workgroups lie past the end; at W=2 the last 128-lane stage-1
# workgroup holds 3 blocks, the last of them 24 elements.
# The bf16 workload's recipe (W=8) at the same size takes the large-grid stage
# 0 from bfloat16 and through the cast option.
RAGGED_N = {5: (1 << 25) + 32 * 5 + 8, 2: (1 << 25) + 32 * 130 + 24, 4: (1 << 25) + 32 * 5 + 8}
CAST = O.BF16_VIA_FP16
RAGGED_CASES = [(5, O.FP, None), (5, O.FP8, None), (5, O.Q6A, None), (5, O.Q4A, None),
                (2, O.FP, None), (2, O.Q8, None), (2, O.Q4, None),
                (4, O.Q6, None), (4, O.FP, None), (4, O.Q4A, CAST), (4, O.FP8, CAST)]


@pytest.mark.parametrize("cfg,codec,dtype", RAGGED_CASES,
                         ids=["cfg%d-%s%s" % (c, I.CODEC_NAMES[k], "-cast" if d == CAST else "")
                              for c, k, d in RAGGED_CASES])
def test_large_shapes_ragged(qr, cfg, codec, dtype):
    _check_full(qr, cfg, codec, n=RAGGED_N[cfg], dtype=dtype)


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


@pytest.mark.parametrize("codec", (O.FP, O.Q8A))
def test_max_size_w8(qr, codec):
    """n = 2^30 elements per rank at W = 8: a receive buffer of 16 GiB (FP) or
    9.7 GiB (Q8A), whose 32-bit offsets split stages 0 and 1 into 5 or 3
    launches over tile ranges.  Windows of blocks straddle every split (the
    split points computed here from the layout: a launch spans
    (2^32 - 1) // (W * tile bytes) - 1 tiles), besides the first, the last and
    random ones; outputs of ranks 0 and 7 against the oracle."""
    n, W, dtype = 1 << 30, 8, O.FP16
    say("max size W=8", codec)
    g = torch.Generator(device="cuda")
    g.manual_seed(8484 + codec)
    xs = [torch.randn(n, generator=g, device="cuda", dtype=torch.float32)
          .to(torch.float16).view(torch.int16) for _ in range(W)]
    ys = [torch.empty_like(xs[0]) for _ in range(W)]
    ws = qr.alloc_workspace(W, codec, n)
    qr.qr_allreduce_sim(codec, xs, ys, ws, dtype=dtype)
    torch.cuda.synchronize()
    nb = n // 32
    per = (2 ** 32 - 1) // (W * recv_tile_bytes(codec)) - 1
    splits = list(range(per * 256, nb, per * 256))
    assert len(splits) == (4 if codec == O.FP else 2)
    windows = sample_windows(nb, count=4, seed=codec) + [(b - 32, b + 32) for b in splits]
    for (lo, hi) in windows:
        e0, e1 = 32 * lo, 32 * hi
        loc = [host16(x[e0:e1]) for x in xs]
        want = O.allreduce(codec, dtype, loc)[0]
        for r in (0, W - 1):
            assert_within_ulp(host16(ys[r][e0:e1]), want, dtype,
                              "max W=8 rank %d y %d..%d" % (r, lo, hi))
    del xs, ys, ws
    torch.cuda.empty_cache()


@pytest.mark.parametrize("codec", (O.FP, O.Q8A), ids=("fp", "q8a"))
def test_max_size_w8_owner(qr, codec):
    """Stage 1 of one owner from the receive buffer at n = 2^30 elements per
    rank, W = 8, for the owner whose chunk crosses the first launch split (a
    launch spans (2^32 - 1) // (W * tile bytes) - 1 tiles): the reduced image
    is cleared first, then the owner's blocks are compared with the oracle in
    windows across the split and at the chunk's ends, and the blocks just
    outside the chunk must still hold the clear pattern."""
    n, W, dtype = 1 << 30, 8, O.FP16
    nb = n // 32
    split = ((2 ** 32 - 1) // (W * recv_tile_bytes(codec)) - 1) * 256
    bpc = (nb + W - 1) // W
    owner = split // bpc
    c_lo, c_hi = owner * bpc, min(nb, (owner + 1) * bpc)
    assert c_lo < split - 32 and split + 32 < c_hi
    say("max size W=8 owner", owner, "codec", codec)
    g = torch.Generator(device="cuda")
    g.manual_seed(9696 + codec)
    xs = [torch.randn(n, generator=g, device="cuda", dtype=torch.float32)
          .to(torch.float16).view(torch.int16) for _ in range(W)]
    recv = qr.alloc_recv(W, codec, n)
    red = qr.alloc_wire(codec, n)
    qr.qr_quantize_recv(codec, xs, recv, dtype=dtype)
    red.fill_(0xA7)
    qr.qr_reduce_recv(codec, W, recv, n, red, dtype, owner=owner)
    torch.cuda.synchronize()
    for (lo, hi) in [(split - 32, split + 32), (c_lo, c_lo + 64), (c_hi - 64, c_hi)]:
        loc = [host16(x[32 * lo:32 * hi]) for x in xs]
        _, want, _ = oracle_whole(codec, dtype, loc)
        mine, theirs = block_ranges(codec, n, lo, hi), block_ranges(codec, 32 * (hi - lo), 0, hi - lo)
        for name, (a, e) in mine.items():
            a2, e2 = theirs[name]
            assert_bytes_equal(hostu8(red[a:e]), want[a2:e2],
                               "owner %d blocks %d..%d %s" % (owner, lo, hi, name))
    for (lo, hi) in [(c_lo - 64, c_lo), (c_hi, c_hi + 64)]:
        for name, (a, e) in block_ranges(codec, n, lo, hi).items():
            assert bool(torch.all(red[a:e] == 0xA7)), ("written outside the chunk", name, lo, hi)
    del xs, recv, red
    torch.cuda.empty_cache()


@pytest.mark.parametrize("cfg,codec", [(4, O.Q6), (3, O.Q4A), (4, O.FP), (3, O.Q8)],
                         ids=("cfg4-q6", "cfg3-q4a", "cfg4-fp", "cfg3-q8"))
def test_cast_option_full(qr, cfg, codec):
    """the bf16 workloads with the bf16 -> fp16 cast option (buffer type 2):
    64 MB (configuration 3's largest size) and 16 MB W=8"""
    _check_full(qr, cfg, codec, n=(1 << 25) if cfg == 3 else None, staged=False,
                dtype=O.BF16_VIA_FP16)


FUSED_EDGE = 2 * 1024 * 1024          # elements: 4 MiB per rank, the single-launch limit


@pytest.mark.parametrize("n", (FUSED_EDGE, FUSED_EDGE + 8), ids=("4MiB-one-launch", "above"))
@pytest.mark.parametrize("codec", (O.FP, O.FP8, O.Q8, O.Q6, O.Q4, O.Q8A, O.Q6A, O.Q4A),
                         ids=[I.CODEC_NAMES[c] for c in (O.FP, O.FP8, O.Q8, O.Q6, O.Q4, O.Q8A,
                                                           O.Q6A, O.Q4A)])
def test_sim_launch_paths(qr, codec, n):
    """qr_allreduce_sim on both sides of the size where it switches from one
    launch to three, W=2 fp16, W=4 bf16 and W=8 bf16"""
    _check_full(qr, 2, codec, n=n, staged=False)
    _check_full(qr, 3, codec, n=n, staged=False)
    _check_full(qr, 4, codec, n=n, staged=False)
