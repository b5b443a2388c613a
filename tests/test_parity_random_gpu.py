"""Parity on randomly drawn cases (fixed seed, so the run is reproducible):
codec, buffer type (fp16, bf16, bf16 through fp16), W, size (any multiple of
8 elements up to 96K, so tails and workgroup counts vary), the input
generator of every workload, and a random owner to run stage 1 for.  Each
case runs the one-call allreduce and the staged calls and compares the wire
images, the reduced image and every output with the oracle, bit for bit."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_bytes_equal, assert_within_ulp, dev16, host16, hostu8, plane_slices, say
from quantized_two_stage_amd import inputs as I

pytestmark = pytest.mark.gpu

CODECS = (O.FP, O.FP8, O.Q8, O.Q6, O.Q4, O.Q8A, O.Q6A, O.Q4A)
CASES = 480


@pytest.fixture(scope="module")
def qr():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_two_stage_amd import qr as q
    return q


def _case(k):
    g = np.random.default_rng(424242 + k)
    codec = int(g.choice(CODECS))
    dtype = int(g.integers(0, 3))                    # 0 fp16, 1 bf16, 2 bf16 through fp16
    W = int(g.choice((2, 4, 8)))
    n = 8 * int(g.integers(1, 12289))
    cfg = int(g.integers(1, 6))
    owner = int(g.integers(0, W))
    return codec, dtype, W, n, cfg, owner


def _inputs(cfg, W, n, dtype, k, codec):
    bits = I.BF16 if dtype else I.FP16
    xs = [I.to_bits(I.draw(cfg, r + 100 * (k + 1), n), bits) for r in range(W)]
    if dtype == O.BF16_VIA_FP16:
        # The cast option's contract: for the quantized codecs, bf16 inputs
        # within the binary16 range (beyond it they become inf on entry).  The
        # FP codec and the one-stage allreduce carry an inf through, so there
        # only negative magnitudes of 2^16 and more are brought into range:
        # positive ones become +inf and every sum holding one is +inf (+inf
        # plus -inf, a NaN, is outside the contract).
        for i, x in enumerate(xs):
            big = (x & 0x7F80) >= 0x4780
            if codec == O.FP:
                big &= (x & 0x8000) != 0
            xs[i] = np.where(big, x & 0x807F | 0x4700, x).astype(np.uint16)
    return xs


@pytest.mark.parametrize("block", range(8))
def test_random_cases(qr, block):
    for k in range(block * CASES // 8, (block + 1) * CASES // 8):
        codec, dtype, W, n, cfg, owner = _case(k)
        label = "case %d: codec %d dtype %d W %d n %d gen %d owner %d" % (
            k, codec, dtype, W, n, cfg, owner)
        say(label)
        xs_np = _inputs(cfg, W, n, dtype, k, codec)
        xs = [dev16(x) for x in xs_np]
        want_wires = [O.quantize(codec, dtype, x) for x in xs_np]
        want_red = O.stage1(codec, dtype, want_wires, n)
        want_ys = O.stage2(codec, dtype, W, want_red, n)
        planes = plane_slices(codec, n)

        # staged calls, stage 1 for one owner's chunk and then for the rest
        wires = [qr.alloc_wire(codec, n) for _ in range(W)]
        qr.qr_quantize_ranks(codec, xs, wires, dtype=dtype)
        red = qr.alloc_wire(codec, n)
        qr.qr_reduce_stage1(codec, wires, n, red, dtype, owner=owner)
        torch.cuda.synchronize()
        lo, hi = O.chunk(W, n, owner)
        part = O.stage1(codec, dtype, want_wires, n, lo, hi)
        assert_bytes_equal(hostu8(red), part, label + " owner chunk")
        qr.qr_reduce_stage1(codec, wires, n, red, dtype)
        ys = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(W)]
        qr.qr_gather_stage2(codec, red, ys, dtype=dtype)
        torch.cuda.synchronize()
        for r in range(W):
            for name, (a, e) in planes.items():
                assert_bytes_equal(hostu8(wires[r])[a:e], want_wires[r][a:e],
                                   "%s wire[%d] %s" % (label, r, name))
        for name, (a, e) in planes.items():
            assert_bytes_equal(hostu8(red)[a:e], want_red[a:e], "%s reduced %s" % (label, name))
        for r in range(W):
            assert_within_ulp(host16(ys[r]), want_ys[r], O.BF16 if dtype else O.FP16,
                              "%s y[%d]" % (label, r))

        # the one-call allreduce
        ys2 = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(W)]
        ws = qr.alloc_workspace(W, codec, n)
        qr.qr_allreduce_sim(codec, xs, ys2, ws, dtype=dtype)
        torch.cuda.synchronize()
        for r in range(W):
            assert_within_ulp(host16(ys2[r]), want_ys[r], O.BF16 if dtype else O.FP16,
                              "%s sim y[%d]" % (label, r))

        # the one-stage allreduce on the same buffers
        qr.qr_allreduce_oneshot(xs, ys2, dtype=dtype)
        torch.cuda.synchronize()
        want_one = O.oneshot(dtype, xs_np)
        for r in range(W):
            assert_within_ulp(host16(ys2[r]), want_one[r], O.BF16 if dtype else O.FP16,
                              "%s one-stage y[%d]" % (label, r))
