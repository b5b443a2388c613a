"""Parity of the one-stage (one-shot) allreduce, qr_allreduce_oneshot, with the
oracle's one-shot, through the C ABI: every rank's output bit-exact (the
method rounds once, so there is nothing for a tolerance to absorb), for both
buffer types and W in {2,4,8}, at sizes with ragged tails and at the full
64 MB workloads on sampled windows; plus the values it must share with the
two-stage FP path, edge values, guard bands and a non-default stream."""
import numpy as np
import pytest
import torch

import oracle as O
import pins
from gpu_util import dev16, host16, sample_windows, say
from quantized_two_stage_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qr():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_two_stage_amd import qr as q
    return q


# dtype 2 = bf16 buffers through binary16: generator 5's +-max-finite blocks
# become +-inf there, and +inf + -inf (a NaN) is outside the contract; the
# edge test covers same-signed overflow
GENS = {O.FP16: (1, 2, 5), O.BF16: (3, 4, 5), O.BF16_VIA_FP16: (3, 4)}
SIZES = (8, 24, 40, 3 * 8192 + 24, 65536 + 8)


def _inputs(cfg, W, n, dtype, salt=0):
    return [I.to_bits(I.draw(cfg, r + 16 * salt, n), dtype) for r in range(W)]


def _run(qr, xs, dtype, stream=None):
    ys = [torch.full_like(xs[0], 0x1357) for _ in xs]
    torch.cuda.synchronize()             # the fills are done before any stream runs
    qr.qr_allreduce_oneshot(xs, ys, dtype=dtype, stream=stream)
    torch.cuda.synchronize()
    return ys


def _assert_equal(got, want, what):
    if not np.array_equal(got, want):
        bad = np.nonzero(got != want)[0]
        raise AssertionError("%s: %d elements differ, first at %d: got %04x want %04x" % (
            what, bad.size, bad[0], got[bad[0]], want[bad[0]]))


def _check(qr, xs_np, dtype, label):
    say("oneshot", label)
    xs = [dev16(x) for x in xs_np]
    ys = _run(qr, xs, dtype)
    want = O.oneshot(dtype, xs_np)
    for r, y in enumerate(ys):
        _assert_equal(host16(y), want[r], "%s y[%d]" % (label, r))
    for r in range(len(xs)):
        assert np.array_equal(host16(xs[r]), xs_np[r]), label       # inputs untouched
    return xs, ys


@pytest.mark.parametrize("W", (2, 4, 8))
@pytest.mark.parametrize("dtype", (O.FP16, O.BF16, O.BF16_VIA_FP16),
                         ids=("fp16", "bf16", "bf16viafp16"))
def test_oneshot_parity(qr, dtype, W):
    for cfg in GENS[dtype]:
        for n in SIZES:
            # the cast option's inputs are bf16 buffers
            _check(qr, _inputs(cfg, W, n, O.BF16 if dtype == O.BF16_VIA_FP16 else dtype), dtype,
                   "W%d n%d gen%d dtype%d" % (W, n, cfg, dtype))


@pytest.mark.parametrize("dtype", (O.FP16, O.BF16), ids=("fp16", "bf16"))
def test_oneshot_equals_two_stage_fp(qr, dtype):
    """the one-stage and the two-stage FP allreduce compute the same values"""
    for W in (2, 4, 8):
        n = 4 * 8192 + 40
        xs_np = _inputs(5, W, n, dtype, salt=1)
        xs, ys = _check(qr, xs_np, dtype, "vs sim W%d" % W)
        ys2 = [torch.empty_like(xs[0]) for _ in range(W)]
        ws = qr.alloc_workspace(W, qr.QR_FP, n)
        qr.qr_allreduce_sim(qr.QR_FP, xs, ys2, ws, dtype=dtype)
        torch.cuda.synchronize()
        for r in range(W):
            _assert_equal(host16(ys[r]), host16(ys2[r]), "oneshot vs sim W%d y[%d]" % (W, r))


@pytest.mark.parametrize("dtype", (O.FP16, O.BF16, O.BF16_VIA_FP16),
                         ids=("fp16", "bf16", "bf16viafp16"))
def test_oneshot_edge_values(qr, dtype):
    """zeros of both signs, sums that overflow to inf, subnormals, identical
    ranks, and cancellation across ranks (dtype 2: bf16 buffers, whose
    largest values become inf in binary16)"""
    W, n = 4, 32 * 10 + 8
    gen_t = O.FP16 if dtype == O.FP16 else O.BF16      # type of the buffers
    one = pins.to_buf([1.0], "fp16" if dtype == O.FP16 else "bf16")[0]
    big = 0x7BFF if dtype == O.FP16 else 0x7F7F
    cases = {
        "zeros": [np.zeros(n, np.uint16)] * W,
        "neg_zeros": [np.full(n, 0x8000, np.uint16)] * W,
        "mixed_zeros": [np.zeros(n, np.uint16), np.full(n, 0x8000, np.uint16)] * 2,
        "constant": [np.full(n, one, np.uint16)] * W,
        "overflow": [np.full(n, big, np.uint16)] * W,
        "overflow_neg": [np.full(n, big | 0x8000, np.uint16)] * W,
        "tiny": [np.full(n, 1, np.uint16) | (np.arange(n, dtype=np.uint16) & 1) * 0x8000] * W,
        "identical": [I.to_bits(I.draw(1, 0, n), gen_t)] * W,
        "cancel": [I.to_bits(I.draw(1, 0, n), gen_t),
                   I.to_bits(I.draw(1, 0, n), gen_t) ^ 0x8000,
                   I.to_bits(I.draw(1, 1, n), gen_t),
                   I.to_bits(I.draw(1, 1, n), gen_t) ^ 0x8000],
    }
    for name, xs_np in cases.items():
        _check(qr, [x.copy() for x in xs_np], dtype, "edge %s" % name)


def test_oneshot_guard_bands(qr):
    """nothing is written outside the outputs"""
    G = 4096
    for W in (2, 8):
        for n in (8, 40, 8192 + 24):
            say("oneshot guard", W, n)
            xs_np = _inputs(5, W, n, O.FP16)
            xs = [dev16(x) for x in xs_np]
            big = [torch.full((n + G,), 0x3C3C, dtype=torch.int16, device="cuda")
                   for _ in range(W)]
            ys = [b[G // 2:G // 2 + n] for b in big]
            qr.qr_allreduce_oneshot(xs, ys, dtype=O.FP16)
            torch.cuda.synchronize()
            want = O.oneshot(O.FP16, xs_np)
            for r, b in enumerate(big):
                h = host16(b)
                assert np.all(h[:G // 2] == 0x3C3C) and np.all(h[G // 2 + n:] == 0x3C3C)
                _assert_equal(h[G // 2:G // 2 + n], want[r], "guard y[%d]" % r)


def test_oneshot_nondefault_stream(qr):
    W, n = 4, 8192 + 8
    xs_np = _inputs(2, W, n, O.FP16)
    xs = [dev16(x) for x in xs_np]
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    ys = _run(qr, xs, O.FP16, stream=s)
    want = O.oneshot(O.FP16, xs_np)
    for r in range(W):
        _assert_equal(host16(ys[r]), want[r], "stream y[%d]" % r)


@pytest.mark.parametrize("cfg", (2, 5, 4))
def test_oneshot_full_size(qr, cfg):
    """the 64 MB (and the 16 MB W=8 bf16) workloads: sampled block windows
    against the oracle, and every element against the two-stage FP path"""
    c = I.CONFIGS[cfg]
    W, n, dtype = c["W"], c["n"], c["dtype"]
    say("oneshot full config", cfg)
    xs_np = I.make(cfg)
    xs = [dev16(x) for x in xs_np]
    ys = _run(qr, xs, dtype)
    nb = (n + 31) // 32
    got = [host16(y) for y in ys]
    for (lo, hi) in sample_windows(nb, count=8, seed=cfg):
        want = O.oneshot(dtype, xs_np, lo, hi)
        for r in range(W):
            _assert_equal(got[r][32 * lo:32 * hi], want[r][32 * lo:32 * hi],
                          "config %d blocks [%d,%d) y[%d]" % (cfg, lo, hi, r))
    ys2 = [torch.empty_like(xs[0]) for _ in range(W)]
    ws = qr.alloc_workspace(W, qr.QR_FP, n)
    qr.qr_allreduce_sim(qr.QR_FP, xs, ys2, ws, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(W):
        _assert_equal(got[r], host16(ys2[r]), "config %d oneshot vs sim y[%d]" % (cfg, r))
