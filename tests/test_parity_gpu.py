"""Parity of the HIP path with the oracle, element by element, through the C
ABI: every wire plane (codes, scales, zeros) and every output bit-exact
(zeros included, with their sign), for every codec x buffer
type x W in {2,4,8}, at sizes that span several 256-lane workgroups and end in
a ragged partial block; plus the hand-worked fixtures, owner-restricted
stage 1, edge cases, guard bands and the no-write-on-error rule."""
import numpy as np
import pytest
import torch

import oracle as O
import pins
from gpu_util import (assert_bytes_equal, assert_recv_equal, assert_within_ulp, dev16,
                      gpu_staged, host16, hostu8, oracle_staged, plane_slices, recv_from_wires,
                      recv_mask, say)
from quantized_two_stage_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qr():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_two_stage_amd import qr as q
    return q


CODECS = (O.FP, O.FP8, O.Q8, O.Q6, O.Q4, O.Q8A, O.Q6A, O.Q4A)
GENS = {O.FP16: (1, 2, 5), O.BF16: (3, 4, 5)}


def _inputs(cfg, W, n, dtype, salt=0):
    return [I.to_bits(I.draw(cfg, r + 16 * salt, n), dtype) for r in range(W)]


def _check_case(qr, codec, dtype, xs_np, label):
    W, n = len(xs_np), xs_np[0].size
    say("case", label)
    xs = [dev16(x) for x in xs_np]
    g_wires, g_red, g_ys = gpu_staged(qr, codec, dtype, xs)
    r_wires, r_red, r_ys = oracle_staged(codec, dtype, xs_np)
    for r in range(W):
        assert_bytes_equal(hostu8(g_wires[r]), r_wires[r], "%s wire[%d]" % (label, r))
    assert_bytes_equal(hostu8(g_red), r_red, "%s reduced" % label)
    for r in range(W):
        assert_within_ulp(host16(g_ys[r]), r_ys[r], dtype, "%s y[%d]" % (label, r))
    # the one-call pipeline gives the same outputs
    ys2 = [torch.empty_like(xs[0]) for _ in range(W)]
    ws = qr.alloc_workspace(W, codec, n)
    ws.fill_(0xA7)           # no reliance on what an earlier call left there
    for y in ys2:
        y.fill_(0x1357)
    qr.qr_allreduce_sim(codec, xs, ys2, ws, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(W):
        assert_within_ulp(host16(ys2[r]), r_ys[r], dtype, "%s sim y[%d]" % (label, r))
    # the workspace holds the receive buffer and the reduced image (whichever
    # launch path the call took), and no padding byte is written
    wb = qr.qr_wire_bytes(codec, n)
    rb = qr.qr_recv_bytes(W, codec, n)
    red_at = (rb + 255) // 256 * 256
    wsh = hostu8(ws)
    assert_recv_equal(wsh[:rb], r_wires, codec, n, "%s sim receive buffer" % label, fill=0xA7)
    assert np.all(wsh[rb:red_at] == 0xA7), (label, "workspace padding written")
    img = wsh[red_at:red_at + wb]
    keep = np.ones(wb, bool)
    for name, (a, e) in plane_slices(codec, n).items():
        assert_bytes_equal(img[a:e], r_red[a:e], "%s sim workspace reduced %s" % (label, name))
        keep[a:e] = False
    assert np.all(img[keep] == 0xA7), (label, "workspace padding written (reduced)")
    # the staged calls through a receive buffer: stage 0 writes it as the
    # layout says, stage 1 reads it back into the same reduced image
    recv = torch.full((qr.qr_recv_bytes(W, codec, n),), 0xA7, dtype=torch.uint8, device="cuda")
    qr.qr_quantize_recv(codec, xs, recv, dtype=dtype)
    red2 = qr.alloc_wire(codec, n)
    qr.qr_reduce_recv(codec, W, recv, n, red2, dtype)
    torch.cuda.synchronize()
    assert_recv_equal(hostu8(recv), r_wires, codec, n, "%s receive buffer" % label, fill=0xA7)
    assert_bytes_equal(hostu8(red2), r_red, "%s reduced from the receive buffer" % label)
    # inputs are never modified
    for r in range(W):
        assert np.array_equal(host16(xs[r]), xs_np[r]), label


SIZES = (8, 24, 40, 3 * 8192 + 24)    # one partial block ... several workgroups + tail


@pytest.mark.parametrize("W", (2, 4, 8))
@pytest.mark.parametrize("dtype", (O.FP16, O.BF16), ids=("fp16", "bf16"))
@pytest.mark.parametrize("codec", CODECS, ids=[I.CODEC_NAMES[c] for c in CODECS])
def test_parity_small(qr, codec, dtype, W):
    for cfg in GENS[dtype]:
        for n in SIZES:
            xs_np = _inputs(cfg, W, n, dtype)
            _check_case(qr, codec, dtype, xs_np, "c%d %s W%d n%d gen%d" % (
                codec, "bf16" if dtype else "fp16", W, n, cfg))


CAST = O.BF16_VIA_FP16                 # bf16 buffers through binary16


def _cast_edges(W, n, salt):
    """bf16 inputs where the cast to binary16 rounds: a bf16 value in the
    binary16 normal range converts exactly, so the inputs spread over every
    binade from 2^-27 to 2^15, with binary16 subnormals, values that underflow
    to +-0, exact ties k*2^-25 (k odd) between binary16 subnormals, and +-0."""
    g = np.random.default_rng(100 + salt)
    out = []
    for r in range(W):
        e = g.uniform(-27.0, 15.5, n)
        v = g.choice([-1.0, 1.0], n) * 2.0 ** e * g.uniform(1.0, 2.0, n)
        ties = g.random(n) < 0.1
        v[ties] = g.choice([-1.0, 1.0], int(ties.sum())) * \
            (2 * g.integers(0, 64, int(ties.sum())) + 1) * 2.0 ** -25
        v[g.random(n) < 0.05] = 0.0
        out.append(pins.torch_f32_to_bf16(np.clip(v, -60000, 60000).astype(np.float32)))
    return out


@pytest.mark.parametrize("W", (2, 4, 8))
@pytest.mark.parametrize("codec", CODECS, ids=[I.CODEC_NAMES[c] for c in CODECS])
def test_parity_cast(qr, codec, W):
    """the bf16 -> fp16 cast option: every wire plane and every output
    bit-exact against the oracle, on the bf16 workloads' generators and
    on inputs spread over binary16's whole range (subnormals, underflow)"""
    for n in SIZES:
        for cfg in (3, 4):
            _check_case(qr, codec, CAST, _inputs(cfg, W, n, O.BF16),
                        "cast c%d W%d n%d gen%d" % (codec, W, n, cfg))
        _check_case(qr, codec, CAST, _cast_edges(W, n, codec * 10 + W),
                    "cast edges c%d W%d n%d" % (codec, W, n))


def _pack_codes(codes, bits):
    """b-bit codes of 32-element blocks into the little-endian bitstream of
    each block (code i at bits [b*i, b*i+b))"""
    c = np.asarray(codes, np.uint64).reshape(-1, 32)
    if bits == 8:
        return c.astype(np.uint8).reshape(-1)
    out = np.zeros((c.shape[0], 32 * bits // 8), np.uint8)
    for i in range(32):
        for j in range(bits):
            bit = bits * i + j
            out[:, bit // 8] |= (((c[:, i] >> np.uint64(j)) & np.uint64(1))
                                 << np.uint64(bit % 8)).astype(np.uint8)
    return out.reshape(-1)


def _rounding_wire(codec, nb, seed):
    """An asymmetric wire image of nb blocks in which every other block has a
    scale s, zero z and code u such that u*s + z, rounded to binary32, lands
    exactly on the midpoint between two binary16 neighbours while the exact
    value does not; returns the wire and how many elements round differently
    when the exact value is rounded straight to binary16."""
    qu = {O.Q8A: 255, O.Q6A: 63, O.Q4A: 15}[codec]
    bits = {O.Q8A: 8, O.Q6A: 6, O.Q4A: 4}[codec]
    g = np.random.default_rng(seed)
    sv = np.arange(1, 0x7c00, dtype=np.uint16)
    sf = sv.view(np.float16).astype(np.float64)
    triples = []                    # (u, scale bits, binade e of the zero)
    for u in range(1, qu + 1):
        for e in range(0, 15):
            m, half = 2.0 ** (e - 11), 2.0 ** (e - 24)
            hit = (np.abs(u * sf - m) < half) & (u * sf != m)
            triples += [(u, int(b), e) for b in sv[hit]]
    codes = g.integers(0, qu + 1, (nb, 32))
    scale = g.integers(0x0400, 0x3000, nb).astype(np.uint16)      # random normal scales
    zero = (g.standard_normal(nb) * 4).astype(np.float16).view(np.uint16)
    if triples:
        for k in range(0, nb, 2):
            u, sb, e = triples[g.integers(len(triples))]
            codes[k, :] = u
            scale[k] = sb
            zero[k] = np.float16(2.0 ** e * (1.0 + g.integers(0, 1024) / 1024.0)).view(np.uint16)
    n = 32 * nb
    wire = np.zeros(O.wire_bytes(codec, n), np.uint8)
    wire[:nb * 32 * bits // 8] = _pack_codes(codes, bits)
    so, zo = O.scale_offset(codec, n), O.zero_offset(codec, n)
    wire[so:so + 2 * nb] = scale.view(np.uint8)
    wire[zo:zo + 2 * nb] = zero.view(np.uint8)
    exact = codes * scale.view(np.float16).astype(np.float64)[:, None] + \
        zero.view(np.float16).astype(np.float64)[:, None]          # exact in binary64
    twice = exact.astype(np.float32).astype(np.float16)
    once = exact.astype(np.float16)
    return wire, int(np.count_nonzero(twice.view(np.uint16) != once.view(np.uint16)))


@pytest.mark.parametrize("codec", (O.Q8A, O.Q6A, O.Q4A), ids=("q8a", "q6a", "q4a"))
def test_dequant_rounds_through_binary32(qr, codec):
    """asymmetric dequantization rounds code*scale + zero to binary32 first and
    then to the buffer type, as the definition does; built wires put many
    binary32 values exactly on binary16 midpoints that the exact values are not
    on (none exist for Q4A: a 4-bit code times a binary16 scale is too short)"""
    nb = 4096
    wire_np, diverging = _rounding_wire(codec, nb, 7 + codec)
    if codec != O.Q4A:
        assert diverging >= 1000, diverging
    n = 32 * nb
    wire = torch.from_numpy(wire_np).cuda()
    for dtype in (O.FP16, O.BF16, O.BF16_VIA_FP16):
        say("double rounding", codec, dtype, diverging)
        y = torch.empty(n, dtype=torch.int16, device="cuda")
        qr.qr_dequantize(codec, wire, y, dtype=dtype)
        ys = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(2)]
        qr.qr_gather_stage2(codec, wire, ys, dtype=dtype)
        torch.cuda.synchronize()
        want = O.dequantize(codec, dtype, wire_np, n)
        for got, what in ((y, "dequantize"), (ys[0], "stage 2"), (ys[1], "stage 2")):
            g_ = host16(got)
            bad = np.nonzero(g_ != want)[0]
            assert bad.size == 0, "%s dtype %d: %d elements differ, first %d got %04x want %04x" % (
                what, dtype, bad.size, bad[0], g_[bad[0]], want[bad[0]])


def test_golden_fixtures_gpu(qr):
    """The hand-worked examples through the HIP path."""
    for case in pins.golden_cases():
        codec, dt = case["codec"], case["dtype"]
        dtype = O.FP16 if dt == "fp16" else O.BF16
        xs_np = [pins.to_buf(x, dt) for x in case["x"]]
        n = xs_np[0].size
        want_y = np.array(case["x"][0] if case["y"] == "x" else case["y"], np.float64)
        say("golden", case["name"])
        xs = [dev16(x) for x in xs_np]
        if case["W"] == 1:
            wire = qr.alloc_wire(codec, n)
            qr.qr_quantize(codec, xs[0], wire, dtype=dtype)
            y = torch.empty_like(xs[0])
            qr.qr_dequantize(codec, wire, y, dtype=dtype)
            torch.cuda.synchronize()
            pins.check_wire_planes(codec, n, hostu8(wire), case["wire"])
            ys = [y]
        else:
            _, red, ys = gpu_staged(qr, codec, dtype, xs)
            pins.check_wire_planes(codec, n, hostu8(red), case["reduced"])
        for y in ys:
            got = pins.from_buf(host16(y), dt)
            assert np.array_equal(got, want_y), (case["name"], got)


@pytest.mark.parametrize("W", (2, 4, 8))
def test_owner_chunks(qr, W):
    """stage 1 for each owner writes exactly its chunk; together they give
    the full reduced image.  847 blocks: at W=2 owner 1 starts at block 424,
    off a 256-block workgroup tile, and spans full and partial tiles.  6
    blocks: at W=4 and W=8 the last owners' chunks are empty (nothing is
    launched and nothing written)."""
    for codec, n in [(c, m) for m in (32 * 5 + 8, 32 * 37 + 16, 32 * 846 + 16)
                     for c in (O.FP, O.Q4, O.Q6A, O.FP8, O.Q8)]:
        xs_np = _inputs(5, W, n, O.FP16, salt=1)
        say("owners", codec, W, n)
        xs = [dev16(x) for x in xs_np]
        wires = [qr.alloc_wire(codec, n) for _ in range(W)]
        qr.qr_quantize_ranks(codec, xs, wires, dtype=O.FP16)
        full = qr.alloc_wire(codec, n)
        qr.qr_reduce_stage1(codec, wires, n, full, O.FP16)
        acc = qr.alloc_wire(codec, n)
        for j in range(W):
            part = qr.alloc_wire(codec, n)
            qr.qr_reduce_stage1(codec, wires, n, part, O.FP16, owner=j)
            torch.cuda.synchronize()
            p = hostu8(part)
            want = O.stage1(codec, O.FP16, [hostu8(w) for w in wires], n,
                            *O.chunk(W, n, j))
            assert_bytes_equal(p, want, "owner %d" % j)
            acc |= part
        torch.cuda.synchronize()
        assert_bytes_equal(hostu8(acc), hostu8(full), "union of owners")
        # the same owners from a receive buffer
        recv = qr.alloc_recv(W, codec, n)
        qr.qr_quantize_recv(codec, xs, recv, dtype=O.FP16)
        acc2 = qr.alloc_wire(codec, n)
        for j in range(W):
            part = qr.alloc_wire(codec, n)
            qr.qr_reduce_recv(codec, W, recv, n, part, O.FP16, owner=j)
            torch.cuda.synchronize()
            want = O.stage1(codec, O.FP16, [hostu8(w) for w in wires], n, *O.chunk(W, n, j))
            assert_bytes_equal(hostu8(part), want, "owner %d from the receive buffer" % j)
            acc2 |= part
        torch.cuda.synchronize()
        assert_bytes_equal(hostu8(acc2), hostu8(full), "union of owners (receive buffer)")


def _random_wire(codec, n, g):
    """A wire image no quantizer wrote: uniformly random code bytes (every
    code, -2^(b-1) included, and junk in the unused slots of a partial last
    block), and binary16 scales and zeros drawn over every finite class:
    +-0, subnormals, normals up to 65504, both signs.  fp8 NaN codes
    (0x7f, 0xff) are moved to 0x7e/0xfe: non-finite values are outside the
    contract.  The FP wire holds random finite binary16 values."""
    wb = O.wire_bytes(codec, n)
    w = g.integers(0, 256, wb, dtype=np.uint8)

    def f16s(k):
        mag = np.where(g.random(k) < 0.3, g.integers(0, 0x400, k),       # 0 and subnormals
                       g.integers(0x400, 0x7C00, k))                       # normals
        mag[g.random(k) < 0.1] = 0
        return (mag | np.where(g.random(k) < 0.3, 0x8000, 0)).astype(np.uint16)

    if codec == O.FP:
        return f16s(n).view(np.uint8).copy()
    if codec == O.FP8:
        cb = O.block_code_bytes(codec) * ((n + 31) // 32)
        c = w[:cb]
        c[(c & 0x7F) == 0x7F] -= 1
    nb = (n + 31) // 32
    so = O.scale_offset(codec, n)
    w[so:so + 2 * nb] = f16s(nb).view(np.uint8)
    if codec & 8:
        zo = O.zero_offset(codec, n)
        w[zo:zo + 2 * nb] = f16s(nb).view(np.uint8)
    return w


def _dev_wire(codec, n, img, qr):
    t = qr.alloc_wire(codec, n)
    t.copy_(torch.from_numpy(img))
    return t


@pytest.mark.parametrize("W", (2, 4, 8))
def test_stage1_any_wire(qr, W):
    """stage 1 on wire images no quantizer wrote (every code value, scales of
    every finite class and sign, junk in unused code slots): the reduced
    image bit-exact against the oracle's stage 1 on the same bytes, for
    every codec.  This reaches the decode of codes stage 0 never writes and
    the saturated requantization of sums beyond the binary16 scale range."""
    n = 3 * 8192 + 24
    for codec in CODECS:
        g = np.random.default_rng(7000 + 10 * W + codec)
        imgs = [_random_wire(codec, n, g) for _ in range(W)]
        say("stage1 any wire", I.CODEC_NAMES[codec], W, n)
        wires = [_dev_wire(codec, n, im, qr) for im in imgs]
        red = qr.alloc_wire(codec, n)
        qr.qr_reduce_stage1(codec, wires, n, red, O.FP16)
        torch.cuda.synchronize()
        # the same bytes through a receive buffer
        rbuf, _ = recv_from_wires(codec, n, imgs)
        recv = torch.from_numpy(rbuf).cuda()
        red2 = qr.alloc_wire(codec, n)
        qr.qr_reduce_recv(codec, W, recv, n, red2, O.FP16)
        torch.cuda.synchronize()
        want = O.stage1(codec, O.FP16, imgs, n)
        for got, how in ((hostu8(red), "wires"), (hostu8(red2), "receive buffer")):
            for name, (a, e) in plane_slices(codec, n).items():
                assert_bytes_equal(got[a:e], want[a:e], "stage1 any wire (%s) %s W%d %s" % (
                    how, I.CODEC_NAMES[codec], W, name))


@pytest.mark.parametrize("dtype", (O.FP16, O.BF16), ids=("fp16", "bf16"))
def test_stage2_any_wire(qr, dtype):
    """stage 2 (and qr_dequantize) on a wire image no quantizer wrote: every
    output bit-exact against the oracle, for every codec."""
    n = 3 * 8192 + 24
    for codec in CODECS:
        g = np.random.default_rng(8000 + codec + 100 * dtype)
        img = _random_wire(codec, n, g)
        say("stage2 any wire", I.CODEC_NAMES[codec], dtype, n)
        red = _dev_wire(codec, n, img, qr)
        ys = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(2)]
        qr.qr_gather_stage2(codec, red, ys, dtype=dtype)
        torch.cuda.synchronize()
        want = O.stage2(codec, dtype, 2, img, n)
        for r in range(2):
            assert_within_ulp(host16(ys[r]), want[r], dtype, "stage2 any wire %s y[%d]" % (
                I.CODEC_NAMES[codec], r))


@pytest.mark.parametrize("dtype", (O.FP16, O.BF16), ids=("fp16", "bf16"))
def test_edge_values(qr, dtype):
    """all-zero, constant, +-0 mixes, sums that overflow to inf, huge and
    tiny magnitudes, identical ranks, and cancellation across ranks."""
    W, n = 4, 32 * 10 + 8
    one = pins.to_buf([1.0], "fp16" if dtype == O.FP16 else "bf16")[0]
    big = 0x7BFF if dtype == O.FP16 else 0x7F7F       # largest finite
    tiny = 0x0001                                       # smallest subnormal
    cases = {
        "zeros": [np.zeros(n, np.uint16)] * W,
        "neg_zeros": [np.full(n, 0x8000, np.uint16)] * W,
        "constant": [np.full(n, one, np.uint16)] * W,
        "overflow": [np.full(n, big, np.uint16)] * W,
        "tiny": [np.full(n, tiny, np.uint16) | (np.arange(n, dtype=np.uint16) & 1) * 0x8000] * W,
        "identical": [I.to_bits(I.draw(1, 0, n), dtype)] * W,
        "cancel": [I.to_bits(I.draw(1, 0, n), dtype),
                   I.to_bits(I.draw(1, 0, n), dtype) ^ 0x8000,
                   I.to_bits(I.draw(1, 1, n), dtype),
                   I.to_bits(I.draw(1, 1, n), dtype) ^ 0x8000],
    }
    for name, xs_np in cases.items():
        for codec in CODECS:
            _check_case(qr, codec, dtype, [x.copy() for x in xs_np],
                        "edge %s c%d" % (name, codec))


def test_single_rank_entry_points(qr):
    """qr_quantize / qr_dequantize on their own (W = 1 of the pipeline)."""
    for dtype in (O.FP16, O.BF16):
        for codec in CODECS:
            n = 8192 + 16
            x_np = I.to_bits(I.draw(5 if dtype == O.FP16 else 4, 7, n), dtype)
            say("single", codec, dtype)
            x = dev16(x_np)
            wire = qr.alloc_wire(codec, n)
            qr.qr_quantize(codec, x, wire, dtype=dtype)
            y = torch.empty_like(x)
            qr.qr_dequantize(codec, wire, y, dtype=dtype)
            torch.cuda.synchronize()
            rw = O.quantize(codec, dtype, x_np)
            assert_bytes_equal(hostu8(wire), rw, "single wire")
            assert_within_ulp(host16(y), O.dequantize(codec, dtype, rw, n), dtype, "single y")


def test_guard_bands(qr):
    """nothing is written outside the buffers: every output sits inside a
    larger allocation filled with a canary pattern."""
    G = 4096
    for codec in CODECS:
        for n in (8, 40, 8192 + 24):
            W = 4
            say("guard", codec, n)
            xs = [dev16(x) for x in _inputs(5, W, n, O.FP16)]
            wb = qr.qr_wire_bytes(codec, n)
            big_w = [torch.full((wb + 2 * G,), 0xA5, dtype=torch.uint8, device="cuda")
                     for _ in range(W + 1)]
            big_y = [torch.full((n + G,), 0x3C3C, dtype=torch.int16, device="cuda")
                     for _ in range(W)]
            wires = [b[G:G + wb] for b in big_w[:W]]
            red = big_w[W][G:G + wb]
            ys = [b[G // 2:G // 2 + n] for b in big_y]
            qr.qr_quantize_ranks(codec, xs, wires, dtype=O.FP16)
            qr.qr_reduce_stage1(codec, wires, n, red, O.FP16)
            qr.qr_gather_stage2(codec, red, ys, dtype=O.FP16)
            torch.cuda.synchronize()
            for b in big_w:
                h = hostu8(b)
                assert np.all(h[:G] == 0xA5) and np.all(h[G + wb:] == 0xA5), codec
                # plane padding is left untouched too
                planes = sorted(plane_slices(codec, n).values())
                inner = h[G:G + wb].copy()
                for a, e in planes:
                    inner[a:e] = 0xA5
                assert np.all(inner == 0xA5), ("padding written", codec, n)
            for b in big_y:
                h = host16(b)
                assert np.all(h[:G // 2] == 0x3C3C) and np.all(h[G // 2 + n:] == 0x3C3C)


def test_sim_guard_bands(qr):
    """qr_allreduce_sim (one launch for W <= 4, three for W = 8) writes
    nothing outside its workspace planes and its outputs"""
    G = 4096
    for codec in CODECS:
        for W in (2, 4, 8):
            for n in (8, 40, 8192 + 24):
                say("sim guard", codec, W, n)
                xs_np = _inputs(5, W, n, O.FP16)
                xs = [dev16(x) for x in xs_np]
                need = qr.qr_sim_workspace_bytes(W, codec, n)
                big_ws = torch.full((need + 2 * G,), 0xA5, dtype=torch.uint8, device="cuda")
                ws = big_ws[G:G + need]
                big_y = [torch.full((n + G,), 0x3C3C, dtype=torch.int16, device="cuda")
                         for _ in range(W)]
                ys = [b[G // 2:G // 2 + n] for b in big_y]
                qr.qr_allreduce_sim(codec, xs, ys, ws, dtype=O.FP16)
                torch.cuda.synchronize()
                h = hostu8(big_ws)
                assert np.all(h[:G] == 0xA5) and np.all(h[G + need:] == 0xA5), (codec, W, n)
                rb = qr.qr_recv_bytes(W, codec, n)
                red_at = (rb + 255) // 256 * 256
                inner = h[G:G + need].copy()
                inner[:rb][recv_mask(codec, n, W)] = 0xA5
                for a, e in plane_slices(codec, n).values():
                    inner[red_at + a:red_at + e] = 0xA5
                assert np.all(inner == 0xA5), ("workspace padding written", codec, W, n)
                want = O.allreduce(codec, O.FP16, xs_np)
                for r, b in enumerate(big_y):
                    hy = host16(b)
                    assert np.all(hy[:G // 2] == 0x3C3C) and np.all(hy[G // 2 + n:] == 0x3C3C)
                    assert_within_ulp(hy[G // 2:G // 2 + n], want[r], O.FP16, "sim guard y")


def test_graph_capture(qr):
    """qr_allreduce_sim and qr_allreduce_oneshot captured in a graph (they
    allocate nothing and issue no memset) and replayed three times, each with
    new inputs copied into the captured buffers and eager work in between:
    every replay equals the oracle"""
    for W, n, codec in ((2, 4096, O.Q4), (4, 3 * 8192 + 24, O.Q6A), (8, 8192, O.FP8),
                        (2, 3 * (1 << 20) + 8, O.Q8)):          # the last one takes three launches
        say("graph", W, n, codec)
        xs = [torch.empty(n, dtype=torch.int16, device="cuda") for _ in range(W)]
        ys = [torch.empty_like(xs[0]) for _ in range(W)]
        y1 = [torch.empty_like(xs[0]) for _ in range(W)]
        ws = qr.alloc_workspace(W, codec, n)
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):                # warm-up outside the capture
            qr.qr_allreduce_sim(codec, xs, ys, ws, dtype=O.FP16)
            qr.qr_allreduce_oneshot(xs, y1, dtype=O.FP16)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            qr.qr_allreduce_sim(codec, xs, ys, ws, dtype=O.FP16)
            qr.qr_allreduce_oneshot(xs, y1, dtype=O.FP16)
        for rep in range(3):
            xs_np = _inputs(1 + rep, W, n, O.FP16, salt=rep)
            for x, h in zip(xs, xs_np):
                x.copy_(dev16(h))
            junk = torch.randn(1 << 16, device="cuda").sum()     # eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            want = O.allreduce(codec, O.FP16, xs_np)
            want1 = O.oneshot(O.FP16, xs_np)
            for r in range(W):
                assert_within_ulp(host16(ys[r]), want[r], O.FP16, "graph replay %d y[%d]" % (rep, r))
                assert np.array_equal(host16(y1[r]), want1[r]), ("graph replay oneshot", rep, r)
            del junk


def test_rejected_call_writes_nothing(qr):
    n, W, codec = 4096, 2, O.Q4
    xs = [dev16(x) for x in _inputs(1, W, n, O.FP16)]
    ybuf = [torch.full((n + 8,), 77, dtype=torch.int16, device="cuda") for _ in range(W)]
    ys = [b[:n] for b in ybuf]
    ws = torch.full((qr.qr_sim_workspace_bytes(W, codec, n),), 9, dtype=torch.uint8,
                    device="cuda")
    say("rejects")
    with pytest.raises(qr.QRError) as e:                        # workspace too small
        qr.qr_allreduce_sim(codec, xs, ys, ws[:-1], dtype=O.FP16)
    assert e.value.code == -5
    with pytest.raises(qr.QRError) as e:                        # misaligned output
        qr.qr_allreduce_sim(codec, xs, [ys[0], ybuf[1][1:n + 1]], ws, dtype=O.FP16)
    assert e.value.code == -4
    with pytest.raises(qr.QRError) as e:                        # y overlaps x
        qr.qr_allreduce_sim(codec, xs, [xs[1], ys[1]], ws, dtype=O.FP16)
    assert e.value.code == -1
    with pytest.raises(qr.QRError) as e:                        # W not in {2,4,8}
        qr.qr_allreduce_sim(codec, xs + [xs[0]], ys + [ybuf[0][8:8 + n]], ws, dtype=O.FP16)
    assert e.value.code == -2
    torch.cuda.synchronize()
    for b in ybuf:
        assert torch.all(b == 77)
    assert torch.all(ws == 9)


def test_nondefault_stream(qr):
    n, W, codec = 8192 * 2, 8, O.Q6
    xs_np = _inputs(5, W, n, O.FP16)
    xs = [dev16(x) for x in xs_np]
    ys = [torch.empty_like(xs[0]) for _ in range(W)]
    ws = qr.alloc_workspace(W, codec, n)
    s = torch.cuda.Stream()
    say("stream")
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        qr.qr_allreduce_sim(codec, xs, ys, ws, dtype=O.FP16)
    s.synchronize()
    want = O.allreduce(codec, O.FP16, xs_np)
    for r in range(W):
        assert_within_ulp(host16(ys[r]), want[r], O.FP16, "stream y")


@pytest.mark.parametrize("dtype", (O.FP16, O.BF16), ids=("fp16", "bf16"))
def test_fp8_every_value(qr, dtype):
    """Every finite fp16 (bf16) value with |v| <= 448 goes through the fp8
    encoder with t = v exactly: each block is 448 followed by 31 of the
    values, so its scale is 448/448 = 1.  Codes (every E4M3 code but NaN
    appears) and the decoded outputs must equal the oracle's."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = (bits.view(np.float16).astype(np.float64) if dtype == O.FP16
            else pins.torch_bf16_to_f32(bits).astype(np.float64))
    keep = bits[np.isfinite(vals) & (np.abs(vals) <= 448)]
    anchor = pins.to_buf([448.0], "fp16" if dtype == O.FP16 else "bf16")[0]
    nblk = -(-keep.size // 31)
    x = np.zeros((nblk, 32), np.uint16)
    x[:, 0] = anchor
    body = np.zeros(nblk * 31, np.uint16)
    body[:keep.size] = keep
    x[:, 1:] = body.reshape(nblk, 31)
    x = x.reshape(-1)
    say("fp8 every value", dtype, x.size)
    xd = dev16(x)
    wire = qr.alloc_wire(O.FP8, x.size)
    qr.qr_quantize(O.FP8, xd, wire, dtype=dtype)
    y = torch.empty_like(xd)
    qr.qr_dequantize(O.FP8, wire, y, dtype=dtype)
    torch.cuda.synchronize()
    rw = O.quantize(O.FP8, dtype, x)
    assert_bytes_equal(hostu8(wire), rw, "fp8 wire")
    codes = set(hostu8(wire)[:32 * nblk].tolist())
    assert len(codes) >= 250, len(codes)
    assert_within_ulp(host16(y), O.dequantize(O.FP8, dtype, rw, x.size), dtype, "fp8 y", ulps=0)


def test_concurrent_host_threads(qr):
    """four host threads, each with its own stream and buffers, issue
    simulated allreduces at the same time (the library keeps no state
    between calls): every result equals the oracle"""
    import threading
    jobs = [(2, O.Q4, 3 * 8192 + 40), (4, O.Q6A, 8192 + 8), (8, O.FP8, 4096),
            (4, O.Q8, 3 * (1 << 20) + 8)]                      # the last takes three launches
    data = []
    for k, (W, codec, n) in enumerate(jobs):
        xs_np = _inputs(2, W, n, O.FP16, salt=20 + k)
        data.append((W, codec, n, xs_np, O.allreduce(codec, O.FP16, xs_np)))
    say("threads", [(W, codec, n) for W, codec, n, _, _ in data])
    bufs = []
    for W, codec, n, xs_np, _ in data:
        xs = [dev16(x) for x in xs_np]
        bufs.append((xs, [torch.empty_like(xs[0]) for _ in range(W)],
                     qr.alloc_workspace(W, codec, n), torch.cuda.Stream()))
    torch.cuda.synchronize()
    bar = threading.Barrier(len(jobs))
    errors = []

    def run(k):
        try:
            W, codec = data[k][0], data[k][1]
            xs, ys, ws, s = bufs[k]
            bar.wait()
            for _ in range(5):
                qr.qr_allreduce_sim(codec, xs, ys, ws, dtype=O.FP16, stream=s)
            s.synchronize()
        except Exception as e:          # reported by the main thread
            errors.append((k, repr(e)))

    ts = [threading.Thread(target=run, args=(k,)) for k in range(len(jobs))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert not errors, errors
    torch.cuda.synchronize()
    for k, (W, codec, n, _, want) in enumerate(data):
        for r in range(W):
            assert_within_ulp(host16(bufs[k][1][r]), want[r], O.FP16,
                              "thread %d y[%d]" % (k, r))
