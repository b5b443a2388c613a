"""Pins for the CPU oracle: checks against what the definitions and the
mathematics fix, never against the oracle itself.

Each ``check_*`` takes a loaded oracle library handle ``L`` and raises
AssertionError on a mismatch, so the same checks run against the real oracle
(tests/test_oracle_pins.py) and against builds of it with a planted mistake
(tests/test_oracle_mutants.py), where at least one must fail.

Independent sources used here: numpy's float16 casts and ``nextafter``,
torch's bfloat16 and float8_e4m3fn casts, brute-force argmin over every code,
closed forms, and the hand-worked
fixtures in tests/golden/.
"""
import json
import math
import os

import numpy as np

import oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
SYM = (O.Q8, O.Q6, O.Q4)
ASYM = (O.Q8A, O.Q6A, O.Q4A)
QUANT = SYM + ASYM + (O.FP8,)
BITS = {O.Q8: 8, O.Q6: 6, O.Q4: 4, O.FP8: 8, O.Q8A: 8, O.Q6A: 6, O.Q4A: 4}
QMAX = {O.Q8: 127, O.Q6: 31, O.Q4: 7, O.FP8: 448, O.Q8A: 255, O.Q6A: 63, O.Q4A: 15}


# ----------------------------------------------------------------------------
# independent helpers (numpy / torch / exact arithmetic)

def f16_bits(v):
    return int(np.array(v, np.float32).astype(np.float16).view(np.uint16))


def f16_val(bits):
    return float(np.array(bits, np.uint16).view(np.float16))


@np.errstate(over="ignore")
def grid_up16(v):
    """least finite float16 >= v (v >= 0), saturated at 65504, by rounding to
    nearest with numpy and stepping with nextafter (vectorised)."""
    v = np.asarray(v, np.float32)
    h = v.astype(np.float16)
    low = np.isfinite(h) & (h.astype(np.float32) < v)
    h = np.where(low, np.nextafter(h, np.float16(np.inf)), h)
    h = np.where(np.isinf(h), np.float16(65504), h)
    return h.view(np.uint16)


@np.errstate(over="ignore")
def grid_down16(v):
    """greatest finite float16 <= v, saturated at -65504 (vectorised)."""
    v = np.asarray(v, np.float32)
    h = v.astype(np.float16)
    high = np.isfinite(h) & (h.astype(np.float32) > v)
    h = np.where(high, np.nextafter(h, np.float16(-np.inf)), h)
    h = np.where(np.isposinf(h), np.float16(65504), h)
    h = np.where(np.isneginf(h), np.float16(-65504), h)
    return h.view(np.uint16)


def torch_bf16_to_f32(bits):
    import torch
    t = torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16).copy())
    return t.view(torch.bfloat16).float().numpy()


def torch_f32_to_bf16(vals):
    import torch
    t = torch.from_numpy(np.asarray(vals, np.float32).copy())
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def e4m3_table():
    """value of every E4M3FN code, from torch's float8_e4m3fn type."""
    import torch
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def e4m3_nearest(t, table):
    """brute force over all 256 codes: the nearest finite E4M3FN value to each
    t (same sign bit as t, so a zero result keeps the sign), ties to the even
    code; saturation falls out because no code above 448 is finite."""
    t = np.atleast_1d(np.asarray(t, np.float64))
    codes = np.arange(256)
    D = np.abs(t[:, None] - table[None, :])       # exact for these ranges
    D[:, np.isnan(table)] = np.inf
    D[np.signbit(t)[:, None] != (codes[None, :] >= 128)] = np.inf
    cand = D == D.min(axis=1, keepdims=True)
    even = cand & (codes[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    return codes[pick]


def nearest_int_even(t, lo, hi):
    """brute force over every integer code in [lo, hi]: nearest to each t,
    ties to the even integer."""
    t = np.atleast_1d(np.asarray(t, np.float64))
    q = np.arange(lo, hi + 1)
    D = np.abs(t[:, None] - q[None, :].astype(np.float64))  # exact: t binary32
    cand = D == D.min(axis=1, keepdims=True)
    even = cand & (q[None, :] % 2 == 0)
    pick = np.where(even.any(axis=1), np.argmax(even, axis=1), np.argmax(cand, axis=1))
    return q[pick]


def random_blocks(seed, count, log2_lo=-30, log2_hi=12):
    """random binary32 blocks of random length 1..32 and random magnitude."""
    g = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        L = int(g.integers(1, 33))
        mag = 2.0 ** g.uniform(log2_lo, log2_hi)
        kind = g.integers(0, 4)
        if kind == 0:
            v = g.standard_normal(L) * mag
        elif kind == 1:
            v = g.uniform(-1, 1, L) * mag + g.uniform(-4, 4) * mag
        elif kind == 2:
            v = g.laplace(0, 1, L) * mag
        else:
            v = np.abs(g.standard_normal(L)) * mag
        out.append(v.astype(np.float32))
    return out


def block_fp16(seed, count):
    """random blocks whose values are float16 numbers (as binary32)."""
    return [b.astype(np.float16).astype(np.float32) for b in
            random_blocks(seed, count, -20, 14)]


# ----------------------------------------------------------------------------
# conversions

def check_h2f_exhaustive(L):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = bits.view(np.float16).astype(np.float32)
    for b, w in zip(bits, want):
        got = O.h2f(int(b), L)
        if math.isnan(w):
            assert math.isnan(got), hex(b)
        else:
            assert np.float32(got).view(np.uint32) == np.float32(w).view(np.uint32), hex(b)


def f16_probe_values(seed=1):
    """float32 values around the float16 grid: every finite float16, every
    midpoint between neighbours, one float32 step either side of each
    midpoint, random values over the whole range, and the overflow edge."""
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float64)
    mids = (pos[:-1] + pos[1:]) / 2.0
    mid32 = mids.astype(np.float32)
    assert np.all(mid32.astype(np.float64) == mids)   # midpoints are exact
    up = np.nextafter(mid32, np.float32(np.inf))
    dn = np.nextafter(mid32, np.float32(-np.inf))
    g = np.random.default_rng(seed)
    rnd = (2.0 ** g.uniform(-30, 17, 20000)).astype(np.float32)
    edge = np.array([65504, 65519.996, 65520, 65536, 1e10, 2.0 ** -25,
                     2.0 ** -24 * 0.75, 2.0 ** -26], np.float32)
    v = np.concatenate([pos.astype(np.float32), mid32, up, dn, rnd, edge])
    return np.concatenate([v, -v])


def check_f2h(L):
    v = f16_probe_values()
    want = v.astype(np.float16).view(np.uint16)
    for x, w in zip(v, want):
        assert O.f2h(float(x), L) == int(w), (float(x), hex(w))
    assert O.f2h(float("inf"), L) == 0x7C00 and O.f2h(float("-inf"), L) == 0xFC00
    assert O.f2h(-0.0, L) == 0x8000


def check_bf16(L):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    want = torch_bf16_to_f32(bits)
    for b, w in zip(bits, want):
        got = O.bf2f(int(b), L)
        if math.isnan(w):
            assert math.isnan(got)
        else:
            assert np.float32(got).view(np.uint32) == np.float32(w).view(np.uint32), hex(b)
    g = np.random.default_rng(2)
    fin = want[np.isfinite(want)].astype(np.float64)
    fin = np.unique(fin[fin > 0])
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    rnd = (2.0 ** g.uniform(-140, 128, 20000)).astype(np.float32)
    v = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)),
                        np.nextafter(mids, np.float32(-np.inf)), rnd,
                        np.array([3.4e38, 3.3961776e38, 1e-45], np.float32)])
    v = np.concatenate([v, -v])
    wantb = torch_f32_to_bf16(v)
    for x, w in zip(v, wantb):
        assert O.f2bf(float(x), L) == int(w), (float(x), hex(w))


def check_ru_rd(L):
    g = np.random.default_rng(3)
    pos = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16).astype(np.float32)
    rnd = (2.0 ** g.uniform(-30, 17, 20000)).astype(np.float32)
    v = np.concatenate([pos, np.nextafter(pos, np.float32(np.inf)),
                        np.nextafter(pos[1:], np.float32(0)), rnd,
                        np.array([65504, 65505, 65519, 65520, 70000, 1e10,
                                  2 ** -25, 2 ** -30], np.float32)])
    up, dn, dnn = grid_up16(v), grid_down16(v), grid_down16(-v)
    for i, x in enumerate(v):
        assert O.ru16(float(x), L) == up[i], float(x)
        assert O.rd16(float(x), L) == dn[i], float(x)
        assert O.rd16(float(-x), L) == dnn[i], float(-x)
    assert O.ru16(0.0, L) == 0 and O.rd16(0.0, L) == 0


def check_e4m3(L):
    table = e4m3_table()
    for c in range(256):
        got = O.e4m3_decode(c, L)
        if math.isnan(table[c]):
            assert math.isnan(got)
        else:
            assert got == table[c], hex(c)
    fin = np.unique(np.abs(table[np.isfinite(table)]))
    mids = (fin[:-1] + fin[1:]) / 2
    g = np.random.default_rng(4)
    t = np.concatenate([fin, mids, np.nextafter(mids.astype(np.float32), np.float32(1e9)),
                        np.nextafter(mids.astype(np.float32), np.float32(0)),
                        g.uniform(0, 500, 3000), 2.0 ** g.uniform(-14, 9, 3000),
                        [448.0, 463.9, 464.0, 1e6, 2.0 ** -10, 2.0 ** -11]]).astype(np.float32)
    t = np.concatenate([t, -t, np.array([0.0, -0.0], np.float32)])
    want = e4m3_nearest(t, table)
    for x, w in zip(t, want):
        assert O.e4m3_encode(float(x), L) == w, float(x)
    # and torch's own encoder (round to nearest even, no saturation) agrees
    # where saturation does not act
    import torch
    tc = torch.from_numpy(np.clip(t, -448, 448).copy())
    tb = tc.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, b in zip(np.clip(t, -448, 448), tb):
        assert O.e4m3_encode(float(x), L) == int(b), float(x)


# ----------------------------------------------------------------------------
# one block

def _signed(code, b):
    return code - (1 << b) if code & (1 << (b - 1)) else code


def check_block_codes(L, count=300):
    """Per block: the scale is the least fp16 >= f32(absmax/qmax) (constant
    block: >= absmax), the zero the greatest fp16 <= min, and every code is
    the brute-force nearest code to t = f32(v * f32(1/s)) (ties to even)."""
    table = e4m3_table()
    f = np.float32
    for codec in QUANT:
        b, qm = BITS[codec], QMAX[codec]
        for v in random_blocks(10 + codec, count):
            codes, s, z = O.quantize_block(codec, v, L)
            mx, mn = float(v.max()), float(v.min())
            if codec in ASYM:
                mn0 = 0.0 if mn == 0 else mn
                assert z == grid_down16(mn0), (codec, mn, hex(z))
                d = f(mx) - f(f16_val(z))
                if not d > 0:
                    assert s == 0 and not codes.any()
                    continue
                assert s == grid_up16(f(d) / f(qm)), (codec, hex(s))
                inv = f(1.0) / f(f16_val(s))
                t = (v - f(f16_val(z))) * inv
                want = nearest_int_even(t, 0, qm)
                assert np.array_equal(codes[:v.size], want), (codec, codes, want)
            else:
                a = max(abs(mx), abs(mn))
                assert z == 0
                if a == 0:
                    assert s == 0 and not codes.any()
                    continue
                arg = f(a) if mx == mn else f(a) / f(qm)
                assert s == grid_up16(arg), (codec, a, hex(s))
                inv = f(1.0) / f(f16_val(s))
                t = v * inv
                if codec == O.FP8:
                    want = e4m3_nearest(t, table)
                    got = codes[:v.size]
                else:
                    want = nearest_int_even(t, -qm, qm)
                    got = np.array([_signed(int(c), b) for c in codes[:v.size]])
                assert np.array_equal(got, want), (codec, got, want)
            assert not codes[v.size:].any()


def _finite_f16_bits():
    """every finite binary16 bit pattern, +-0 and subnormals included"""
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    return b[(b & 0x7C00) != 0x7C00]


def _unpack_codes(codes_plane, nb, b):
    """code i of each block from bits [b*i, b*i+b) of the block's
    little-endian bitstring, by numpy's unpackbits (independent of the
    oracle's packing code)"""
    blk = codes_plane[:nb * 4 * b].reshape(nb, 4 * b)
    bits = np.unpackbits(blk, axis=1, bitorder="little").reshape(nb, 32, b)
    return (bits.astype(np.int64) << np.arange(b)).sum(axis=2)


def check_one_element_sweep(L):
    """Exhaustive in one element: two fixed blocks of binary16 values, one
    element of which takes every finite binary16 value (63488 blocks each),
    quantized by the oracle in one call per codec.  Every block's scale (and
    zero) must be the binary16 grid neighbour of the binary32 quotient found
    by nextafter; every code the nearest (ties to even) to t = v * (1/s),
    by numpy's rint (binary32) or torch's float8_e4m3fn cast, clamped; the
    varying element's code also by brute force over every code."""
    g = np.random.default_rng(31)
    sweep = _finite_f16_bits()
    f = np.float32
    bases = [(g.standard_normal(32).astype(np.float16).view(np.uint16), 0),
             ((g.standard_normal(32) * 1e-3).astype(np.float16).view(np.uint16), 17)]
    table = e4m3_table()
    for codec in QUANT:
        b, qm = BITS[codec], QMAX[codec]
        for base, j in bases:
            x = np.tile(base, (sweep.size, 1))
            x[:, j] = sweep
            nb = sweep.size
            wire = O.quantize(codec, O.FP16, x.ravel(), L=L)
            # plane offsets from the layout's definition: each plane starts at
            # the next 256-byte boundary after the previous one
            so = (nb * 4 * b + 255) // 256 * 256
            s = wire[so:so + 2 * nb].view(np.uint16)
            codes = _unpack_codes(wire, nb, b)
            v = x.view(np.float16).astype(np.float32)
            mx, mn = v.max(axis=1), v.min(axis=1)
            if codec in ASYM:
                zo = (so + 2 * nb + 255) // 256 * 256
                z = wire[zo:zo + 2 * nb].view(np.uint16)
                mn0 = np.where(mn == 0, f(0.0), mn)
                assert np.array_equal(z, grid_down16(mn0)), codec
                zf = z.view(np.float16).astype(np.float32)
                d = mx - zf
                with np.errstate(divide="ignore", over="ignore"):
                    want_s = np.where(d > 0, grid_up16(d / f(qm)), 0).astype(np.uint16)
                assert np.array_equal(s, want_s), codec
                inv = np.where(s > 0, f(1.0) / np.maximum(s.view(np.float16).astype(f), f(6e-8)),
                               f(0.0)).astype(f)
                t = (v - zf[:, None]) * inv[:, None]
                want = np.clip(np.rint(t), 0, qm).astype(np.int64)
                got = codes
            else:
                a = np.maximum(np.abs(mx), np.abs(mn))
                arg = np.where(mx == mn, a, a / f(qm)).astype(f)
                want_s = np.where(a > 0, grid_up16(arg), 0).astype(np.uint16)
                assert np.array_equal(s, want_s), codec
                inv = np.where(s > 0, f(1.0) / np.maximum(s.view(np.float16).astype(f), f(6e-8)),
                               f(0.0)).astype(f)
                t = v * inv[:, None]
                if codec == O.FP8:
                    import torch
                    tc = torch.from_numpy(np.clip(t, -448, 448))
                    want = tc.to(torch.float8_e4m3fn).view(torch.uint8).numpy().astype(np.int64)
                    want[s == 0] = 0
                    got = codes
                else:
                    want = np.clip(np.rint(t), -qm, qm).astype(np.int64)
                    got = np.where(codes >= 1 << (b - 1), codes - (1 << b), codes)
            bad = np.nonzero(got != want)
            assert bad[0].size == 0, (codec, j, bad[0][:3], bad[1][:3])
            # the varying element by brute force over every code
            tj = t[:, j].astype(np.float64)
            if codec == O.FP8:
                wj = e4m3_nearest(tj, table)
                wj[s == 0] = 0
            else:
                lo = 0 if codec in ASYM else -qm
                wj = np.concatenate([nearest_int_even(tj[k:k + 4096], lo, qm)
                                     for k in range(0, tj.size, 4096)])
            assert np.array_equal(got[:, j], wj), codec


def check_error_bound(L, count=400):
    """|v - dequant| within half a step (plus binary32 slop) per element."""
    for codec in QUANT:
        for v in random_blocks(20 + codec, count):
            codes, s, z = O.quantize_block(codec, v, L)
            fs, fz = f16_val(s), f16_val(z)
            for i, x in enumerate(v.astype(np.float64)):
                xh = float(O.dequant_code(codec, int(codes[i]), s, z, L))
                err = abs(x - xh)
                if codec in SYM:
                    bound = fs * (0.5 + 2.0 ** -15)
                elif codec in ASYM:
                    bound = 0.5 * fs + 2.0 ** -21 * (abs(x) + abs(fz))
                else:
                    t = abs(x) / fs if fs else 0.0
                    e = max(math.floor(math.log2(t)) if t > 0 else -6, -6)
                    bound = fs * 2.0 ** (e - 4) * (1 + 2.0 ** -20) + 2.0 ** -21 * abs(x)
                if fs == 0:
                    bound = 0.0
                assert err <= bound, (codec, i, x, xh, fs)


def check_zero_blocks(L):
    for codec in QUANT:
        for L_ in (1, 8, 32):
            for v in (np.zeros(L_, np.float32), -np.zeros(L_, np.float32),
                      np.array(([0.0, -0.0] * 16)[:L_], np.float32)):
                codes, s, z = O.quantize_block(codec, v, L)
                assert s == 0 and z == 0 and not codes.any(), codec
                for c in codes[:L_]:
                    assert O.dequant_code(codec, int(c), s, z, L) == 0.0


def check_idempotent(L, count=300):
    """Symmetric codecs: requantizing the dequantized block gives the same
    codes and scale (normal-range blocks whose dequantized values are not all
    equal; a constant result falls under the constant-block rule)."""
    for codec in SYM + (O.FP8,):
        for v in random_blocks(30 + codec, count, -8, 12):
            codes, s, z = O.quantize_block(codec, v, L)
            if s == 0:
                continue
            xh = np.array([O.dequant_code(codec, int(c), s, z, L) for c in codes[:v.size]],
                          np.float32)
            if xh.max() == xh.min():
                continue        # dequantizes to a constant: the constant rule applies
            codes2, s2, _ = O.quantize_block(codec, xh, L)
            assert s2 == s and np.array_equal(codes2, codes), (codec, v, xh)


# ----------------------------------------------------------------------------
# whole buffers

def check_constants_exhaustive(L, codecs=QUANT):
    """Every finite fp16 value as a constant block survives the W=1 pipeline
    exactly, for every codec; bf16: every bf16 value fp16 can represent."""
    h = np.arange(0, 0x7C00, dtype=np.uint16)
    h = np.concatenate([h, h | 0x8000])
    xf16 = np.repeat(h, 32)
    vals = torch_bf16_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    ok = np.isfinite(vals) & (np.abs(vals) <= 65504)
    f16of = vals.astype(np.float16)
    exact = ok & (f16of.astype(np.float32) == vals)
    bfb = np.arange(65536, dtype=np.uint32).astype(np.uint16)[exact]
    xbf16 = np.repeat(bfb, 32)
    for codec in codecs:
        for dtype, x, conv in ((O.FP16, xf16, lambda a: a.view(np.float16).astype(np.float64)),
                               (O.BF16, xbf16, lambda a: torch_bf16_to_f32(a).astype(np.float64))):
            y = O.allreduce(codec, dtype, [x], L=L)[0]
            bad = np.nonzero(conv(y) != conv(x))[0]
            assert bad.size == 0, (codec, dtype, bad[:4], x[bad[:4]], y[bad[:4]])


def _fp_cases(seed):
    """Raw inputs of every W in (1, 2, 3, 4, 8) and both buffer types, with
    the expected allreduce: the binary32 sum in rank order 0..W-1 (numpy
    float32 additions in that order), rounded once by numpy/torch casts.
    For W >= 3 a quarter of the elements cancel: one rank holds +2^15, a later
    one -2^15 and an earlier one 2^-9, so the binary32 sum depends on the
    order; magnitudes up to 2^10 * N(0,1) also reach the binary16 overflow."""
    g = np.random.default_rng(seed)
    for W in (1, 2, 3, 4, 8):
        for dtype in (O.FP16, O.BF16):
            n = 8 * int(g.integers(1, 200))
            xs64 = [g.standard_normal(n) * 2.0 ** g.uniform(-10, 10, n) for _ in range(W)]
            if W >= 3:
                idx = g.choice(n, n // 4, replace=False)
                for e in idx:
                    r = sorted(g.choice(W, 3, replace=False))
                    sg = 1.0 if g.random() < 0.5 else -1.0
                    for q in range(W):
                        xs64[q][e] = 0.0
                    xs64[r[0]][e] = 2.0 ** -9 * sg
                    xs64[r[1]][e] = 2.0 ** 15
                    xs64[r[2]][e] = -2.0 ** 15
            if dtype == O.FP16:
                xs = [x.astype(np.float16).view(np.uint16) for x in xs64]
                vals = [x.view(np.float16).astype(np.float32) for x in xs]
            else:
                xs = [torch_f32_to_bf16(x.astype(np.float32)) for x in xs64]
                vals = [torch_bf16_to_f32(x) for x in xs]
            acc = vals[0].copy()
            for v in vals[1:]:
                acc = (acc + v).astype(np.float32)
            want = acc.astype(np.float16).view(np.uint16) if dtype == O.FP16 else \
                torch_f32_to_bf16(acc)
            yield W, dtype, xs, want


def check_fp_closed_form(L):
    """FP codec: output = the binary32 sum in rank order 0..W-1, rounded once."""
    for W, dtype, xs, want in _fp_cases(5):
        ys = O.allreduce(O.FP, dtype, xs, L=L)
        for y in ys:
            assert np.array_equal(y, want), (W, dtype)


def check_oneshot_closed_form(L):
    """One-stage allreduce: every rank's output = the binary32 sum in rank
    order 0..W-1, rounded once; also on block sub-ranges (elements outside
    the range untouched)."""
    for W, dtype, xs, want in _fp_cases(6):
        ys = O.oneshot(dtype, xs, L=L)
        for y in ys:
            assert np.array_equal(y, want), (W, dtype)
        n = xs[0].size
        nb = (n + 31) // 32
        lo, hi = nb // 3, max(nb // 3 + 1, (2 * nb) // 3)
        sentinel = [np.full(n, 0xABCD, np.uint16) for _ in range(W)]
        O.oneshot(dtype, xs, lo, hi, ys=sentinel, L=L)
        e_lo, e_hi = 32 * lo, min(n, 32 * hi)
        for y in sentinel:
            assert np.array_equal(y[e_lo:e_hi], want[e_lo:e_hi]), (W, dtype, "range")
            assert np.all(y[:e_lo] == 0xABCD) and np.all(y[e_hi:] == 0xABCD), (W, dtype)


def check_cast_option(L):
    """bf16 buffers through binary16 (dtype 2): the allreduce, the one-stage
    allreduce and every wire image equal those of the binary16 pipeline run on
    the binary16 roundings of the inputs (numpy's cast of the bf16 values),
    with the binary16 results rounded to bf16 (torch's cast).  Inputs span
    binary16 subnormals, values that flush to zero, ties of the bf16 grid, and
    (FP paths only) magnitudes that overflow binary16."""
    g = np.random.default_rng(9)
    CAST = 2
    for W in (1, 2, 4, 8):
        n = 8 * int(g.integers(4, 120))
        for codec in (O.FP, O.FP8, O.Q8, O.Q6, O.Q4, O.Q8A, O.Q6A, O.Q4A):
            hi = 17.0 if codec == O.FP else 15.0            # 2^17 overflows binary16
            xs64 = [g.standard_normal(n) * 2.0 ** g.uniform(-30, hi, n) for _ in range(W)]
            # overflows are all positive: +inf + -inf (a NaN) is outside the contract
            xs64 = [np.where(np.abs(x) > 60000.0, np.abs(x), x) for x in xs64]
            xs = [torch_f32_to_bf16(np.clip(x, -65000.0, 65000.0).astype(np.float32))
                  if codec != O.FP else torch_f32_to_bf16(x.astype(np.float32)) for x in xs64]
            xs16 = [torch_bf16_to_f32(x).astype(np.float16).view(np.uint16) for x in xs]
            want = [torch_f32_to_bf16(y.view(np.float16).astype(np.float32))
                    for y in O.allreduce(codec, O.FP16, xs16, L=L)]
            got = O.allreduce(codec, CAST, xs, L=L)
            for r in range(W):
                assert np.array_equal(got[r], want[r]), (W, codec, r)
            for r in range(W):
                assert np.array_equal(O.quantize(codec, CAST, xs[r], L=L),
                                      O.quantize(codec, O.FP16, xs16[r], L=L)), (W, codec)
            if codec == O.FP:
                got1 = O.oneshot(CAST, xs, L=L)
                want1 = [torch_f32_to_bf16(y.view(np.float16).astype(np.float32))
                         for y in O.oneshot(O.FP16, xs16, L=L)]
                for r in range(W):
                    assert np.array_equal(got1[r], want1[r]), (W, "oneshot")


def _planes(codec, n, wire, L=None):
    nb = (n + 31) // 32
    cb = nb * 32 * BITS[codec] // 8
    so = O.scale_offset(codec, n, L)
    s = wire[so:so + 2 * nb].view(np.uint16)
    z = None
    if codec in ASYM:
        zo = O.zero_offset(codec, n, L)
        z = wire[zo:zo + 2 * nb].view(np.uint16)
    return wire[:cb], s, z


def check_end_to_end_bound(L):
    """Per element |y - sum x_r| <= sum of the rank quantization bounds + the
    stage-1 requantization bound + rounding of the binary32 sum and of the
    final cast (all from the recorded scales, in binary64)."""
    g = np.random.default_rng(6)
    for W in (2, 4, 8):
        for codec in QUANT:
            n = 32 * 24 + 16
            xs64 = [g.standard_normal(n) * 2.0 ** g.uniform(-6, 6) for _ in range(W)]
            xs = [x.astype(np.float16).view(np.uint16) for x in xs64]
            xv = [x.view(np.float16).astype(np.float64) for x in xs]
            wires = [O.quantize(codec, O.FP16, x, L=L) for x in xs]
            red = O.stage1(codec, O.FP16, wires, n, L=L)
            ys = O.stage2(codec, O.FP16, W, red, n, L=L)
            assert all(np.array_equal(ys[0], y) for y in ys[1:])
            y = ys[0].view(np.float16).astype(np.float64)
            exact = np.sum(xv, axis=0)

            def step_bound(wire, nvals):
                _, s, z = _planes(codec, n, wire, L)
                fs = np.repeat(s.view(np.float16).astype(np.float64), 32)[:n]
                if codec in SYM:
                    return fs * (0.5 + 2.0 ** -15)
                if codec in ASYM:
                    fz = np.repeat(z.view(np.float16).astype(np.float64), 32)[:n]
                    return 0.5 * fs + 2.0 ** -21 * (np.abs(nvals) + np.abs(fz))
                # half a step of E4M3 at t = v/s: 2^-4 |t| in the normal range,
                # 2^-10 in the subnormal range
                return fs * 2.0 ** -10 + (2.0 ** -4 + 2.0 ** -20) * np.abs(nvals)

            bound = sum(step_bound(w, x) for w, x in zip(wires, xv))
            absum = np.sum(np.abs(xv), axis=0) + bound
            bound = bound + step_bound(red, np.abs(exact) + bound) + \
                (W - 1) * 2.0 ** -23 * absum
            bound = bound + np.abs(y) * 2.0 ** -11 + 2.0 ** -24
            assert np.all(np.abs(y - exact) <= bound), (W, codec)


def _decode_wire_numpy(codec, n, wire):
    """Every element of a quantized wire image as binary32, decoded with
    numpy alone: code fields by np.unpackbits, the scale (and zero) planes at
    their 256-byte boundaries, symmetric codes sign-extended, fp8 codes
    through torch's float8_e4m3fn table.  The product code * scale is exact in
    binary32 (at most 8 + 11 significant bits); an asymmetric value adds the
    zero with one binary32 rounding (numpy float32 addition)."""
    nb = (n + 31) // 32
    b = BITS[codec]
    f = np.uint16
    codes = _unpack_codes(wire, nb, b)
    so = (nb * 4 * b + 255) // 256 * 256
    s = wire[so:so + 2 * nb].view(f).view(np.float16).astype(np.float64)[:, None]
    if codec == O.FP8:
        vals = (e4m3_table()[codes] * s).astype(np.float32)
    elif codec in SYM:
        q = np.where(codes >= 1 << (b - 1), codes - (1 << b), codes)
        vals = (q * s).astype(np.float32)
    else:
        zo = (so + 2 * nb + 255) // 256 * 256
        z = wire[zo:zo + 2 * nb].view(f).view(np.float16).astype(np.float32)[:, None]
        vals = (codes * s).astype(np.float32) + z
    return vals.reshape(-1)[:n]


def _stage1_cases(seed):
    """Rank buffers for the stage-1 composition pin: W in (2, 3, 4, 8), both
    buffer types, a ragged tail.  Block kinds, drawn per block:
      - cancellation: one rank holds small values (2^-9 scale), two others
        hold +B and -B with B near 2^14, the rest zero; in binary32 the small
        terms are absorbed or not depending on the order of the additions;
      - mixed magnitudes: every rank N(0,1) times its own 2^U(-6, 6), so the
        binary32 sums carry more significant bits than the buffer type;
      - plain N(0,1)."""
    g = np.random.default_rng(seed)
    for W in (2, 3, 4, 8):
        for dtype in (O.FP16, O.BF16):
            nb = 48
            n = 32 * nb - 8 * int(g.integers(0, 4))
            xs64 = [np.zeros(n) for _ in range(W)]
            for k in range(nb):
                lo, hi = 32 * k, min(n, 32 * k + 32)
                L = hi - lo
                kind = k % 3
                if kind == 0 and W >= 3:
                    a, b, c = g.choice(W, 3, replace=False)
                    big = g.uniform(0.5, 1.0, L) * 2.0 ** 14
                    xs64[a][lo:hi] = g.standard_normal(L) * 2.0 ** -9
                    xs64[b][lo:hi] = big
                    xs64[c][lo:hi] = -big
                elif kind == 1:
                    for r in range(W):
                        xs64[r][lo:hi] = g.standard_normal(L) * 2.0 ** g.uniform(-6, 6)
                else:
                    for r in range(W):
                        xs64[r][lo:hi] = g.standard_normal(L)
            if dtype == O.FP16:
                xs = [x.astype(np.float16).view(np.uint16) for x in xs64]
            else:
                xs = [torch_f32_to_bf16(x.astype(np.float32)) for x in xs64]
            yield W, dtype, n, xs


def check_stage1_composition(L):
    """Stage 1 of every quantized codec is the composition of three pinned
    parts: the W wire images (the oracle's quantizer, pinned by the checks
    above) are decoded with numpy, summed in numpy binary32 in rank order
    0..W-1, and every block of the reduced image must equal the oracle's block
    quantizer applied to those binary32 sums (codes, scale and zero).  The
    cancellation blocks make the order and the precision of the sum visible,
    the mixed-magnitude blocks the requantization of sums that the buffer type
    cannot hold."""
    for W, dtype, n, xs in _stage1_cases(12):
        for codec in QUANT:
            wires = [O.quantize(codec, dtype, x, L=L) for x in xs]
            vals = [_decode_wire_numpy(codec, n, w) for w in wires]
            acc = vals[0].copy()
            for v in vals[1:]:
                acc = (acc + v).astype(np.float32)
            red = O.stage1(codec, dtype, wires, n, L=L)
            nb = (n + 31) // 32
            b = BITS[codec]
            got_codes = _unpack_codes(red, nb, b)
            _, got_s, got_z = _planes(codec, n, red, L)
            for k in range(nb):
                codes, s, z = O.quantize_block(codec, acc[32 * k:min(n, 32 * k + 32)], L)
                assert np.array_equal(got_codes[k], codes.astype(np.int64)), (W, dtype, codec, k)
                assert got_s[k] == s, (W, dtype, codec, k, got_s[k], s)
                if codec in ASYM:
                    assert got_z[k] == z, (W, dtype, codec, k)


def check_chunks(L):
    for W in (1, 2, 3, 4, 8):
        for n in (8, 16, 40, 256, 2048, 2056, 32 * 7 + 8, 32 * 1000):
            nb = (n + 31) // 32
            bpc = -(-nb // W)
            prev = 0
            for j in range(W):
                lo, hi = O.chunk(W, n, j, L)
                assert lo == min(nb, j * bpc) and hi == min(nb, (j + 1) * bpc)
                assert lo == prev
                prev = hi
            assert prev == nb


def check_layout(L):
    """Plane sizes and offsets, by hand from the wire definition."""
    n = 32 * 1024 * 1024
    want = {O.FP: 67108864, O.FP8: 35651584, O.Q8: 35651584, O.Q8A: 37748736,
            O.Q6: 27262976, O.Q6A: 29360128, O.Q4: 18874368, O.Q4A: 20971520}
    for c, w in want.items():
        assert O.wire_bytes(c, n, L) == w, c
    assert O.wire_bytes(O.Q8, 2048, L) == 2176
    assert O.wire_bytes(O.Q4A, 2048, L) == 1024 + 128 + 128 + 128     # 1408
    assert O.wire_bytes(O.Q6, 8 * 1024 * 1024, L) == 6815744
    assert O.wire_bytes(O.Q4, 40, L) == 256 + 4
    assert O.scale_offset(O.Q6, 40, L) == 256 and O.zero_offset(O.Q6A, 40, L) == 512
    assert O.wire_bytes(O.Q6A, 32 * 100, L) == 2560 + 256 + 200   # codes 2400 -> 2560


def check_owner_split(L):
    """Stage 1 restricted to each owner's chunk, together, equals stage 1
    over all blocks; no owner writes outside its chunk."""
    g = np.random.default_rng(7)
    for W in (2, 3, 4, 8):
        for codec in (O.FP, O.Q4, O.Q6A, O.FP8):
            n = 32 * int(g.integers(1, 40)) + 8 * int(g.integers(0, 4))
            xs = [(g.standard_normal(n)).astype(np.float16).view(np.uint16) for _ in range(W)]
            wires = [O.quantize(codec, O.FP16, x, L=L) for x in xs]
            full = O.stage1(codec, O.FP16, wires, n, L=L)
            acc = np.zeros_like(full)
            for j in range(W):
                lo, hi = O.chunk(W, n, j, L)
                part = O.stage1(codec, O.FP16, wires, n, lo, hi, L=L)
                if codec != O.FP:
                    c, s, z = _planes(codec, n, part, L)
                    cb = 32 * BITS[codec] // 8
                    assert not c[:lo * cb].any() and not c[hi * cb:].any()
                    assert not s[:lo].any() and not s[hi:].any()
                acc |= part
            assert np.array_equal(acc, full), (W, codec)


# ----------------------------------------------------------------------------
# hand-worked fixtures

def golden_cases():
    with open(os.path.join(GOLDEN, "hand_worked.json")) as f:
        return json.load(f)["cases"]


def to_buf(vals, dtype):
    a = np.array(vals, np.float64)
    if dtype == "fp16":
        return a.astype(np.float16).view(np.uint16)
    return torch_f32_to_bf16(a.astype(np.float32))


def from_buf(buf, dtype):
    if dtype == "fp16":
        return buf.view(np.float16).astype(np.float64)
    return torch_bf16_to_f32(buf).astype(np.float64)


def check_wire_planes(codec, n, wire, exp):
    """codes at 0, scales at the next 256-byte boundary, zeros (asymmetric)
    at the next 256-byte boundary after the scales."""
    nb = (n + 31) // 32
    c = bytes.fromhex(exp["codes"])
    assert len(c) == nb * 32 * BITS[codec] // 8
    assert bytes(wire[:len(c)]) == c, (bytes(wire[:len(c)]).hex(), exp["codes"])
    so = (len(c) + 255) // 256 * 256
    s = bytes.fromhex(exp["scales"])
    assert bytes(wire[so:so + 2 * nb]) == s, (bytes(wire[so:so + 2 * nb]).hex(), exp["scales"])
    end = so + 2 * nb
    if codec in ASYM:
        zo = (end + 255) // 256 * 256
        z = bytes.fromhex(exp["zeros"])
        assert bytes(wire[zo:zo + 2 * nb]) == z, bytes(wire[zo:zo + 2 * nb]).hex()
        end = zo + 2 * nb
    assert wire.size == end == exp["wire_bytes"], (wire.size, end)


def check_golden(L):
    for case in golden_cases():
        codec, dt = case["codec"], case["dtype"]
        dtype = O.FP16 if dt == "fp16" else O.BF16
        xs = [to_buf(x, dt) for x in case["x"]]
        n = xs[0].size
        want_y = np.array(case["x"][0] if case["y"] == "x" else case["y"], np.float64)
        if case["W"] == 1:
            wire = O.quantize(codec, dtype, xs[0], L=L)
            check_wire_planes(codec, n, wire, case["wire"])
            y = O.dequantize(codec, dtype, wire, n, L=L)
        else:
            wires = [O.quantize(codec, dtype, x, L=L) for x in xs]
            red = O.stage1(codec, dtype, wires, n, L=L)
            check_wire_planes(codec, n, red, case["reduced"])
            y = O.allreduce(codec, dtype, xs, L=L)[0]
        assert np.array_equal(from_buf(y, dt), want_y), (case["name"], from_buf(y, dt))


QUICK_CHECKS = [check_golden, check_layout, check_chunks, check_zero_blocks,
                check_f2h, check_ru_rd, check_e4m3, check_bf16,
                check_block_codes, check_error_bound, check_idempotent,
                check_fp_closed_form, check_oneshot_closed_form, check_cast_option,
                check_end_to_end_bound, check_stage1_composition,
                check_owner_split, check_one_element_sweep]
