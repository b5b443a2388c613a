"""Helpers for the GPU parity tests: device/host transfer of raw 16-bit
buffers, the HIP pipeline run stage by stage through the C ABI, the same
pipeline on the oracle, and the comparisons the parity bar asks for."""
import sys

import numpy as np
import torch

import oracle as O


def say(*a):
    """name the case before a GPU step (flushed, so it survives a crash)."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy()).cuda()


def host16(t):
    return t.cpu().numpy().view(np.uint16)


def hostu8(t):
    return t.cpu().numpy()


def gpu_staged(qr, codec, dtype, xs, fill=0x5A5A):
    """quantize_ranks -> reduce_stage1(all owners) -> gather_stage2."""
    W, n = len(xs), xs[0].numel()
    wires = [qr.alloc_wire(codec, n) for _ in range(W)]
    qr.qr_quantize_ranks(codec, xs, wires, dtype=dtype)
    red = qr.alloc_wire(codec, n)
    qr.qr_reduce_stage1(codec, wires, n, red, dtype)
    ys = [torch.full((n,), fill - 65536 if fill > 32767 else fill, dtype=torch.int16,
                     device="cuda") for _ in range(W)]
    qr.qr_gather_stage2(codec, red, ys, dtype=dtype)
    torch.cuda.synchronize()
    return wires, red, ys


def oracle_staged(codec, dtype, xs_np, lo=0, hi=O.ALL):
    W, n = len(xs_np), xs_np[0].size
    wires = [O.quantize(codec, dtype, x, lo, hi) for x in xs_np]
    red = O.stage1(codec, dtype, wires, n, lo, hi)
    ys = O.stage2(codec, dtype, W, red, n, lo, hi)
    return wires, red, ys


def ordered(bits):
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, -(b & 0x7FFF), b)


def ulp_distance(a, b):
    return np.abs(ordered(a) - ordered(b))


def assert_bytes_equal(got, want, what):
    got, want = np.asarray(got), np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "%s: %d bytes differ, first at %d (got %02x want %02x)" % (
        what, bad.size, bad[0], got[bad[0]], want[bad[0]])


def _is_nan(bits, dtype):
    exp = 0x7C00 if dtype == O.FP16 else 0x7F80
    man = 0x03FF if dtype == O.FP16 else 0x007F
    return ((bits & exp) == exp) & ((bits & man) != 0)


def _is_inf(bits, dtype):
    return (bits & 0x7FFF) == (0x7C00 if dtype == O.FP16 else 0x7F80)


def assert_within_ulp(got, want, dtype, what, ulps=0, signed_zero=True):
    """outputs within `ulps` units in the last place of the buffer type
    (ordered-integer distance; inf only equals inf of the same sign; with
    signed_zero, a zero must also carry the expected sign); returns how many
    elements are not bit-identical.  The default is 0 ulps: the kernels
    round exactly as the definition does (binary32, then the buffer type), so
    any 1-ulp difference is a rounding-order bug (one such, a binary32 result
    rounded straight to binary16 by a merged instruction, differed by exactly
    1 ulp on rare elements, and turned -0 into +0)."""
    got, want = np.asarray(got, np.uint16), np.asarray(want, np.uint16)
    assert got.shape == want.shape
    assert np.array_equal(_is_nan(got, dtype), _is_nan(want, dtype)), what
    inf_g, inf_w = _is_inf(got, dtype), _is_inf(want, dtype)
    assert np.array_equal(inf_g, inf_w), (what, np.nonzero(inf_g != inf_w)[0][:5])
    assert np.array_equal(got[inf_g], want[inf_w]), what
    fin = ~(inf_g | _is_nan(got, dtype))
    d = ulp_distance(got[fin], want[fin])
    worst = int(d.max()) if d.size else 0
    assert worst <= ulps, "%s: %d ulp (index %d)" % (what, worst, np.nonzero(fin)[0][np.argmax(d)])
    if signed_zero:
        zs = np.nonzero((((got | want) & 0x7FFF) == 0) & (got != want))[0]
        assert zs.size == 0, "%s: %d zeros of the wrong sign (first at %d: got %04x want %04x)" % (
            what, zs.size, zs[0], got[zs[0]], want[zs[0]])
    return int(np.count_nonzero((got != want) & ~(((got | want) & 0x7FFF) == 0)))


def plane_slices(codec, n):
    """byte ranges of the codes, scales and zeros planes of a wire image."""
    if codec == O.FP:
        return {"raw": (0, 2 * n)}
    nb = (n + 31) // 32
    cb = O.block_code_bytes(codec)
    so = O.scale_offset(codec, n)
    out = {"codes": (0, nb * cb), "scales": (so, so + 2 * nb)}
    if codec & 8:
        zo = O.zero_offset(codec, n)
        out["zeros"] = (zo, zo + 2 * nb)
    return out


def block_ranges(codec, n, lo, hi):
    """byte ranges of blocks [lo, hi) in each plane of a wire image."""
    if codec == O.FP:
        return {"raw": (64 * lo, min(64 * hi, 2 * n))}
    cb = O.block_code_bytes(codec)
    so = O.scale_offset(codec, n)
    out = {"codes": (cb * lo, cb * hi), "scales": (so + 2 * lo, so + 2 * hi)}
    if codec & 8:
        zo = O.zero_offset(codec, n)
        out["zeros"] = (zo + 2 * lo, zo + 2 * hi)
    return out


def assert_wire_blocks(got, want, codec, n, lo, hi, what):
    for name, (a, b) in block_ranges(codec, n, lo, hi).items():
        assert_bytes_equal(got[a:b], want[a:b], "%s %s blocks %d..%d" % (what, name, lo, hi))


def sample_windows(nb, count=12, width=64, seed=0):
    """block windows spread over [0, nb): the first, the last, and random."""
    g = np.random.default_rng(seed)
    w = min(width, nb)
    starts = {0, nb - w}
    if nb > w:
        starts.update(int(s) for s in g.integers(0, nb - w, count))
    return sorted((s, s + w) for s in starts)


def recv_tile_bytes(codec):
    """bytes of one rank's tile of 256 blocks in the receive buffer: the
    tile's codes, scales (and zeros); FP: 256 blocks of raw 16-bit data"""
    if codec == O.FP:
        return 256 * 64
    return 256 * (O.block_code_bytes(codec) + 2 + (2 if codec & 8 else 0))


def recv_word_bytes(codec):
    """a tile's codes sit in the receive buffer word-major, in words of this
    many bytes: word k of the tile's 256 blocks is contiguous"""
    return 8 if O.block_code_bytes(codec) == 24 else 16


def _rank_tiles(codec, n, wire):
    """one rank's tiles of the receive buffer from its planar wire image, as
    (tiles, defined) arrays of shape (tile count, tile bytes), from the
    layout's definition: a tile holds blocks [256t, 256t+256): their codes,
    word-major (word k, bytes [kS, kS+S) of each block's codes, of all 256
    blocks one after the other, then word k+1), then their binary16 scales,
    then their binary16 zeros; FP: the blocks' raw data.  Slots of blocks
    past the last one are undefined."""
    nb = (n + 31) // 32
    nt = (nb + 255) // 256
    T = recv_tile_bytes(codec)

    def padded(src, size):
        v, d = np.zeros(size, np.uint8), np.zeros(size, bool)
        v[:src.size], d[:src.size] = src, True
        return v, d

    if codec == O.FP:
        v, d = padded(np.asarray(wire[:2 * n]), nt * T)
        return v.reshape(nt, T), d.reshape(nt, T)
    cb, S = O.block_code_bytes(codec), recv_word_bytes(codec)
    parts = []
    v, d = padded(np.asarray(wire[:nb * cb]), nt * 256 * cb)
    parts.append(tuple(x.reshape(nt, 256, cb // S, S).transpose(0, 2, 1, 3).reshape(nt, 256 * cb)
                       for x in (v, d)))
    planes = [O.scale_offset(codec, n)] + ([O.zero_offset(codec, n)] if codec & 8 else [])
    for off in planes:
        v, d = padded(np.asarray(wire[off:off + 2 * nb]), nt * 512)
        parts.append((v.reshape(nt, 512), d.reshape(nt, 512)))
    return (np.concatenate([p[0] for p in parts], axis=1),
            np.concatenate([p[1] for p in parts], axis=1))


def recv_from_wires(codec, n, wires, fill=0):
    """the receive buffer holding W planar wire images (numpy), with the
    mask of its defined bytes; padding bytes hold `fill`.  Tile t of rank r
    starts at byte (t*W + r) * T."""
    W = len(wires)
    tiles = [_rank_tiles(codec, n, w) for w in wires]
    nt, T = tiles[0][0].shape
    buf = np.full((nt, W, T), fill, np.uint8)
    mask = np.zeros((nt, W, T), bool)
    for r, (v, d) in enumerate(tiles):
        buf[:, r] = np.where(d, v, np.uint8(fill))
        mask[:, r] = d
    return buf.ravel(), mask.ravel()


def recv_mask(codec, n, W):
    """the defined bytes of a receive buffer of W ranks"""
    wb = O.wire_bytes(codec, n)
    return recv_from_wires(codec, n, [np.zeros(wb, np.uint8)] * W)[1]


def assert_recv_equal(got, wires, codec, n, what, fill=None):
    """a receive buffer against W planar wire images: every defined byte
    equal; with `fill`, every padding byte still holds it"""
    want, mask = recv_from_wires(codec, n, wires)
    got = np.asarray(got)
    assert got.size == want.size, (what, got.size, want.size)
    assert_bytes_equal(got[mask], want[mask], what)
    if fill is not None:
        assert np.all(got[~mask] == fill), (what, "receive-buffer padding written")


def oracle_threads():
    """host threads for the oracle: the CPUs this process may use, at most 16"""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def oracle_whole(codec, dtype, xs_np, threads=None):
    """The oracle over whole buffers, split by block range over host threads
    (the oracle is called on each range; ctypes releases the GIL): the W
    planar wire images, the reduced image, and the output every rank gets
    (stage 2 dequantizes the one reduced image on every rank)."""
    import threading
    O.lib()                  # loaded once, before the threads
    W, n = len(xs_np), xs_np[0].size
    nb = (n + 31) // 32
    T = threads or oracle_threads()
    bounds = np.linspace(0, nb, T + 1).astype(np.int64)
    wb = O.wire_bytes(codec, n)
    wires = [np.zeros(wb, np.uint8) for _ in range(W)]
    red = np.zeros(wb, np.uint8)
    y = np.zeros(n, np.uint16)

    def par(fn):
        ts = [threading.Thread(target=fn, args=(int(bounds[i]), int(bounds[i + 1])))
              for i in range(T) if bounds[i] < bounds[i + 1]]
        for t in ts:
            t.start()
        for t in ts:
            t.join()

    def q(lo, hi):
        for r in range(W):
            O.quantize(codec, dtype, xs_np[r], lo, hi, wire=wires[r])
    par(q)
    par(lambda lo, hi: O.stage1(codec, dtype, wires, n, lo, hi, reduced=red))
    par(lambda lo, hi: O.dequantize(codec, dtype, red, n, lo, hi, y=y))
    return wires, red, y

