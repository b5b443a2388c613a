"""The receive buffer's layout as the GPU tests state it (gpu_util), held to
a byte-by-byte restatement of its definition in include/qr.h: tile t of rank
r at (t*W + r) * T; in a tile, the codes word-major in words of S bytes (8
for 6-bit codes, else 16), then the binary16 scales, then the zeros; FP the
raw data; slots past the last block undefined."""
import numpy as np

import oracle as O
from gpu_util import recv_from_wires, recv_mask, recv_tile_bytes

CODECS = (O.FP, O.FP8, O.Q8, O.Q6, O.Q4, O.Q8A, O.Q6A, O.Q4A)


def _by_byte(codec, n, wires, fill):
    W, nb, T = len(wires), (n + 31) // 32, recv_tile_bytes(codec)
    size = (nb + 255) // 256 * W * T
    want, mask = np.full(size, fill, np.uint8), np.zeros(size, bool)
    for r in range(W):
        for blk in range(nb):
            t, b = divmod(blk, 256)
            base = (t * W + r) * T
            if codec == O.FP:
                for i in range(min(64, 2 * n - 64 * blk)):
                    want[base + 64 * b + i] = wires[r][64 * blk + i]
                    mask[base + 64 * b + i] = True
                continue
            cb = O.block_code_bytes(codec)
            S = 8 if cb == 24 else 16
            for i in range(cb):
                k, o = divmod(i, S)
                d = base + k * 256 * S + b * S + o
                want[d], mask[d] = wires[r][cb * blk + i], True
            offs = [O.scale_offset(codec, n)] + ([O.zero_offset(codec, n)] if codec & 8 else [])
            for p, off in enumerate(offs):
                for i in range(2):
                    d = base + 256 * cb + 512 * p + 2 * b + i
                    want[d], mask[d] = wires[r][off + 2 * blk + i], True
    return want, mask


def test_receive_buffer_layout():
    g = np.random.default_rng(7)
    for codec in CODECS:
        for n, W in ((8, 2), (40, 4), (8192 + 24, 8), (3 * 8192, 2)):
            wires = [g.integers(0, 256, O.wire_bytes(codec, n)).astype(np.uint8)
                     for _ in range(W)]
            got, gmask = recv_from_wires(codec, n, wires, fill=7)
            want, wmask = _by_byte(codec, n, wires, 7)
            assert np.array_equal(got, want) and np.array_equal(gmask, wmask), (codec, n, W)
            assert np.array_equal(recv_mask(codec, n, W), wmask), (codec, n, W)
