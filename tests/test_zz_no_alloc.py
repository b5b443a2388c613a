"""qr_allreduce_sim_noalloc through the C ABI: the simulated allreduce with the
library's own workspace buffer gives, bit for bit, what qr_allreduce_sim gives
with a caller workspace; two calls in a row, the second on a smaller input,
on the single-launch path (up to 4 MiB per rank buffer) and on the
three-launch path; the largest accepted size; a refused size writes
nothing."""
import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import dev16, host16, say
from quantized_two_stage_amd import inputs as I

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qr():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from quantized_two_stage_amd import qr as q
    return q


def _xs(W, n, dtype, seed):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(W):
        v = g.standard_normal(n) * 2.0 ** g.uniform(-4, 4)
        out.append(I.to_bits(v, O.BF16 if dtype in (O.BF16, O.BF16_VIA_FP16) else O.FP16))
    return out


def _both(qr, codec, dtype, W, n, seed):
    """the no-alloc call and qr_allreduce_sim on the same inputs; outputs
    pre-filled with different patterns so that an unwritten element shows"""
    xs_np = _xs(W, n, dtype, seed)
    xs = [dev16(x) for x in xs_np]
    ys_a = [torch.full((n,), 0x1357, dtype=torch.int16, device="cuda") for _ in range(W)]
    ys_b = [torch.full((n,), 0x2468, dtype=torch.int16, device="cuda") for _ in range(W)]
    ws = qr.alloc_workspace(W, codec, n)
    say("noalloc W=%d codec=%d dtype=%d n=%d" % (W, codec, dtype, n))
    qr.qr_allreduce_sim_noalloc(codec, xs, ys_a, dtype=dtype)
    qr.qr_allreduce_sim(codec, xs, ys_b, ws, dtype=dtype)
    torch.cuda.synchronize()
    for r in range(W):
        a, b = host16(ys_a[r]), host16(ys_b[r])
        bad = np.nonzero(a != b)[0]
        assert bad.size == 0, "W=%d codec=%d n=%d rank %d: %d elements differ (first %d)" % (
            W, codec, n, r, bad.size, bad[0])
    return xs_np, [host16(y) for y in ys_a]


# (W, codec, buffer type, first n, second n): the first call on the
# three-launch path or at the single launch's largest size, the second smaller
CASES = [
    (2, O.Q4, O.FP16, 1 << 22, 2048 + 8),          # 8 MiB (three launches), then 4 KB
    (8, O.FP, O.FP16, 1 << 21, 1000),              # 4 MiB, 36 MiB of workspace
    (4, O.Q6A, O.BF16, 1 << 21, 8),
    (8, O.Q8A, O.BF16_VIA_FP16, (1 << 21) - 8, 4096 + 24),
    (2, O.FP8, O.FP16, 3 << 21, (1 << 20) + 8),    # 12 MiB (three launches), then 2 MiB
    (4, O.Q8, O.FP16, 1 << 20, (1 << 19) + 8),
]


@pytest.mark.parametrize("W,codec,dtype,n1,n2", CASES)
def test_noalloc_matches_sim_twice(qr, W, codec, dtype, n1, n2):
    assert n2 < n1
    assert qr.qr_sim_workspace_bytes(W, codec, n1) <= qr.QR_SCRATCH_BYTES
    _both(qr, codec, dtype, W, n1, seed=100 + W + codec)
    xs_np, ys = _both(qr, codec, dtype, W, n2, seed=200 + W + codec)
    if n2 <= 1 << 16:
        want = O.allreduce(codec, dtype, xs_np)
        for r in range(W):
            assert np.array_equal(ys[r], want[r]), (W, codec, n2, r)


def test_noalloc_largest_size_and_refusal(qr):
    W, codec, dtype = 2, O.FP, O.FP16
    n = 8
    while qr.qr_sim_workspace_bytes(W, codec, n + 8) <= qr.QR_SCRATCH_BYTES:
        n += 8
    _both(qr, codec, dtype, W, n, seed=7)
    xs = [torch.zeros(n + 8, dtype=torch.int16, device="cuda") for _ in range(W)]
    ys = [torch.full((n + 8,), 0x1357, dtype=torch.int16, device="cuda") for _ in range(W)]
    say("noalloc refused size n=%d" % (n + 8))
    with pytest.raises(qr.QRError) as e:
        qr.qr_allreduce_sim_noalloc(codec, xs, ys, dtype=dtype)
    assert e.value.code == -5
    torch.cuda.synchronize()
    for y in ys:
        assert bool((y == 0x1357).all())
