"""Seeded synthetic inputs for the simulated allreduce.

This module draws numbers and nothing else: it holds none of the method's
arithmetic, and both the tests (for the oracle and the HIP path alike) and the
benchmark take their inputs from here.

Every buffer is drawn in float64 with numpy's PCG64 generator, seeded with
``1000*config + rank`` (draws shared by all ranks use ``1000*config + 999``),
then rounded to the buffer type: float16 by numpy's cast, bfloat16 by way of
float32 with torch's CPU cast (both round to nearest, ties to even).  Buffers
are returned as raw 16-bit patterns (numpy ``uint16``).

The shapes follow the pages' sweep of allreduce sizes (the tp2 timing table of
"Integrate quick allreduce and select the best allreduce implementation",
4 KB to 64 MB per rank buffer, binary units as in the vLLM quick_all_reduce
docs page's ``MB = 1024 * 1024``); the value distributions are synthetic
stand-ins for activations (the pages measure on no dataset).
"""
import numpy as np

FP, Q8, Q6, Q4, FP8, Q8A, Q6A, Q4A = 0, 1, 2, 3, 5, 9, 10, 11
FP16, BF16 = 0, 1
CODEC_NAMES = {FP: "fp", Q8: "q8", Q6: "q6", Q4: "q4", FP8: "fp8",
               Q8A: "q8a", Q6A: "q6a", Q4A: "q4a"}
ALL_CODECS = (FP, FP8, Q8, Q6, Q4, Q8A, Q6A, Q4A)
MB = 1024 * 1024

# The five workloads: ranks W, buffer type, elements per rank, codecs.
CONFIGS = {
    1: dict(W=2, dtype=FP16, n=2048, codecs=(Q8,),
            desc="W=2 fp16 4 KB/rank, Q8 symmetric, N(0,1)"),
    2: dict(W=2, dtype=FP16, n=64 * MB // 2, codecs=(FP, FP8, Q8, Q6, Q4),
            desc="W=2 fp16 64 MB/rank, N(0,1) with 0.1% x50 outliers"),
    3: dict(W=4, dtype=BF16, n=None, codecs=(Q4A,),
            sizes=tuple(2 ** k for k in range(11, 26)),
            desc="W=4 bf16 4 KB..64 MB/rank, Q4 asymmetric, N(0,0.5)+row bias"),
    4: dict(W=8, dtype=BF16, n=1024 * 8192, codecs=(Q6,),
            desc="W=8 bf16 16 MB/rank [1024 tokens x 8192 hidden], Q6 symmetric, "
                 "Laplace(0,1) x per-channel scale 10^U(-3,1)"),
    5: dict(W=8, dtype=FP16, n=64 * MB // 2, codecs=ALL_CODECS,
            desc="W=8 fp16 64 MB/rank, adversarial blocks (zero/constant/spike/"
                 "+-max-finite) 1:1:1:1 interleaved with N(0,1) blocks"),
}

ROW = 8192        # config 3: bias rows of 8192 contiguous elements
HIDDEN = 8192     # config 4: hidden size (channels run along the buffer)
BLOCK = 32        # config 5: the pattern is laid out on 32-element blocks


def rng(config, rank):
    return np.random.Generator(np.random.PCG64(1000 * config + rank))


def shared_rng(config):
    return np.random.Generator(np.random.PCG64(1000 * config + 999))


def draw(config, rank, n, W=None):
    """float64 values of one rank's buffer for a workload."""
    g = rng(config, rank)
    if config in (1, 0):
        return g.standard_normal(n)
    if config == 2:
        # each element independently x50 with probability 0.001: the number of
        # outliers is binomial, their positions a uniform sample without repeats
        v = g.standard_normal(n)
        k = int(g.binomial(n, 0.001))
        v[g.choice(n, k, replace=False)] *= 50.0
        return v
    if config == 3:
        v = g.normal(0.0, 0.5, n)
        rows = (n + ROW - 1) // ROW
        bias = g.uniform(-2.0, 2.0, rows)
        full = n // ROW
        v[:full * ROW].reshape(full, ROW)[:] += bias[:full, None]
        if full < rows:
            v[full * ROW:] += bias[full]
        return v
    if config == 4:
        sigma = 10.0 ** shared_rng(config).uniform(-3.0, 1.0, HIDDEN)
        v = g.laplace(0.0, 1.0, n)
        full = n // HIDDEN
        v[:full * HIDDEN].reshape(full, HIDDEN)[:] *= sigma[None, :]
        v[full * HIDDEN:] *= sigma[:n - full * HIDDEN]
        return v
    if config == 5:
        return _adversarial(g, shared_rng(config), n)
    raise ValueError("unknown config %r" % (config,))


def _adversarial(g, gs, n):
    """Block pattern by block index k: odd k are N(0,1); even k have type
    (k/2) mod 4, the same on every rank: 0 all zero, 1 one constant drawn
    N(0,1) per rank, 2 a single spike at a position shared by the ranks with
    value +-2^U(-14,15), 3 each element +-65504 with probability 1/2, else
    N(0,1)."""
    nb = (n + BLOCK - 1) // BLOCK
    v = g.standard_normal(nb * BLOCK).reshape(nb, BLOCK)
    k = np.arange(nb)
    kind = np.where(k % 2 == 1, -1, (k // 2) % 4)
    v[kind == 0] = 0.0
    c1 = np.nonzero(kind == 1)[0]
    v[c1] = g.standard_normal(c1.size)[:, None]
    c2 = np.nonzero(kind == 2)[0]
    pos = gs.integers(0, BLOCK, nb)[c2]               # shared across ranks
    val = np.exp2(g.uniform(-14.0, 15.0, c2.size)) * np.where(
        g.random(c2.size) < 0.5, -1.0, 1.0)
    v[c2] = 0.0
    v[c2, pos] = val
    c3 = np.nonzero(kind == 3)[0]
    pick = g.random((c3.size, BLOCK)) < 0.5
    sign = np.where(g.random((c3.size, BLOCK)) < 0.5, -1.0, 1.0)
    v[c3] = np.where(pick, 65504.0 * sign, v[c3])
    return v.reshape(-1)[:n]


def to_bits(v64, dtype):
    """Round float64 values to the buffer type; return raw uint16 patterns."""
    if dtype == FP16:
        return v64.astype(np.float16).view(np.uint16)
    import torch
    f32 = torch.from_numpy(np.ascontiguousarray(v64, dtype=np.float32))
    return f32.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def make(config, W=None, n=None, dtype=None):
    """Raw uint16 buffers of all ranks for a workload (defaults: its own)."""
    c = CONFIGS.get(config, CONFIGS[1])
    W = c["W"] if W is None else W
    n = c["n"] if n is None else n
    dtype = c["dtype"] if dtype is None else dtype
    return [to_bits(draw(config, r, n, W), dtype) for r in range(W)]
