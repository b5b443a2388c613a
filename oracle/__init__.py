"""CPU oracle for the two-stage quantized allreduce -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never does.

A thin ctypes layer over ``qr_oracle.c`` (plain scalar C, see its header for
the passages of the pages it follows and the readings taken where they are
silent).  Arrays are numpy: raw 16-bit buffers are ``uint16``, wire images are
``uint8``.
"""
import ctypes
import os

import numpy as np

from . import build as _build

FP, Q8, Q6, Q4, FP8, Q8A, Q6A, Q4A = 0, 1, 2, 3, 5, 9, 10, 11
FP16, BF16, BF16_VIA_FP16 = 0, 1, 2
BLK = 32
ALL = ctypes.c_size_t(-1).value

_lib = None


def lib():
    """Load the oracle library, building it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _lib = _declare(ctypes.CDLL(_build.LIB))
    return _lib


def load_variant(path):
    """Load another build of the oracle source (used by the mutation tests)."""
    return _declare(ctypes.CDLL(path))


def _declare(L):
    sz, u16, u8, f32, i32 = (ctypes.c_size_t, ctypes.c_uint16, ctypes.c_uint8,
                             ctypes.c_float, ctypes.c_int)
    P = ctypes.c_void_p
    sig = {
        "ref_h2f": (f32, [u16]), "ref_f2h": (u16, [f32]),
        "ref_bf2f": (f32, [u16]), "ref_f2bf": (u16, [f32]),
        "ref_ru16": (u16, [f32]), "ref_rd16": (u16, [f32]),
        "ref_e4m3_decode": (f32, [u8]), "ref_e4m3_encode": (u8, [f32]),
        "ref_codec_qmax": (f32, [i32]),
        "ref_block_code_bytes": (sz, [i32]),
        "ref_scale_offset": (sz, [i32, sz]), "ref_zero_offset": (sz, [i32, sz]),
        "ref_wire_bytes": (sz, [i32, sz]),
        "ref_quantize_block": (None, [i32, P, i32, P, P, P]),
        "ref_dequant_code": (f32, [i32, ctypes.c_uint32, u16, u16]),
        "ref_quantize": (i32, [i32, i32, P, sz, P, sz, sz]),
        "ref_dequantize": (i32, [i32, i32, P, sz, P, sz, sz]),
        "ref_chunk": (None, [i32, sz, i32, P, P]),
        "ref_stage1": (i32, [i32, i32, i32, P, sz, P, sz, sz]),
        "ref_stage2": (i32, [i32, i32, i32, P, sz, P, sz, sz]),
        "ref_allreduce": (i32, [i32, i32, i32, P, P, sz, sz, sz]),
        "ref_oneshot": (i32, [i32, i32, P, P, sz, sz, sz]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _ptrs(arrs):
    return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])


def _check(rc, what):
    if rc != 0:
        raise ValueError("oracle %s failed (%d)" % (what, rc))


# -- scalar conversions -------------------------------------------------------
def h2f(h, L=None):
    return (L or lib()).ref_h2f(int(h))


def f2h(v, L=None):
    return (L or lib()).ref_f2h(float(v))


def bf2f(b, L=None):
    return (L or lib()).ref_bf2f(int(b))


def f2bf(v, L=None):
    return (L or lib()).ref_f2bf(float(v))


def ru16(v, L=None):
    return (L or lib()).ref_ru16(float(v))


def rd16(v, L=None):
    return (L or lib()).ref_rd16(float(v))


def e4m3_encode(t, L=None):
    return (L or lib()).ref_e4m3_encode(float(t))


def e4m3_decode(c, L=None):
    return (L or lib()).ref_e4m3_decode(int(c))


def qmax(codec, L=None):
    return (L or lib()).ref_codec_qmax(codec)


# -- layout --------------------------------------------------------------------
def wire_bytes(codec, n, L=None):
    return (L or lib()).ref_wire_bytes(codec, n)


def scale_offset(codec, n, L=None):
    return (L or lib()).ref_scale_offset(codec, n)


def zero_offset(codec, n, L=None):
    return (L or lib()).ref_zero_offset(codec, n)


def block_code_bytes(codec, L=None):
    return (L or lib()).ref_block_code_bytes(codec)


def chunk(W, n, j, L=None):
    lo, hi = ctypes.c_size_t(), ctypes.c_size_t()
    (L or lib()).ref_chunk(W, n, j, ctypes.byref(lo), ctypes.byref(hi))
    return lo.value, hi.value


# -- one block -----------------------------------------------------------------
def quantize_block(codec, v, L=None):
    """Quantize up to 32 binary32 values; returns (codes[32] uint32, s, z)."""
    v = np.ascontiguousarray(v, dtype=np.float32)
    assert 1 <= v.size <= BLK
    codes = np.zeros(BLK, np.uint32)
    s, z = ctypes.c_uint16(), ctypes.c_uint16()
    (L or lib()).ref_quantize_block(codec, _p(v), v.size, _p(codes),
                                    ctypes.byref(s), ctypes.byref(z))
    return codes, s.value, z.value


def dequant_code(codec, code, s, z=0, L=None):
    return (L or lib()).ref_dequant_code(codec, int(code), int(s), int(z))


# -- the pipeline ----------------------------------------------------------------
def quantize(codec, dtype, x, lo=0, hi=ALL, wire=None, L=None):
    x = np.ascontiguousarray(x, dtype=np.uint16)
    if wire is None:
        wire = np.zeros(wire_bytes(codec, x.size, L), np.uint8)
    _check((L or lib()).ref_quantize(codec, dtype, _p(x), x.size, _p(wire), lo, hi),
           "quantize")
    return wire


def dequantize(codec, dtype, wire, n, lo=0, hi=ALL, y=None, L=None):
    wire = np.ascontiguousarray(wire, dtype=np.uint8)
    if y is None:
        y = np.zeros(n, np.uint16)
    _check((L or lib()).ref_dequantize(codec, dtype, _p(wire), n, _p(y), lo, hi),
           "dequantize")
    return y


def stage1(codec, dtype, wires, n, lo=0, hi=ALL, reduced=None, L=None):
    wires = [np.ascontiguousarray(w, dtype=np.uint8) for w in wires]
    if reduced is None:
        reduced = np.zeros(wire_bytes(codec, n, L), np.uint8)
    _check((L or lib()).ref_stage1(codec, dtype, len(wires), _ptrs(wires), n,
                                   _p(reduced), lo, hi), "stage1")
    return reduced


def stage2(codec, dtype, W, reduced, n, lo=0, hi=ALL, L=None):
    reduced = np.ascontiguousarray(reduced, dtype=np.uint8)
    ys = [np.zeros(n, np.uint16) for _ in range(W)]
    _check((L or lib()).ref_stage2(codec, dtype, W, _p(reduced), n, _ptrs(ys),
                                   lo, hi), "stage2")
    return ys


def allreduce(codec, dtype, xs, lo=0, hi=ALL, ys=None, L=None):
    xs = [np.ascontiguousarray(x, dtype=np.uint16) for x in xs]
    n = xs[0].size
    if ys is None:
        ys = [np.zeros(n, np.uint16) for _ in xs]
    _check((L or lib()).ref_allreduce(len(xs), dtype, codec, _ptrs(xs), _ptrs(ys),
                                      n, lo, hi), "allreduce")
    return ys


def oneshot(dtype, xs, lo=0, hi=ALL, ys=None, L=None):
    """The one-stage (one-shot) FP allreduce of W raw buffers."""
    xs = [np.ascontiguousarray(x, dtype=np.uint16) for x in xs]
    n = xs[0].size
    if ys is None:
        ys = [np.zeros(n, np.uint16) for _ in xs]
    _check((L or lib()).ref_oneshot(len(xs), dtype, _ptrs(xs), _ptrs(ys), n, lo, hi),
           "oneshot")
    return ys
