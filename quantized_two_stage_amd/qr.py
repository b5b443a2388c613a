"""Python binding of the C ABI in include/qr.h (argument marshalling only).

Every function has the name of the C entry point it calls and takes torch
tensors on the GPU; all work happens in libqr.so's HIP kernels, on the current
torch stream unless `stream` is given.  There is no other implementation: if
libqr.so is missing this module raises on import.  Since the C ABI sees only
pointers, each function first checks what only the tensors know (enough
bytes behind every pointer, contiguous, in device memory, as many outputs as
inputs) and raises ValueError before any call.
"""
import ctypes
import os

import torch

QR_FP, QR_Q8, QR_Q6, QR_Q4, QR_FP8 = 0, 1, 2, 3, 5
QR_Q8_ASYM, QR_Q6_ASYM, QR_Q4_ASYM = 9, 10, 11
QR_FP16, QR_BF16, QR_BF16_VIA_FP16 = 0, 1, 2
CODECS = (QR_FP, QR_FP8, QR_Q8, QR_Q6, QR_Q4, QR_Q8_ASYM, QR_Q6_ASYM, QR_Q4_ASYM)
CODEC_NAMES = {QR_FP: "fp", QR_Q8: "q8", QR_Q6: "q6", QR_Q4: "q4", QR_FP8: "fp8",
               QR_Q8_ASYM: "q8a", QR_Q6_ASYM: "q6a", QR_Q4_ASYM: "q4a"}
ERRORS = {-1: "QR_ERR_ARG", -2: "QR_ERR_UNSUPPORTED", -3: "QR_ERR_SIZE",
          -4: "QR_ERR_ALIGN", -5: "QR_ERR_WORKSPACE", -6: "QR_ERR_HIP"}
QR_MAX_BYTES = 1 << 31
QR_SCRATCH_BYTES = 64 << 20

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libqr.so")


class QRError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__("%s (%d): %s" % (ERRORS.get(code, "?"), code, msg))
        self.code = code


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libqr.so is not built (%s); run "
                          "quantized_two_stage_amd/build.py" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    sz, i32, P = ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p
    PP = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "qr_wire_bytes": (sz, [i32, sz]),
        "qr_sim_workspace_bytes": (sz, [i32, i32, sz]),
        "qr_recv_bytes": (sz, [i32, i32, sz]),
        "qr_quantize_recv": (i32, [i32, i32, i32, PP, sz, P, P]),
        "qr_reduce_recv": (i32, [i32, i32, i32, P, sz, i32, P, P]),
        "qr_quantize": (i32, [i32, i32, P, sz, P, P]),
        "qr_dequantize": (i32, [i32, i32, P, sz, P, P]),
        "qr_quantize_ranks": (i32, [i32, i32, i32, PP, sz, PP, P]),
        "qr_reduce_stage1": (i32, [i32, i32, i32, PP, sz, i32, P, P]),
        "qr_gather_stage2": (i32, [i32, i32, i32, P, sz, PP, P]),
        "qr_allreduce_sim": (i32, [i32, i32, i32, PP, PP, sz, P, sz, P]),
        "qr_allreduce_oneshot": (i32, [i32, i32, PP, PP, sz, P]),
        "qr_allreduce_sim_noalloc": (i32, [i32, i32, i32, PP, PP, sz, P]),
        "qr_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    return L


LIB = _load()
EXPORTS = ("qr_wire_bytes", "qr_sim_workspace_bytes", "qr_recv_bytes", "qr_quantize",
           "qr_dequantize", "qr_quantize_ranks", "qr_quantize_recv", "qr_reduce_stage1",
           "qr_reduce_recv", "qr_gather_stage2",
           "qr_allreduce_sim", "qr_allreduce_oneshot", "qr_allreduce_sim_noalloc",
           "qr_last_error")


def _check(rc):
    if rc != 0:
        raise QRError(rc, LIB.qr_last_error().decode())


def _dtype_of(t, dtype):
    if dtype is not None:
        return dtype
    if t.dtype == torch.float16:
        return QR_FP16
    if t.dtype == torch.bfloat16:
        return QR_BF16
    raise TypeError("pass dtype= for a %s buffer" % t.dtype)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _ptrs(ts):
    return (ctypes.c_void_p * len(ts))(*[t.data_ptr() for t in ts])


def _n16(t):
    return t.numel() * t.element_size() // 2


def _nbytes(t):
    return t.numel() * t.element_size()


def _bufs(*groups):
    """The C ABI sees only pointers: refuse, before any call, a tensor the
    kernels would run past (too small or not contiguous) or one not in
    device memory.  groups: (name, tensors, bytes each must hold)."""
    for what, ts, need in groups:
        for i, t in enumerate(ts):
            if not t.is_contiguous():
                raise ValueError("%s[%d] is not contiguous" % (what, i))
            if _nbytes(t) < need:
                raise ValueError("%s[%d] holds %d bytes, %d needed" % (what, i, _nbytes(t),
                                                                       need))
    for what, ts, _ in groups:
        for i, t in enumerate(ts):
            if not t.is_cuda:
                raise ValueError("%s[%d] is not in GPU memory" % (what, i))


def _same_count(xs, ys, a, b):
    if len(xs) != len(ys):
        raise ValueError("%d %s but %d %s" % (len(xs), a, len(ys), b))


def qr_last_error():
    return LIB.qr_last_error().decode()


def qr_wire_bytes(codec, n):
    return LIB.qr_wire_bytes(codec, n)


def qr_sim_workspace_bytes(W, codec, n):
    return LIB.qr_sim_workspace_bytes(W, codec, n)


def qr_recv_bytes(W, codec, n):
    return LIB.qr_recv_bytes(W, codec, n)


def qr_quantize(codec, x, wire, dtype=None, stream=None):
    n = _n16(x)
    _bufs(("x", [x], 2 * n), ("wire", [wire], qr_wire_bytes(codec, n)))
    _check(LIB.qr_quantize(codec, _dtype_of(x, dtype), _ptr(x), _n16(x), _ptr(wire),
                           _stream(stream)))
    return wire


def qr_dequantize(codec, wire, y, dtype=None, stream=None):
    n = _n16(y)
    _bufs(("wire", [wire], qr_wire_bytes(codec, n)), ("y", [y], 2 * n))
    _check(LIB.qr_dequantize(codec, _dtype_of(y, dtype), _ptr(wire), _n16(y), _ptr(y),
                             _stream(stream)))
    return y


def qr_quantize_ranks(codec, xs, wires, dtype=None, stream=None):
    _same_count(xs, wires, "inputs", "wire images")
    n = _n16(xs[0])
    _bufs(("xs", xs, 2 * n), ("wires", wires, qr_wire_bytes(codec, n)))
    _check(LIB.qr_quantize_ranks(codec, _dtype_of(xs[0], dtype), len(xs), _ptrs(xs),
                                 _n16(xs[0]), _ptrs(wires), _stream(stream)))
    return wires


def qr_quantize_recv(codec, xs, recv, dtype=None, stream=None):
    """stage 0 of W ranks into one receive buffer (qr_recv_bytes bytes)"""
    n = _n16(xs[0])
    _bufs(("xs", xs, 2 * n), ("recv", [recv], qr_recv_bytes(len(xs), codec, n)))
    _check(LIB.qr_quantize_recv(codec, _dtype_of(xs[0], dtype), len(xs), _ptrs(xs), n,
                                _ptr(recv), _stream(stream)))
    return recv


def qr_reduce_recv(codec, W, recv, n, reduced, dtype, owner=-1, stream=None):
    """stage 1 of W ranks from a receive buffer"""
    _bufs(("recv", [recv], qr_recv_bytes(W, codec, n)),
          ("reduced", [reduced], qr_wire_bytes(codec, n)))
    _check(LIB.qr_reduce_recv(codec, dtype, W, _ptr(recv), n, owner, _ptr(reduced),
                              _stream(stream)))
    return reduced


def qr_reduce_stage1(codec, wires, n, reduced, dtype, owner=-1, stream=None):
    _bufs(("wires", wires, qr_wire_bytes(codec, n)),
          ("reduced", [reduced], qr_wire_bytes(codec, n)))
    _check(LIB.qr_reduce_stage1(codec, dtype, len(wires), _ptrs(wires), n, owner,
                                _ptr(reduced), _stream(stream)))
    return reduced


def qr_gather_stage2(codec, reduced, ys, dtype=None, stream=None):
    n = _n16(ys[0])
    _bufs(("reduced", [reduced], qr_wire_bytes(codec, n)), ("ys", ys, 2 * n))
    _check(LIB.qr_gather_stage2(codec, _dtype_of(ys[0], dtype), len(ys), _ptr(reduced),
                                _n16(ys[0]), _ptrs(ys), _stream(stream)))
    return ys


def qr_allreduce_sim(codec, xs, ys, workspace, dtype=None, stream=None):
    """ys[r] = the simulated two-stage allreduce of xs (out-of-place)."""
    _same_count(xs, ys, "inputs", "outputs")
    n = _n16(xs[0])
    # the workspace's size is passed to the call, which checks it
    _bufs(("xs", xs, 2 * n), ("ys", ys, 2 * n), ("workspace", [workspace], 0))
    ws_bytes = _nbytes(workspace)
    _check(LIB.qr_allreduce_sim(len(xs), _dtype_of(xs[0], dtype), codec, _ptrs(xs),
                                _ptrs(ys), n, _ptr(workspace), ws_bytes, _stream(stream)))
    return ys


def qr_allreduce_sim_noalloc(codec, xs, ys, dtype=None, stream=None):
    """qr_allreduce_sim with the library's own workspace buffer: allocates
    nothing (for callers that cannot); calls on one GPU must not overlap."""
    _same_count(xs, ys, "inputs", "outputs")
    n = _n16(xs[0])
    _bufs(("xs", xs, 2 * n), ("ys", ys, 2 * n))
    _check(LIB.qr_allreduce_sim_noalloc(len(xs), _dtype_of(xs[0], dtype), codec, _ptrs(xs),
                                        _ptrs(ys), n, _stream(stream)))
    return ys


def qr_allreduce_oneshot(xs, ys, dtype=None, stream=None):
    """ys[r] = the one-stage allreduce of xs: every rank sums all W buffers."""
    _same_count(xs, ys, "inputs", "outputs")
    n = _n16(xs[0])
    _bufs(("xs", xs, 2 * n), ("ys", ys, 2 * n))
    _check(LIB.qr_allreduce_oneshot(len(xs), _dtype_of(xs[0], dtype), _ptrs(xs), _ptrs(ys),
                                    _n16(xs[0]), _stream(stream)))
    return ys


def alloc_wire(codec, n, device="cuda"):
    """A device buffer for one wire image (padding bytes start at zero)."""
    return torch.zeros(qr_wire_bytes(codec, n), dtype=torch.uint8, device=device)


def alloc_recv(W, codec, n, device="cuda"):
    """A device buffer for a receive buffer (padding bytes start at zero)."""
    return torch.zeros(qr_recv_bytes(W, codec, n), dtype=torch.uint8, device=device)


def alloc_workspace(W, codec, n, device="cuda"):
    return torch.empty(qr_sim_workspace_bytes(W, codec, n), dtype=torch.uint8,
                       device=device)
