"""The C-ABI library on the host (no GPU needed): it loads, exports every
function include/qr.h declares, sizes wire images and workspaces as the wire
definition says, and rejects every invalid argument with the documented code
before anything is launched (the pointers below are fake, never touched)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qr.h")


def _lib():
    from quantized_two_stage_amd import qr
    return qr


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qr_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("qr_quantize", "qr_dequantize", "qr_reduce_stage1", "qr_gather_stage2",
                 "qr_allreduce_sim", "qr_wire_bytes", "qr_sim_workspace_bytes",
                 "qr_last_error", "qr_quantize_ranks", "qr_allreduce_oneshot",
                 "qr_recv_bytes", "qr_quantize_recv", "qr_reduce_recv",
                 "qr_allreduce_sim_noalloc"):
        assert must in names


def test_library_exports_every_declared_symbol():
    qr = _lib()
    for name in declared_functions():
        assert hasattr(qr.LIB, name), name
        assert name in qr.EXPORTS, name
    # the binding exposes each under the same name
    for name in declared_functions():
        assert callable(getattr(qr, name)), name


def test_wire_bytes_matches_definition():
    qr = _lib()
    n = 32 * 1024 * 1024
    want = {qr.QR_FP: 67108864, qr.QR_FP8: 35651584, qr.QR_Q8: 35651584,
            qr.QR_Q8_ASYM: 37748736, qr.QR_Q6: 27262976, qr.QR_Q6_ASYM: 29360128,
            qr.QR_Q4: 18874368, qr.QR_Q4_ASYM: 20971520}
    for c, w in want.items():
        assert qr.qr_wire_bytes(c, n) == w
    assert qr.qr_wire_bytes(qr.QR_Q8, 2048) == 2176
    assert qr.qr_wire_bytes(qr.QR_Q4_ASYM, 2048) == 1408
    assert qr.qr_wire_bytes(qr.QR_Q4, 40) == 260
    assert qr.qr_wire_bytes(4, 2048) == 0                     # NONE is not a codec
    # receive buffer: one tile of 256 blocks per rank (256 * (32 + 2) bytes),
    # then the reduced image at the next 256-byte boundary
    assert qr.qr_recv_bytes(2, qr.QR_Q8, 2048) == 2 * 256 * 34
    assert qr.qr_recv_bytes(8, qr.QR_Q4_ASYM, n) == (n // 32 // 256) * 8 * 256 * 20
    assert qr.qr_recv_bytes(4, qr.QR_FP, 8192 * 3 + 8) == 4 * 4 * 256 * 64
    assert qr.qr_sim_workspace_bytes(2, qr.QR_Q8, 2048) == 2 * 256 * 34 + 2304
    assert qr.qr_sim_workspace_bytes(3, qr.QR_Q8, 2048) == 0


def test_wire_bytes_agree_with_oracle():
    import oracle
    qr = _lib()
    for c in qr.CODECS:
        for n in (8, 16, 24, 32, 40, 2048, 2056, 8192 * 3 + 8, 1 << 20):
            assert qr.qr_wire_bytes(c, n) == oracle.wire_bytes(c, n), (c, n)


FAKE = 0x7f0000000000          # 16-byte aligned, never dereferenced


def _pp(vals):
    return (ctypes.c_void_p * len(vals))(*vals)


def _call_sim(W=2, dtype=0, codec=1, xs=None, ys=None, n=2048, ws=None, ws_bytes=None):
    qr = _lib()
    xs = xs if xs is not None else [FAKE + i * 0x100000 for i in range(W)]
    ys = ys if ys is not None else [FAKE + 0x10000000 + i * 0x100000 for i in range(W)]
    ws = FAKE + 0x40000000 if ws is None else ws
    need = qr.qr_sim_workspace_bytes(max(W, 2) if W in (2, 4, 8) else 2, codec
                                     if codec in qr.CODECS else 1, n)
    ws_bytes = need if ws_bytes is None else ws_bytes
    return qr.LIB.qr_allreduce_sim(W, dtype, codec, _pp(xs), _pp(ys), n,
                                   ctypes.c_void_p(ws), ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=3), -2), (dict(W=1), -2), (dict(W=16), -2),
    (dict(dtype=3), -2), (dict(codec=4), -2), (dict(codec=7), -2), (dict(codec=12), -2),
    (dict(n=0), -3), (dict(n=2044), -3), (dict(n=(1 << 30) + 8), -3),
    (dict(ws_bytes=100), -5),
    (dict(xs=[FAKE + 4, FAKE + 0x100000]), -4),
    (dict(ys=[FAKE + 0x10000000, FAKE + 0x10000008]), -4),
    (dict(ws=FAKE + 0x40000008), -4),
    (dict(xs=[0, FAKE + 0x100000]), -1),
    (dict(ws=0), -1),
    (dict(ys=[FAKE, FAKE + 0x10000000]), -1),               # y aliases x
    (dict(ys=[FAKE + 0x10000000, FAKE + 0x10000000]), -1),  # two ys alias
    (dict(ws=FAKE), -1),                                   # workspace over x
])
def test_allreduce_sim_rejects(kw, code):
    qr = _lib()
    assert _call_sim(**kw) == code
    assert qr.LIB.qr_last_error().decode() != ""


def test_stage_entry_points_reject():
    qr = _lib()
    L = qr.LIB
    P = ctypes.c_void_p
    a, b = P(FAKE), P(FAKE + 0x1000000)
    # quantize / dequantize
    assert L.qr_quantize(4, 0, a, 2048, b, None) == -2
    assert L.qr_quantize(1, 0, a, 2047, b, None) == -3
    assert L.qr_quantize(1, 0, P(FAKE + 8), 2048, b, None) == -4
    assert L.qr_quantize(1, 0, a, 2048, P(0), None) == -1
    assert L.qr_quantize(1, 0, a, 2048, P(FAKE + 1024), None) == -1   # overlap
    assert L.qr_dequantize(1, 1, a, 2048, P(FAKE + 0x10), None) == -1  # overlap
    assert L.qr_dequantize(1, 3, a, 2048, b, None) == -2
    # stage 1
    w2 = _pp([FAKE, FAKE + 0x1000000])
    assert L.qr_reduce_stage1(1, 0, 2, w2, 2048, 2, P(FAKE + 0x2000000), None) == -1
    assert L.qr_reduce_stage1(1, 0, 2, w2, 2048, -2, P(FAKE + 0x2000000), None) == -1
    assert L.qr_reduce_stage1(1, 0, 3, _pp([FAKE] * 3), 2048, -1, P(FAKE + 0x2000000),
                              None) == -2
    assert L.qr_reduce_stage1(1, 0, 2, w2, 2048, -1, P(FAKE + 0x1000010), None) == -1
    assert L.qr_reduce_stage1(1, 0, 2, None, 2048, -1, P(FAKE + 0x2000000), None) == -1
    # stage 2 and batched quantize
    assert L.qr_gather_stage2(1, 0, 0, a, 2048, _pp([FAKE + 0x1000000]), None) == -2
    assert L.qr_gather_stage2(1, 0, 9, a, 2048, _pp([FAKE] * 9), None) == -2
    assert L.qr_gather_stage2(1, 0, 2, a, 2048, _pp([FAKE + 0x1000000] * 2), None) == -1
    assert L.qr_quantize_ranks(1, 0, 2, _pp([FAKE, FAKE + 0x1000]), 2048,
                               _pp([FAKE + 0x2000000, FAKE + 0x2000010]), None) == -1
    assert "overlap" in L.qr_last_error().decode()


def _call_oneshot(W=2, dtype=0, xs=None, ys=None, n=2048):
    qr = _lib()
    xs = xs if xs is not None else [FAKE + i * 0x100000 for i in range(W)]
    ys = ys if ys is not None else [FAKE + 0x10000000 + i * 0x100000 for i in range(W)]
    return qr.LIB.qr_allreduce_oneshot(W, dtype, _pp(xs), _pp(ys), n, None)


@pytest.mark.parametrize("kw,code", [
    (dict(W=3), -2), (dict(W=1), -2), (dict(W=16), -2), (dict(dtype=3), -2),
    (dict(n=0), -3), (dict(n=2044), -3), (dict(n=(1 << 30) + 8), -3),
    (dict(xs=[FAKE + 4, FAKE + 0x100000]), -4),
    (dict(ys=[FAKE + 0x10000000, FAKE + 0x10000008]), -4),
    (dict(xs=[0, FAKE + 0x100000]), -1),
    (dict(ys=[FAKE + 0x100000 + 16, FAKE + 0x10000000]), -1),  # y overlaps x
    (dict(ys=[FAKE + 0x10000000, FAKE + 0x10000000]), -1),     # two ys alias
])
def test_allreduce_oneshot_rejects(kw, code):
    qr = _lib()
    assert _call_oneshot(**kw) == code
    assert qr.LIB.qr_last_error().decode() != ""
    assert qr.LIB.qr_allreduce_oneshot(2, 0, None, _pp([FAKE, FAKE]), 2048, None) == -1


def test_allreduce_sim_noalloc_rejects():
    """The entry point without a workspace: the argument checks of
    qr_allreduce_sim, then QR_ERR_WORKSPACE for a workspace beyond the
    library's buffer, all before any GPU call."""
    qr = _lib()
    L = qr.LIB
    xs = _pp([FAKE, FAKE + 0x10000000])
    ys = _pp([FAKE + 0x20000000, FAKE + 0x30000000])
    assert qr.QR_SCRATCH_BYTES == 64 << 20
    n = 8
    while qr.qr_sim_workspace_bytes(2, qr.QR_FP, n + 8) <= qr.QR_SCRATCH_BYTES:
        n += 8
    assert n == (64 << 20) // 3 // 2 // 256 * 256 // 8 * 8 or n > 0
    assert L.qr_allreduce_sim_noalloc(2, 0, qr.QR_FP, xs, ys, n + 8, None) == -5
    assert "workspace" in L.qr_last_error().decode()
    assert L.qr_allreduce_sim_noalloc(8, 0, qr.QR_Q8_ASYM, _pp([FAKE + i * 0x10000000
                                                              for i in range(8)]),
                                      _pp([FAKE + (8 + i) * 0x10000000 for i in range(8)]),
                                      1 << 24, None) == -5
    assert L.qr_allreduce_sim_noalloc(3, 0, qr.QR_Q4, xs, ys, 64, None) == -2
    assert L.qr_allreduce_sim_noalloc(2, 0, 4, xs, ys, 64, None) == -2
    assert L.qr_allreduce_sim_noalloc(2, 0, qr.QR_Q4, xs, ys, 12, None) == -3
    assert L.qr_allreduce_sim_noalloc(2, 0, qr.QR_Q4, xs, xs, 64, None) == -1
    assert L.qr_allreduce_sim_noalloc(2, 0, qr.QR_Q4, None, ys, 64, None) == -1
    assert L.qr_allreduce_sim_noalloc(2, 0, qr.QR_Q4, _pp([FAKE + 4, FAKE + 0x10000000]), ys,
                                      64, None) == -4


def test_last_error_is_per_thread():
    """each host thread reads back its own last error: two threads fail with
    different errors, meet at a barrier, then each reads its message"""
    import threading
    qr = _lib()
    bar = threading.Barrier(2)
    got = {}

    def run(name, kw):
        code = _call_sim(**kw)
        bar.wait()                       # both calls have failed before either reads
        got[name] = (code, qr.LIB.qr_last_error().decode())

    ts = [threading.Thread(target=run, args=("w", dict(W=3))),
          threading.Thread(target=run, args=("n", dict(n=0)))]
    for t in ts:
        t.start()
    for t in ts:
        t.join()
    assert got["w"][0] == -2 and "W = 3" in got["w"][1], got
    assert got["n"][0] == -3 and "n must be > 0" in got["n"][1], got


def test_binding_refuses_tensors_the_kernels_would_overrun():
    """the Python binding checks what only the tensors know, before any call:
    as many outputs as inputs, enough bytes behind every pointer, contiguous
    memory, device memory (CPU tensors here: each check fires before any
    library call)"""
    import torch
    qr = _lib()
    n, W, c = 4096, 2, qr.QR_Q4
    xs = [torch.zeros(n, dtype=torch.float16) for _ in range(W)]
    ys = [torch.zeros(n, dtype=torch.float16) for _ in range(W)]
    ws = torch.zeros(qr.qr_sim_workspace_bytes(W, c, n), dtype=torch.uint8)
    wire = torch.zeros(qr.qr_wire_bytes(c, n), dtype=torch.uint8)
    cases = [
        (lambda: qr.qr_allreduce_sim(c, xs, ys[:1], ws), "2 inputs but 1 outputs"),
        (lambda: qr.qr_allreduce_sim(c, xs, [ys[0], ys[1][:n - 8]], ws), "ys[1] holds"),
        (lambda: qr.qr_allreduce_sim(c, [xs[0], torch.zeros(2 * n, dtype=torch.float16)[::2]],
                                     ys, ws), "xs[1] is not contiguous"),
        (lambda: qr.qr_allreduce_sim(c, xs, ys, ws), "not in GPU memory"),
        (lambda: qr.qr_allreduce_oneshot(xs, ys[:1]), "2 inputs but 1 outputs"),
        (lambda: qr.qr_quantize(c, xs[0], wire[:-1]), "wire[0] holds"),
        (lambda: qr.qr_dequantize(c, wire[:-2], ys[0]), "wire[0] holds"),
        (lambda: qr.qr_quantize_ranks(c, xs, [wire]), "2 inputs but 1 wire images"),
        (lambda: qr.qr_reduce_stage1(c, [wire, wire], n, wire[:100], 0), "reduced[0] holds"),
        (lambda: qr.qr_gather_stage2(c, wire, [ys[0], ys[1][:10]]), "ys[1] holds"),
    ]
    for call, msg in cases:
        with pytest.raises(ValueError) as e:
            call()
        assert msg in str(e.value), (msg, str(e.value))


def test_pattern_library_exports_its_header_and_rejects():
    """libqr_pattern.so (the stage-1 access pattern the benchmark times) loads,
    exports every function include/qr_pattern.h declares, and refuses invalid
    arguments with -1 before launching (fake pointers, never touched)."""
    from quantized_two_stage_amd import build as qbuild
    src = open(os.path.join(ROOT, "include", "qr_pattern.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = sorted(set(re.findall(r"\b(qrp_[a-z0-9_]+)\s*\(", src)))
    assert names == ["qrp_stage1_pattern", "qrp_stream"]
    L = ctypes.CDLL(qbuild.PATTERN_LIB)
    for name in names:
        assert hasattr(L, name), name
    f = L.qrp_stage1_pattern
    f.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t,
                  ctypes.c_void_p, ctypes.c_void_p]
    f.restype = ctypes.c_int
    good = dict(codec=3, W=8, recv=1 << 20, n=1 << 10, red=1 << 24)
    bad = [dict(codec=4), dict(codec=12), dict(W=3), dict(W=1), dict(n=0), dict(n=12),
           dict(recv=0), dict(red=0), dict(recv=(1 << 20) + 8), dict(red=(1 << 24) + 4),
           dict(n=1 << 30)]        # offsets beyond 32 bits at W=8
    for b in bad:
        a = dict(good, **b)
        assert f(a["codec"], a["W"], a["recv"], a["n"], a["red"], None) == -1, b
    g = L.qrp_stream
    g.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_size_t, ctypes.c_void_p]
    g.restype = ctypes.c_int
    good = dict(kind=2, k=4, nt=1, src=1 << 20, dst=1 << 24, nbytes=1 << 20)
    bad = [dict(kind=3), dict(kind=-1), dict(k=2), dict(k=0), dict(nt=2), dict(nbytes=0),
           dict(nbytes=48), dict(nbytes=(1 << 36) + 32), dict(dst=0), dict(dst=(1 << 24) + 8),
           dict(src=0), dict(src=(1 << 20) + 4), dict(kind=0, src=0)]
    for b in bad:
        a = dict(good, **b)
        assert g(a["kind"], a["k"], a["nt"], a["src"], a["dst"], a["nbytes"], None) == -1, b
