// qr_api.cpp -- the extern "C" entry points declared in include/qr.h.
//
// Everything here runs on the host: argument checks (done before anything is
// launched, so a rejected call writes nothing), the wire layout, and the
// kernel launches of qr_kernels.hip.  The library keeps no state between
// calls other than the text of the last error (per thread) and, once
// qr_allreduce_sim_noalloc has run on a GPU, the address of that GPU's
// workspace buffer.
#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>

#include "qr.h"
#include "qr_internal.h"

namespace qr {

bool codec_valid(int c) {
  return c == QR_FP || c == QR_Q8 || c == QR_Q6 || c == QR_Q4 || c == QR_FP8 ||
         c == QR_Q8_ASYM || c == QR_Q6_ASYM || c == QR_Q4_ASYM;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int code_bits(int c) {
  switch (c & 7) {
    case QR_Q6: return 6;
    case QR_Q4: return 4;
    default: return 8;     // Q8, FP8
  }
}

Layout make_layout(int codec, size_t n) {
  Layout L;
  L.n = n;
  L.nb = (n + 31) / 32;
  L.nslices = 2 * L.nb;
  L.ntiles = (L.nb + kTileBlocks - 1) / kTileBlocks;
  if (codec == QR_FP) {
    L.code_bytes = 2 * n;
    L.total = 2 * n;
    L.tile_bytes = (size_t)kTileBlocks * 64;
    return L;
  }
  const size_t cb = (size_t)(32 * code_bits(codec) / 8);
  L.code_bytes = L.nb * cb;
  L.off_s = align256(L.code_bytes);
  L.total = L.off_s + 2 * L.nb;
  if (codec & 8) {
    L.off_z = align256(L.total);
    L.total = L.off_z + 2 * L.nb;
  }
  L.tile_bytes = (size_t)kTileBlocks * (cb + 2 + ((codec & 8) ? 2 : 0));
  return L;
}

}  // namespace qr

// qr_allreduce_sim runs its three stages as one launch (each workgroup
// carrying its tile of blocks through all three) up to this many bytes per
// rank buffer, and as three launches above.  Measured on MI355X: up to 4 MiB
// the single launch halves the time of a call (about 4.5-6 us instead of
// 9-11 us at W = 2, 4 and 8); above, the launches are no longer the cost.
#ifndef QR_FUSED_MAX_BYTES
#define QR_FUSED_MAX_BYTES ((size_t)4 << 20)
#endif

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = 0;
  return QR_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(QR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool w_sim(int W) { return W == 2 || W == 4 || W == 8; }

int check_kind(int codec, int dtype, size_t n) {
  if (!qr::codec_valid(codec))
    return fail(QR_ERR_UNSUPPORTED, "unsupported codec %d", codec);
  if (dtype != QR_FP16 && dtype != QR_BF16 && dtype != QR_BF16_VIA_FP16)
    return fail(QR_ERR_UNSUPPORTED, "unsupported dtype %d", dtype);
  if (n == 0) return fail(QR_ERR_SIZE, "n must be > 0");
  if (n % 8 != 0)
    return fail(QR_ERR_SIZE, "n = %zu: the byte size must be a multiple of 16", n);
  if (n > QR_MAX_BYTES / 2)
    return fail(QR_ERR_SIZE, "n = %zu exceeds QR_MAX_BYTES", n);
  return QR_OK;
}

int check_ptr(const void* p, const char* what, int idx) {
  if (p == nullptr) return fail(QR_ERR_ARG, "%s[%d] is NULL", what, idx);
  if (((uintptr_t)p & 15u) != 0)
    return fail(QR_ERR_ALIGN, "%s[%d] is not 16-byte aligned", what, idx);
  return QR_OK;
}

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

#define QR_TRY(expr)          \
  do {                        \
    int rc_ = (expr);         \
    if (rc_ != QR_OK) return rc_; \
  } while (0)

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// outputs must be pairwise disjoint and disjoint from every input
int check_disjoint(const void* const* ins, int nin, size_t in_bytes,
                   const void* const* outs, int nout, size_t out_bytes) {
  for (int i = 0; i < nout; i++) {
    for (int j = 0; j < nin; j++)
      if (overlap(outs[i], out_bytes, ins[j], in_bytes))
        return fail(QR_ERR_ARG, "output %d overlaps input %d", i, j);
    for (int j = 0; j < i; j++)
      if (overlap(outs[i], out_bytes, outs[j], out_bytes))
        return fail(QR_ERR_ARG, "outputs %d and %d overlap", j, i);
  }
  return QR_OK;
}

// arguments of the simulated allreduce other than its workspace
int check_sim(int W, int dtype, int codec, const void* const* xs, void* const* ys, size_t n) {
  QR_TRY(check_kind(codec, dtype, n));
  if (!w_sim(W)) return fail(QR_ERR_UNSUPPORTED, "W = %d not in {2,4,8}", W);
  if (xs == nullptr || ys == nullptr) return fail(QR_ERR_ARG, "NULL pointer array");
  for (int r = 0; r < W; r++) {
    QR_TRY(check_ptr(xs[r], "xs", r));
    QR_TRY(check_ptr(ys[r], "ys", r));
  }
  return check_disjoint(xs, W, 2 * n, (const void* const*)ys, W, 2 * n);
}

int check_workspace_disjoint(int W, const void* const* xs, void* const* ys, size_t n,
                             const void* ws, size_t need) {
  for (int r = 0; r < W; r++) {
    if (overlap(ws, need, xs[r], 2 * n)) return fail(QR_ERR_ARG, "workspace overlaps xs[%d]", r);
    if (overlap(ws, need, ys[r], 2 * n)) return fail(QR_ERR_ARG, "workspace overlaps ys[%d]", r);
  }
  return QR_OK;
}

// rank r's base pointer in a receive buffer: the start of its first tile
void recv_ptrs(uint8_t* recv, int W, const qr::Layout& L, qr::OutPtrs& out, qr::InPtrs& in) {
  for (int r = 0; r < W; r++) {
    out.p[r] = recv + (size_t)r * L.tile_bytes;
    in.p[r] = out.p[r];
  }
}

// the launches of the simulated allreduce, arguments already checked: the
// receive buffer at the start of `ws`, the reduced image at the next
// 256-byte boundary after it
int run_sim(int W, int dtype, int codec, const void* const* xs, void* const* ys, size_t n,
            uint8_t* ws, hipStream_t st) {
  const qr::Layout L = qr::make_layout(codec, n);
  qr::InPtrs in{}, wires_in{};
  qr::OutPtrs wires_out{}, out{};
  recv_ptrs(ws, W, L, wires_out, wires_in);
  for (int r = 0; r < W; r++) {
    in.p[r] = static_cast<const uint8_t*>(xs[r]);
    out.p[r] = static_cast<uint8_t*>(ys[r]);
  }
  uint8_t* reduced = ws + qr::align256(L.recv_bytes(W));
  (void)hipGetLastError();
  if (2 * n <= QR_FUSED_MAX_BYTES)
    return hip_status(qr::launch_fused(codec, dtype, W, in, wires_out, reduced, out, L, st),
                      "fused launch");
  QR_TRY(hip_status(qr::launch_quantize(codec, dtype, W, in, wires_out, true, L, st),
                    "quantize launch"));
  QR_TRY(hip_status(qr::launch_stage1(codec, dtype, W, wires_in, true, reduced, 0, L.nb, L,
                                      st),
                    "stage-1 launch"));
  return hip_status(qr::launch_dequantize(codec, dtype, W, reduced, out, L, st),
                    "stage-2 launch");
}

// owner j's blocks [j*bpc, min(nb, (j+1)*bpc)), bpc = ceil(nb/W); all blocks for -1
void owner_range(int W, int owner, const qr::Layout& L, size_t& lo, size_t& hi) {
  lo = 0;
  hi = L.nb;
  if (owner >= 0) {
    const size_t bpc = (L.nb + W - 1) / W;
    lo = (size_t)owner * bpc < L.nb ? (size_t)owner * bpc : L.nb;
    hi = lo + bpc < L.nb ? lo + bpc : L.nb;
  }
}

}  // namespace

extern "C" {

size_t qr_wire_bytes(qr_codec codec, size_t n) {
  if (!qr::codec_valid(codec)) return 0;
  return qr::make_layout(codec, n).total;
}

size_t qr_recv_bytes(int W, qr_codec codec, size_t n) {
  if (W < 1 || W > qr::kMaxRanks || !qr::codec_valid(codec)) return 0;
  return qr::make_layout(codec, n).recv_bytes(W);
}

size_t qr_sim_workspace_bytes(int W, qr_codec codec, size_t n) {
  if (!w_sim(W) || !qr::codec_valid(codec)) return 0;
  const qr::Layout L = qr::make_layout(codec, n);
  return qr::align256(L.recv_bytes(W)) + qr::align256(L.total);
}

const char* qr_last_error(void) { return g_err; }

int qr_quantize(qr_codec codec, qr_dtype dtype, const void* x, size_t n,
                void* wire, void* stream) {
  QR_TRY(check_kind(codec, dtype, n));
  QR_TRY(check_ptr(x, "x", 0));
  QR_TRY(check_ptr(wire, "wire", 0));
  const qr::Layout L = qr::make_layout(codec, n);
  const void* outs[1] = {wire};
  QR_TRY(check_disjoint(&x, 1, 2 * n, outs, 1, L.total));
  qr::InPtrs in{};
  qr::OutPtrs out{};
  in.p[0] = static_cast<const uint8_t*>(x);
  out.p[0] = static_cast<uint8_t*>(wire);
  (void)hipGetLastError();
  return hip_status(qr::launch_quantize(codec, dtype, 1, in, out, false, L, as_stream(stream)),
                    "quantize launch");
}

int qr_dequantize(qr_codec codec, qr_dtype dtype, const void* wire, size_t n,
                  void* y, void* stream) {
  QR_TRY(check_kind(codec, dtype, n));
  QR_TRY(check_ptr(wire, "wire", 0));
  QR_TRY(check_ptr(y, "y", 0));
  const qr::Layout L = qr::make_layout(codec, n);
  const void* outs[1] = {y};
  QR_TRY(check_disjoint(&wire, 1, L.total, outs, 1, 2 * n));
  qr::OutPtrs out{};
  out.p[0] = static_cast<uint8_t*>(y);
  (void)hipGetLastError();
  return hip_status(qr::launch_dequantize(codec, dtype, 1,
                                          static_cast<const uint8_t*>(wire), out, L,
                                          as_stream(stream)),
                    "dequantize launch");
}

int qr_quantize_ranks(qr_codec codec, qr_dtype dtype, int W, const void* const* xs,
                      size_t n, void* const* wires, void* stream) {
  QR_TRY(check_kind(codec, dtype, n));
  if (W < 1 || W > qr::kMaxRanks)
    return fail(QR_ERR_UNSUPPORTED, "W = %d outside 1..%d", W, qr::kMaxRanks);
  if (xs == nullptr || wires == nullptr) return fail(QR_ERR_ARG, "NULL pointer array");
  for (int r = 0; r < W; r++) {
    QR_TRY(check_ptr(xs[r], "xs", r));
    QR_TRY(check_ptr(wires[r], "wires", r));
  }
  const qr::Layout L = qr::make_layout(codec, n);
  QR_TRY(check_disjoint(xs, W, 2 * n, (const void* const*)wires, W, L.total));
  qr::InPtrs in{};
  qr::OutPtrs out{};
  for (int r = 0; r < W; r++) {
    in.p[r] = static_cast<const uint8_t*>(xs[r]);
    out.p[r] = static_cast<uint8_t*>(wires[r]);
  }
  (void)hipGetLastError();
  return hip_status(qr::launch_quantize(codec, dtype, W, in, out, false, L, as_stream(stream)),
                    "quantize launch");
}

int qr_reduce_stage1(qr_codec codec, qr_dtype dtype, int W, const void* const* wires,
                     size_t n, int owner, void* reduced_wire, void* stream) {
  QR_TRY(check_kind(codec, dtype, n));
  if (!w_sim(W)) return fail(QR_ERR_UNSUPPORTED, "W = %d not in {2,4,8}", W);
  if (owner < -1 || owner >= W)
    return fail(QR_ERR_ARG, "owner = %d outside -1..W-1", owner);
  if (wires == nullptr) return fail(QR_ERR_ARG, "NULL pointer array");
  for (int r = 0; r < W; r++) QR_TRY(check_ptr(wires[r], "wires", r));
  QR_TRY(check_ptr(reduced_wire, "reduced_wire", 0));
  const qr::Layout L = qr::make_layout(codec, n);
  const void* outs[1] = {reduced_wire};
  QR_TRY(check_disjoint(wires, W, L.total, outs, 1, L.total));
  size_t lo, hi;
  owner_range(W, owner, L, lo, hi);
  qr::InPtrs in{};
  for (int r = 0; r < W; r++) in.p[r] = static_cast<const uint8_t*>(wires[r]);
  (void)hipGetLastError();
  return hip_status(qr::launch_stage1(codec, dtype, W, in, false,
                                      static_cast<uint8_t*>(reduced_wire), lo, hi, L,
                                      as_stream(stream)),
                    "stage-1 launch");
}

int qr_quantize_recv(qr_codec codec, qr_dtype dtype, int W, const void* const* xs, size_t n,
                     void* recv, void* stream) {
  QR_TRY(check_kind(codec, dtype, n));
  if (!w_sim(W)) return fail(QR_ERR_UNSUPPORTED, "W = %d not in {2,4,8}", W);
  if (xs == nullptr) return fail(QR_ERR_ARG, "NULL pointer array");
  for (int r = 0; r < W; r++) QR_TRY(check_ptr(xs[r], "xs", r));
  QR_TRY(check_ptr(recv, "recv", 0));
  const qr::Layout L = qr::make_layout(codec, n);
  const void* outs[1] = {recv};
  QR_TRY(check_disjoint(xs, W, 2 * n, outs, 1, L.recv_bytes(W)));
  qr::InPtrs in{}, unused{};
  qr::OutPtrs out{};
  recv_ptrs(static_cast<uint8_t*>(recv), W, L, out, unused);
  for (int r = 0; r < W; r++) in.p[r] = static_cast<const uint8_t*>(xs[r]);
  (void)hipGetLastError();
  return hip_status(qr::launch_quantize(codec, dtype, W, in, out, true, L, as_stream(stream)),
                    "quantize launch");
}

int qr_reduce_recv(qr_codec codec, qr_dtype dtype, int W, const void* recv, size_t n,
                   int owner, void* reduced_wire, void* stream) {
  QR_TRY(check_kind(codec, dtype, n));
  if (!w_sim(W)) return fail(QR_ERR_UNSUPPORTED, "W = %d not in {2,4,8}", W);
  if (owner < -1 || owner >= W)
    return fail(QR_ERR_ARG, "owner = %d outside -1..W-1", owner);
  QR_TRY(check_ptr(recv, "recv", 0));
  QR_TRY(check_ptr(reduced_wire, "reduced_wire", 0));
  const qr::Layout L = qr::make_layout(codec, n);
  const void* outs[1] = {reduced_wire};
  QR_TRY(check_disjoint(&recv, 1, L.recv_bytes(W), outs, 1, L.total));
  size_t lo, hi;
  owner_range(W, owner, L, lo, hi);
  qr::InPtrs in{};
  qr::OutPtrs unused{};
  recv_ptrs(const_cast<uint8_t*>(static_cast<const uint8_t*>(recv)), W, L, unused, in);
  (void)hipGetLastError();
  return hip_status(qr::launch_stage1(codec, dtype, W, in, true,
                                      static_cast<uint8_t*>(reduced_wire), lo, hi, L,
                                      as_stream(stream)),
                    "stage-1 launch");
}

int qr_gather_stage2(qr_codec codec, qr_dtype dtype, int W, const void* reduced_wire,
                     size_t n, void* const* ys, void* stream) {
  QR_TRY(check_kind(codec, dtype, n));
  if (W < 1 || W > qr::kMaxRanks)
    return fail(QR_ERR_UNSUPPORTED, "W = %d outside 1..%d", W, qr::kMaxRanks);
  if (ys == nullptr) return fail(QR_ERR_ARG, "NULL pointer array");
  QR_TRY(check_ptr(reduced_wire, "reduced_wire", 0));
  for (int r = 0; r < W; r++) QR_TRY(check_ptr(ys[r], "ys", r));
  const qr::Layout L = qr::make_layout(codec, n);
  QR_TRY(check_disjoint(&reduced_wire, 1, L.total, (const void* const*)ys, W, 2 * n));
  qr::OutPtrs out{};
  for (int r = 0; r < W; r++) out.p[r] = static_cast<uint8_t*>(ys[r]);
  (void)hipGetLastError();
  return hip_status(qr::launch_dequantize(codec, dtype, W,
                                          static_cast<const uint8_t*>(reduced_wire), out,
                                          L, as_stream(stream)),
                    "stage-2 launch");
}

int qr_allreduce_sim(int W, qr_dtype dtype, qr_codec codec, const void* const* xs,
                     void* const* ys, size_t n, void* workspace, size_t ws_bytes,
                     void* stream) {
  QR_TRY(check_sim(W, dtype, codec, xs, ys, n));
  QR_TRY(check_ptr(workspace, "workspace", 0));
  const size_t need = qr_sim_workspace_bytes(W, codec, n);
  if (ws_bytes < need)
    return fail(QR_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", ws_bytes, need);
  QR_TRY(check_workspace_disjoint(W, xs, ys, n, workspace, need));
  return run_sim(W, dtype, codec, xs, ys, n, static_cast<uint8_t*>(workspace),
                 as_stream(stream));
}

int qr_allreduce_sim_noalloc(int W, qr_dtype dtype, qr_codec codec, const void* const* xs,
                             void* const* ys, size_t n, void* stream) {
  QR_TRY(check_sim(W, dtype, codec, xs, ys, n));
  const size_t need = qr_sim_workspace_bytes(W, codec, n);
  if (need > QR_SCRATCH_BYTES)
    return fail(QR_ERR_WORKSPACE,
                "W = %d, codec %d, n = %zu needs a %zu-byte workspace, more than the "
                "library's %zu-byte buffer",
                W, (int)codec, n, need, (size_t)QR_SCRATCH_BYTES);
  void* ws = nullptr;
  QR_TRY(hip_status(qr::scratch_address(&ws), "workspace buffer lookup"));
  QR_TRY(check_workspace_disjoint(W, xs, ys, n, ws, need));
  return run_sim(W, dtype, codec, xs, ys, n, static_cast<uint8_t*>(ws), as_stream(stream));
}

int qr_allreduce_oneshot(int W, qr_dtype dtype, const void* const* xs, void* const* ys,
                         size_t n, void* stream) {
  QR_TRY(check_kind(QR_FP, dtype, n));
  if (!w_sim(W)) return fail(QR_ERR_UNSUPPORTED, "W = %d not in {2,4,8}", W);
  if (xs == nullptr || ys == nullptr) return fail(QR_ERR_ARG, "NULL pointer array");
  for (int r = 0; r < W; r++) {
    QR_TRY(check_ptr(xs[r], "xs", r));
    QR_TRY(check_ptr(ys[r], "ys", r));
  }
  QR_TRY(check_disjoint(xs, W, 2 * n, (const void* const*)ys, W, 2 * n));
  qr::InPtrs in{};
  qr::OutPtrs out{};
  for (int r = 0; r < W; r++) {
    in.p[r] = static_cast<const uint8_t*>(xs[r]);
    out.p[r] = static_cast<uint8_t*>(ys[r]);
  }
  (void)hipGetLastError();
  return hip_status(qr::launch_oneshot(dtype, W, in, out, n, as_stream(stream)),
                    "one-stage launch");
}

}  // extern "C"
