// abi_host_check.cpp -- test program: the C ABI's host code (qr_api.cpp)
// without a GPU, built with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer.  The kernel launchers of qr_internal.h and the
// two HIP runtime calls qr_api.cpp makes are replaced here by stubs that
// record every launch, so the program checks what each entry point would
// launch, and with which arguments:
//   - qr_allreduce_sim: one fused launch up to 4 MiB per rank, above that
//     quantize -> stage 1 over all blocks -> stage 2, with the W wire images
//     and the reduced image at 256-byte-aligned strides of the workspace;
//   - qr_reduce_stage1 per owner: blocks [j*bpc, min(nb, (j+1)*bpc));
//   - every rejected call returns its documented code and launches nothing;
//   - a failed launch returns QR_ERR_HIP, names the stage, and the staged
//     sim launches nothing after it;
//   - qr_allreduce_sim_noalloc launches what qr_allreduce_sim launches, with
//     the library's buffer (the stubbed lookup's address) as the workspace,
//     and rejects a workspace beyond QR_SCRATCH_BYTES without looking it up.
// Device pointers are fake addresses; nothing dereferences them.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <vector>

#include "qr.h"
#include "qr_internal.h"

namespace {

struct Call {
  const char* what;
  int codec, dtype, W;
  bool recv;
  const void* in[qr::kMaxRanks];
  const void* out[qr::kMaxRanks];
  const void* red;
  size_t lo, hi, n, total;
};

std::vector<Call> g_calls;
hipError_t g_fail_on = hipSuccess;     // error the next launch returns
const char* g_fail_what = nullptr;     // ... if it is this launch
int g_checks = 0, g_bad = 0;

hipError_t record(const Call& c) {
  g_calls.push_back(c);
  if (g_fail_what && strcmp(g_fail_what, c.what) == 0) return g_fail_on;
  return hipSuccess;
}

void expect(bool ok, const char* what, int line) {
  g_checks++;
  if (!ok) {
    g_bad++;
    fprintf(stderr, "FAILED line %d: %s\n", line, what);
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

}  // namespace

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }
extern "C" const char* hipGetErrorString(hipError_t e) {
  return e == hipSuccess ? "no error" : "stubbed launch failure";
}

namespace qr {

hipError_t launch_quantize(int codec, int dtype, int W, const InPtrs& xs, const OutPtrs& wires,
                           bool recv, const Layout& L, hipStream_t) {
  Call c{"quantize", codec, dtype, W, recv, {}, {}, nullptr, 0, 0, L.n, L.total};
  for (int r = 0; r < W; r++) c.in[r] = xs.p[r], c.out[r] = wires.p[r];
  return record(c);
}
hipError_t launch_stage1(int codec, int dtype, int W, const InPtrs& wires, bool recv,
                         uint8_t* reduced, size_t blk_lo, size_t blk_hi, const Layout& L,
                         hipStream_t) {
  Call c{"stage1", codec, dtype, W, recv, {}, {}, reduced, blk_lo, blk_hi, L.n, L.total};
  for (int r = 0; r < W; r++) c.in[r] = wires.p[r];
  if (blk_hi <= blk_lo) return hipSuccess;   // the real launcher launches nothing then
  return record(c);
}
hipError_t launch_dequantize(int codec, int dtype, int W, const uint8_t* wire, const OutPtrs& ys,
                             const Layout& L, hipStream_t) {
  Call c{"stage2", codec, dtype, W, false, {}, {}, wire, 0, 0, L.n, L.total};
  for (int r = 0; r < W; r++) c.out[r] = ys.p[r];
  return record(c);
}
hipError_t launch_fused(int codec, int dtype, int W, const InPtrs& xs, const OutPtrs& wires,
                        uint8_t* reduced, const OutPtrs& ys, const Layout& L, hipStream_t) {
  Call c{"fused", codec, dtype, W, true, {}, {}, reduced, 0, 0, L.n, L.total};
  for (int r = 0; r < W; r++) c.in[r] = wires.p[r], c.out[r] = ys.p[r];
  (void)xs;
  return record(c);
}
int g_scratch_lookups = 0;
hipError_t scratch_address(void** p) {
  g_scratch_lookups++;
  *p = reinterpret_cast<void*>((uintptr_t)0x7f0000000000ull + ((uintptr_t)30 << 36));
  return hipSuccess;
}
hipError_t launch_oneshot(int dtype, int W, const InPtrs& xs, const OutPtrs& ys, size_t n,
                          hipStream_t) {
  Call c{"oneshot", 0, dtype, W, false, {}, {}, nullptr, 0, 0, n, 0};
  for (int r = 0; r < W; r++) c.in[r] = xs.p[r], c.out[r] = ys.p[r];
  return record(c);
}

}  // namespace qr

namespace {

// fake, 256-byte-aligned device addresses far apart
void* dev(int i) { return reinterpret_cast<void*>((uintptr_t)0x7f0000000000ull + ((uintptr_t)i << 36)); }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// one rank's tile of 256 blocks in the receive buffer, from its definition
size_t tile_bytes(int codec) {
  if (codec == QR_FP) return 256 * 64;
  const size_t cb = (codec & 7) == QR_Q6 ? 24 : (codec & 7) == QR_Q4 ? 16 : 32;
  return 256 * (cb + 2 + ((codec & 8) ? 2 : 0));
}

const int CODECS[] = {QR_FP, QR_Q8, QR_Q6, QR_Q4, QR_FP8, QR_Q8_ASYM, QR_Q6_ASYM, QR_Q4_ASYM};

void sim_paths() {
  for (int codec : CODECS) {
    for (int W : {2, 4, 8}) {
      for (size_t n : {(size_t)8, (size_t)2048 + 8, (size_t)2 << 20, ((size_t)2 << 20) + 8,
                       (size_t)1 << 25}) {
        const void* xs[8];
        void* ys[8];
        for (int r = 0; r < W; r++) xs[r] = dev(r), ys[r] = dev(8 + r);
        void* ws = dev(20);
        const size_t need = qr_sim_workspace_bytes(W, (qr_codec)codec, n);
        const size_t tile = tile_bytes(codec), nt = ((n + 31) / 32 + 255) / 256;
        const size_t recv = qr_recv_bytes(W, (qr_codec)codec, n);
        EXPECT(recv == nt * W * tile);
        const size_t red_at = align256(recv);
        EXPECT(need == red_at + align256(qr_wire_bytes((qr_codec)codec, n)));
        g_calls.clear();
        int rc = qr_allreduce_sim(W, QR_FP16, (qr_codec)codec, xs, ys, n, ws, need, nullptr);
        EXPECT(rc == QR_OK);
        const uint8_t* base = static_cast<const uint8_t*>(ws);
        if (2 * n <= ((size_t)4 << 20)) {
          EXPECT(g_calls.size() == 1 && strcmp(g_calls[0].what, "fused") == 0);
          if (!g_calls.empty()) {
            EXPECT(g_calls[0].red == base + red_at && g_calls[0].recv);
            for (int r = 0; r < W; r++) EXPECT(g_calls[0].in[r] == base + r * tile);
          }
        } else {
          EXPECT(g_calls.size() == 3);
          if (g_calls.size() == 3) {
            EXPECT(strcmp(g_calls[0].what, "quantize") == 0);
            EXPECT(strcmp(g_calls[1].what, "stage1") == 0);
            EXPECT(strcmp(g_calls[2].what, "stage2") == 0);
            EXPECT(g_calls[0].recv && g_calls[1].recv);
            for (int r = 0; r < W; r++) {
              EXPECT(g_calls[0].in[r] == xs[r]);
              EXPECT(g_calls[0].out[r] == base + r * tile);
              EXPECT(g_calls[1].in[r] == base + r * tile);
              EXPECT(g_calls[2].out[r] == ys[r]);
            }
            EXPECT(g_calls[1].red == base + red_at && g_calls[2].red == base + red_at);
            EXPECT(g_calls[1].lo == 0 && g_calls[1].hi == (n + 31) / 32);
          }
        }
        // the staged calls through a receive buffer launch the same kernels
        g_calls.clear();
        EXPECT(qr_quantize_recv((qr_codec)codec, QR_FP16, W, xs, n, (void*)base, nullptr) == QR_OK);
        EXPECT(qr_reduce_recv((qr_codec)codec, QR_FP16, W, base, n, -1, (void*)(base + red_at),
                              nullptr) == QR_OK);
        EXPECT(g_calls.size() == 2);
        if (g_calls.size() == 2) {
          EXPECT(g_calls[0].recv && g_calls[1].recv);
          for (int r = 0; r < W; r++)
            EXPECT(g_calls[0].out[r] == base + r * tile && g_calls[1].in[r] == base + r * tile);
          EXPECT(g_calls[1].lo == 0 && g_calls[1].hi == (n + 31) / 32);
        }
        for (const Call& c : g_calls) EXPECT(c.n == n && c.W == W && c.codec == codec);
      }
    }
  }
}

void owner_ranges() {
  for (int W : {2, 4, 8}) {
    for (size_t n : {(size_t)8, (size_t)40, (size_t)32 * 37 + 16, (size_t)32 * 846 + 16,
                     (size_t)1 << 20}) {
      const size_t nb = (n + 31) / 32, bpc = (nb + W - 1) / W;
      const void* wires[8];
      for (int r = 0; r < W; r++) wires[r] = dev(r);
      size_t covered = 0;
      for (int j = 0; j < W; j++) {
        g_calls.clear();
        EXPECT(qr_reduce_stage1(QR_Q4, QR_FP16, W, wires, n, j, dev(9), nullptr) == QR_OK);
        EXPECT(qr_reduce_recv(QR_Q4, QR_FP16, W, dev(0), n, j, dev(9), nullptr) == QR_OK);
        size_t lo = j * bpc < nb ? j * bpc : nb, hi = lo + bpc < nb ? lo + bpc : nb;
        if (lo == hi) {
          EXPECT(g_calls.empty());
        } else {
          EXPECT(g_calls.size() == 2);
          for (const Call& c : g_calls) EXPECT(c.lo == lo && c.hi == hi);
          covered += hi - lo;
        }
      }
      EXPECT(covered == nb);
    }
  }
}

void rejections() {
  const void* xs[8];
  void* ys[8];
  for (int r = 0; r < 8; r++) xs[r] = dev(r), ys[r] = dev(8 + r);
  const size_t n = 4096, need = qr_sim_workspace_bytes(2, QR_Q4, n);
  struct Case { int rc, expect; } cases[] = {
      {qr_allreduce_sim(3, QR_FP16, QR_Q4, xs, ys, n, dev(20), need, nullptr), QR_ERR_UNSUPPORTED},
      {qr_allreduce_sim(2, (qr_dtype)7, QR_Q4, xs, ys, n, dev(20), need, nullptr), QR_ERR_UNSUPPORTED},
      {qr_allreduce_sim(2, QR_FP16, (qr_codec)4, xs, ys, n, dev(20), need, nullptr), QR_ERR_UNSUPPORTED},
      {qr_allreduce_sim(2, QR_FP16, QR_Q4, xs, ys, 0, dev(20), need, nullptr), QR_ERR_SIZE},
      {qr_allreduce_sim(2, QR_FP16, QR_Q4, xs, ys, 12, dev(20), need, nullptr), QR_ERR_SIZE},
      {qr_allreduce_sim(2, QR_FP16, QR_Q4, xs, ys, ((size_t)1 << 30) + 8, dev(20), need, nullptr),
       QR_ERR_SIZE},
      {qr_allreduce_sim(2, QR_FP16, QR_Q4, xs, ys, n, dev(20), need - 1, nullptr), QR_ERR_WORKSPACE},
      {qr_allreduce_sim(2, QR_FP16, QR_Q4, xs, ys, n, (uint8_t*)dev(20) + 8, need, nullptr),
       QR_ERR_ALIGN},
      {qr_allreduce_sim(2, QR_FP16, QR_Q4, xs, ys, n, nullptr, need, nullptr), QR_ERR_ARG},
      {qr_allreduce_sim(2, QR_FP16, QR_Q4, nullptr, ys, n, dev(20), need, nullptr), QR_ERR_ARG},
      {qr_allreduce_sim(2, QR_FP16, QR_Q4, xs, (void* const*)xs, n, dev(20), need, nullptr),
       QR_ERR_ARG},                                   // outputs alias inputs
      {qr_allreduce_sim(2, QR_FP16, QR_Q4, xs, ys, n, (void*)xs[1], need, nullptr), QR_ERR_ARG},
      {qr_reduce_stage1(QR_Q4, QR_FP16, 2, xs, n, 2, dev(9), nullptr), QR_ERR_ARG},  // owner
      {qr_reduce_stage1(QR_Q4, QR_FP16, 2, xs, n, -2, dev(9), nullptr), QR_ERR_ARG},
      {qr_reduce_stage1(QR_Q4, QR_FP16, 2, xs, n, -1, (void*)xs[0], nullptr), QR_ERR_ARG},
      {qr_quantize_ranks(QR_Q4, QR_FP16, 9, xs, n, ys, nullptr), QR_ERR_UNSUPPORTED},
      {qr_gather_stage2(QR_Q4, QR_FP16, 0, xs[0], n, ys, nullptr), QR_ERR_UNSUPPORTED},
      {qr_allreduce_oneshot(5, QR_FP16, xs, ys, n, nullptr), QR_ERR_UNSUPPORTED},
      {qr_quantize(QR_Q4, QR_FP16, xs[0], n, (uint8_t*)xs[0] + 16, nullptr), QR_ERR_ARG},
      {qr_quantize_recv(QR_Q4, QR_FP16, 3, xs, n, dev(20), nullptr), QR_ERR_UNSUPPORTED},
      {qr_quantize_recv(QR_Q4, QR_FP16, 2, xs, n, (uint8_t*)xs[1] + 256, nullptr), QR_ERR_ARG},
      {qr_quantize_recv(QR_Q4, QR_FP16, 2, xs, n, (uint8_t*)dev(20) + 8, nullptr), QR_ERR_ALIGN},
      {qr_quantize_recv(QR_Q4, QR_FP16, 2, nullptr, n, dev(20), nullptr), QR_ERR_ARG},
      {qr_reduce_recv(QR_Q4, QR_FP16, 2, dev(20), n, 2, dev(21), nullptr), QR_ERR_ARG},
      {qr_reduce_recv(QR_Q4, QR_FP16, 4, dev(20), n, -1, (uint8_t*)dev(20) + 4096, nullptr),
       QR_ERR_ARG},                                   // reduced image inside the buffer
      {qr_reduce_recv(QR_Q4, QR_FP16, 8, dev(20), 12, -1, dev(21), nullptr), QR_ERR_SIZE},
      {qr_reduce_recv((qr_codec)4, QR_FP16, 2, dev(20), n, -1, dev(21), nullptr),
       QR_ERR_UNSUPPORTED},
      {qr_dequantize(QR_Q4, QR_FP16, xs[0], n, (uint8_t*)ys[0] + 4, nullptr), QR_ERR_ALIGN},
  };
  g_calls.clear();
  for (const Case& c : cases) EXPECT(c.rc == c.expect);
  EXPECT(g_calls.empty());
  EXPECT(strlen(qr_last_error()) > 0);
  EXPECT(qr_wire_bytes((qr_codec)4, 8) == 0 && qr_sim_workspace_bytes(3, QR_Q4, 8) == 0);
  // the largest rank buffer: sizes computed without overflow
  const size_t nmax = (size_t)1 << 30;
  EXPECT(qr_wire_bytes(QR_FP, nmax) == 2 * nmax);
  EXPECT(qr_wire_bytes(QR_Q8_ASYM, nmax) == align256(align256(nmax) + nmax / 16) + nmax / 16);
  EXPECT(qr_sim_workspace_bytes(8, QR_FP, nmax) == 9 * 2 * nmax);
  EXPECT(qr_recv_bytes(8, QR_FP, nmax) == 8 * 2 * nmax);
  EXPECT(qr_recv_bytes(8, QR_Q8_ASYM, nmax) == (nmax / 32 / 256) * 8 * 256 * 36);
  EXPECT(qr_recv_bytes(9, QR_Q4, 8) == 0 && qr_recv_bytes(0, QR_Q4, 8) == 0);
  EXPECT(qr_recv_bytes(1, QR_Q4, 8) == 256 * 18);
}

void failed_launch() {
  const void* xs[2] = {dev(0), dev(1)};
  void* ys[2] = {dev(8), dev(9)};
  const size_t n = (size_t)1 << 22;      // staged path
  const size_t need = qr_sim_workspace_bytes(2, QR_Q8, n);
  g_fail_what = "stage1";
  g_fail_on = hipErrorLaunchFailure;
  g_calls.clear();
  EXPECT(qr_allreduce_sim(2, QR_FP16, QR_Q8, xs, ys, n, dev(20), need, nullptr) == QR_ERR_HIP);
  EXPECT(g_calls.size() == 2);                       // quantize, stage1; no stage 2
  EXPECT(strstr(qr_last_error(), "stage-1") != nullptr);
  g_fail_what = nullptr;
  g_calls.clear();
  EXPECT(qr_allreduce_sim(2, QR_FP16, QR_Q8, xs, ys, n, dev(20), need, nullptr) == QR_OK);
  EXPECT(g_calls.size() == 3 && qr_last_error()[0] == 0);
}

void noalloc_paths() {
  const uint8_t* base = static_cast<const uint8_t*>(dev(30));   // the stubbed buffer
  for (int codec : CODECS) {
    for (int W : {2, 4, 8}) {
      for (size_t n : {(size_t)8, (size_t)2048 + 8, (size_t)2 << 20, ((size_t)2 << 20) + 8,
                       (size_t)1 << 25}) {
        const void* xs[8];
        void* ys[8];
        for (int r = 0; r < W; r++) xs[r] = dev(r), ys[r] = dev(8 + r);
        const size_t need = qr_sim_workspace_bytes(W, (qr_codec)codec, n);
        const size_t red_at = align256(qr_recv_bytes(W, (qr_codec)codec, n));
        g_calls.clear();
        const int before = qr::g_scratch_lookups;
        int rc = qr_allreduce_sim_noalloc(W, QR_FP16, (qr_codec)codec, xs, ys, n, nullptr);
        if (need > QR_SCRATCH_BYTES) {
          EXPECT(rc == QR_ERR_WORKSPACE && g_calls.empty());
          EXPECT(qr::g_scratch_lookups == before);
          continue;
        }
        EXPECT(rc == QR_OK);
        std::vector<Call> mine = g_calls;
        g_calls.clear();
        EXPECT(qr_allreduce_sim(W, QR_FP16, (qr_codec)codec, xs, ys, n, (void*)base, need,
                                nullptr) == QR_OK);
        EXPECT(mine.size() == g_calls.size());
        EXPECT(!mine.empty() && mine.back().red == base + red_at);
        for (size_t i = 0; i < mine.size() && i < g_calls.size(); i++) {
          EXPECT(strcmp(mine[i].what, g_calls[i].what) == 0 && mine[i].recv == g_calls[i].recv);
          EXPECT(mine[i].red == g_calls[i].red);
          EXPECT(mine[i].lo == g_calls[i].lo && mine[i].hi == g_calls[i].hi);
          for (int r = 0; r < W; r++)
            EXPECT(mine[i].in[r] == g_calls[i].in[r] && mine[i].out[r] == g_calls[i].out[r]);
        }
      }
    }
  }
  // the largest accepted size is the buffer's; one element block more is refused
  const void* xs[2] = {dev(0), dev(1)};
  void* ys[2] = {dev(8), dev(9)};
  size_t n = 8;
  while (qr_sim_workspace_bytes(2, QR_FP, n + 8) <= QR_SCRATCH_BYTES) n += 8;
  g_calls.clear();
  EXPECT(qr_allreduce_sim_noalloc(2, QR_FP16, QR_FP, xs, ys, n, nullptr) == QR_OK);
  EXPECT(qr_allreduce_sim_noalloc(2, QR_FP16, QR_FP, xs, ys, n + 8, nullptr) == QR_ERR_WORKSPACE);
  EXPECT(strstr(qr_last_error(), "workspace") != nullptr);
  EXPECT(g_calls.size() == 3);                       // the accepted call only (staged)
  // argument checks come first, as for qr_allreduce_sim
  EXPECT(qr_allreduce_sim_noalloc(3, QR_FP16, QR_Q4, xs, ys, 64, nullptr) == QR_ERR_UNSUPPORTED);
  EXPECT(qr_allreduce_sim_noalloc(2, QR_FP16, QR_Q4, xs, (void* const*)xs, 64, nullptr) ==
         QR_ERR_ARG);
  EXPECT(qr_allreduce_sim_noalloc(2, QR_FP16, QR_Q4, xs, ys, 12, nullptr) == QR_ERR_SIZE);
}

}  // namespace

int main() {
  sim_paths();
  owner_ranges();
  rejections();
  failed_launch();
  noalloc_paths();
  printf("C ABI host code: %d checks, %d failed\n", g_checks, g_bad);
  return g_bad == 0 ? 0 : 1;
}
