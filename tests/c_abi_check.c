/* c_abi_check.c -- test program: the C ABI of include/qr.h used from plain C
 * (C11, gcc, no C++ and no torch): device memory from the HIP runtime's C
 * API, the library's entry points called directly, every output compared
 * bit for bit with the CPU oracle (oracle/libqr_oracle.so, test
 * infrastructure) on the same inputs.
 *
 * Covered: qr_allreduce_sim for every codec, both buffer types and W = 2, 4,
 * 8 at a size with a ragged last block (one launch) and, for two codecs, at a
 * size above the single-launch limit (three launches); the staged calls
 * (qr_quantize_ranks, qr_reduce_stage1 per owner, qr_gather_stage2) against
 * the same oracle outputs; qr_allreduce_oneshot; and a rejected call, which
 * must return its code, leave a message and write nothing.
 *
 * Inputs: a counter-based generator (splitmix64) of binary16 / bfloat16 bit
 * patterns of finite values of moderate size, the same arrays fed to both.
 * Prints one line per case group and "ALL OK" when every comparison holds. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "qr.h"

/* the oracle (oracle/qr_oracle.c) */
int ref_allreduce(int W, int dtype, int c, const uint16_t* const* xs, uint16_t* const* ys,
                  size_t n, size_t blk_lo, size_t blk_hi);
int ref_oneshot(int W, int dtype, const uint16_t* const* xs, uint16_t* const* ys, size_t n,
                size_t blk_lo, size_t blk_hi);

#define CK(x)                                                                   \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);     \
      exit(2);                                                                  \
    }                                                                           \
  } while (0)

static uint64_t mix64(uint64_t z) {
  z += 0x9e3779b97f4a7c15ull;
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}

/* finite values with exponents spread over about 2^-8 .. 2^7, both signs */
static uint16_t draw(int dtype, uint64_t key) {
  const uint64_t r = mix64(key);
  const uint16_t sign = (uint16_t)((r & 1) << 15);
  if (dtype == QR_FP16) {
    const uint16_t e = (uint16_t)(7 + (r >> 1) % 16);   /* biased exponent 7..22 */
    return (uint16_t)(sign | (e << 10) | ((r >> 8) & 0x3ff));
  }
  const uint16_t e = (uint16_t)(119 + (r >> 1) % 16);   /* biased exponent 119..134 */
  return (uint16_t)(sign | (e << 7) | ((r >> 8) & 0x7f));
}

static int failures = 0;

static void expect_equal(const uint16_t* got, const uint16_t* want, size_t n, const char* what,
                         int W, int codec, int dtype, int r) {
  for (size_t i = 0; i < n; i++) {
    if (got[i] != want[i]) {
      printf("MISMATCH %s W=%d codec=%d dtype=%d rank %d element %zu: got %04x want %04x\n",
             what, W, codec, dtype, r, i, got[i], want[i]);
      failures++;
      return;
    }
  }
}

/* one allreduce case: sim (and, if staged, the staged calls) vs the oracle */
static void run_case(int W, int codec, int dtype, size_t n, int staged, uint64_t seed) {
  const int in_t = dtype == QR_BF16_VIA_FP16 ? QR_BF16 : dtype;
  uint16_t *hx[8], *hy[8], *want[8];
  void *dx[8], *dy[8];
  for (int r = 0; r < W; r++) {
    hx[r] = malloc(2 * n);
    hy[r] = malloc(2 * n);
    want[r] = malloc(2 * n);
    if (!hx[r] || !hy[r] || !want[r]) { printf("host allocation failed\n"); exit(2); }
    for (size_t i = 0; i < n; i++) hx[r][i] = draw(in_t, seed * 1000003ull + (uint64_t)r * n + i);
    CK(hipMalloc(&dx[r], 2 * n));
    CK(hipMalloc(&dy[r], 2 * n));
    CK(hipMemcpy(dx[r], hx[r], 2 * n, hipMemcpyHostToDevice));
  }
  if (ref_allreduce(W, dtype, codec, (const uint16_t* const*)hx, want, n, 0, (size_t)-1) != 0) {
    printf("oracle refused W=%d codec=%d dtype=%d\n", W, codec, dtype);
    exit(2);
  }
  const size_t ws_bytes = qr_sim_workspace_bytes(W, (qr_codec)codec, n);
  void* ws;
  CK(hipMalloc(&ws, ws_bytes));
  int rc = qr_allreduce_sim(W, (qr_dtype)dtype, (qr_codec)codec, (const void* const*)dx,
                            (void* const*)dy, n, ws, ws_bytes, NULL);
  if (rc != QR_OK) {
    printf("qr_allreduce_sim returned %d: %s\n", rc, qr_last_error());
    failures++;
  }
  CK(hipDeviceSynchronize());
  for (int r = 0; r < W; r++) {
    CK(hipMemcpy(hy[r], dy[r], 2 * n, hipMemcpyDeviceToHost));
    expect_equal(hy[r], want[r], n, "sim", W, codec, dtype, r);
  }
  if (staged) {
    /* the staged calls, with stage 1 issued owner by owner */
    const size_t wb = qr_wire_bytes((qr_codec)codec, n);
    void *wires[8], *red;
    for (int r = 0; r < W; r++) CK(hipMalloc(&wires[r], wb));
    CK(hipMalloc(&red, wb));
    for (int r = 0; r < W; r++) CK(hipMemset(dy[r], 0, 2 * n));
    rc = qr_quantize_ranks((qr_codec)codec, (qr_dtype)dtype, W, (const void* const*)dx, n,
                           (void* const*)wires, NULL);
    for (int j = 0; j < W && rc == QR_OK; j++)
      rc = qr_reduce_stage1((qr_codec)codec, (qr_dtype)dtype, W, (const void* const*)wires, n, j,
                            red, NULL);
    if (rc == QR_OK)
      rc = qr_gather_stage2((qr_codec)codec, (qr_dtype)dtype, W, red, n, (void* const*)dy, NULL);
    if (rc != QR_OK) {
      printf("staged call returned %d: %s\n", rc, qr_last_error());
      failures++;
    }
    CK(hipDeviceSynchronize());
    for (int r = 0; r < W; r++) {
      CK(hipMemcpy(hy[r], dy[r], 2 * n, hipMemcpyDeviceToHost));
      expect_equal(hy[r], want[r], n, "staged", W, codec, dtype, r);
    }
    /* the same through a receive buffer, stage 1 owner by owner */
    void* recv;
    CK(hipMalloc(&recv, qr_recv_bytes(W, (qr_codec)codec, n)));
    for (int r = 0; r < W; r++) CK(hipMemset(dy[r], 0, 2 * n));
    rc = qr_quantize_recv((qr_codec)codec, (qr_dtype)dtype, W, (const void* const*)dx, n, recv,
                          NULL);
    for (int j = 0; j < W && rc == QR_OK; j++)
      rc = qr_reduce_recv((qr_codec)codec, (qr_dtype)dtype, W, recv, n, j, red, NULL);
    if (rc == QR_OK)
      rc = qr_gather_stage2((qr_codec)codec, (qr_dtype)dtype, W, red, n, (void* const*)dy, NULL);
    if (rc != QR_OK) {
      printf("receive-buffer call returned %d: %s\n", rc, qr_last_error());
      failures++;
    }
    CK(hipDeviceSynchronize());
    for (int r = 0; r < W; r++) {
      CK(hipMemcpy(hy[r], dy[r], 2 * n, hipMemcpyDeviceToHost));
      expect_equal(hy[r], want[r], n, "recv", W, codec, dtype, r);
    }
    CK(hipFree(recv));
    for (int r = 0; r < W; r++) CK(hipFree(wires[r]));
    CK(hipFree(red));
  }
  CK(hipFree(ws));
  for (int r = 0; r < W; r++) {
    CK(hipFree(dx[r]));
    CK(hipFree(dy[r]));
    free(hx[r]);
    free(hy[r]);
    free(want[r]);
  }
}

static void run_oneshot(int W, int dtype, size_t n, uint64_t seed) {
  const int in_t = dtype == QR_BF16_VIA_FP16 ? QR_BF16 : dtype;
  uint16_t *hx[8], *hy[8], *want[8];
  void *dx[8], *dy[8];
  for (int r = 0; r < W; r++) {
    hx[r] = malloc(2 * n);
    hy[r] = malloc(2 * n);
    want[r] = malloc(2 * n);
    if (!hx[r] || !hy[r] || !want[r]) { printf("host allocation failed\n"); exit(2); }
    for (size_t i = 0; i < n; i++) hx[r][i] = draw(in_t, seed * 1000003ull + (uint64_t)r * n + i);
    CK(hipMalloc(&dx[r], 2 * n));
    CK(hipMalloc(&dy[r], 2 * n));
    CK(hipMemcpy(dx[r], hx[r], 2 * n, hipMemcpyHostToDevice));
  }
  if (ref_oneshot(W, dtype, (const uint16_t* const*)hx, want, n, 0, (size_t)-1) != 0) exit(2);
  const int rc = qr_allreduce_oneshot(W, (qr_dtype)dtype, (const void* const*)dx,
                                      (void* const*)dy, n, NULL);
  if (rc != QR_OK) {
    printf("qr_allreduce_oneshot returned %d: %s\n", rc, qr_last_error());
    failures++;
  }
  CK(hipDeviceSynchronize());
  for (int r = 0; r < W; r++) {
    CK(hipMemcpy(hy[r], dy[r], 2 * n, hipMemcpyDeviceToHost));
    expect_equal(hy[r], want[r], n, "oneshot", W, -1, dtype, r);
    CK(hipFree(dx[r]));
    CK(hipFree(dy[r]));
    free(hx[r]);
    free(hy[r]);
    free(want[r]);
  }
}

/* a rejected call (W = 3) returns its code, leaves a message, writes nothing */
static void run_rejected(void) {
  const size_t n = 4096;
  void *dx[3], *dy[3];
  uint16_t h[4096];
  for (int r = 0; r < 3; r++) {
    CK(hipMalloc(&dx[r], 2 * n));
    CK(hipMalloc(&dy[r], 2 * n));
    CK(hipMemset(dx[r], 0, 2 * n));
    CK(hipMemset(dy[r], 0x5a, 2 * n));
  }
  void* ws;
  const size_t wsb = qr_sim_workspace_bytes(2, QR_Q8, n) * 2;
  CK(hipMalloc(&ws, wsb));
  const int rc = qr_allreduce_sim(3, QR_FP16, QR_Q8, (const void* const*)dx, (void* const*)dy, n,
                                  ws, wsb, NULL);
  CK(hipDeviceSynchronize());
  if (rc != QR_ERR_UNSUPPORTED || qr_last_error()[0] == '\0') {
    printf("rejected call: returned %d, message \"%s\"\n", rc, qr_last_error());
    failures++;
  }
  for (int r = 0; r < 3; r++) {
    CK(hipMemcpy(h, dy[r], 2 * n, hipMemcpyDeviceToHost));
    for (size_t i = 0; i < n; i++)
      if (h[i] != 0x5a5a) {
        printf("rejected call wrote output %d element %zu\n", r, i);
        failures++;
        break;
      }
    CK(hipFree(dx[r]));
    CK(hipFree(dy[r]));
  }
  CK(hipFree(ws));
}

int main(void) {
  static const int codecs[8] = {QR_FP, QR_FP8, QR_Q8, QR_Q6, QR_Q4,
                                QR_Q8_ASYM, QR_Q6_ASYM, QR_Q4_ASYM};
  static const int dtypes[3] = {QR_FP16, QR_BF16, QR_BF16_VIA_FP16};
  static const int Ws[3] = {2, 4, 8};
  int cases = 0;
  uint64_t seed = 1;
  for (int wi = 0; wi < 3; wi++)
    for (int di = 0; di < 3; di++)
      for (int ci = 0; ci < 8; ci++) {
        run_case(Ws[wi], codecs[ci], dtypes[di], 3 * 8192 + 40, di == 0, seed++);
        cases++;
      }
  printf("qr_allreduce_sim (one launch), staged calls for fp16: %d cases, %d failures\n", cases,
         failures);
  /* above the single-launch limit: three launches */
  run_case(2, QR_Q4, QR_FP16, (2u << 20) + 8, 1, seed++);
  run_case(4, QR_Q6_ASYM, QR_BF16, (2u << 20) + 8, 0, seed++);
  printf("qr_allreduce_sim (three launches): 2 cases, %d failures so far\n", failures);
  for (int wi = 0; wi < 3; wi++)
    for (int di = 0; di < 3; di++) run_oneshot(Ws[wi], dtypes[di], 8192 + 24, seed++);
  printf("qr_allreduce_oneshot: 9 cases, %d failures so far\n", failures);
  run_rejected();
  printf("rejected call: %d failures so far\n", failures);
  printf("%s\n", failures == 0 ? "ALL OK" : "FAILURES");
  return failures == 0 ? 0 : 1;
}
