/* oracle_sanitize.c -- test program: drives every entry point of the CPU
 * oracle (oracle/qr_oracle.c, compiled into this program) under
 * AddressSanitizer and UndefinedBehaviorSanitizer.  Every buffer is
 * allocated at exactly the size the oracle's interface states, so a read or
 * write past it lands in a redzone; a sanitizer report aborts the program.
 *
 * Covered: the number-format conversions over all 16-bit patterns and random
 * binary32 values; the block quantizer for every codec and block length
 * 1..32; the decode of every code; quantize, dequantize, stage 1 (whole and
 * per owner chunk), stage 2, the whole allreduce and the one-stage allreduce
 * for every codec, buffer type (fp16, bf16, bf16 through fp16), W in
 * {1, 2, 3, 4, 8} and ragged sizes.  Inputs are finite (non-finite values
 * are outside the oracle's contract); bf16 inputs reach far beyond the
 * binary16 range, which exercises the saturated scales and clamped codes.
 * Prints one line and exits 0 when nothing was reported. */
#include <stddef.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

float ref_h2f(uint16_t h);
uint16_t ref_f2h(float v);
float ref_bf2f(uint16_t b);
uint16_t ref_f2bf(float v);
uint16_t ref_ru16(float v);
uint16_t ref_rd16(float v);
float ref_e4m3_decode(uint8_t c);
uint8_t ref_e4m3_encode(float t);
float ref_codec_qmax(int c);
size_t ref_block_code_bytes(int c);
size_t ref_wire_bytes(int c, size_t n);
void ref_quantize_block(int c, const float* v, int L, uint32_t* codes, uint16_t* s,
                        uint16_t* z);
float ref_dequant_code(int c, uint32_t code, uint16_t s, uint16_t z);
int ref_quantize(int c, int dtype, const uint16_t* x, size_t n, uint8_t* wire, size_t lo,
                 size_t hi);
int ref_dequantize(int c, int dtype, const uint8_t* wire, size_t n, uint16_t* y, size_t lo,
                   size_t hi);
void ref_chunk(int W, size_t n, int j, size_t* lo, size_t* hi);
int ref_stage1(int c, int dtype, int W, const uint8_t* const* wires, size_t n,
               uint8_t* reduced, size_t lo, size_t hi);
int ref_stage2(int c, int dtype, int W, const uint8_t* reduced, size_t n, uint16_t* const* ys,
               size_t lo, size_t hi);
int ref_allreduce(int W, int dtype, int c, const uint16_t* const* xs, uint16_t* const* ys,
                  size_t n, size_t lo, size_t hi);
int ref_oneshot(int W, int dtype, const uint16_t* const* xs, uint16_t* const* ys, size_t n,
                size_t lo, size_t hi);

static const size_t ALL = (size_t)-1;
static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

static uint32_t next32(void) {           /* xorshift64* */
  rng_state ^= rng_state >> 12;
  rng_state ^= rng_state << 25;
  rng_state ^= rng_state >> 27;
  return (uint32_t)((rng_state * 0x2545f4914f6cdd1dull) >> 32);
}

/* a random finite 16-bit pattern of the buffer type (0 fp16, else bf16) */
static uint16_t finite16(int bf16) {
  for (;;) {
    uint16_t b = (uint16_t)next32();
    uint16_t e = bf16 ? 0x7f80 : 0x7c00;
    if ((b & e) != e) return b;
  }
}

static float finite32(void) {
  for (;;) {
    uint32_t u = next32();
    if ((u & 0x7f800000u) != 0x7f800000u) {
      float f;
      memcpy(&f, &u, 4);
      return f;
    }
  }
}

static void* alloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static long calls = 0;

static void fail(const char* what, int rc) {
  fprintf(stderr, "%s returned %d\n", what, rc);
  exit(1);
}

static void formats(void) {
  volatile float sink = 0.0f;
  for (uint32_t h = 0; h < 65536; h++) {
    sink += ref_h2f((uint16_t)h) * 0.0f;
    if (((h & 0x7f80) != 0x7f80)) sink += ref_bf2f((uint16_t)h) * 0.0f;
  }
  for (int i = 0; i < 200000; i++) {
    float f = finite32();
    sink += (float)(ref_f2h(f) + ref_f2bf(f) + ref_e4m3_encode(f));
    float a = f < 0 ? -f : f;
    sink += (float)(ref_ru16(a) + ref_rd16(f));
  }
  for (int c = 0; c < 256; c++) sink += ref_e4m3_decode((uint8_t)c) * 0.0f;
  (void)sink;
  calls += 65536 * 2 + 200000 * 5 + 256;
}

static const int CODECS[] = {0, 1, 2, 3, 5, 9, 10, 11};
static const int NCODECS = 8;

static void blocks(void) {
  for (int k = 1; k < NCODECS; k++) {
    int c = CODECS[k];
    for (int L = 1; L <= 32; L++) {
      for (int rep = 0; rep < 50; rep++) {
        float* v = alloc((size_t)L * sizeof(float));
        int scale = (int)(next32() % 60) - 30;
        for (int i = 0; i < L; i++) {
          uint16_t h = finite16(0);
          v[i] = ref_h2f(h) * (scale >= 0 ? (float)(1u << (scale / 3)) : 1.0f / (float)(1u << (-scale / 3)));
        }
        if (rep % 10 == 0)
          for (int i = 0; i < L; i++) v[i] = v[0];            /* constant block */
        if (rep % 10 == 1)
          for (int i = 0; i < L; i++) v[i] = 0.0f;            /* zero block */
        uint32_t* codes = alloc(32 * sizeof(uint32_t));
        uint16_t s, z;
        ref_quantize_block(c, v, L, codes, &s, &z);
        volatile float sink = 0.0f;
        for (int i = 0; i < L; i++) sink += ref_dequant_code(c, codes[i], s, z);
        (void)sink;
        free(codes);
        free(v);
        calls += 1 + L;
      }
    }
    uint32_t ncodes = c == 2 || c == 10 ? 64u : c == 3 || c == 11 ? 16u : 256u;
    for (uint32_t code = 0; code < ncodes; code++) {
      volatile float sink = ref_dequant_code(c, code, finite16(0) & 0x7fff, finite16(0));
      (void)sink;
      calls++;
    }
  }
}

static void pipeline(void) {
  static const size_t NS[] = {8, 16, 24, 32, 40, 1000, 8 * 1001, 8192 + 24};
  static const int WS[] = {1, 2, 3, 4, 8};
  for (size_t in = 0; in < sizeof NS / sizeof NS[0]; in++) {
    size_t n = NS[in];
    for (int iw = 0; iw < 5; iw++) {
      int W = WS[iw];
      for (int dtype = 0; dtype <= 2; dtype++) {
        uint16_t** xs = alloc((size_t)W * sizeof(uint16_t*));
        uint16_t** ys = alloc((size_t)W * sizeof(uint16_t*));
        for (int r = 0; r < W; r++) {
          xs[r] = alloc(n * 2);
          ys[r] = alloc(n * 2);
          for (size_t i = 0; i < n; i++) xs[r][i] = finite16(dtype != 0);
          if (dtype == 2)                     /* cast option: keep inputs fp16-finite */
            for (size_t i = 0; i < n; i++) xs[r][i] &= 0xc77f;
        }
        int rc = ref_oneshot(W, dtype, (const uint16_t* const*)xs, ys, n, 0, ALL);
        if (rc) fail("ref_oneshot", rc);
        calls++;
        for (int k = 0; k < NCODECS; k++) {
          int c = CODECS[k];
          size_t wb = ref_wire_bytes(c, n);
          uint8_t** wires = alloc((size_t)W * sizeof(uint8_t*));
          for (int r = 0; r < W; r++) {
            wires[r] = alloc(wb);
            memset(wires[r], 0, wb);
            rc = ref_quantize(c, dtype, xs[r], n, wires[r], 0, ALL);
            if (rc) fail("ref_quantize", rc);
          }
          uint8_t* red = alloc(wb);
          memset(red, 0, wb);
          rc = ref_stage1(c, dtype, W, (const uint8_t* const*)wires, n, red, 0, ALL);
          if (rc) fail("ref_stage1", rc);
          for (int j = 0; j < W; j++) {          /* owner chunks */
            size_t lo, hi;
            ref_chunk(W, n, j, &lo, &hi);
            rc = ref_stage1(c, dtype, W, (const uint8_t* const*)wires, n, red, lo, hi);
            if (rc) fail("ref_stage1 (owner)", rc);
            rc = ref_stage2(c, dtype, W, red, n, ys, lo, hi);
            if (rc) fail("ref_stage2 (owner)", rc);
          }
          rc = ref_stage2(c, dtype, W, red, n, ys, 0, ALL);
          if (rc) fail("ref_stage2", rc);
          rc = ref_dequantize(c, dtype, wires[0], n, ys[0], 0, ALL);
          if (rc) fail("ref_dequantize", rc);
          rc = ref_allreduce(W, dtype, c, (const uint16_t* const*)xs, ys, n, 0, ALL);
          if (rc) fail("ref_allreduce", rc);
          /* a wire image no quantizer wrote: random bytes (finite scales) */
          for (size_t i = 0; i < wb; i++) red[i] = (uint8_t)next32();
          if (c != 0) {
            size_t nb = (n + 31) / 32, so = (nb * ref_block_code_bytes(c) + 255) / 256 * 256;
            for (size_t b = 0; b < 2 * nb; b += 2) {
              uint16_t h = finite16(0);
              memcpy(red + so + b, &h, 2);
            }
            if (c & 8) {
              size_t zo = (so + 2 * nb + 255) / 256 * 256;
              for (size_t b = 0; b < 2 * nb; b += 2) {
                uint16_t h = finite16(0);
                memcpy(red + zo + b, &h, 2);
              }
            }
            if (c == 5)
              for (size_t i = 0; i < nb * 32; i++)
                if ((red[i] & 0x7f) == 0x7f) red[i] = 0;   /* no fp8 NaN codes */
          } else {
            for (size_t i = 0; i < n; i++) {
              uint16_t h = finite16(dtype == 1);
              memcpy(red + 2 * i, &h, 2);
            }
          }
          rc = ref_stage2(c, dtype, W, red, n, ys, 0, ALL);
          if (rc) fail("ref_stage2 (any wire)", rc);
          calls += 3 * W + 4;
          for (int r = 0; r < W; r++) free(wires[r]);
          free(wires);
          free(red);
        }
        for (int r = 0; r < W; r++) {
          free(xs[r]);
          free(ys[r]);
        }
        free(xs);
        free(ys);
      }
    }
  }
}

int main(void) {
  formats();
  blocks();
  pipeline();
  printf("oracle under ASan+UBSan: %ld calls, no report\n", calls);
  return 0;
}
