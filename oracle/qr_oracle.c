/*
 * qr_oracle.c -- plain, slow, scalar CPU oracle for the two-stage quantized
 * allreduce.  TEST INFRASTRUCTURE ONLY: nothing in the product library links,
 * loads or calls this file; only the tests, the smoke check and the CPU
 * baseline of the benchmark do.  It shares no code, header, table or constant
 * generator with the HIP path.
 *
 * What it follows
 *   - "Integrate quick allreduce and select the best allreduce implementation"
 *     (vLLM PR #18473), PR description item 2: the two-stage allreduce with
 *     wire formats f16, fp8, Q8, Q6, Q4.
 *   - "Add quickreduce as alternative to custom allreduce" (vLLM PR #16804),
 *     PR description: int4/int8 symmetric and asymmetric quantization.
 *   - vLLM API docs, vllm.distributed.device_communicators.quick_all_reduce,
 *     QuickReduceRegime (FP=0, INT8=1, INT6=2, INT4=3, NONE=4) and
 *     QuickAllReduce.quick_all_reduce (out-of-place; input never modified).
 *   - PR #18473's description item 2 and its tp2 timing table name a second,
 *     one-stage ("1stage", f16 only) allreduce.  The review thread of "Add
 *     quickreduce as alternative to custom allreduce" (vLLM PR #16804)
 *     proposes the one-shot kind (every rank reads every rank's buffer and
 *     reduces locally) for small buffers and two shots for larger ones.
 *
 * The pages name the formats only.  The readings taken where they are silent
 * (all stated again next to the code that implements them):
 *   32-element blocks; one fp16 scale per block (rounded up to the fp16 grid,
 *   saturating), plus one fp16 zero offset (rounded down) for the asymmetric
 *   codecs; codes are clamp(round-half-even(v / scale)); symmetric code range
 *   +-(2^(b-1)-1); fp8 is OCP E4M3FN with a per-block scale absmax/448;
 *   stage 1 sums the W dequantized ranks in binary32 in rank order
 *   0..W-1 and requantizes the binary32 sums with the same codec; stage 2
 *   dequantizes and rounds once to the buffer type.
 *
 * Arithmetic: IEEE binary32 for every step of the method (the method's own
 * precision: binary32 sums, binary16 scale/zero), each operation rounded
 * separately -- build with -O2 -ffp-contract=off, no fast-math, no FTZ.
 * Conversions are written from the value definition of each format, using
 * binary64 where that is exact, not by bit tricks.
 *
 * Every exported function works on a block range [blk_lo, blk_hi) so a test
 * can check sampled blocks of a large buffer; blk_hi = (size_t)-1 means "to
 * the last block".
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* codec numbering: low values are QuickReduceRegime's, fp8 and the
 * asymmetric variants are added (asymmetric = symmetric | 8). */
enum { C_FP = 0, C_Q8 = 1, C_Q6 = 2, C_Q4 = 3, C_FP8 = 5,
       C_Q8A = 9, C_Q6A = 10, C_Q4A = 11 };
/* buffer types; T_BF16_VIA_FP16 = bfloat16 buffers that are converted to
 * binary16 on entry and back on exit (see ld/st below) */
enum { T_FP16 = 0, T_BF16 = 1, T_BF16_VIA_FP16 = 2 };

#define BLK 32

/* ------------------------------------------------------------------ */
/* binary16 (IEEE 754 half): 1 sign, 5 exponent (bias 15), 10 fraction */

/* exact value of a binary16 bit pattern */
float ref_h2f(uint16_t h) {
  int sign = h >> 15;
  int e = (h >> 10) & 0x1F;
  int m = h & 0x3FF;
  double v;
  if (e == 0x1F) {
    if (m != 0) return NAN;
    v = INFINITY;
  } else if (e == 0) {
    v = ldexp((double)m, -24);               /* subnormal: m * 2^-24 */
  } else {
    v = ldexp(1.0 + m / 1024.0, e - 15);     /* normal */
  }
  return (float)(sign ? -v : v);             /* exact: fits binary32 */
}

/* spacing of the binary16 grid in the binade holding |a| (a finite, >0) */
static double h_quantum(double a) {
  int k;
  if (a < ldexp(1.0, -14)) return ldexp(1.0, -24);
  frexp(a, &k);                               /* a = f * 2^k, f in [0.5,1) */
  return ldexp(1.0, (k - 1) - 10);
}

/* bit pattern of a binary16-representable magnitude r (finite, >= 0) */
static uint16_t h_encode_mag(double r) {
  int k;
  if (r == 0.0) return 0;
  if (r < ldexp(1.0, -14)) return (uint16_t)(r / ldexp(1.0, -24));
  frexp(r, &k);
  int e = k - 1;                              /* r = (1 + m/1024) * 2^e */
  double m = (r / ldexp(1.0, e) - 1.0) * 1024.0;
  return (uint16_t)(((e + 15) << 10) | (int)m);
}

/* binary32 -> binary16, round to nearest, ties to even; overflow -> inf */
uint16_t ref_f2h(float v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs((double)v);
  if (isnan(v)) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00;    /* 65520 = halfway 65504..65536 */
  double q = h_quantum(a);
  double r = nearbyint(a / q) * q;            /* a/q exact; nearbyint is RNE */
  if (r > 65504.0) return sign | 0x7C00;
  return sign | h_encode_mag(r);
}

/* least binary16 >= v, for v >= 0; saturated at 65504 (never inf) */
uint16_t ref_ru16(float v) {
  double a = (double)v;
  if (!(a > 0.0)) return 0;                   /* v == 0 (either sign) */
  if (a > 65504.0) return 0x7BFF;
  double q = h_quantum(a);
  double r = ceil(a / q) * q;
  if (r > 65504.0) r = 65504.0;
  return h_encode_mag(r);
}

/* greatest binary16 <= v; saturated at -65504 (never -inf) */
uint16_t ref_rd16(float v) {
  double a = (double)v;
  if (a < 0.0) return 0x8000 | ref_ru16((float)-a);
  if (a >= 65504.0) return 0x7BFF;
  uint16_t sign = signbit(v) ? 0x8000 : 0;    /* keeps -0 as -0 */
  if (a == 0.0) return sign;
  double q = h_quantum(a);
  double r = floor(a / q) * q;
  return sign | h_encode_mag(r);
}

/* ------------------------------------------------------------------ */
/* bfloat16: the upper half of a binary32 (8 exponent, 7 fraction bits) */

float ref_bf2f(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* binary32 -> bfloat16, round to nearest, ties to even; overflow -> inf */
uint16_t ref_f2bf(float v) {
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  if (isnan(v)) return 0x7FC0;
  double a = fabs((double)v);
  if (isinf(v)) return sign | 0x7F80;
  if (a == 0.0) return sign;
  double q;                                   /* grid spacing of bf16 at a */
  if (a < ldexp(1.0, -126)) {
    q = ldexp(1.0, -133);                     /* subnormal binade */
  } else {
    int k;
    frexp(a, &k);
    q = ldexp(1.0, (k - 1) - 7);
  }
  double r = nearbyint(a / q) * q;
  if (r >= ldexp(1.0, 128)) return sign | 0x7F80;
  float rf = (float)r;                        /* exact: r has <= 8 bits */
  uint32_t u;
  memcpy(&u, &rf, 4);
  return sign | (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------ */
/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 fraction; no infinity,
 * 0x7F/0xFF are NaN, largest finite 448. */

float ref_e4m3_decode(uint8_t c) {
  int sign = c >> 7, e = (c >> 3) & 0xF, m = c & 7;
  double v;
  if (e == 0xF && m == 7) return NAN;
  if (e == 0) v = ldexp((double)m, -9);                 /* subnormal */
  else v = ldexp(1.0 + m / 8.0, e - 7);
  return (float)(sign ? -v : v);
}

/* nearest finite E4M3 value, ties to even, saturating at 448; the sign is
 * kept even when the magnitude rounds to zero */
uint8_t ref_e4m3_encode(float t) {
  uint8_t sign = signbit(t) ? 0x80 : 0;
  double a = fabs((double)t);
  if (isnan(t)) return 0x7F;
  if (a >= 448.0) return sign | 0x7E;
  double q;
  if (a < ldexp(1.0, -6)) {
    q = ldexp(1.0, -9);
  } else {
    int k;
    frexp(a, &k);
    q = ldexp(1.0, (k - 1) - 3);
  }
  double r = nearbyint(a / q) * q;            /* <= 448 because a < 448 */
  if (r == 0.0) return sign;
  if (r < ldexp(1.0, -6)) return sign | (uint8_t)(r / ldexp(1.0, -9));
  int k;
  frexp(r, &k);
  int e = k - 1;
  int m = (int)((r / ldexp(1.0, e) - 1.0) * 8.0);
  return sign | (uint8_t)(((e + 7) << 3) | m);
}

/* ------------------------------------------------------------------ */
/* codec properties */

static int codec_valid(int c) {
  return c == C_FP || c == C_Q8 || c == C_Q6 || c == C_Q4 || c == C_FP8 ||
         c == C_Q8A || c == C_Q6A || c == C_Q4A;
}
static int codec_bits(int c) {
  switch (c & 7) {
    case C_Q8: return 8;
    case C_Q6: return 6;
    case C_Q4: return 4;
    case C_FP8: return 8;
    default: return 16;
  }
}
static int codec_asym(int c) { return (c & 8) != 0; }

/* symmetric: largest code magnitude; asymmetric: largest unsigned code */
float ref_codec_qmax(int c) {
  if (c == C_FP8) return 448.0f;
  int b = codec_bits(c);
  if (codec_asym(c)) return (float)((1 << b) - 1);       /* 255, 63, 15 */
  return (float)((1 << (b - 1)) - 1);                    /* 127, 31, 7 */
}

/* ------------------------------------------------------------------ */
/* wire image of one rank: plane 0 = codes (nb * 32*b/8 bytes), plane 1 =
 * fp16 scales at the next 256-byte boundary, plane 2 (asymmetric only) =
 * fp16 zeros at the next 256-byte boundary.  FP: the raw 2n bytes. */

static size_t align256(size_t x) { return (x + 255) / 256 * 256; }
static size_t nblocks(size_t n) { return (n + BLK - 1) / BLK; }

size_t ref_block_code_bytes(int c) { return (size_t)BLK * codec_bits(c) / 8; }
size_t ref_scale_offset(int c, size_t n) {
  return align256(nblocks(n) * ref_block_code_bytes(c));
}
size_t ref_zero_offset(int c, size_t n) {
  return align256(ref_scale_offset(c, n) + 2 * nblocks(n));
}
size_t ref_wire_bytes(int c, size_t n) {
  if (!codec_valid(c)) return 0;
  if (c == C_FP) return 2 * n;
  if (codec_asym(c)) return ref_zero_offset(c, n) + 2 * nblocks(n);
  return ref_scale_offset(c, n) + 2 * nblocks(n);
}

/* code i of a block occupies bits [b*i, b*i+b) of the block's little-endian
 * bitstring (bit 0 = least significant bit of byte 0) */
static void put_code(uint8_t* blk, int b, int i, uint32_t code) {
  for (int j = 0; j < b; j++) {
    int bit = b * i + j;
    if ((code >> j) & 1u) blk[bit / 8] |= (uint8_t)(1u << (bit % 8));
    else blk[bit / 8] &= (uint8_t)~(1u << (bit % 8));
  }
}
static uint32_t get_code(const uint8_t* blk, int b, int i) {
  uint32_t code = 0;
  for (int j = 0; j < b; j++) {
    int bit = b * i + j;
    code |= (uint32_t)((blk[bit / 8] >> (bit % 8)) & 1u) << j;
  }
  return code;
}

/* ------------------------------------------------------------------ */
/* one block: quantize L (1..32) binary32 values.  codes[i] receives the
 * b-bit code (two's complement for symmetric, unsigned for asymmetric, the
 * E4M3 byte for fp8); slots i >= L get 0.  *s and *z receive the binary16
 * scale and zero (z = 0 for symmetric codecs). */
void ref_quantize_block(int c, const float* v, int L, uint32_t* codes,
                        uint16_t* s, uint16_t* z) {
  int b = codec_bits(c);
  float qmax = ref_codec_qmax(c);
  float mx = v[0], mn = v[0];
  for (int i = 1; i < L; i++) {
    if (v[i] > mx) mx = v[i];
    if (v[i] < mn) mn = v[i];
  }
  for (int i = 0; i < BLK; i++) codes[i] = 0;
  *s = 0;
  *z = 0;

  if (!codec_asym(c)) {
    /* symmetric: scale from the absolute maximum; a constant block takes
     * its own magnitude as the scale so that it is reproduced exactly */
    float a = fabsf(mx) > fabsf(mn) ? fabsf(mx) : fabsf(mn);
    if (a == 0.0f) return;                    /* all zero: s = +0, codes 0 */
    float arg = (mx == mn) ? a : a / qmax;    /* one binary32 division */
    *s = ref_ru16(arg);
    float inv = 1.0f / ref_h2f(*s);
    for (int i = 0; i < L; i++) {
      float t = v[i] * inv;
      if (c == C_FP8) {
        codes[i] = ref_e4m3_encode(t);
      } else {
        float q = nearbyintf(t);              /* ties to even */
        if (q > qmax) q = qmax;
        if (q < -qmax) q = -qmax;
        int qi = (int)q;
        codes[i] = (uint32_t)qi & ((1u << b) - 1u);
      }
    }
  } else {
    /* asymmetric: zero = block minimum rounded down to binary16 (a zero
     * minimum is taken as +0), scale = range / qu rounded up */
    if (mn == 0.0f) mn = 0.0f;
    *z = ref_rd16(mn);
    float fz = ref_h2f(*z);
    float d = mx - fz;
    if (!(d > 0.0f)) return;                  /* constant block: s = +0 */
    *s = ref_ru16(d / qmax);
    float inv = 1.0f / ref_h2f(*s);
    for (int i = 0; i < L; i++) {
      float t = (v[i] - fz) * inv;
      float u = nearbyintf(t);
      if (u > qmax) u = qmax;
      if (u < 0.0f) u = 0.0f;
      codes[i] = (uint32_t)(int)u;
    }
  }
}

/* dequantize code i of a block with scale s and zero z: exact product, and
 * for asymmetric one rounded addition of the zero */
float ref_dequant_code(int c, uint32_t code, uint16_t s, uint16_t z) {
  float fs = ref_h2f(s);
  if (c == C_FP8) return ref_e4m3_decode((uint8_t)code) * fs;
  int b = codec_bits(c);
  if (codec_asym(c)) {
    float p = (float)code * fs;
    return p + ref_h2f(z);
  }
  int q = (int)code;
  if (q & (1 << (b - 1))) q -= (1 << b);      /* sign-extend b bits */
  return (float)q * fs;
}

/* ------------------------------------------------------------------ */
/* element conversion for the buffer type */
/* The bf16 -> fp16 cast option of the vLLM quick_all_reduce docs page
 * (QuickAllReduce.init_quick_all_reduce, VLLM_ROCM_QUICK_REDUCE_CAST_BF16_TO_FP16:
 * bf16 inputs are converted to fp16 and the fp16 kernels run).  Reading
 * taken: each bf16 input is rounded to binary16 (nearest even, overflow to
 * inf), the whole allreduce then runs exactly as for binary16 buffers (the FP
 * wire holds binary16), and each binary16 result is rounded to bfloat16. */
static float ld(int dtype, uint16_t x) {
  if (dtype == T_BF16_VIA_FP16) return ref_h2f(ref_f2h(ref_bf2f(x)));
  return dtype == T_BF16 ? ref_bf2f(x) : ref_h2f(x);
}
static uint16_t st(int dtype, float v) {
  if (dtype == T_BF16_VIA_FP16) return ref_f2bf(ref_h2f(ref_f2h(v)));
  return dtype == T_BF16 ? ref_f2bf(v) : ref_f2h(v);
}
/* type of the raw values in an FP wire image */
static int wire_type(int dtype) { return dtype == T_BF16_VIA_FP16 ? T_FP16 : dtype; }

/* write one quantized block k of a wire image from binary32 values */
static void wire_put_block(int c, uint8_t* wire, size_t n, size_t k,
                           const float* v, int L) {
  uint32_t codes[BLK];
  uint16_t s, z;
  ref_quantize_block(c, v, L, codes, &s, &z);
  int b = codec_bits(c);
  uint8_t* blk = wire + k * ref_block_code_bytes(c);
  for (int i = 0; i < BLK; i++) put_code(blk, b, i, codes[i]);
  memcpy(wire + ref_scale_offset(c, n) + 2 * k, &s, 2);
  if (codec_asym(c)) memcpy(wire + ref_zero_offset(c, n) + 2 * k, &z, 2);
}

/* dequantize block k of a wire image to binary32 values */
static void wire_get_block(int c, const uint8_t* wire, size_t n, size_t k,
                           float* v, int L) {
  uint16_t s, z = 0;
  int b = codec_bits(c);
  const uint8_t* blk = wire + k * ref_block_code_bytes(c);
  memcpy(&s, wire + ref_scale_offset(c, n) + 2 * k, 2);
  if (codec_asym(c)) memcpy(&z, wire + ref_zero_offset(c, n) + 2 * k, 2);
  for (int i = 0; i < L; i++)
    v[i] = ref_dequant_code(c, get_code(blk, b, i), s, z);
}

static int block_len(size_t n, size_t k) {
  size_t rest = n - k * BLK;
  return rest < BLK ? (int)rest : BLK;
}
static size_t clamp_hi(size_t n, size_t hi) {
  size_t nb = nblocks(n);
  return hi > nb ? nb : hi;
}
static int args_ok(int c, int dtype, size_t n) {
  return codec_valid(c) && dtype >= T_FP16 && dtype <= T_BF16_VIA_FP16 && n > 0;
}

/* ------------------------------------------------------------------ */
/* the pipeline */

/* stage 0: quantize one rank's buffer x (n raw 16-bit values) into wire */
int ref_quantize(int c, int dtype, const uint16_t* x, size_t n, uint8_t* wire,
                 size_t blk_lo, size_t blk_hi) {
  if (!args_ok(c, dtype, n)) return -1;
  blk_hi = clamp_hi(n, blk_hi);
  for (size_t k = blk_lo; k < blk_hi; k++) {
    int L = block_len(n, k);
    if (c == C_FP) {                          /* FP: the wire is the raw data */
      uint16_t* w = (uint16_t*)wire + k * BLK;
      for (int i = 0; i < L; i++)
        w[i] = st(wire_type(dtype), ld(dtype, x[k * BLK + i]));
      continue;
    }
    float v[BLK];
    for (int i = 0; i < L; i++) v[i] = ld(dtype, x[k * BLK + i]);
    wire_put_block(c, wire, n, k, v, L);
  }
  return 0;
}

/* dequantize one wire image into y (rounded once to the buffer type) */
int ref_dequantize(int c, int dtype, const uint8_t* wire, size_t n,
                   uint16_t* y, size_t blk_lo, size_t blk_hi) {
  if (!args_ok(c, dtype, n)) return -1;
  blk_hi = clamp_hi(n, blk_hi);
  for (size_t k = blk_lo; k < blk_hi; k++) {
    int L = block_len(n, k);
    if (c == C_FP) {
      const uint16_t* w = (const uint16_t*)wire + k * BLK;
      for (int i = 0; i < L; i++) y[k * BLK + i] = st(dtype, ld(wire_type(dtype), w[i]));
      continue;
    }
    float v[BLK];
    wire_get_block(c, wire, n, k, v, L);
    for (int i = 0; i < L; i++) y[k * BLK + i] = st(dtype, v[i]);
  }
  return 0;
}

/* chunk of blocks owned by rank j: [j*bpc, min(nb, (j+1)*bpc)), bpc = ceil(nb/W) */
void ref_chunk(int W, size_t n, int j, size_t* lo, size_t* hi) {
  size_t nb = nblocks(n);
  size_t bpc = (nb + (size_t)W - 1) / (size_t)W;
  size_t a = (size_t)j * bpc, e = a + bpc;
  if (a > nb) a = nb;
  if (e > nb) e = nb;
  *lo = a;
  *hi = e;
}

/* stage 1 (owner reduce) on blocks [blk_lo, blk_hi): dequantize every
 * rank's block, sum in binary32 in rank order 0..W-1, requantize the sums
 * with the same codec (FP: round the sums once to the buffer type). */
int ref_stage1(int c, int dtype, int W, const uint8_t* const* wires, size_t n,
               uint8_t* reduced, size_t blk_lo, size_t blk_hi) {
  if (!args_ok(c, dtype, n) || W < 1) return -1;
  blk_hi = clamp_hi(n, blk_hi);
  for (size_t k = blk_lo; k < blk_hi; k++) {
    int L = block_len(n, k);
    float acc[BLK], v[BLK];
    for (int r = 0; r < W; r++) {
      if (c == C_FP) {
        const uint16_t* xr = (const uint16_t*)wires[r] + k * BLK;
        for (int i = 0; i < L; i++) v[i] = ld(wire_type(dtype), xr[i]);
      } else {
        wire_get_block(c, wires[r], n, k, v, L);
      }
      for (int i = 0; i < L; i++) acc[i] = (r == 0) ? v[i] : acc[i] + v[i];
    }
    if (c == C_FP) {
      uint16_t* out = (uint16_t*)reduced + k * BLK;
      for (int i = 0; i < L; i++) out[i] = st(wire_type(dtype), acc[i]);
    } else {
      wire_put_block(c, reduced, n, k, acc, L);
    }
  }
  return 0;
}

/* stage 2: every rank dequantizes the reduced wire into its own output */
int ref_stage2(int c, int dtype, int W, const uint8_t* reduced, size_t n,
               uint16_t* const* ys, size_t blk_lo, size_t blk_hi) {
  if (W < 1) return -1;
  for (int r = 0; r < W; r++) {
    int rc = ref_dequantize(c, dtype, reduced, n, ys[r], blk_lo, blk_hi);
    if (rc) return rc;
  }
  return 0;
}

/* the whole simulated allreduce of W buffers on blocks [blk_lo, blk_hi):
 * quantize each rank, stage 1, stage 2.  Wire images are allocated here. */
int ref_allreduce(int W, int dtype, int c, const uint16_t* const* xs,
                  uint16_t* const* ys, size_t n, size_t blk_lo, size_t blk_hi) {
  if (!args_ok(c, dtype, n) || W < 1) return -1;
  size_t wb = ref_wire_bytes(c, n);
  uint8_t** wires = (uint8_t**)calloc((size_t)W, sizeof(uint8_t*));
  uint8_t* red = (uint8_t*)calloc(wb, 1);
  int rc = (wires && red) ? 0 : -2;
  for (int r = 0; r < W && rc == 0; r++) {
    wires[r] = (uint8_t*)calloc(wb, 1);
    if (!wires[r]) rc = -2;
    else rc = ref_quantize(c, dtype, xs[r], n, wires[r], blk_lo, blk_hi);
  }
  if (rc == 0)
    rc = ref_stage1(c, dtype, W, (const uint8_t* const*)wires, n, red, blk_lo,
                    blk_hi);
  if (rc == 0) rc = ref_stage2(c, dtype, W, red, n, ys, blk_lo, blk_hi);
  if (wires)
    for (int r = 0; r < W; r++) free(wires[r]);
  free(wires);
  free(red);
  return rc;
}

/* the one-stage (one-shot) allreduce of PR #18473 ("1stage", f16): every
 * rank reads all W buffers and rounds their binary32 sum, taken in rank
 * order 0..W-1, once to the buffer type; no wire format is involved.  On
 * the elements of blocks [blk_lo, blk_hi) (32-element blocks, used here only
 * as the unit of the range). */
int ref_oneshot(int W, int dtype, const uint16_t* const* xs, uint16_t* const* ys,
                size_t n, size_t blk_lo, size_t blk_hi) {
  if (dtype < T_FP16 || dtype > T_BF16_VIA_FP16 || n == 0 || W < 1) return -1;
  blk_hi = clamp_hi(n, blk_hi);
  size_t e_lo = blk_lo * BLK, e_hi = blk_hi * BLK < n ? blk_hi * BLK : n;
  for (size_t i = e_lo; i < e_hi; i++) {
    float acc = ld(dtype, xs[0][i]);
    for (int r = 1; r < W; r++) acc = acc + ld(dtype, xs[r][i]);
    uint16_t y = st(dtype, acc);
    for (int r = 0; r < W; r++) ys[r][i] = y;
  }
  return 0;
}
