// qr_device.h -- device helpers of the two-stage quantized allreduce for
// gfx950: number formats, code packing/unpacking and the block quantizer.
//
// Two work decompositions are used (see qr_kernels.hip):
//   - one lane per 32-element block (stage 1): the block's codes are 16, 24
//     or 32 bytes (one, three or two words in the receive buffer's word-major
//     tiles), its statistics and scale are computed once, in registers, with
//     no cross-lane traffic;
//   - four lanes per block, 8 elements each (stage 0 and stage 2): every lane
//     reads or writes 16 contiguous bytes of 16-bit data, so those planes
//     stream at full coalescing; stage 0 combines the block's max/min across
//     the four lanes with two DPP quad permutes.
//
// The numerics follow the readings taken for the formats named in "Integrate
// quick allreduce and select the best allreduce implementation" (vLLM PR
// #18473, PR description item 2) and "Add quickreduce as alternative to
// custom allreduce" (vLLM PR #16804, PR description): 32-element blocks, a
// binary16 scale rounded up (and a binary16 zero rounded down for the
// asymmetric codecs), codes = clamp(round-half-even(v * (1/scale))),
// binary32 sums.  Every operation below is a single IEEE binary32 operation
// with round-to-nearest-even (the library is built with contraction off and
// denormals kept), so the results are bit-for-bit those of the definition.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qr {

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

enum Codec { kFP = 0, kQ8 = 1, kQ6 = 2, kQ4 = 3, kFP8 = 5,
             kQ8A = 9, kQ6A = 10, kQ4A = 11 };
// buffer types; kBF16H = bfloat16 buffers converted to binary16 on entry
// and back on exit (the bf16 -> fp16 cast option)
enum DType { kF16 = 0, kBF16 = 1, kBF16H = 2 };

constexpr int kBlock = 32;   // elements per block

template <int C>
struct CodecT {
  static constexpr int base = C & 7;
  static constexpr bool asym = (C & 8) != 0;
  static constexpr bool fp8 = C == kFP8;
  static constexpr int bits = base == kQ6 ? 6 : base == kQ4 ? 4 : 8;
  static constexpr float qmax =
      fp8 ? 448.0f
          : asym ? float((1 << bits) - 1) : float((1 << (bits - 1)) - 1);
  static constexpr int block_bytes = kBlock * bits / 8;   // 16, 24, 32
  static constexpr int words = block_bytes / 4;           // 4, 6, 8
  // symmetric 4-bit codes are unpacked as 16*q (see code_values)
  static constexpr float unpack_scale = (!asym && bits == 4) ? 0.0625f : 1.0f;
};

// ---------------------------------------------------------------------------
// number formats

__device__ __forceinline__ float h2f(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);   // exact
}
// binary32 -> binary16, nearest-even, overflow to inf (v_cvt_f16_f32)
__device__ __forceinline__ uint32_t f2h(float f) {
  return __builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float bf2f(uint32_t b) {
  return (float)__builtin_bit_cast(__bf16, (uint16_t)b);      // exact
}
// binary32 -> bfloat16, nearest-even, overflow to inf (v_cvt_pk_bf16_f32;
// for every non-NaN binary32 input this is round-to-nearest-even on the bit
// pattern)
__device__ __forceinline__ uint32_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// a buffer element as binary32; with the cast option, the bfloat16 input is
// first rounded to binary16
template <int D>
__device__ __forceinline__ float ld16(uint32_t bits) {
  if constexpr (D == kBF16H) return h2f(f2h(bf2f(bits)));
  return D == kBF16 ? bf2f(bits) : h2f(bits);
}
// A binary32 value the compiler must produce as such.  Without it, an fma
// (or add) followed by a conversion to binary16 may be merged into one
// mixed-precision instruction (v_fma_mixlo_f16) that rounds the exact result
// once, straight to binary16; the definition rounds to binary32 first, and the
// two differ when the binary32 value lands on a binary16 midpoint.
__device__ __forceinline__ float as_f32(float v) {
  asm("" : "+v"(v));
  return v;
}

// a binary32 result as a buffer element (rounded from the binary32 value);
// with the cast option, rounded to binary16 and that to bfloat16
template <int D>
__device__ __forceinline__ uint32_t st16(float v) {
  v = as_f32(v);
  if constexpr (D == kBF16H) return f2bf(h2f(f2h(v)));
  return D == kBF16 ? f2bf(v) : f2h(v);
}
// two 16-bit values of a packed word
template <int D>
__device__ __forceinline__ uint32_t st16x2(float lo, float hi) {
  return st16<D>(lo) | (st16<D>(hi) << 16);
}

// least binary16 >= v (v >= 0), saturated at 65504: round to nearest, then
// step up one unit where that fell below v
__device__ __forceinline__ uint32_t ru16(float v) {
  v = as_f32(v);
  uint32_t h = f2h(v);
  if (h2f(h) < v) h += 1u;
  return h >= 0x7c00u ? 0x7bffu : h;
}

// greatest binary16 <= v, saturated at -65504
__device__ __forceinline__ uint32_t rd16(float v) {
  v = as_f32(v);
  uint32_t h = f2h(v);
  if (h2f(h) > v) h = (h & 0x8000u) ? h + 1u : (h == 0u ? 0x8001u : h - 1u);
  return (h & 0x7fffu) >= 0x7c00u ? (h & 0x8000u) | 0x7bffu : h;
}

// OCP E4M3FN (bias 7, 3 fraction bits, largest finite 448, 0x7f/0xff NaN).
// gfx950's conversions use this format: v_cvt_pk_fp8_f32 rounds to nearest,
// ties to even, keeps the sign of a zero result, and gives 448 for
// 448 <= |t| <= 464 (NaN above: callers clamp first where that can occur);
// v_cvt_f32_fp8 decodes exactly.
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, uint32_t old, bool hi) {
  return hi ? (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, true)
            : (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, false);
}
template <int Byte>
__device__ __forceinline__ float e4m3_dec(uint32_t word) {
  return __builtin_amdgcn_cvt_f32_fp8((int)word, Byte);
}

// Round-half-even to an integer by one binary32 addition: for |c| <= 2^22,
// c + 1.5*2^23 lies in [2^23, 2^24), where the spacing is 1, so the sum is
// 1.5*2^23 + rint(c) exactly and its low fraction bits hold rint(c) in two's
// complement.
constexpr float kRoundMagic = 12582912.0f;
__device__ __forceinline__ uint32_t rint_bits(float c) {
  return __builtin_bit_cast(uint32_t, c + kRoundMagic);
}

// rint_bits(t)'s low byte written into byte Byte of w in the same
// instruction (an SDWA destination select on the v_add_f32): byte 0 clears
// the other bytes, bytes 1..3 keep them.  One instruction per 8- or 4-bit
// code instead of an add and a funnel shift.
template <int Byte>
__device__ __forceinline__ void rint_byte(uint32_t& w, float t) {
  const float m = kRoundMagic;
  if constexpr (Byte == 0)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD "
        "src1_sel:DWORD" : "=v"(w) : "v"(t), "v"(m));
  else if constexpr (Byte == 1)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:DWORD" : "+v"(w) : "v"(t), "v"(m));
  else if constexpr (Byte == 2)
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:DWORD" : "+v"(w) : "v"(t), "v"(m));
  else
    asm("v_add_f32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD "
        "src1_sel:DWORD" : "+v"(w) : "v"(t), "v"(m));
}

// a / D, correctly rounded, for the integer codecs' divisors (D = 127, 31,
// 7, 255, 63, 15): q0 = a*R with R = RN(1/D), then one residual step
// q0 + RN(a - q0*D)*R with two fused multiply-adds.  For each of these D this
// equals the IEEE quotient for every positive binary32 a (checked
// exhaustively on gfx950 by tests/gpu_arith_check.hip).  fp8's divisor 448
// does not have this property for subnormal a and keeps the IEEE division.
template <int D>
__device__ __forceinline__ float div_by(float a) {
  if constexpr (D == 448) {
    return a / 448.0f;
  } else {
    constexpr float R = 1.0f / (float)D;
    const float q0 = a * R;
    return __builtin_fmaf(__builtin_fmaf(-q0, (float)D, a), R, q0);
  }
}

// 1/s, correctly rounded, for s a positive finite binary16 value: the
// hardware reciprocal (within 1 ulp) and one Newton step.  Equals the IEEE
// quotient for every such s (checked exhaustively by
// tests/gpu_arith_check.hip).
__device__ __forceinline__ float recip_f16(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  return __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
}

// value held by another lane of this lane's quad (DPP quad permute)
template <int Ctrl>
__device__ __forceinline__ float quad_perm(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), Ctrl, 0xf, 0xf, false));
}
template <int Ctrl>
__device__ __forceinline__ uint32_t quad_perm_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, Ctrl, 0xf, 0xf, false);
}
constexpr int kSwap1 = 0xb1;    // quad_perm [1,0,3,2]
constexpr int kSwap2 = 0x4e;    // quad_perm [2,3,0,1]
constexpr int kFromOdd = 0xf5;  // quad_perm [1,1,3,3]
constexpr int kFromNext = 0xf9; // quad_perm [1,2,3,3]

// ---------------------------------------------------------------------------
// code packing: code i at bits [b*i, b*i+b) of a little-endian bitstring

// Packs N b-bit codes, code i taken from the low bits of c[i] (higher bits
// are ignored), into ceil(N*b/32) words: each code is shifted in at the top
// of the current word with one funnel shift (v_alignbit_b32); a code that
// straddles two words is shifted in as two pieces.  The bits of a last,
// partly filled word beyond N*b are zero.
template <int B, int N>
__device__ __forceinline__ void pack_bits(const uint32_t (&c)[N],
                                          uint32_t (&w)[(N * B + 31) / 32]) {
  constexpr int nw = (N * B + 31) / 32;
#pragma unroll
  for (int k = 0; k < nw; k++) {
    uint32_t acc = 0;
    int filled = 0;
#pragma unroll
    for (int i = 0; i < N; i++) {
      const int lo = B * i, hi = lo + B;             // code i's bit range
      const int a = lo > 32 * k ? lo : 32 * k;       // its part in word k
      const int e = hi < 32 * (k + 1) ? hi : 32 * (k + 1);
      if (a < e) {
        const uint32_t piece = a > lo ? c[i] >> (a - lo) : c[i];
        acc = __builtin_amdgcn_alignbit(piece, acc, e - a);
        filled += e - a;
      }
    }
    w[k] = filled == 32 ? acc : acc >> (32 - filled);
  }
}

// Scaled values t[i] (v*inv, or (v-z)*inv) -> packed codes.  `sat` marks a
// block whose scale or zero saturated at the binary16 range, the only case in
// which t can leave the code range (see block_params): then t is clamped
// first, as the definition does (one v_med3_f32: t is never NaN, the inputs
// being finite), otherwise the clamp is the identity and skipped.
template <int C, int N>
__device__ __forceinline__ void encode(float (&t)[N], bool sat,
                                       uint32_t (&w)[(N * CodecT<C>::bits + 31) / 32]) {
  using T = CodecT<C>;
  if (sat) {
    const float lo = T::asym ? 0.0f : -T::qmax;
#pragma unroll
    for (int i = 0; i < N; i++) t[i] = __builtin_amdgcn_fmed3f(t[i], lo, T::qmax);
  }
  if constexpr (T::fp8) {
#pragma unroll
    for (int k = 0; k < N / 4; k++)
      w[k] = e4m3_pack2(t[4 * k + 2], t[4 * k + 3],
                        e4m3_pack2(t[4 * k], t[4 * k + 1], 0u, false), true);
  } else if constexpr (T::bits == 8) {
#pragma unroll
    for (int k = 0; k < N / 4; k++) {
      rint_byte<0>(w[k], t[4 * k]);
      rint_byte<1>(w[k], t[4 * k + 1]);
      rint_byte<2>(w[k], t[4 * k + 2]);
      rint_byte<3>(w[k], t[4 * k + 3]);
    }
  } else if constexpr (T::bits == 4) {
    // even codes as the bytes of `ev`, odd codes as the bytes of `od`, then
    // the low nibbles interleaved: code i at bits [4i, 4i+4)
#pragma unroll
    for (int k = 0; k < N / 8; k++) {
      uint32_t ev, od;
      rint_byte<0>(ev, t[8 * k]);
      rint_byte<1>(ev, t[8 * k + 2]);
      rint_byte<2>(ev, t[8 * k + 4]);
      rint_byte<3>(ev, t[8 * k + 6]);
      rint_byte<0>(od, t[8 * k + 1]);
      rint_byte<1>(od, t[8 * k + 3]);
      rint_byte<2>(od, t[8 * k + 5]);
      rint_byte<3>(od, t[8 * k + 7]);
      w[k] = (ev & 0x0f0f0f0fu) | ((od << 4) & 0xf0f0f0f0u);
    }
  } else {
    uint32_t c[N];
#pragma unroll
    for (int i = 0; i < N; i++) c[i] = rint_bits(t[i]);
    pack_bits<T::bits, N>(c, w);
  }
}

// a & m computed once per word.  Opaque to the optimizer on purpose: seen
// through, the mask is folded into every byte extraction below, which then
// takes two instructions per code instead of one sign- or zero-extending byte
// select inside the conversion (SDWA).
__device__ __forceinline__ uint32_t and_word(uint32_t a, uint32_t m) {
  uint32_t r;
  asm("v_and_b32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(m));
  return r;
}

// Code values of N codes packed from bit 0 of w, as binary32: q (or 16*q for
// symmetric 4-bit codes, so that a sign-extended byte select does the
// unpacking), u for asymmetric codes, the decoded value for fp8.  The value
// of a code is then cv[i] * (s * unpack_scale) (+ z): the product is exact.
template <int C, int N>
__device__ __forceinline__ void code_values(const uint32_t* w, float (&cv)[N]) {
  using T = CodecT<C>;
  constexpr int b = T::bits;
  if constexpr (T::fp8) {
#pragma unroll
    for (int k = 0; k < N / 4; k++) {
      cv[4 * k] = e4m3_dec<0>(w[k]);
      cv[4 * k + 1] = e4m3_dec<1>(w[k]);
      cv[4 * k + 2] = e4m3_dec<2>(w[k]);
      cv[4 * k + 3] = e4m3_dec<3>(w[k]);
    }
  } else if constexpr (b == 8) {
#pragma unroll
    for (int k = 0; k < N / 4; k++)
#pragma unroll
      for (int m = 0; m < 4; m++)
        cv[4 * k + m] = T::asym ? (float)((w[k] >> (8 * m)) & 0xffu)
                                : (float)(int)(int8_t)(w[k] >> (8 * m));
  } else if constexpr (b == 4) {
#pragma unroll
    for (int k = 0; k < N / 8; k++) {
      // even codes of the word in the bytes of `ev`, odd codes in `od`
      const uint32_t ev = T::asym ? and_word(w[k], 0x0f0f0f0fu)
                                  : and_word(w[k] << 4, 0xf0f0f0f0u);
      const uint32_t od = T::asym ? and_word(w[k] >> 4, 0x0f0f0f0fu)
                                  : and_word(w[k], 0xf0f0f0f0u);
#pragma unroll
      for (int m = 0; m < 4; m++) {
        cv[8 * k + 2 * m] = T::asym ? (float)((ev >> (8 * m)) & 0xffu)
                                    : (float)(int)(int8_t)(ev >> (8 * m));
        cv[8 * k + 2 * m + 1] = T::asym ? (float)((od >> (8 * m)) & 0xffu)
                                        : (float)(int)(int8_t)(od >> (8 * m));
      }
    }
  } else {                                           // 6-bit
#pragma unroll
    for (int i = 0; i < N; i++) {
      const int off = b * i, k = off >> 5, sh = off & 31;
      const uint32_t x = (sh + b <= 32) ? w[k] : __builtin_amdgcn_alignbit(w[k + 1], w[k], sh);
      const int s = (sh + b <= 32) ? sh : 0;
      // (the bit-field builtins return unsigned: the signed field must be
      // converted as int)
      cv[i] = T::asym ? (float)__builtin_amdgcn_ubfe(x, s, b)
                      : (float)(int)__builtin_amdgcn_sbfe((int)x, s, b);
    }
  }
}

// ---------------------------------------------------------------------------
// block quantizer

// max and min of p[0..8), or (-inf, +inf) when the group holds no value
__device__ __forceinline__ void group_max_min(const float* p, bool any, float& mx,
                                              float& mn) {
  // chains, so that each pair of new values takes one v_max3/v_min3
  mx = fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(fmaxf(p[0], p[1]), p[2]), p[3]), p[4]), p[5]),
                   p[6]), p[7]);
  mn = fminf(fminf(fminf(fminf(fminf(fminf(fminf(p[0], p[1]), p[2]), p[3]), p[4]), p[5]),
                   p[6]), p[7]);
  mx = any ? mx : -__builtin_inff();
  mn = any ? mn : __builtin_inff();
}

// One rank's term of the stage-1 sum, in rank order: acc = x_0 for the first
// rank, acc = acc + x_r after it.  A symmetric/fp8 term cv*s is exact, so
// acc + cv*s is one fused multiply-add; an asymmetric term cv*s + z is
// rounded once (the product is exact) and then added.
template <int C, int N>
__device__ __forceinline__ void add_rank(float (&acc)[N], const float (&cv)[N], float s, float z,
                                         bool first) {
#pragma unroll
  for (int i = 0; i < N; i++) {
    if constexpr (CodecT<C>::asym) {
      const float x = __builtin_fmaf(cv[i], s, z);
      acc[i] = first ? x : acc[i] + x;
    } else {
      acc[i] = first ? cv[i] * s : __builtin_fmaf(cv[i], s, acc[i]);
    }
  }
}

// fma(h, S, z) in binary32 with h the binary16 value in half Hi of `h2`
// (v_fma_mix_f32): the conversion of h is exact and the result is rounded
// once.  Written as inline asm: the compiler converts the half with a
// separate instruction instead.
template <bool Hi>
__device__ __forceinline__ float fma_mix16(uint32_t h2, float S, float z) {
  float r;
  if constexpr (Hi)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
        : "=v"(r) : "v"(h2), "v"(S), "v"(z));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,0]"
        : "=v"(r) : "v"(h2), "v"(S), "v"(z));
  return r;
}

// q/16 for the signed 4-bit field in bits [0, 4) of byte Byte of w
// (v_cvt_off_f32_i4 with an SDWA byte select): exact, and the other 28 bits
// of w are ignored.  One instruction per symmetric 4-bit code: the even code
// of a byte is its low nibble, the odd code the low nibble of the same byte
// of w >> 4.
template <int Byte>
__device__ __forceinline__ float off_i4(uint32_t w) {
  float r;
  if constexpr (Byte == 0)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_0"
        : "=v"(r) : "v"(w));
  else if constexpr (Byte == 1)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_1"
        : "=v"(r) : "v"(w));
  else if constexpr (Byte == 2)
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_2"
        : "=v"(r) : "v"(w));
  else
    asm("v_cvt_off_f32_i4_sdwa %0, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3"
        : "=v"(r) : "v"(w));
  return r;
}

// bit 5 (the sign bit) of every 6-bit field of a block's 192-bit string, as
// it falls in word k
constexpr uint32_t six_sign_mask(int k) {
  uint32_t m = 0;
  for (int b = 5; b < 192; b += 6)
    if (b >= 32 * k && b < 32 * k + 32) m |= 1u << (b - 32 * k);
  return m;
}

// add_rank on the rank's code words directly.  Asymmetric 4-bit codes
// (unsigned) are masked into the two 16-bit halves of a word, where a field
// f < 1024 reads as the binary16 subnormal f * 2^-24; with the scale taken
// as s * 2^24 (s * 2^20 for a code shifted up by 4 bits) one v_fma_mix_f32
// gives the term u*s + z, exactly as the definition rounds it (the product
// is exact).  This replaces a conversion and an FMA per code (stage 1 3-6%
// faster; for 8-bit codes the same scheme measured no gain).
// Symmetric 4-bit codes (s here is the scale times 1/16, unpack_scale):
//   - first rank: flipping bit 3 of every nibble gives u = q + 8 in
//     [0, 16), read as a binary16 subnormal as above; fma(u, s*2^24, -8s) is
//     u*s - 8s = q*s, exact, so one v_fma_mix_f32 per code forms the term.
//   - later ranks: off_i4 gives q/16 in one instruction per code, and
//     fma(q/16, 16s, acc) rounds acc + q*s once (the product is exact).
// 6-bit codes, read the same way: a field extracted zero-extended is the
// binary16 subnormal f * 2^-24, and one v_fma_mix_f32 with s * 2^24 forms the
// term.  Asymmetric: u*s + z for every rank (instead of a convert and an
// FMA).  Symmetric, first rank: with bit 5 of every field flipped (one XOR
// per word) the field is q + 32, and fma(q + 32, s, -32s) = q*s exactly.
// Other codecs, and later ranks of symmetric 6-bit codes, go through
// code_values and add_rank.
template <int C, int N>
__device__ __forceinline__ void add_codes(float (&acc)[N], const uint32_t* w, float s, float z,
                                          bool first) {
  using T = CodecT<C>;
  if constexpr (!T::asym && T::bits == 4) {
    // s = scale / 16 (exact); every constant below is a power-of-two multiple
    if (first) {
      const float S0 = s * 268435456.0f, S4 = s * 16777216.0f;     // scale * 2^24, * 2^20
      const float Z = s * -128.0f;                                   // -8 * scale
#pragma unroll
      for (int k = 0; k < N / 8; k++) {
        const uint32_t x = w[k] ^ 0x88888888u;
        const uint32_t a = x & 0x000f000fu, b = x & 0x00f000f0u;
        const uint32_t c = (x >> 8) & 0x000f000fu, d = (x >> 8) & 0x00f000f0u;
        acc[8 * k + 0] = fma_mix16<false>(a, S0, Z);
        acc[8 * k + 4] = fma_mix16<true>(a, S0, Z);
        acc[8 * k + 1] = fma_mix16<false>(b, S4, Z);
        acc[8 * k + 5] = fma_mix16<true>(b, S4, Z);
        acc[8 * k + 2] = fma_mix16<false>(c, S0, Z);
        acc[8 * k + 6] = fma_mix16<true>(c, S0, Z);
        acc[8 * k + 3] = fma_mix16<false>(d, S4, Z);
        acc[8 * k + 7] = fma_mix16<true>(d, S4, Z);
      }
    } else {
      const float S = s * 256.0f;                                    // 16 * scale
#pragma unroll
      for (int k = 0; k < N / 8; k++) {
        const uint32_t h = w[k] >> 4;
        const float cv[8] = {off_i4<0>(w[k]), off_i4<0>(h), off_i4<1>(w[k]), off_i4<1>(h),
                             off_i4<2>(w[k]), off_i4<2>(h), off_i4<3>(w[k]), off_i4<3>(h)};
#pragma unroll
        for (int i = 0; i < 8; i++) acc[8 * k + i] = __builtin_fmaf(cv[i], S, acc[8 * k + i]);
      }
    }
  } else if constexpr (T::bits == 6) {
    if (T::asym || first) {
      constexpr int nw = (N * 6 + 31) / 32;
      uint32_t x[nw];
#pragma unroll
      for (int k = 0; k < nw; k++) x[k] = T::asym ? w[k] : w[k] ^ six_sign_mask(k);
      const float S = s * 16777216.0f;                               // s * 2^24
      const float Z = T::asym ? z : s * -32.0f;
#pragma unroll
      for (int i = 0; i < N; i++) {
        const int off = 6 * i, k = off >> 5, sh = off & 31;
        const uint32_t f = sh + 6 <= 32
                               ? __builtin_amdgcn_ubfe(x[k], sh, 6)
                               : __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(x[k + 1], x[k], sh),
                                                       0, 6);
        const float t = fma_mix16<false>(f, S, Z);
        acc[i] = first ? t : acc[i] + t;
      }
    } else {
      float cv[N];
      code_values<C, N>(w, cv);
      add_rank<C, N>(acc, cv, s, z, false);
    }
  } else if constexpr (T::asym && T::bits == 4) {
    const float S0 = s * 16777216.0f, S4 = s * 1048576.0f;        // s * 2^24, s * 2^20
#pragma unroll
    for (int k = 0; k < N / 8; k++) {
      // code i of the word sits at bits 4i: halves of a = codes 0 and 4,
      // b = 1 and 5 (shifted by 4), c = 2 and 6, d = 3 and 7 (shifted by 4)
      const uint32_t a = w[k] & 0x000f000fu, b = w[k] & 0x00f000f0u;
      const uint32_t c = (w[k] >> 8) & 0x000f000fu, d = (w[k] >> 8) & 0x00f000f0u;
      float x[8];
      x[0] = fma_mix16<false>(a, S0, z);
      x[4] = fma_mix16<true>(a, S0, z);
      x[1] = fma_mix16<false>(b, S4, z);
      x[5] = fma_mix16<true>(b, S4, z);
      x[2] = fma_mix16<false>(c, S0, z);
      x[6] = fma_mix16<true>(c, S0, z);
      x[3] = fma_mix16<false>(d, S4, z);
      x[7] = fma_mix16<true>(d, S4, z);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[8 * k + i] = first ? x[i] : acc[8 * k + i] + x[i];
    }
  } else {
    float cv[N];
    code_values<C, N>(w, cv);
    add_rank<C, N>(acc, cv, s, z, first);
  }
}

// The binary16 value in the low half of h, times k, in binary32 (one
// v_fma_mix_f32: the conversion is exact, and so is the product for k a power
// of two).  The addend is -0 (the inline constant 0, negated by the source
// modifier), so that -0 * k stays -0 (with +0 it would round to +0).  The
// high half of h is ignored.
__device__ __forceinline__ float h2f_times(uint32_t h, float k) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, neg(0) op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h), "v"(k));
  return r;
}

// fma_mix16 with the addend given as the binary16 value in the low half of
// zh, converted exactly inside the same instruction: fma(h, S, z) rounded
// once, as fma_mix16(h2, S, h2f(zh)).
template <bool Hi>
__device__ __forceinline__ float fma_mix16h(uint32_t h2, float S, uint32_t zh) {
  float r;
  if constexpr (Hi)
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,1]"
        : "=v"(r) : "v"(h2), "v"(S), "v"(zh));
  else
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,0,0] op_sel_hi:[1,0,1]"
        : "=v"(r) : "v"(h2), "v"(S), "v"(zh));
  return r;
}

// add_codes for the asymmetric 4- and 6-bit codes with the rank's scale and
// zero taken as their binary16 bits: S0 = s * 2^24 and S4 = s * 2^20 come from
// one v_fma_mix_f32 each (h2f_times) and the zero enters every term as a
// binary16 operand (fma_mix16h), which saves the two conversions and two
// multiplies per rank that the binary32 forms need.  The terms and sums are
// those of add_codes, bit for bit.
template <int C, int N>
__device__ __forceinline__ void add_codes_asym(float (&acc)[N], const uint32_t* w, float S0,
                                               float S4, uint32_t zh, bool first) {
  using T = CodecT<C>;
  static_assert(T::asym && (T::bits == 4 || T::bits == 6), "asymmetric 4- and 6-bit codes");
  if constexpr (T::bits == 4) {
#pragma unroll
    for (int k = 0; k < N / 8; k++) {
      const uint32_t a = w[k] & 0x000f000fu, b = w[k] & 0x00f000f0u;
      const uint32_t c = (w[k] >> 8) & 0x000f000fu, d = (w[k] >> 8) & 0x00f000f0u;
      float x[8];
      x[0] = fma_mix16h<false>(a, S0, zh);
      x[4] = fma_mix16h<true>(a, S0, zh);
      x[1] = fma_mix16h<false>(b, S4, zh);
      x[5] = fma_mix16h<true>(b, S4, zh);
      x[2] = fma_mix16h<false>(c, S0, zh);
      x[6] = fma_mix16h<true>(c, S0, zh);
      x[3] = fma_mix16h<false>(d, S4, zh);
      x[7] = fma_mix16h<true>(d, S4, zh);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[8 * k + i] = first ? x[i] : acc[8 * k + i] + x[i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < N; i++) {
      const int off = 6 * i, k = off >> 5, sh = off & 31;
      const uint32_t f = sh + 6 <= 32
                             ? __builtin_amdgcn_ubfe(w[k], sh, 6)
                             : __builtin_amdgcn_ubfe(__builtin_amdgcn_alignbit(w[k + 1], w[k], sh),
                                                     0, 6);
      const float t = fma_mix16h<false>(f, S0, zh);
      acc[i] = first ? t : acc[i] + t;
    }
  }
}

// max and min of a whole block p[0..32): one chain each, so that every pair
// of new values takes one v_max3/v_min3
__device__ __forceinline__ void block_max_min(const float* p, float& mx, float& mn) {
  mx = fmaxf(p[0], p[1]);
  mn = fminf(p[0], p[1]);
#pragma unroll
  for (int i = 2; i < kBlock; i++) {
    mx = fmaxf(mx, p[i]);
    mn = fminf(mn, p[i]);
  }
}

// Scale and zero of a block from its max and min, and the parameters that
// turn a value into t = (v - tz) * inv.
template <int C>
struct BlockParams {
  uint32_t s = 0, z = 0;   // binary16 scale and zero (z = 0: symmetric)
  float tz = 0.0f;         // subtracted before scaling (the zero)
  float inv = 0.0f;        // 1/s, or 0 for a block whose codes are all 0
  bool sat = false;        // scale or zero saturated at the binary16 range
};

template <int C>
__device__ __forceinline__ BlockParams<C> block_params(float mx, float mn) {
  using T = CodecT<C>;
  BlockParams<C> p;
  // t lies within qmax*(1 + 3*2^-24) < qmax + 1/2 of the code range whenever
  // the scale (and zero) are not saturated: s >= f32(range/qmax) and 1/s is
  // rounded once.  Rounding t then already gives a code in range; the clamp
  // of the definition is only executed for saturated blocks (|x| beyond the
  // binary16 range), where it matters.
  if constexpr (!T::asym) {
    const float a = fmaxf(fabsf(mx), fabsf(mn));
    // a constant block takes its own magnitude as the scale
    const float arg = (mx == mn) ? a : div_by<(int)T::qmax>(a);
    p.s = a != 0.0f ? ru16(arg) : 0u;
    // all-zero block: scale +0 and codes 0 (inv = 0 gives t = +-0)
    p.inv = a != 0.0f ? recip_f16(h2f(p.s)) : 0.0f;
    p.sat = p.s == 0x7bffu;
  } else {
    if (mn == 0.0f) mn = 0.0f;                // a zero minimum is +0
    p.z = rd16(mn);
    p.tz = h2f(p.z);
    const float d = mx - p.tz;
    p.s = d > 0.0f ? ru16(div_by<(int)T::qmax>(d)) : 0u;
    // d <= 0 (constant block): scale +0, codes 0 (inv = 0 gives t = +-0)
    p.inv = d > 0.0f ? recip_f16(h2f(p.s)) : 0.0f;
    p.sat = p.s == 0x7bffu || p.z == 0xfbffu;
  }
  return p;
}

// Quantizes N values of a block with its parameters.  For fp8 an all-zero
// block (s = 0) must give code 0x00 even for -0 inputs: the codes are masked.
template <int C, int N>
__device__ __forceinline__ void quantize_values(const float (&v)[N], const BlockParams<C>& p,
                                                uint32_t (&w)[(N * CodecT<C>::bits + 31) / 32]) {
  using T = CodecT<C>;
  float t[N];
#pragma unroll
  for (int i = 0; i < N; i++) t[i] = T::asym ? (v[i] - p.tz) * p.inv : v[i] * p.inv;
  encode<C, N>(t, p.sat, w);
  if constexpr (T::fp8) {
    const uint32_t keep = p.s != 0u ? 0xffffffffu : 0u;
#pragma unroll
    for (int k = 0; k < N / 4; k++) w[k] &= keep;
  }
}

}  // namespace qr
