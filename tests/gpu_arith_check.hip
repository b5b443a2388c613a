// gpu_arith_check.hip -- test program: exhaustive checks, on the GPU, of the
// arithmetic identities the kernels in quantized_two_stage_amd/csrc rely on.
// Each device helper of qr_device.h is compared with a plain reference
// written here, for every input in its domain:
//   1. div_by<D>(a) == a / D (IEEE) for every positive finite binary32 a,
//      D = 127, 31, 7, 255, 63, 15
//   2. recip_f16(s) == 1 / s (IEEE) for every positive finite binary16 s
//   3. rint_bits(c) holds round-half-even(c) in its low bits, |c| <= 256
//   4. e4m3_pack2 (v_cvt_pk_fp8_f32) == nearest-even E4M3FN with saturation
//      for every binary32 |t| <= 464, both halves of the word, both signs
//   5. e4m3_dec<k> (v_cvt_f32_fp8) == exact E4M3FN value, all codes, k = 0..3
//   6. f2bf (v_cvt_pk_bf16_f32) == nearest-even on the bit pattern for every
//      non-NaN binary32
//   7. f2h (v_cvt_f16_f32) == nearest-even binary16 (subnormals, overflow to
//      inf) for every non-NaN binary32, against an integer conversion written
//      from the two formats' definitions
//   8. fma_mix16<Hi> (v_fma_mix_f32 on a binary16 half) reads every non-NaN
//      binary16 in either half exactly, whatever the other half holds
//   9. fma_mix16<Hi>(f, S, z) == fmaf(f * 2^-24, S, z) for every field
//      f < 1024 (the subnormals the asymmetric codes are read as), every
//      positive finite binary16 scale s with S = s * 2^24 and S = s * 2^20,
//      and a binary16 zero point z drawn per case
//  10. rint_byte<B> (an SDWA byte write of the rounding add) holds
//      round-half-even(c) in byte B, keeps the other bytes (B > 0) or clears
//      them (B = 0), for every |c| <= 256
//  11. off_i4<B>(w) (v_cvt_off_f32_i4, SDWA byte B) == q/16 for the signed
//      4-bit field in bits [8B, 8B+4) of w, for every 32-bit w and B = 0..3
//  12. the symmetric 4-bit first-rank term: fma_mix16 on the offset field
//      (bit 3 flipped) at bit 0 or bit 4 of either half, with the scale
//      constants add_codes uses, == q * s exactly, for every code q and every
//      positive finite binary16 scale s
//  13. the same for the symmetric 6-bit first-rank term: the field with bit 5
//      flipped, read as a binary16 subnormal, fma'd with s * 2^24 and -32s,
//      == q * s exactly for every 6-bit code q and every positive finite
//      binary16 scale s
//  14. h2f_times(h, k) (v_fma_mix_f32 reading the low half) == h2f(h) * k
//      exactly for every non-NaN binary16 h, k = 2^24 and 2^20, whatever the
//      high half holds
//  15. fma_mix16h<Hi>(f, S, zh) (the addend read as binary16) ==
//      fmaf(f * 2^-24, S, h2f(zh)) for every field f < 1024 in either half and
//      every finite binary16 zh, with S = s * 2^24 or s * 2^20 for a binary16
//      scale s drawn per case, junk in the other halves
// Prints one line per check and exits 0 only if every count is zero.
// Grid-stride loops with explicit bounds; counters in one small array.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "../quantized_two_stage_amd/csrc/qr_device.h"

using namespace qr;

enum { kDiv = 0, kRcp = 6, kRint = 7, kEnc = 8, kDec = 9, kBf = 10, kF2h = 11, kMixCvt = 12,
       kMixFma = 13, kRByte = 14, kOffI4 = 15, kSymMix = 16, kSym6Mix = 17, kH2fTimes = 18,
       kMixFmaH = 19, kSlots = 20 };

__device__ void miss(uint32_t* c, int slot) { atomicAdd(&c[slot], 1u); }

template <int D>
__global__ void k_div(uint32_t* c, int slot) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x + 1; i < 0x7f800000ull;
       i += stride) {
    const float a = __builtin_bit_cast(float, (uint32_t)i);
    if (__builtin_bit_cast(uint32_t, div_by<D>(a)) != __builtin_bit_cast(uint32_t, a / (float)D))
      miss(c, slot);
  }
}

__global__ void k_rcp(uint32_t* c) {
  const uint32_t h = blockIdx.x * blockDim.x + threadIdx.x + 1;
  if (h >= 0x7c00u) return;
  const float s = h2f(h);
  if (__builtin_bit_cast(uint32_t, recip_f16(s)) != __builtin_bit_cast(uint32_t, 1.0f / s))
    miss(c, kRcp);
}

__global__ void k_rint(uint32_t* c) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2ull * 0x43800001ull;
       i += stride) {
    const uint32_t u = (uint32_t)(i % 0x43800001ull) | (i >= 0x43800001ull ? 0x80000000u : 0u);
    const float x = __builtin_bit_cast(float, u);         // |x| <= 256
    const int want = (int)__builtin_rintf(x);
    if ((rint_bits(x) & 0x3ffu) != ((uint32_t)want & 0x3ffu)) miss(c, kRint);
  }
}

// reference E4M3FN encoder: nearest, ties to even, saturating at 448,
// sign kept; from the format's value grid
__device__ uint32_t e4m3_ref(float t) {
  const uint32_t u = __builtin_bit_cast(uint32_t, t);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(t);
  if (a >= 448.0f) return sign | 0x7eu;
  const int e = a < 0.015625f ? -6 : (int)((__builtin_bit_cast(uint32_t, a) >> 23) & 0xff) - 127;
  const float step = __builtin_ldexpf(1.0f, e - 3);       // grid spacing at a
  const float m = __builtin_rintf(a / step);              // a/step is exact
  const float r = m * step;                               // exact
  if (r == 0.0f) return sign;
  if (r < 0.015625f) return sign | (uint32_t)(r * 512.0f);
  const int er = (int)((__builtin_bit_cast(uint32_t, r) >> 23) & 0xff) - 127;
  const uint32_t frac = (__builtin_bit_cast(uint32_t, r) >> 20) & 7u;
  return sign | ((uint32_t)(er + 7) << 3) | frac;
}

__global__ void k_enc(uint32_t* c) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  const uint64_t end = 0x43e80001ull;                     // |t| <= 464
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < end; i += stride) {
    const float t = __builtin_bit_cast(float, (uint32_t)i);
    const uint32_t lo = e4m3_pack2(t, -t, 0x5a5a0000u, false);
    const uint32_t hi = e4m3_pack2(-t, t, 0x00003c3cu, true);
    const uint32_t rp = e4m3_ref(t), rn = e4m3_ref(-t);
    if (lo != (0x5a5a0000u | rp | (rn << 8)) || hi != (0x00003c3cu | (rn << 16) | (rp << 24)))
      miss(c, kEnc);
  }
}

__global__ void k_dec(uint32_t* c) {
  const uint32_t code = threadIdx.x;                      // 0..255
  if (code >= 256u || (code & 0x7fu) == 0x7fu) return;    // NaN codes
  const uint32_t e = (code >> 3) & 0xfu, m = code & 7u;
  float v = e == 0 ? __builtin_ldexpf((float)m, -9) : __builtin_ldexpf(1.0f + m / 8.0f, (int)e - 7);
  v = (code & 0x80u) ? -v : v;
  const uint32_t want = __builtin_bit_cast(uint32_t, v);
  const uint32_t w = 0x11223344u;
  if (__builtin_bit_cast(uint32_t, e4m3_dec<0>((w & 0xffffff00u) | code)) != want) miss(c, kDec);
  if (__builtin_bit_cast(uint32_t, e4m3_dec<1>((w & 0xffff00ffu) | (code << 8))) != want) miss(c, kDec);
  if (__builtin_bit_cast(uint32_t, e4m3_dec<2>((w & 0xff00ffffu) | (code << 16))) != want) miss(c, kDec);
  if (__builtin_bit_cast(uint32_t, e4m3_dec<3>((w & 0x00ffffffu) | (code << 24))) != want) miss(c, kDec);
}

__device__ uint32_t hash32(uint32_t x) {
  x ^= x >> 16; x *= 0x7feb352du; x ^= x >> 15; x *= 0x846ca68bu; x ^= x >> 16;
  return x;
}

__global__ void k_rint_byte(uint32_t* c) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < 2ull * 0x43800001ull;
       i += stride) {
    const uint32_t u = (uint32_t)(i % 0x43800001ull) | (i >= 0x43800001ull ? 0x80000000u : 0u);
    const float x = __builtin_bit_cast(float, u);         // |x| <= 256
    const uint32_t want = (uint32_t)(int)__builtin_rintf(x) & 0xffu;
    const uint32_t junk = hash32(u);
    uint32_t w0 = junk, w1 = junk, w2 = junk, w3 = junk;
    rint_byte<0>(w0, x);
    rint_byte<1>(w1, x);
    rint_byte<2>(w2, x);
    rint_byte<3>(w3, x);
    if (w0 != want) miss(c, kRByte);
    if (w1 != ((junk & 0xffff00ffu) | (want << 8))) miss(c, kRByte);
    if (w2 != ((junk & 0xff00ffffu) | (want << 16))) miss(c, kRByte);
    if (w3 != ((junk & 0x00ffffffu) | (want << 24))) miss(c, kRByte);
  }
}

__global__ void k_mix_cvt(uint32_t* c) {
  const uint32_t p = blockIdx.x * blockDim.x + threadIdx.x;     // 0..65535
  if (p >= 65536u || (p & 0x7fffu) > 0x7c00u) return;             // NaN patterns
  const uint32_t want = __builtin_bit_cast(uint32_t, h2f(p));
  const uint32_t junk = hash32(p) & 0xffffu;
  if (__builtin_bit_cast(uint32_t, fma_mix16<false>((junk << 16) | p, 1.0f, -0.0f)) != want)
    miss(c, kMixCvt);
  if (__builtin_bit_cast(uint32_t, fma_mix16<true>((p << 16) | junk, 1.0f, -0.0f)) != want)
    miss(c, kMixCvt);
}

__global__ void k_mix_fma(uint32_t* c) {
  const uint64_t n = 2ull * 0x7bffull * 1024ull;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t f = (uint32_t)(i & 1023u);
    const uint32_t sb = (uint32_t)((i >> 10) % 0x7bffull) + 1u;     // 0x0001 .. 0x7bff
    const bool shifted = i >= n / 2;
    const float S = h2f(sb) * (shifted ? 1048576.0f : 16777216.0f);
    uint32_t zb = hash32((uint32_t)i) & 0xffffu;
    if ((zb & 0x7fffu) >= 0x7c00u) zb &= 0x83ffu;                    // keep z finite
    const float z = h2f(zb);
    const float want = __builtin_fmaf((float)f * 5.9604644775390625e-8f, S, z);   // f * 2^-24
    const uint32_t junk = hash32((uint32_t)i ^ 0x9e3779b9u) & 0xffffu;
    if (__builtin_bit_cast(uint32_t, fma_mix16<false>((junk << 16) | f, S, z)) !=
        __builtin_bit_cast(uint32_t, want))
      miss(c, kMixFma);
    if (__builtin_bit_cast(uint32_t, fma_mix16<true>((f << 16) | junk, S, z)) !=
        __builtin_bit_cast(uint32_t, want))
      miss(c, kMixFma);
  }
}

__global__ void k_off_i4(uint32_t* c) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32); i += stride) {
    const uint32_t w = (uint32_t)i;
    const float got[4] = {off_i4<0>(w), off_i4<1>(w), off_i4<2>(w), off_i4<3>(w)};
    for (int b = 0; b < 4; b++) {
      const int q = (int)((w >> (8 * b)) & 0xfu) - (int)((w >> (8 * b)) & 0x8u) * 2;
      if (__builtin_bit_cast(uint32_t, got[b]) != __builtin_bit_cast(uint32_t, (float)q / 16.0f))
        miss(c, kOffI4);
    }
  }
}

__global__ void k_sym_mix(uint32_t* c) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t nib = i & 15u, sb = (i >> 4) + 1u;               // code bits, scale 0x0001..
  if (sb >= 0x7c00u) return;
  const int q = (int)nib - (int)(nib & 8u) * 2;
  const float want = (float)q * h2f(sb);                          // exact
  const float s = h2f(sb) * 0.0625f;                              // as add_codes receives it
  const float S0 = s * 268435456.0f, S4 = s * 16777216.0f, Z = s * -128.0f;
  const uint32_t f = nib ^ 8u, junk = hash32(i) & 0xffffu;
  const float got[4] = {fma_mix16<false>((junk << 16) | f, S0, Z),
                        fma_mix16<true>((f << 16) | junk, S0, Z),
                        fma_mix16<false>(((junk & 0xff0fu) << 16) | (f << 4), S4, Z),
                        fma_mix16<true>((f << 20) | (junk & 0xff0fu), S4, Z)};
  for (int k = 0; k < 4; k++)
    if (__builtin_bit_cast(uint32_t, got[k]) != __builtin_bit_cast(uint32_t, want))
      miss(c, kSymMix);
}

__global__ void k_sym6_mix(uint32_t* c) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t field = i & 63u, sb = (i >> 6) + 1u;             // code bits, scale 0x0001..
  if (sb >= 0x7c00u) return;
  const int q = (int)field - (int)(field & 32u) * 2;
  const float want = (float)q * h2f(sb);                          // exact
  const float s = h2f(sb);
  const uint32_t f = field ^ 32u, junk = hash32(i) & 0xffffu;
  const float got[2] = {fma_mix16<false>((junk << 16) | f, s * 16777216.0f, s * -32.0f),
                        fma_mix16<true>((f << 16) | junk, s * 16777216.0f, s * -32.0f)};
  for (int k = 0; k < 2; k++)
    if (__builtin_bit_cast(uint32_t, got[k]) != __builtin_bit_cast(uint32_t, want))
      miss(c, kSym6Mix);
}

__global__ void k_h2f_times(uint32_t* c) {
  const uint32_t p = blockIdx.x * blockDim.x + threadIdx.x;     // 0..65535
  if (p >= 65536u || (p & 0x7fffu) > 0x7c00u) return;             // NaN patterns
  const uint32_t junk = hash32(p) & 0xffffu;
  const float ks[2] = {16777216.0f, 1048576.0f};
  for (int k = 0; k < 2; k++)
    if (__builtin_bit_cast(uint32_t, h2f_times((junk << 16) | p, ks[k])) !=
        __builtin_bit_cast(uint32_t, h2f(p) * ks[k]))
      miss(c, kH2fTimes);
}

__global__ void k_mix_fma_h(uint32_t* c) {
  const uint64_t n = 1024ull * 65536ull;                           // field x zero pattern
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    const uint32_t f = (uint32_t)(i & 1023u), zb = (uint32_t)(i >> 10);
    if ((zb & 0x7fffu) >= 0x7c00u) continue;                       // z finite
    const uint32_t hsh = hash32((uint32_t)i);
    const uint32_t sb = hsh % 0x7bffu + 1u;                        // 0x0001 .. 0x7bff
    const float S = h2f(sb) * ((hsh >> 31) ? 1048576.0f : 16777216.0f);
    const float want = __builtin_fmaf((float)f * 5.9604644775390625e-8f, S, h2f(zb));
    const uint32_t junk = hash32((uint32_t)i ^ 0x9e3779b9u);
    const uint32_t zh = (junk & 0xffff0000u) | zb;
    if (__builtin_bit_cast(uint32_t, fma_mix16h<false>(((junk & 0xffffu) << 16) | f, S, zh)) !=
        __builtin_bit_cast(uint32_t, want))
      miss(c, kMixFmaH);
    if (__builtin_bit_cast(uint32_t, fma_mix16h<true>((f << 16) | (junk & 0xffffu), S, zh)) !=
        __builtin_bit_cast(uint32_t, want))
      miss(c, kMixFmaH);
  }
}

__global__ void k_bf(uint32_t* c) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32); i += stride) {
    const uint32_t u = (uint32_t)i;
    if ((u & 0x7fffffffu) > 0x7f800000u) continue;        // NaN
    const uint32_t want = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    if (f2bf(__builtin_bit_cast(float, u)) != want) miss(c, kBf);
  }
}

// reference binary32 -> binary16, round to nearest even, from the formats:
// binary16 normals start at 2^-14 (binary32 biased exponent 113), its
// subnormals are multiples of 2^-24, and magnitudes from 65520 up round to inf
__device__ uint32_t f2h_ref(uint32_t u) {
  const uint32_t sign = (u >> 16) & 0x8000u;
  const uint32_t a = u & 0x7fffffffu;
  if (a >= 0x477ff000u) return sign | 0x7c00u;
  const uint32_t e = a >> 23;
  if (e >= 113u) {
    const uint32_t m = a & 0x7fffffu;
    uint32_t h = ((e - 112u) << 10) | (m >> 13);
    const uint32_t rest = m & 0x1fffu;
    if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u;
    return sign | h;
  }
  if (e < 102u) return sign;                              // below 2^-25
  const uint32_t mant = (a & 0x7fffffu) | 0x800000u;     // value = mant * 2^(e-150)
  const uint32_t sh = 126u - e;                           // 14 .. 24
  uint32_t q = mant >> sh;                                // value / 2^-24, truncated
  const uint32_t rest = mant & ((1u << sh) - 1u), half = 1u << (sh - 1u);
  if (rest > half || (rest == half && (q & 1u))) q += 1u;
  return sign | q;
}

__global__ void k_f2h(uint32_t* c) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < (1ull << 32); i += stride) {
    const uint32_t u = (uint32_t)i;
    if ((u & 0x7fffffffu) > 0x7f800000u) continue;        // NaN
    if (f2h(__builtin_bit_cast(float, u)) != f2h_ref(u)) miss(c, kF2h);
  }
}

#define CK(x)                                                                       \
  do {                                                                              \
    hipError_t e_ = (x);                                                            \
    if (e_ != hipSuccess) {                                                         \
      printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);         \
      return 2;                                                                     \
    }                                                                               \
  } while (0)

int main() {
  uint32_t* c;
  CK(hipMalloc(&c, kSlots * sizeof(uint32_t)));
  CK(hipMemset(c, 0, kSlots * sizeof(uint32_t)));
  k_div<127><<<8192, 256>>>(c, kDiv + 0);
  k_div<31><<<8192, 256>>>(c, kDiv + 1);
  k_div<7><<<8192, 256>>>(c, kDiv + 2);
  k_div<255><<<8192, 256>>>(c, kDiv + 3);
  k_div<63><<<8192, 256>>>(c, kDiv + 4);
  k_div<15><<<8192, 256>>>(c, kDiv + 5);
  k_rcp<<<(0x7c00 + 255) / 256, 256>>>(c);
  k_rint<<<8192, 256>>>(c);
  k_enc<<<8192, 256>>>(c);
  k_dec<<<1, 256>>>(c);
  k_bf<<<8192, 256>>>(c);
  k_f2h<<<8192, 256>>>(c);
  k_mix_cvt<<<256, 256>>>(c);
  k_mix_fma<<<8192, 256>>>(c);
  k_rint_byte<<<8192, 256>>>(c);
  k_off_i4<<<8192, 256>>>(c);
  k_sym_mix<<<(16 * 0x7bff + 255) / 256, 256>>>(c);
  k_sym6_mix<<<(64 * 0x7bff + 255) / 256, 256>>>(c);
  k_h2f_times<<<256, 256>>>(c);
  k_mix_fma_h<<<8192, 256>>>(c);
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  uint32_t h[kSlots];
  CK(hipMemcpy(h, c, sizeof h, hipMemcpyDeviceToHost));
  CK(hipFree(c));
  const char* div_names[6] = {"127", "31", "7", "255", "63", "15"};
  uint32_t total = 0;
  for (int k = 0; k < 6; k++) {
    printf("div_by<%s>: %u mismatches over all positive finite binary32\n", div_names[k], h[kDiv + k]);
    total += h[kDiv + k];
  }
  printf("recip_f16: %u mismatches over all positive finite binary16\n", h[kRcp]);
  printf("rint_bits: %u mismatches over all |c| <= 256\n", h[kRint]);
  printf("e4m3_pack2: %u mismatches over all |t| <= 464\n", h[kEnc]);
  printf("e4m3_dec: %u mismatches over all non-NaN codes, 4 byte positions\n", h[kDec]);
  printf("f2bf: %u mismatches over all non-NaN binary32\n", h[kBf]);
  printf("f2h: %u mismatches over all non-NaN binary32\n", h[kF2h]);
  printf("fma_mix16 read: %u mismatches over all non-NaN binary16, both halves\n", h[kMixCvt]);
  printf("fma_mix16 fma: %u mismatches over all fields < 1024 x positive finite binary16 scales"
         " x (2^24, 2^20), both halves\n", h[kMixFma]);
  printf("rint_byte: %u mismatches over all |c| <= 256, 4 byte positions\n", h[kRByte]);
  printf("off_i4: %u mismatches over all 32-bit words, 4 byte positions\n", h[kOffI4]);
  printf("symmetric 4-bit fma_mix term: %u mismatches over all codes x positive finite binary16"
         " scales, both halves, both nibble positions\n", h[kSymMix]);
  printf("symmetric 6-bit fma_mix term: %u mismatches over all codes x positive finite binary16"
         " scales, both halves\n", h[kSym6Mix]);
  printf("h2f_times: %u mismatches over all non-NaN binary16 x (2^24, 2^20)\n", h[kH2fTimes]);
  printf("fma_mix16h (binary16 addend): %u mismatches over all fields < 1024 x all finite"
         " binary16 zeros, both halves\n", h[kMixFmaH]);
  total += h[kRcp] + h[kRint] + h[kEnc] + h[kDec] + h[kBf] + h[kF2h] + h[kMixCvt] + h[kMixFma] +
           h[kRByte] + h[kOffI4] + h[kSymMix] + h[kSym6Mix] + h[kH2fTimes] + h[kMixFmaH];
  printf("%s\n", total == 0 ? "ALL OK" : "MISMATCHES");
  return total == 0 ? 0 : 1;
}
