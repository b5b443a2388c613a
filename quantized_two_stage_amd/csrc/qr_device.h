// qr_device.h -- device helpers of the two-stage quantized allreduce for
// gfx950: number formats, the per-lane block quantizer and the wire-slice
// code I/O.
//
// Work decomposition used by every kernel: a 32-element block is handled by
// a pair of adjacent lanes, each owning a 16-element "slice" (lane 2j takes
// elements 0..15 of block j, lane 2j+1 elements 16..31).  A slice is 32
// bytes of fp16/bf16 input (two 128-bit accesses) and 16*b/8 bytes of codes
// (8 for 4-bit, 12 for 6-bit, 16 for 8-bit codes), so consecutive lanes
// touch consecutive bytes in every plane.  The block statistics (max/min)
// need one exchange between the two lanes of a pair (a DPP quad permute).
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
enum DType { kF16 = 0, kBF16 = 1 };

constexpr int kSlice = 16;   // elements per lane
constexpr int kBlock = 32;   // elements per block (a lane pair)

template <int C>
struct CodecT {
  static constexpr int base = C & 7;
  static constexpr bool asym = (C & 8) != 0;
  static constexpr bool fp8 = C == kFP8;
  static constexpr int bits = base == kQ6 ? 6 : base == kQ4 ? 4 : 8;
  static constexpr float qmax =
      fp8 ? 448.0f
          : asym ? float((1 << bits) - 1) : float((1 << (bits - 1)) - 1);
  static constexpr int slice_bytes = kSlice * bits / 8;
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
  return __builtin_bit_cast(float, b << 16);
}
// binary32 -> bfloat16, nearest-even on the bit pattern, overflow to inf
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int D>
__device__ __forceinline__ float ld16(uint32_t bits) {
  return D == kBF16 ? bf2f(bits) : h2f(bits);
}
template <int D>
__device__ __forceinline__ uint32_t st16(float v) {
  return D == kBF16 ? f2bf(v) : f2h(v);
}

// least binary16 >= v (v >= 0), saturated at 65504: round to nearest, then
// step up one unit where that fell below v
__device__ __forceinline__ uint32_t ru16(float v) {
  uint32_t h = f2h(v);
  if (h2f(h) < v) h += 1u;
  return h >= 0x7c00u ? 0x7bffu : h;
}

// greatest binary16 <= v, saturated at -65504
__device__ __forceinline__ uint32_t rd16(float v) {
  uint32_t h = f2h(v);
  if (h2f(h) > v) h = (h & 0x8000u) ? h + 1u : (h == 0u ? 0x8001u : h - 1u);
  return (h & 0x7fffu) >= 0x7c00u ? (h & 0x8000u) | 0x7bffu : h;
}

// OCP E4M3FN encode: nearest, ties to even, saturating at 448; the sign of
// t is kept when the magnitude rounds to zero
__device__ __forceinline__ uint32_t e4m3_enc(float t) {
  uint32_t u = __builtin_bit_cast(uint32_t, t);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t au = u & 0x7fffffffu;
  float a = __builtin_bit_cast(float, au);
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7eu;
  } else if (a < 0.015625f) {                 // below 2^-6: steps of 2^-9
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {                                    // round the fraction to 3 bits
    code = ((au + 0x7ffffu + ((au >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return code | sign;
}

// OCP E4M3FN decode (exact); code 0x7f/0xff (NaN) is never produced here
__device__ __forceinline__ float e4m3_dec(uint32_t c) {
  uint32_t em = c & 0x7fu;
  float mag = em < 8u ? (float)em * 0.001953125f
                      : __builtin_bit_cast(float, (em + (120u << 3)) << 20);
  return __builtin_bit_cast(float,
                            __builtin_bit_cast(uint32_t, mag) | ((c & 0x80u) << 24));
}

// value held by the other lane of this lane's pair (DPP quad_perm [1,0,3,2])
__device__ __forceinline__ float pair_other(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xb1, 0xf, 0xf,
                                      false));
}

// ---------------------------------------------------------------------------
// block quantizer: the lane's 16 values (first `valid` of them real, valid in
// {0, 8, 16}) together with the partner lane's form one block.  Writes the
// lane's 16 codes (b-bit patterns, zero for invalid slots) and the block's
// binary16 scale and zero (identical in both lanes).

template <int C>
__device__ __forceinline__ void quantize_slice(const float (&v)[kSlice], int valid,
                                               uint32_t (&code)[kSlice],
                                               uint32_t& s_out, uint32_t& z_out) {
  using T = CodecT<C>;
  float mx = v[0], mn = v[0];
#pragma unroll
  for (int i = 1; i < 8; i++) {
    mx = fmaxf(mx, v[i]);
    mn = fminf(mn, v[i]);
  }
  if (valid == kSlice) {
#pragma unroll
    for (int i = 8; i < kSlice; i++) {
      mx = fmaxf(mx, v[i]);
      mn = fminf(mn, v[i]);
    }
  }
  if (valid == 0) {
    mx = -__builtin_inff();
    mn = __builtin_inff();
  }
  mx = fmaxf(mx, pair_other(mx));
  mn = fminf(mn, pair_other(mn));

  uint32_t s = 0, z = 0;
#pragma unroll
  for (int i = 0; i < kSlice; i++) code[i] = 0;

  if constexpr (!T::asym) {
    float a = fmaxf(fabsf(mx), fabsf(mn));
    if (a != 0.0f) {
      // a constant block takes its own magnitude as the scale
      float arg = (mx == mn) ? a : a / T::qmax;
      s = ru16(arg);
      float inv = 1.0f / h2f(s);
#pragma unroll
      for (int i = 0; i < kSlice; i++) {
        float t = v[i] * inv;
        uint32_t c;
        if constexpr (T::fp8) {
          c = e4m3_enc(t);
        } else {
          float q = fminf(fmaxf(__builtin_rintf(t), -T::qmax), T::qmax);
          c = (uint32_t)(int)q & ((1u << T::bits) - 1u);
        }
        code[i] = (i < valid) ? c : 0u;
      }
    }
  } else {
    if (mn == 0.0f) mn = 0.0f;                  // a zero minimum is +0
    z = rd16(mn);
    float fz = h2f(z);
    float d = mx - fz;
    if (d > 0.0f) {
      s = ru16(d / T::qmax);
      float inv = 1.0f / h2f(s);
#pragma unroll
      for (int i = 0; i < kSlice; i++) {
        float t = (v[i] - fz) * inv;
        float u = fminf(fmaxf(__builtin_rintf(t), 0.0f), T::qmax);
        code[i] = (i < valid) ? (uint32_t)(int)u : 0u;
      }
    }
  }
  s_out = s;
  z_out = z;
}

// ---------------------------------------------------------------------------
// slice code words: 16 codes of b bits, little-endian bitstream

template <int C>
struct SliceWords {
  static constexpr int nw = CodecT<C>::slice_bytes / 4;   // 2, 3 or 4
  uint32_t w[nw];
};

template <int C>
__device__ __forceinline__ SliceWords<C> load_slice(const uint8_t* p) {
  SliceWords<C> r;
  if constexpr (SliceWords<C>::nw == 4) {
    u32x4 q = *reinterpret_cast<const u32x4*>(p);
    r.w[0] = q.x; r.w[1] = q.y; r.w[2] = q.z; r.w[3] = q.w;
  } else if constexpr (SliceWords<C>::nw == 2) {
    u32x2 q = *reinterpret_cast<const u32x2*>(p);
    r.w[0] = q.x; r.w[1] = q.y;
  } else {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    r.w[0] = q[0]; r.w[1] = q[1]; r.w[2] = q[2];
  }
  return r;
}

template <int C>
__device__ __forceinline__ void store_slice(uint8_t* p, const SliceWords<C>& r) {
  if constexpr (SliceWords<C>::nw == 4) {
    *reinterpret_cast<u32x4*>(p) = u32x4{r.w[0], r.w[1], r.w[2], r.w[3]};
  } else if constexpr (SliceWords<C>::nw == 2) {
    *reinterpret_cast<u32x2*>(p) = u32x2{r.w[0], r.w[1]};
  } else {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
    q[0] = r.w[0]; q[1] = r.w[1]; q[2] = r.w[2];
  }
}

// raw b-bit field i of the slice (zero-extended)
template <int C>
__device__ __forceinline__ uint32_t get_field(const SliceWords<C>& r, int i) {
  constexpr int b = CodecT<C>::bits;
  const int off = b * i, k = off >> 5, sh = off & 31;
  uint32_t x;
  if (sh + b <= 32 || k + 1 >= SliceWords<C>::nw)
    x = r.w[k] >> sh;
  else
    x = __builtin_amdgcn_alignbit(r.w[k + 1], r.w[k], sh);
  return x & ((1u << b) - 1u);
}

template <int C>
__device__ __forceinline__ SliceWords<C> pack_slice(const uint32_t (&code)[kSlice]) {
  constexpr int b = CodecT<C>::bits;
  SliceWords<C> r;
#pragma unroll
  for (int k = 0; k < SliceWords<C>::nw; k++) r.w[k] = 0;
#pragma unroll
  for (int i = 0; i < kSlice; i++) {
    const int off = b * i, k = off >> 5, sh = off & 31;
    r.w[k] |= code[i] << sh;
    if (sh + b > 32) r.w[k + 1] |= code[i] >> (32 - sh);
  }
  return r;
}

// dequantized value of field i: code*s exact, plus z for asymmetric codecs
template <int C>
__device__ __forceinline__ float dequant_field(const SliceWords<C>& r, int i,
                                               float s, float z) {
  using T = CodecT<C>;
  uint32_t f = get_field<C>(r, i);
  if constexpr (T::fp8) {
    return e4m3_dec(f) * s;
  } else if constexpr (T::asym) {
    return __builtin_fmaf((float)f, s, z);    // f*s is exact: one rounding
  } else {
    int q = (int)(f << (32 - T::bits)) >> (32 - T::bits);
    return (float)q * s;
  }
}

}  // namespace qr
