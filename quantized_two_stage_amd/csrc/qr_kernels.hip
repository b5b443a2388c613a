// qr_kernels.hip -- gfx950 kernels of the two-stage quantized allreduce.
//
//   k_quantize   stage 0: binary16/bfloat16 -> codes + scale (+ zero)
//   k_stage1     stage 1: W wire blocks -> dequantize -> binary32 sum in rank
//                order -> requantize (one pass over HBM per byte)
//   k_stage1_fp  stage 1 of the FP codec: sum of the raw buffers, rounded once
//   k_dequant    stage 2 / dequantize: codes -> binary16/bfloat16, W outputs
//   k_copy       stages 0 and 2 of the FP codec (the wire is the raw data)
//
// The method is the 2-stage allreduce of "Integrate quick allreduce and
// select the best allreduce implementation" (vLLM PR #18473, PR description
// item 2), with the symmetric/asymmetric integer codecs of "Add quickreduce
// as alternative to custom allreduce" (vLLM PR #16804, PR description).
//
// Every kernel is HBM-streaming: one 64-lane wave handles 32 blocks = 1024
// elements, each lane a 16-element slice; every plane is read and written
// with consecutive lanes on consecutive addresses (128-bit accesses for the
// 16-bit data and the 8-bit codes, 96/64-bit for 6/4-bit codes).  No LDS and
// no MFMA: nothing here is a contraction.
#include "qr_device.h"
#include "qr_internal.h"

namespace qr {
namespace {

constexpr int kThreads = 256;

struct Geo {
  uint32_t n;        // elements per rank
  uint32_t off_s;    // scale plane offset
  uint32_t off_z;    // zero plane offset
};

__device__ __forceinline__ int slice_valid(uint32_t slice, uint32_t n) {
  uint32_t e0 = slice * kSlice;
  return e0 >= n ? 0 : (n - e0 >= (uint32_t)kSlice ? kSlice : (int)(n - e0));
}

template <int D>
__device__ __forceinline__ void load_vals(const uint8_t* x, int valid,
                                          float (&v)[kSlice]) {
  u32x4 a = {0u, 0u, 0u, 0u}, b = {0u, 0u, 0u, 0u};
  if (valid >= 8) a = *reinterpret_cast<const u32x4*>(x);
  if (valid >= 16) b = *reinterpret_cast<const u32x4*>(x + 16);
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int k = 0; k < 8; k++) {
    v[2 * k] = ld16<D>(w[k] & 0xffffu);
    v[2 * k + 1] = ld16<D>(w[k] >> 16);
  }
}

template <int D>
__device__ __forceinline__ void store_vals(uint8_t* y, int valid,
                                           const float (&v)[kSlice]) {
  uint32_t w[8];
#pragma unroll
  for (int k = 0; k < 8; k++) w[k] = st16<D>(v[2 * k]) | (st16<D>(v[2 * k + 1]) << 16);
  if (valid >= 8) *reinterpret_cast<u32x4*>(y) = u32x4{w[0], w[1], w[2], w[3]};
  if (valid >= 16) *reinterpret_cast<u32x4*>(y + 16) = u32x4{w[4], w[5], w[6], w[7]};
}

__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}
__device__ __forceinline__ void st_u16(uint8_t* p, uint32_t v) {
  *reinterpret_cast<uint16_t*>(p) = (uint16_t)v;
}

// acc + dequant(field i).  For symmetric and fp8 codes the product code*s is
// exact in binary32, so one fused multiply-add rounds exactly like the
// separate add of the exact product.
template <int C>
__device__ __forceinline__ float accumulate(const SliceWords<C>& r, int i, float s,
                                            float z, float acc) {
  using T = CodecT<C>;
  if constexpr (T::asym) {
    return acc + dequant_field<C>(r, i, s, z);
  } else if constexpr (T::fp8) {
    return __builtin_fmaf(e4m3_dec(get_field<C>(r, i)), s, acc);
  } else {
    uint32_t f = get_field<C>(r, i);
    int q = (int)(f << (32 - T::bits)) >> (32 - T::bits);
    return __builtin_fmaf((float)q, s, acc);
  }
}

// ---------------------------------------------------------------------------
// stage 0

template <int C, int D>
__global__ __launch_bounds__(kThreads) void k_quantize(InPtrs xs, OutPtrs wires,
                                                       uint32_t nslices, Geo g) {
  using T = CodecT<C>;
  const uint32_t slice = blockIdx.x * kThreads + threadIdx.x;
  if (slice >= nslices) return;               // nslices is even: pairs stay whole
  const int r = blockIdx.y;
  const int valid = slice_valid(slice, g.n);
  float v[kSlice];
  load_vals<D>(xs.p[r] + (size_t)slice * (2 * kSlice), valid, v);
  uint32_t code[kSlice], s, z;
  quantize_slice<C>(v, valid, code, s, z);
  uint8_t* w = wires.p[r];
  store_slice<C>(w + (size_t)slice * T::slice_bytes, pack_slice<C>(code));
  if ((slice & 1u) == 0u) {
    st_u16(w + g.off_s + (size_t)(slice >> 1) * 2, s);
    if constexpr (T::asym) st_u16(w + g.off_z + (size_t)(slice >> 1) * 2, z);
  }
}

// stages 0 and 2 of FP: dst.p[r] <- src.p[r], 32 bytes per lane
__global__ __launch_bounds__(kThreads) void k_copy(InPtrs src, OutPtrs dst,
                                                   uint32_t nslices, uint32_t n) {
  const uint32_t slice = blockIdx.x * kThreads + threadIdx.x;
  if (slice >= nslices) return;
  const int r = blockIdx.y;
  const int valid = slice_valid(slice, n);
  const uint8_t* s = src.p[r] + (size_t)slice * (2 * kSlice);
  uint8_t* d = dst.p[r] + (size_t)slice * (2 * kSlice);
  if (valid >= 8) *reinterpret_cast<u32x4*>(d) = *reinterpret_cast<const u32x4*>(s);
  if (valid >= 16)
    *reinterpret_cast<u32x4*>(d + 16) = *reinterpret_cast<const u32x4*>(s + 16);
}

// ---------------------------------------------------------------------------
// stage 1

template <int C, int D, int W>
__global__ __launch_bounds__(kThreads) void k_stage1(InPtrs wires, uint8_t* red,
                                                     uint32_t slice_lo,
                                                     uint32_t slice_hi, Geo g) {
  using T = CodecT<C>;
  const uint32_t slice = slice_lo + blockIdx.x * kThreads + threadIdx.x;
  if (slice >= slice_hi) return;
  const uint32_t blk = slice >> 1;
  const int valid = slice_valid(slice, g.n);

  SliceWords<C> cw[W];
  float sc[W], zc[W];
#pragma unroll
  for (int r = 0; r < W; r++) {
    cw[r] = load_slice<C>(wires.p[r] + (size_t)slice * T::slice_bytes);
    sc[r] = h2f(ld_u16(wires.p[r] + g.off_s + (size_t)blk * 2));
    zc[r] = T::asym ? h2f(ld_u16(wires.p[r] + g.off_z + (size_t)blk * 2)) : 0.0f;
  }
  float acc[kSlice];
#pragma unroll
  for (int i = 0; i < kSlice; i++) acc[i] = dequant_field<C>(cw[0], i, sc[0], zc[0]);
#pragma unroll
  for (int r = 1; r < W; r++) {
#pragma unroll
    for (int i = 0; i < kSlice; i++) acc[i] = accumulate<C>(cw[r], i, sc[r], zc[r], acc[i]);
  }
  uint32_t code[kSlice], s, z;
  quantize_slice<C>(acc, valid, code, s, z);
  store_slice<C>(red + (size_t)slice * T::slice_bytes, pack_slice<C>(code));
  if ((slice & 1u) == 0u) {
    st_u16(red + g.off_s + (size_t)blk * 2, s);
    if constexpr (T::asym) st_u16(red + g.off_z + (size_t)blk * 2, z);
  }
}

template <int D, int W>
__global__ __launch_bounds__(kThreads) void k_stage1_fp(InPtrs xs, uint8_t* red,
                                                        uint32_t slice_lo,
                                                        uint32_t slice_hi, uint32_t n) {
  const uint32_t slice = slice_lo + blockIdx.x * kThreads + threadIdx.x;
  if (slice >= slice_hi) return;
  const int valid = slice_valid(slice, n);
  const size_t off = (size_t)slice * (2 * kSlice);
  float v[W][kSlice];
#pragma unroll
  for (int r = 0; r < W; r++) load_vals<D>(xs.p[r] + off, valid, v[r]);
  float acc[kSlice];
#pragma unroll
  for (int i = 0; i < kSlice; i++) {
    acc[i] = v[0][i];
#pragma unroll
    for (int r = 1; r < W; r++) acc[i] = acc[i] + v[r][i];
  }
  store_vals<D>(red + off, valid, acc);
}

// ---------------------------------------------------------------------------
// stage 2 / dequantize

template <int C, int D>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t* wire, OutPtrs ys,
                                                      uint32_t nslices, Geo g) {
  using T = CodecT<C>;
  const uint32_t slice = blockIdx.x * kThreads + threadIdx.x;
  if (slice >= nslices) return;
  const int r = blockIdx.y;
  const uint32_t blk = slice >> 1;
  const int valid = slice_valid(slice, g.n);
  SliceWords<C> cw = load_slice<C>(wire + (size_t)slice * T::slice_bytes);
  float s = h2f(ld_u16(wire + g.off_s + (size_t)blk * 2));
  float z = T::asym ? h2f(ld_u16(wire + g.off_z + (size_t)blk * 2)) : 0.0f;
  float v[kSlice];
#pragma unroll
  for (int i = 0; i < kSlice; i++) v[i] = dequant_field<C>(cw, i, s, z);
  store_vals<D>(ys.p[r] + (size_t)slice * (2 * kSlice), valid, v);
}

// ---------------------------------------------------------------------------
// dispatch

Geo geo(const Layout& L) {
  return Geo{(uint32_t)L.n, (uint32_t)L.off_s, (uint32_t)L.off_z};
}

dim3 grid_for(size_t slices, int ranks) {
  return dim3((unsigned)((slices + kThreads - 1) / kThreads), (unsigned)ranks, 1);
}

template <int C, int D>
void q_launch(int W, const InPtrs& xs, const OutPtrs& wires, const Layout& L,
              hipStream_t st) {
  hipLaunchKernelGGL((k_quantize<C, D>), grid_for(L.nslices, W), dim3(kThreads), 0,
                     st, xs, wires, (uint32_t)L.nslices, geo(L));
}

template <int C, int D>
void dq_launch(int W, const uint8_t* wire, const OutPtrs& ys, const Layout& L,
               hipStream_t st) {
  hipLaunchKernelGGL((k_dequant<C, D>), grid_for(L.nslices, W), dim3(kThreads), 0,
                     st, wire, ys, (uint32_t)L.nslices, geo(L));
}

template <int C, int D, int W>
void s1_launch(const InPtrs& wires, uint8_t* red, uint32_t lo, uint32_t hi,
               const Layout& L, hipStream_t st) {
  if constexpr (C == kFP) {
    hipLaunchKernelGGL((k_stage1_fp<D, W>), grid_for(hi - lo, 1), dim3(kThreads), 0,
                       st, wires, red, lo, hi, (uint32_t)L.n);
  } else {
    hipLaunchKernelGGL((k_stage1<C, D, W>), grid_for(hi - lo, 1), dim3(kThreads), 0,
                       st, wires, red, lo, hi, geo(L));
  }
}

template <int C, int D>
void s1_by_w(int W, const InPtrs& wires, uint8_t* red, uint32_t lo, uint32_t hi,
             const Layout& L, hipStream_t st) {
  switch (W) {
    case 2: s1_launch<C, D, 2>(wires, red, lo, hi, L, st); break;
    case 4: s1_launch<C, D, 4>(wires, red, lo, hi, L, st); break;
    case 8: s1_launch<C, D, 8>(wires, red, lo, hi, L, st); break;
    default: break;
  }
}

// calls F<codec, dtype>::run(args...) for the runtime (codec, dtype)
#define QR_DISPATCH(codec, dtype, FN, ...)                                    \
  do {                                                                        \
    const bool bf = (dtype) == kBF16;                                         \
    switch (codec) {                                                          \
      case kFP: bf ? FN<kFP, kBF16>(__VA_ARGS__) : FN<kFP, kF16>(__VA_ARGS__); break;     \
      case kQ8: bf ? FN<kQ8, kBF16>(__VA_ARGS__) : FN<kQ8, kF16>(__VA_ARGS__); break;     \
      case kQ6: bf ? FN<kQ6, kBF16>(__VA_ARGS__) : FN<kQ6, kF16>(__VA_ARGS__); break;     \
      case kQ4: bf ? FN<kQ4, kBF16>(__VA_ARGS__) : FN<kQ4, kF16>(__VA_ARGS__); break;     \
      case kFP8: bf ? FN<kFP8, kBF16>(__VA_ARGS__) : FN<kFP8, kF16>(__VA_ARGS__); break;  \
      case kQ8A: bf ? FN<kQ8A, kBF16>(__VA_ARGS__) : FN<kQ8A, kF16>(__VA_ARGS__); break;  \
      case kQ6A: bf ? FN<kQ6A, kBF16>(__VA_ARGS__) : FN<kQ6A, kF16>(__VA_ARGS__); break;  \
      case kQ4A: bf ? FN<kQ4A, kBF16>(__VA_ARGS__) : FN<kQ4A, kF16>(__VA_ARGS__); break;  \
      default: break;                                                         \
    }                                                                         \
  } while (0)

template <int C, int D>
void q_dispatch(int W, const InPtrs& xs, const OutPtrs& wires, const Layout& L,
                hipStream_t st) {
  if constexpr (C == kFP) {
    hipLaunchKernelGGL(k_copy, grid_for(L.nslices, W), dim3(kThreads), 0, st, xs, wires,
                       (uint32_t)L.nslices, (uint32_t)L.n);
  } else {
    q_launch<C, D>(W, xs, wires, L, st);
  }
}

template <int C, int D>
void dq_dispatch(int W, const uint8_t* wire, const OutPtrs& ys, const Layout& L,
                 hipStream_t st) {
  if constexpr (C == kFP) {
    InPtrs src;
    for (int r = 0; r < kMaxRanks; r++) src.p[r] = wire;
    hipLaunchKernelGGL(k_copy, grid_for(L.nslices, W), dim3(kThreads), 0, st, src, ys,
                       (uint32_t)L.nslices, (uint32_t)L.n);
  } else {
    dq_launch<C, D>(W, wire, ys, L, st);
  }
}

}  // namespace

hipError_t launch_quantize(int codec, int dtype, int W, const InPtrs& xs,
                           const OutPtrs& wires, const Layout& L, hipStream_t st) {
  QR_DISPATCH(codec, dtype, q_dispatch, W, xs, wires, L, st);
  return hipGetLastError();
}

hipError_t launch_stage1(int codec, int dtype, int W, const InPtrs& wires,
                         uint8_t* reduced, size_t blk_lo, size_t blk_hi,
                         const Layout& L, hipStream_t st) {
  if (blk_hi <= blk_lo) return hipSuccess;
  const uint32_t lo = (uint32_t)(2 * blk_lo), hi = (uint32_t)(2 * blk_hi);
  QR_DISPATCH(codec, dtype, s1_by_w, W, wires, reduced, lo, hi, L, st);
  return hipGetLastError();
}

hipError_t launch_dequantize(int codec, int dtype, int W, const uint8_t* wire,
                             const OutPtrs& ys, const Layout& L, hipStream_t st) {
  QR_DISPATCH(codec, dtype, dq_dispatch, W, wire, ys, L, st);
  return hipGetLastError();
}

}  // namespace qr
