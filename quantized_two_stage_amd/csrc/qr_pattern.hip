// qr_pattern.hip -- the benchmark's access-pattern reference for stage 1, built
// into its own library (libqr_pattern.so), not into libqr.so.
//
// qrp_stage1_pattern issues exactly the loads and stores of the stage-1
// kernel that reads a receive buffer (the same grid, the same lanes, the same
// addresses and access widths, through the helpers of qr_stage_io.h) and
// replaces the dequantize-sum-requantize arithmetic by an XOR of the W ranks'
// words.  Its time is what the memory system needs for stage 1's bytes in
// stage 1's pattern: the ceiling the benchmark reports beside the kernel.
#include <stdint.h>

#include "qr.h"
#include "qr_device.h"
#include "qr_pattern.h"
#include "qr_internal.h"
#include "qr_stage_io.h"

namespace qr {
namespace {

template <int C, int W, int TB>
__global__ __launch_bounds__(kThreads) void k_stage1_pattern(InPtrs wires, uint8_t* red,
                                                             uint32_t nb, Geo g) {
  using T = CodecT<C>;
  const uint32_t blk = blockIdx.x * TB + threadIdx.x;
  if (blk >= nb) return;
  S1In<C, W> in;
  s1_load<C, W, true>(wires, blk, g, in);
  uint32_t w[T::words];
  uint32_t s = in.sh[0], z = in.zh[0];
#pragma unroll
  for (int k = 0; k < T::words; k++) w[k] = in.cw[0][k];
#pragma unroll
  for (int r = 1; r < W; r++) {
#pragma unroll
    for (int k = 0; k < T::words; k++) w[k] ^= in.cw[r][k];
    s ^= in.sh[r];
    z ^= in.zh[r];
  }
  s1_store<C>(red, blk, g, w, s, z);
}

// the FP codec's stage 1 (k_sum_fp over a receive buffer): the same 16-byte
// chunks, four per lane, W loads each, one store
template <int W>
__global__ __launch_bounds__(kThreads) void k_sum_pattern(InPtrs xs, uint8_t* red,
                                                          uint32_t nchunks, uint32_t tstride) {
  const uint32_t base = blockIdx.x * (kThreads * kPerLane) + threadIdx.x;
  u32x4 q[kPerLane][W];
#pragma unroll
  for (int j = 0; j < kPerLane; j++) {
    const uint32_t c = base + j * kThreads;
    const uint32_t off = fp_chunk<true>(tstride, 0u, c < nchunks ? c : 0u);
#pragma unroll
    for (int r = 0; r < W; r++)
      q[j][r] = ld_in<kS1Load<W>>(reinterpret_cast<const u32x4*>(xs.p[r] + off));
  }
#pragma unroll
  for (int j = 0; j < kPerLane; j++) {
    const uint32_t c = base + j * kThreads;
    if (c >= nchunks) break;
    u32x4 o = q[j][0];
#pragma unroll
    for (int r = 1; r < W; r++) o ^= q[j][r];
    st_out<kStage1>(reinterpret_cast<u32x4*>(red) + c, o);
  }
}

// plain streams: kind 0 read, 1 write, 2 copy; K 16-byte accesses per lane,
// access k of lane l at chunk 256k + l of the workgroup's 256K chunks
template <int Kind, int K, bool NT>
__global__ __launch_bounds__(kThreads) void k_stream(const u32x4* src, u32x4* dst,
                                                     uint64_t nchunks, uint32_t* out) {
  const uint64_t base = (uint64_t)blockIdx.x * (kThreads * K) + threadIdx.x;
  if constexpr (Kind == 0) {
    u32x4 acc = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int k = 0; k < K; k++) {
      const uint64_t c = base + (uint64_t)k * kThreads;
      if (c < nchunks) acc ^= NT ? __builtin_nontemporal_load(src + c) : src[c];
    }
    // never true for the benchmark's data, but the loads cannot be dropped
    if ((acc.x ^ acc.y ^ acc.z ^ acc.w) == 0x9e3779b9u) out[blockIdx.x] = acc.x;
  } else if constexpr (Kind == 1) {
#pragma unroll
    for (int k = 0; k < K; k++) {
      const uint64_t c = base + (uint64_t)k * kThreads;
      const u32x4 v = {(uint32_t)c, 1u, 2u, 3u};
      if (c < nchunks) {
        if constexpr (NT)
          __builtin_nontemporal_store(v, dst + c);
        else
          dst[c] = v;
      }
    }
  } else {
    u32x4 v[K];
#pragma unroll
    for (int k = 0; k < K; k++) {
      const uint64_t c = base + (uint64_t)k * kThreads;
      if (c < nchunks) v[k] = NT ? __builtin_nontemporal_load(src + c) : src[c];
    }
#pragma unroll
    for (int k = 0; k < K; k++) {
      const uint64_t c = base + (uint64_t)k * kThreads;
      if (c < nchunks) dst[c] = v[k];
    }
  }
}

template <int Kind, int K, bool NT>
void stream_launch(const void* src, void* dst, uint64_t nchunks, hipStream_t st) {
  const unsigned ng = (unsigned)((nchunks + kThreads * K - 1) / (kThreads * K));
  hipLaunchKernelGGL((k_stream<Kind, K, NT>), dim3(ng), dim3(kThreads), 0, st,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), nchunks,
                     static_cast<uint32_t*>(dst));
}

template <int Kind>
void stream_by(int K, bool nt, const void* src, void* dst, uint64_t nchunks, hipStream_t st) {
  if (K == 1)
    nt ? stream_launch<Kind, 1, true>(src, dst, nchunks, st)
       : stream_launch<Kind, 1, false>(src, dst, nchunks, st);
  else
    nt ? stream_launch<Kind, 4, true>(src, dst, nchunks, st)
       : stream_launch<Kind, 4, false>(src, dst, nchunks, st);
}

size_t a256(size_t x) { return (x + 255) & ~(size_t)255; }

template <int C, int W>
void launch(const InPtrs& in, uint8_t* red, size_t n, hipStream_t st) {
  const size_t nb = (n + 31) / 32;
  // at W=8 in full rounds, as stage 1 launches (round_cap_lds)
  if constexpr (C == kFP) {
    const uint32_t nc = (uint32_t)(n / 8);
    constexpr auto K = k_sum_pattern<W>;
    const unsigned ng = (nc + kThreads * kPerLane - 1) / (kThreads * kPerLane);
    hipLaunchKernelGGL(K, dim3(ng), dim3(kThreads), W == 8 ? round_cap_lds<K>(kThreads, ng) : 0,
                       st, in, red, nc, (uint32_t)(W * kTileBlocks * 64));
  } else {
    using T = CodecT<C>;
    const size_t off_s = a256(nb * T::block_bytes);
    const size_t off_z = a256(off_s + 2 * nb);
    const uint32_t tile = kTileBlocks * (T::block_bytes + 2 + (T::asym ? 2 : 0));
    const Geo g{(uint32_t)n, (uint32_t)nb, (uint32_t)off_s, (uint32_t)off_z, W * tile, 0u};
    // the workgroup size stage 1 takes for this size (s1_lanes_per_workgroup)
    if (s1_lanes_per_workgroup(W, nb) == 128) {
      constexpr auto K = k_stage1_pattern<C, W, 128>;
      const unsigned ng = (unsigned)((nb + 127) / 128);
      hipLaunchKernelGGL(K, dim3(ng), dim3(128), 0, st, in, red, (uint32_t)nb, g);
    } else {
      constexpr auto K = k_stage1_pattern<C, W, kThreads>;
      const unsigned ng = (unsigned)((nb + kThreads - 1) / kThreads);
      hipLaunchKernelGGL(K, dim3(ng), dim3(kThreads), W == 8 ? round_cap_lds<K>(kThreads, ng) : 0,
                         st, in, red, (uint32_t)nb, g);
    }
  }
}

template <int C>
void by_w(int W, const InPtrs& in, uint8_t* red, size_t n, hipStream_t st) {
  if (W == 2) launch<C, 2>(in, red, n, st);
  if (W == 4) launch<C, 4>(in, red, n, st);
  if (W == 8) launch<C, 8>(in, red, n, st);
}

}  // namespace
}  // namespace qr

extern "C" {

// declared, with its arguments, in qr_pattern.h
int qrp_stage1_pattern(int codec, int W, const void* recv, size_t n, void* reduced,
                       void* stream) {
  using namespace qr;
  if (!(W == 2 || W == 4 || W == 8) || n == 0 || n % 8 != 0 || n > QR_MAX_BYTES / 2 ||
      recv == nullptr || reduced == nullptr || ((uintptr_t)recv & 15u) != 0 ||
      ((uintptr_t)reduced & 15u) != 0)
    return -1;
  if (!(codec == QR_FP || codec == QR_Q8 || codec == QR_Q6 || codec == QR_Q4 ||
        codec == QR_FP8 || codec == QR_Q8_ASYM || codec == QR_Q6_ASYM || codec == QR_Q4_ASYM))
    return -1;
  // bytes of one rank's tile of the receive buffer: the codes (FP: the raw
  // data) of 256 blocks, then their scales and zeros
  const size_t cb = codec == QR_FP ? 64 : (codec & 7) == QR_Q6 ? 24 : (codec & 7) == QR_Q4 ? 16 : 32;
  const size_t tile = (size_t)kTileBlocks * (codec == QR_FP ? cb : cb + 2 + ((codec & 8) ? 2 : 0));
  // one launch: the receive buffer's offsets must fit in 32 bits
  const size_t tiles = ((n + 31) / 32 + kTileBlocks - 1) / kTileBlocks;
  if ((tiles + 1) * (size_t)W * tile >= ((size_t)1 << 32)) return -1;
  InPtrs in{};
  for (int r = 0; r < W; r++) in.p[r] = static_cast<const uint8_t*>(recv) + (size_t)r * tile;
  uint8_t* red = static_cast<uint8_t*>(reduced);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  switch (codec) {
    case QR_FP: by_w<kFP>(W, in, red, n, st); break;
    case QR_Q8: by_w<kQ8>(W, in, red, n, st); break;
    case QR_Q6: by_w<kQ6>(W, in, red, n, st); break;
    case QR_Q4: by_w<kQ4>(W, in, red, n, st); break;
    case QR_FP8: by_w<kFP8>(W, in, red, n, st); break;
    case QR_Q8_ASYM: by_w<kQ8A>(W, in, red, n, st); break;
    case QR_Q6_ASYM: by_w<kQ6A>(W, in, red, n, st); break;
    case QR_Q4_ASYM: by_w<kQ4A>(W, in, red, n, st); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// declared, with its arguments, in qr_pattern.h
int qrp_stream(int kind, int per_lane, int nontemporal, const void* src, void* dst,
               size_t bytes, void* stream) {
  using namespace qr;
  if (kind < 0 || kind > 2 || (per_lane != 1 && per_lane != 4) ||
      (nontemporal != 0 && nontemporal != 1) || bytes == 0 || bytes % 32 != 0 ||
      bytes > ((size_t)1 << 36) || dst == nullptr || ((uintptr_t)dst & 15u) != 0 ||
      (kind != 1 && (src == nullptr || ((uintptr_t)src & 15u) != 0)))
    return -1;
  // a copy moves bytes / 2 each way
  const uint64_t nchunks = (kind == 2 ? bytes / 2 : bytes) / 16;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (kind == 0)
    stream_by<0>(per_lane, nontemporal != 0, src, dst, nchunks, st);
  else if (kind == 1)
    stream_by<1>(per_lane, nontemporal != 0, src, dst, nchunks, st);
  else
    stream_by<2>(per_lane, nontemporal != 0, src, dst, nchunks, st);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
