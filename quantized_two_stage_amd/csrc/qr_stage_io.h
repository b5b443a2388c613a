// qr_stage_io.h -- launch geometry, wire-data addressing and the stage-1
// loads and stores of the gfx950 kernels, shared by qr_kernels.hip and the
// benchmark's access-pattern reference (qr_pattern.hip), so that the
// reference issues exactly the loads and stores of the stage-1 kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "qr_device.h"
#include "qr_internal.h"

namespace qr {
namespace {

constexpr int kThreads = 256;
constexpr int kPerLane = 4;        // quarters / chunks per lane (k_quantize and
                                   // the FP kernels of stages 0 and 1)
// Launch shapes chosen by size.  Finer work items (fewer quarters per lane,
// smaller workgroups) measured faster on the largest grids and slower on
// mid-size ones (8-32 MB per rank), where the coarser form's fewer
// workgroups win; the thresholds sit between the measured points.
//   stage 0: quarters per lane of k_quantize (the quad quantizer's slots):
//            2 from W*n >= 2^28 elements (1% faster at W=8, 64 MB per rank),
//            else 4 (2 was 3% slower at W*n = 2^26, the same at 2^27);
//            8-bit codes keep 4 at every size: with the inputs streamed in,
//            their quantizer is VALU-heavy, and 4 slots spread each lane's
//            share of the block parameters over 32 elements instead of 16
//            (W=8, 64 MB per rank: FP8, Q8 and Q8A 1.5-2% faster per
//            allreduce; the 6- and 4-bit codes equal or up to 2% slower);
//   stage 2: quarters per lane of k_dequant and the FP copy: 1 from
//            W*n >= 2^26 (1-3% faster at W = 4 and 8), else 4;
//   stage 1: lanes per workgroup, one block per lane: 128 at W = 2 from
//            2^20 blocks per rank (3-5% faster at 64 MB per rank), else 256.
inline int s0_quarters_per_lane(int W, size_t n, int bits) {
  return (uint64_t)W * n >= (1ull << 28) && bits != 8 ? 2 : 4;
}
inline int s2_quarters_per_lane(int W, size_t n) {
  return (uint64_t)W * n >= (1ull << 26) ? 1 : 4;
}
inline int s1_lanes_per_workgroup(int W, size_t nb) {
  return W == 2 && nb >= (1u << 20) ? 128 : kThreads;
}

// Full rounds.  A stage-1 grid gives each CU few workgroups (16 at 64 MB per
// rank), and when the kernel's occupancy does not divide that number the
// last round runs part-empty: 16 workgroups at 5 per CU run as 5 + 5 + 5 + 1.
// round_cap_lds<Kernel> gives the dynamic LDS, which the kernels leave
// unused, that caps a launch of `groups` workgroups at the fewest workgroups
// per CU that keep its number of rounds (here 4 per CU: four full rounds);
// 0 where the kernel's own occupancy already does, where the cap would go
// below 3, or where the occupancy calculator does not confirm that exact cap
// (LDS is allocated in granules).  Host code; lookups are cached per device.
// Measured cold, alternating with uncapped launches: at W=8 and 64 MB per
// rank Q4A 2.5-4.1% faster, Q6A between 0.4% slower and 1.8% faster (the
// other codecs' registers allow 3 or 4 per CU: no cap); at W=4 the same caps
// made Q4A and Q6A 0.5-1.7% slower at 16-64 MB per rank.  So stage 1 takes
// it at W=8 only: the launch whose arithmetic is heaviest against its bytes.
constexpr int kRoundDevices = 64;
constexpr int kRoundMaxCap = 32;

inline int round_device() {
  int d = -1;
  return hipGetDevice(&d) == hipSuccess && d >= 0 && d < kRoundDevices ? d : -1;
}

// CUs and LDS bytes per CU of device dev (-1 where the runtime gives none)
inline void round_resources(int dev, int& cus, int& lds) {
  static std::atomic<int> c_cus[kRoundDevices], c_lds[kRoundDevices];   // 0: not looked up
  cus = c_cus[dev].load(std::memory_order_acquire);
  if (cus == 0) {
    int a = -1, b = -1;
    if (hipDeviceGetAttribute(&a, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) a = -1;
    if (hipDeviceGetAttribute(&b, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
        hipSuccess)
      b = -1;
    c_lds[dev].store(b > 0 ? b : -1, std::memory_order_relaxed);
    c_cus[dev].store(a > 0 ? a : -1, std::memory_order_release);
    cus = a > 0 ? a : -1;
  }
  lds = c_lds[dev].load(std::memory_order_relaxed);
}

template <auto Kernel>
size_t round_cap_lds(int threads, size_t groups) {
  const int dev = round_device();
  if (dev < 0 || groups == 0) return 0;
  int cus = 0, lds = 0;
  round_resources(dev, cus, lds);
  if (cus <= 0 || lds <= 0) return 0;
  // workgroups per CU the kernel's own resources allow (threads is the same
  // at every launch of one kernel)
  static std::atomic<int> c_nat[kRoundDevices];                          // 0: not looked up
  int nat = c_nat[dev].load(std::memory_order_relaxed);
  if (nat == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &nat, reinterpret_cast<const void*>(Kernel), threads, 0) != hipSuccess || nat <= 0)
      nat = -1;
    c_nat[dev].store(nat, std::memory_order_relaxed);
  }
  if (nat <= 1) return 0;
  const size_t per_cu = (groups + cus - 1) / cus;
  const size_t rounds = (per_cu + nat - 1) / nat;
  const size_t cap = (per_cu + rounds - 1) / rounds;
  if (cap >= (size_t)nat || cap < 3 || cap >= (size_t)kRoundMaxCap) return 0;
  const size_t bytes = (size_t)lds / cap / 1024 * 1024;
  // whether that many bytes give exactly `cap` workgroups per CU
  static std::atomic<int> c_ok[kRoundDevices][kRoundMaxCap];             // 0: not checked
  int ok = c_ok[dev][cap].load(std::memory_order_relaxed);
  if (ok == 0) {
    int got = 0;
    ok = hipOccupancyMaxActiveBlocksPerMultiprocessor(
             &got, reinterpret_cast<const void*>(Kernel), threads, bytes) == hipSuccess &&
                 got == (int)cap
             ? 1
             : -1;
    c_ok[dev][cap].store(ok, std::memory_order_relaxed);
  }
  return ok > 0 ? bytes : 0;
}

// Tuning knobs (compile-time; the defaults are the measured best on MI355X):
// QR_NT_STORE bit mask of the stages (1 = stage 0, 2 = stage 1, 4 = stage 2)
//             whose streamed outputs are written with non-temporal stores.
//             Default 4: the outputs of stage 2 (the result; through the
//             caches those lines stay dirty and the next kernel pays for
//             their write-back: the W=8 step was 12-14% slower).  Stage 1's
//             reduced image stays cached because stage 2 reads it W times,
//             and so do stage 0's wire data, which stage 1 reads next (with
//             stage 0's loads non-temporal, cached stores made the W=8 step
//             1.5% faster: FP 5%, Q4 3%, the asymmetric 8- and 4-bit codes 1%
//             slower).
// QR_NT_LOAD  bit mask of the stages whose read-once inputs are loaded with
//             non-temporal loads.  Default 3: the inputs of stage 0 and the
//             wire data of stage 1 from W = 4 up (kS1Stream), wherever each
//             load instruction of a wave reads one contiguous range (Stream
//             below).  Cold at W=8, 64 MB per rank, against cached loads:
//             stage 1 of Q4A 11% faster, Q4 9%, FP 7%; the stage-1 reads then
//             also leave the reduced image in the Infinity Cache for stage
//             2's W reads (with cached stage-1 loads the W=8 FP allreduce took
//             444 us instead of 395, the 8-bit codes 6-11% longer); and the
//             whole step 3% faster from stage 0's.  At W = 4 stage 1 is 3-5%
//             faster cold.  At W = 2 cached loads are better (cold stage 1
//             3-6% faster, the allreduce 0.5%), so stage 1 keeps them there.
//             Where two instructions read halves of the same lines (32-byte
//             code blocks read as two 16-byte words per lane), non-temporal
//             loads made stage 1 about 10% slower, so those stay cached: the
//             receive buffer stores such codes word-major (WireAt) so that
//             stage 1 can stream them, and the planar wire images keep cached
//             loads for them.  Stage 2 and the one-stage allreduce re-read
//             their inputs and always load through the caches.
#ifndef QR_NT_STORE
#define QR_NT_STORE 4
#endif
#ifndef QR_NT_LOAD
#define QR_NT_LOAD 3
#endif
constexpr int kStage0 = 1, kStage1 = 2, kStage2 = 4;
constexpr int kKeep = 0;           // store policy: always through the caches
// stage 1's wire-data loads stream (non-temporal, QR_NT_LOAD) from W = 4 up
template <int W>
constexpr int kS1Load = W >= 4 ? kStage1 : kKeep;

template <int Stage, typename V>
__device__ __forceinline__ void st_out(V* p, V v) {
  if constexpr ((QR_NT_STORE & Stage) != 0)
    __builtin_nontemporal_store(v, p);
  else
    *p = v;
}
// Stream: every load instruction of a wave at this site reads one contiguous
// range, so no line is fetched by two instructions.  Stage kKeep: cached.
template <int Stage, bool Stream = true, typename V>
__device__ __forceinline__ V ld_in(const V* p) {
  if constexpr ((QR_NT_LOAD & Stage) != 0 && Stream)
    return __builtin_nontemporal_load(p);
  else
    return *p;
}

struct Geo {
  uint32_t n;        // elements per rank
  uint32_t nb;       // blocks per rank
  uint32_t off_s;    // scale plane offset
  uint32_t off_z;    // zero plane offset
  uint32_t tstride;  // receive buffer: bytes from one tile of a rank to its next (W tiles)
  uint32_t tile0;    // receive buffer: the tile the ranks' base pointers point at
};

// Byte offsets of block blk's codes, scale and zero from a rank's base
// pointer, in 32 bits (a uniform 64-bit base plus a 32-bit offset: the
// loads and stores take the base in scalar registers and one offset register
// serves every rank).  Recv == false: the planar wire image (codes at
// blk * CB, scales and zeros in their planes; a wire image is below 4 GiB).
// Recv == true: the rank's tiles in the receive buffer, the base being its
// tile tile0; tile t = blk / kTileBlocks starts (t - tile0) * tstride further
// and holds kTileBlocks blocks' codes, then their scales, then their zeros
// (the host launches tile ranges whose offsets stay below 4 GiB).  A tile's
// codes are stored word-major: the blocks' code bytes are cut into words of
// kWord bytes (16; 8 for 24-byte blocks) and word k of all kTileBlocks
// blocks is contiguous, so that a wave whose lanes take consecutive blocks
// reads one contiguous range with each load instruction (16-byte blocks are
// one word: their layout is the planar one's).
template <int CB, bool Recv>
struct WireAt {
  static constexpr uint32_t kTB = kTileBlocks;
  static constexpr uint32_t kWord = CB == 24 ? 8 : 16;
  __device__ static __forceinline__ uint32_t tile(const Geo& g, uint32_t blk) {
    return (blk / kTB - g.tile0) * g.tstride;
  }
  // byte o (< CB) of block blk's codes
  __device__ static __forceinline__ uint32_t code_at(const Geo& g, uint32_t blk, uint32_t o) {
    if constexpr (Recv)
      return tile(g, blk) + (o / kWord) * (kTB * kWord) + (blk % kTB) * kWord + o % kWord;
    return blk * (uint32_t)CB + o;
  }
  __device__ static __forceinline__ uint32_t scale(const Geo& g, uint32_t blk) {
    if constexpr (Recv) return tile(g, blk) + kTB * CB + (blk % kTB) * 2u;
    return g.off_s + blk * 2u;
  }
  __device__ static __forceinline__ uint32_t zero(const Geo& g, uint32_t blk) {
    if constexpr (Recv) return tile(g, blk) + kTB * (CB + 2) + (blk % kTB) * 2u;
    return g.off_z + blk * 2u;
  }
};
template <int C, bool Recv>
using At = WireAt<CodecT<C>::block_bytes, Recv>;

__device__ __forceinline__ uint32_t ld_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}
__device__ __forceinline__ void st_u16(uint8_t* p, uint32_t v) {
  *reinterpret_cast<uint16_t*>(p) = (uint16_t)v;
}

// Byte offset (32 bits, as above) of 16-byte chunk c of a rank's raw data
// (the FP codec's wire): planar, or in the rank's tiles of the receive
// buffer from its tile tile0 (a tile holds the kTileBlocks * 4 chunks of its
// blocks).
template <bool Recv>
__device__ __forceinline__ uint32_t fp_chunk(uint32_t tstride, uint32_t tile0, uint32_t c) {
  constexpr uint32_t kTC = kTileBlocks * 4;
  if constexpr (Recv) return (c / kTC - tile0) * tstride + (c % kTC) * 16u;
  return c * 16u;
}

// the W code blocks and scales (and zeros) of one block index
template <int C, int W>
struct S1In {
  uint32_t cw[W][CodecT<C>::words];
  uint32_t sh[W], zh[W];     // binary16 scale and zero bits
};

// the W ranks' code blocks and scales (and zeros) of block blk; Recv: from
// the ranks' tiles of the receive buffer (the W tiles of one workgroup's
// blocks are consecutive there, so the workgroup reads one contiguous range)
template <int C, int W, bool Recv>
__device__ __forceinline__ void s1_load(const InPtrs& wires, uint32_t blk, const Geo& g,
                                        S1In<C, W>& in) {
  using T = CodecT<C>;
  // word k of every lane's block: one contiguous range per wave in the
  // receive buffer (word-major) and for 16-byte blocks (one word)
  constexpr bool kStream = Recv || T::block_bytes == 16;
  const uint32_t so = At<C, Recv>::scale(g, blk), zo = At<C, Recv>::zero(g, blk);
#pragma unroll
  for (int r = 0; r < W; r++) {
    if constexpr (T::words == 6) {
#pragma unroll
      for (int k = 0; k < 3; k++) {
        const u32x2 q = ld_in<kS1Load<W>, kStream>(
            reinterpret_cast<const u32x2*>(wires.p[r] + At<C, Recv>::code_at(g, blk, 8 * k)));
        in.cw[r][2 * k] = q.x;
        in.cw[r][2 * k + 1] = q.y;
      }
    } else {
#pragma unroll
      for (int k = 0; k < T::words / 4; k++) {
        const u32x4 q = ld_in<kS1Load<W>, kStream>(
            reinterpret_cast<const u32x4*>(wires.p[r] + At<C, Recv>::code_at(g, blk, 16 * k)));
        in.cw[r][4 * k] = q.x; in.cw[r][4 * k + 1] = q.y;
        in.cw[r][4 * k + 2] = q.z; in.cw[r][4 * k + 3] = q.w;
      }
    }
    in.sh[r] = ld_u16(wires.p[r] + so);
    in.zh[r] = T::asym ? ld_u16(wires.p[r] + zo) : 0u;
    // Loads issue rank by rank, and all before any arithmetic.  Loads
    // retire in issue order, so rank 0's sum can start once its own three
    // have landed; left to itself the scheduler groups all codes before all
    // scales and zeros, or holds back the last ranks' loads to save
    // registers, and either way more of the latency is exposed at W=8.
    __builtin_amdgcn_sched_barrier(0);
  }
}

// the reduced block's codes w, scale s and zero z into the reduced image (a
// planar wire image)
template <int C>
__device__ __forceinline__ void s1_store(uint8_t* red, uint32_t blk, const Geo& g,
                                         const uint32_t (&w)[CodecT<C>::words], uint32_t s,
                                         uint32_t z) {
  using T = CodecT<C>;
  uint8_t* cb = red + At<C, false>::code_at(g, blk, 0);
  const uint32_t so = At<C, false>::scale(g, blk), zo = At<C, false>::zero(g, blk);
  if constexpr (T::words == 6) {
#pragma unroll
    for (int k = 0; k < 3; k++)
      st_out<kStage1>(reinterpret_cast<u32x2*>(cb) + k, u32x2{w[2 * k], w[2 * k + 1]});
  } else {
#pragma unroll
    for (int k = 0; k < T::words / 4; k++)
      st_out<kStage1>(reinterpret_cast<u32x4*>(cb) + k,
                      u32x4{w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]});
  }
  st_u16(red + so, s);
  if constexpr (T::asym) st_u16(red + zo, z);
}

}  // namespace
}  // namespace qr
