// qr_kernels.hip -- gfx950 kernels of the two-stage quantized allreduce.
//
//   k_quantize   stage 0: binary16/bfloat16 -> codes + scale (+ zero)
//   k_stage1     stage 1: W wire blocks -> dequantize -> binary32 sum in rank
//                order -> requantize (one pass over HBM per byte)
//   k_sum_fp     stage 1 of the FP codec, and the one-stage allreduce: sum of
//                the raw buffers, rounded once
//   k_dequant    stage 2 / dequantize: codes -> binary16/bfloat16, W outputs
//   k_copy       stages 0 and 2 of the FP codec (the wire is the raw data;
//                converted under the bf16 -> fp16 cast option)
//   k_fused      all three stages in one launch for small buffers, each
//   k_fused_fp   workgroup taking its tile of blocks through all three
//
// The method is the 2-stage allreduce of "Integrate quick allreduce and
// select the best allreduce implementation" (vLLM PR #18473, PR description
// item 2), with the symmetric/asymmetric integer codecs of "Add quickreduce
// as alternative to custom allreduce" (vLLM PR #16804, PR description).
//
// Every kernel streams HBM; nothing is a contraction, so no MFMA and no LDS.
//   - k_quantize and k_dequant work on quarter blocks (8 elements = 16
//     contiguous bytes of 16-bit data, consecutive lanes on consecutive
//     quarters).  k_quantize takes U = 4 or 2 quarters per lane (by size and
//     code width, s0_quarters_per_lane), issued before any is used, so that a quad of
//     lanes holds the quarters of U blocks: it reduces each block's max/min
//     with DPP quad permutes, lane j derives the scale of block j mod U, and
//     1/s reaches the other lanes by a DPP broadcast (a few instructions,
//     instead of a round trip through LDS).  k_dequant takes 4 or 1 quarters
//     per lane (s2_quarters_per_lane).
//   - k_stage1 gives each lane a whole block: W code blocks of 16/24/32
//     bytes and W scales in, one code block and scale out; the per-block
//     work (max/min, two divisions, rounding of the scale) is done once,
//     which matters because this kernel is the one closest to the VALU limit
//     (W=2, 4-bit codes: 1.7 bytes of HBM per element).  From the receive
//     buffer, whose tiles hold the codes word-major, each load instruction of
//     a wave reads one contiguous range, so from W = 4 up the wire data
//     stream in with non-temporal loads (QR_NT_LOAD).
//   - the FP kernels give each lane 16-byte chunks, four per lane (stage
//     2: as k_dequant).
//   - k_fused gives each lane one quarter block of every rank (a workgroup
//     holds 64 blocks) and quantizes four ranks at a time as the four slots
//     of the quad quantizer.
#include <atomic>
#include <mutex>

#include "qr.h"
#include "qr_device.h"
#include "qr_internal.h"
#include "qr_stage_io.h"

// The workspace of qr_allreduce_sim_noalloc: one buffer per GPU, held for the
// life of the process.  In host code `scratch` names a host-side stand-in,
// not device memory: kernels receive the address that hipGetSymbolAddress
// returns for the current device (scratch_address below), never the name.
static __device__ __align__(256) uint8_t scratch[QR_SCRATCH_BYTES];

namespace qr {
namespace {

// Bytes of codes of quarter j (0..3) of a block: 8 codes = 8*b bits starting
// at bit 8*b*j of the block's bitstring.  Returned as words with the first
// code at bit 0: for 6-bit codes two words hold the 48 bits (quarters 1 and 3
// start in the middle of a word).
template <int C>
struct QuarterIO {
  static constexpr int b = CodecT<C>::bits;
  static constexpr int nw = (8 * b + 31) / 32;     // 1 (4-bit), 2 (6/8-bit)

  __device__ static void load(const uint8_t* blk, int j, uint32_t (&w)[nw]) {
    if constexpr (b == 4) {
      w[0] = reinterpret_cast<const uint32_t*>(blk)[j];
    } else if constexpr (b == 8) {
      const u32x2 q = reinterpret_cast<const u32x2*>(blk)[j];
      w[0] = q.x;
      w[1] = q.y;
    } else {                                         // 6-bit: bits [48j, 48j+48)
      const uint32_t* p = reinterpret_cast<const uint32_t*>(blk) + ((3 * j) >> 1);
      const uint32_t a = p[0], c = p[1];
      const int sh = (j & 1) * 16;
      w[0] = __builtin_amdgcn_alignbit(c, a, sh);
      w[1] = c >> sh;
    }
  }
  // the same quarter of block blk from a rank's tiles of the receive buffer
  // (base: the rank's tile g.tile0; word-major codes)
  __device__ static void load_recv(const uint8_t* base, const Geo& g, uint32_t blk, int j,
                                   uint32_t (&w)[nw]) {
    using A = At<C, true>;
    if constexpr (b == 4) {
      w[0] = *reinterpret_cast<const uint32_t*>(base + A::code_at(g, blk, 4 * j));
    } else if constexpr (b == 8) {
      const u32x2 q = *reinterpret_cast<const u32x2*>(base + A::code_at(g, blk, 8 * j));
      w[0] = q.x;
      w[1] = q.y;
    } else {
      const uint32_t i0 = (3 * j) >> 1;              // its first 32-bit word of the block
      const uint32_t a = *reinterpret_cast<const uint32_t*>(base + A::code_at(g, blk, 4 * i0));
      const uint32_t c =
          *reinterpret_cast<const uint32_t*>(base + A::code_at(g, blk, 4 * i0 + 4));
      const int sh = (j & 1) * 16;
      w[0] = __builtin_amdgcn_alignbit(c, a, sh);
      w[1] = c >> sh;
    }
  }
};

// ---------------------------------------------------------------------------
// stage 0: quarter blocks, U (4 or 2) per lane.  For each u the four
// lanes of a quad hold the four quarters of one block, so a quad covers U
// blocks.  Every lane reduces the max/min of all U blocks across the quad,
// then lane j derives the scale (and zero) of block j mod U and hands 1/s,
// the zero and two flags to the others (DPP quad broadcasts): with U = 4 each
// block's divisions and roundings run once, with U = 2 twice.

// max/min with a quad neighbour in one instruction: the DPP permute is the
// first source of v_max_f32/v_min_f32 itself.  (Written as a permute and an
// fmaxf, or as med3 with an infinite bound, the compiler emits a permute, a
// canonicalizing v_max of the permuted value and the max: three
// instructions; the values here are never NaN, for which canonicalizing is a
// no-op.)  The s_nop gives the two wait states a DPP read needs after a VALU
// write of its source, which the compiler does not insert for inline asm.
template <int Ctrl>
__device__ __forceinline__ float quad_max(float v) {
  static_assert(Ctrl == kSwap1 || Ctrl == kSwap2, "quad swaps only");
  float r;
  if constexpr (Ctrl == kSwap1)
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "=&v"(r) : "v"(v));
  else
    asm("s_nop 1\n\tv_max_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "=&v"(r) : "v"(v));
  return r;
}
template <int Ctrl>
__device__ __forceinline__ float quad_min(float v) {
  static_assert(Ctrl == kSwap1 || Ctrl == kSwap2, "quad swaps only");
  float r;
  if constexpr (Ctrl == kSwap1)
    asm("s_nop 1\n\tv_min_f32_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
        : "=&v"(r) : "v"(v));
  else
    asm("s_nop 1\n\tv_min_f32_dpp %0, %1, %1 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
        : "=&v"(r) : "v"(v));
  return r;
}

// quad_perm [u,u,u,u]: the value of lane u of the quad
template <int U>
__device__ __forceinline__ float from_lane(float v) { return quad_perm<U * 0x55>(v); }
template <int U>
__device__ __forceinline__ uint32_t from_lane_u(uint32_t v) { return quad_perm_u<U * 0x55>(v); }

// Quantizes U slots of 8 values per lane (U = 1, 2 or 4): slot u holds
// quarter q[u] of the wire image wire[u], and in every slot the four lanes of
// a quad hold the four quarters of one block (lane j quarter j).  Block
// statistics come through quad permutes; lane j derives the parameters of
// slot (j mod U)'s block, lane j < U stores that block's scale (and zero) and
// hands 1/s, the zero and two flags to the quad; every lane then encodes and
// stores its own quarter of every slot.  own_wire and own_q are wire[j mod U]
// and q[j mod U], which the caller can form more cheaply than a select.
// Quarters at or past q_end store nothing; quarters holding no element
// (8q >= n) are left out of the statistics and get code 0.  q_end is a
// multiple of 4, so a quad is wholly in or out.  Full: the caller guarantees
// that every quarter holds 8 elements and lies below q_end (no range checks
// are made).  Recv: the wire data go to a rank's tiles of the receive buffer
// (wire[u] the rank's base there) instead of a planar wire image.
template <int C, int Stage, bool Full, int U, bool Recv>
__device__ __forceinline__ void quantize_core(float (&v)[U][8], uint8_t* const (&wire)[U],
                                              const uint32_t (&q)[U], uint8_t* own_wire,
                                              uint32_t own_q, uint32_t q_end, const Geo& g) {
  static_assert(U == 1 || U == 2 || U == 4, "slots per lane");
  using T = CodecT<C>;
  constexpr int nw = (8 * T::bits + 31) / 32;
  const int j = threadIdx.x & 3;                // this lane's quarter of each block
  // every lane stays active through the quad exchanges below; quarters past
  // the end compute on stand-in data and store nothing
  float mx[U], mn[U];
#pragma unroll
  for (int u = 0; u < U; u++) {
    group_max_min(v[u], Full || 8 * q[u] < g.n, mx[u], mn[u]);
    mx[u] = quad_max<kSwap2>(quad_max<kSwap1>(mx[u]));
    mn[u] = quad_min<kSwap2>(quad_min<kSwap1>(mn[u]));
  }
  // lane j: parameters of slot j mod U
  float bx = mx[0], bn = mn[0];
#pragma unroll
  for (int u = 1; u < U; u++) {
    if (j % U == u) {
      bx = mx[u];
      bn = mn[u];
    }
  }
  const BlockParams<C> p = block_params<C>(bx, bn);
  if (j < U && (Full || own_q < q_end)) {
    const uint32_t own_blk = own_q >> 2;
    st_u16(own_wire + At<C, Recv>::scale(g, own_blk), p.s);
    if constexpr (T::asym) st_u16(own_wire + At<C, Recv>::zero(g, own_blk), p.z);
  }
  const uint32_t flags = (p.sat ? 1u : 0u) | (p.s != 0u ? 2u : 0u);
  float inv[U], tz[U];
  uint32_t fl[U];
  inv[0] = from_lane<0>(p.inv);
  fl[0] = from_lane_u<0>(flags);
  if constexpr (T::asym) tz[0] = from_lane<0>(p.tz);
  if constexpr (U > 1) {
    inv[1] = from_lane<1>(p.inv);
    fl[1] = from_lane_u<1>(flags);
    if constexpr (T::asym) tz[1] = from_lane<1>(p.tz);
  }
  if constexpr (U > 2) {
    inv[2] = from_lane<2>(p.inv); inv[3] = from_lane<3>(p.inv);
    fl[2] = from_lane_u<2>(flags); fl[3] = from_lane_u<3>(flags);
    if constexpr (T::asym) {
      tz[2] = from_lane<2>(p.tz);
      tz[3] = from_lane<3>(p.tz);
    }
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; i++) t[i] = T::asym ? (v[u][i] - tz[u]) * inv[u] : v[u][i] * inv[u];
    uint32_t w[nw];
    encode<C, 8>(t, (fl[u] & 1u) != 0u, w);
    // fp8: an all-zero block gives code 0x00 even for -0 inputs; every codec:
    // quarters beyond the buffer hold code 0
    const bool keep = (Full || 8 * q[u] < g.n) && (!T::fp8 || (fl[u] & 2u) != 0u);
#pragma unroll
    for (int k = 0; k < nw; k++) w[k] = keep ? w[k] : 0u;
    const uint32_t blk = q[u] >> 2;
    if constexpr (T::bits == 6 && Recv) {
      // word-major 8-byte words: lanes 0, 1, 2 of the quad each write word j,
      // bits [64j, 64j+64) of the block's bitstring: the top of their own 48
      // bits (from bit 16j) and the bottom of the next lane's
      const uint32_t n0 = quad_perm_u<kFromNext>(w[0]);
      const uint32_t n1 = quad_perm_u<kFromNext>(w[1]);
      const uint64_t a = ((uint64_t)(w[1] & 0xffffu) << 32) | w[0];
      const uint64_t b = ((uint64_t)(n1 & 0xffffu) << 32) | n0;
      const uint64_t word = (a >> (16 * j)) | (b << (48 - 16 * j));
      if ((Full || q[u] < q_end) && j < 3)
        st_out<Stage>(reinterpret_cast<u32x2*>(wire[u] + At<C, true>::code_at(g, blk, 8 * j)),
                      u32x2{(uint32_t)word, (uint32_t)(word >> 32)});
    } else if constexpr (T::bits == 6) {
      uint8_t* cb = wire[u] + At<C, false>::code_at(g, blk, 0);
      // lanes 0 and 2 of the quad each write 96 bits (their own 48 and their
      // odd neighbour's 48)
      const uint32_t o0 = quad_perm_u<kFromOdd>(w[0]);
      const uint32_t o1 = quad_perm_u<kFromOdd>(w[1]);
      if ((Full || q[u] < q_end) && (j & 1) == 0) {
        uint32_t* d = reinterpret_cast<uint32_t*>(cb) + 3 * (j >> 1);
        st_out<Stage>(d, w[0]);
        st_out<Stage>(d + 1, (w[1] & 0xffffu) | (o0 << 16));
        st_out<Stage>(d + 2, (o0 >> 16) | (o1 << 16));
      }
    } else if (Full || q[u] < q_end) {
      // quarter j: bytes [4j, 4j+4) or [8j, 8j+8) of the block's codes
      uint8_t* d = wire[u] + At<C, Recv>::code_at(g, blk, T::bits * j);
      if constexpr (T::bits == 4)
        st_out<Stage>(reinterpret_cast<uint32_t*>(d), w[0]);
      else
        st_out<Stage>(reinterpret_cast<u32x2*>(d), u32x2{w[0], w[1]});
    }
  }
}

// U quarters q0 + 256u (u < U) of one wire image: in slot u a quad holds the
// four quarters of one block, and lane j derives (and lane j < U stores) the
// parameters of slot j mod U
template <int C, int Stage, bool Full, bool Recv, int U>
__device__ __forceinline__ void quantize_quarters(float (&v)[U][8], uint32_t q0,
                                                  uint32_t q_end, uint8_t* wire,
                                                  const Geo& g) {
  uint8_t* wp[U];
  uint32_t qs[U];
#pragma unroll
  for (int u = 0; u < U; u++) {
    wp[u] = wire;
    qs[u] = q0 + u * kThreads;
  }
  quantize_core<C, Stage, Full, U, Recv>(v, wp, qs, wire,
                                         q0 + ((threadIdx.x & 3) % U) * kThreads, q_end, g);
}

template <int C, int D, bool Full, bool Recv, int U, int Stage = kStage0>
__device__ __forceinline__ void quantize_tile(const u32x4 (&raw)[U], uint32_t q0,
                                              uint8_t* wire, const Geo& g) {
  float v[U][8];
#pragma unroll
  for (int u = 0; u < U; u++) {
    const uint32_t rw[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
    for (int k = 0; k < 4; k++) {
      v[u][2 * k] = ld16<D>(rw[k] & 0xffffu);
      v[u][2 * k + 1] = ld16<D>(rw[k] >> 16);
    }
  }
  quantize_quarters<C, Stage, Full, Recv, U>(v, q0, 4 * g.nb, wire, g);
}

template <bool Full, int U>
__device__ __forceinline__ void load_tile(const uint8_t* x, uint32_t q0, uint32_t n,
                                          u32x4 (&raw)[U]) {
#pragma unroll
  for (int u = 0; u < U; u++) {
    const uint32_t q = q0 + u * kThreads;
    raw[u] = ld_in<kStage0>(reinterpret_cast<const u32x4*>(x) + (Full || 8 * q < n ? q : 0u));
  }
}

// The (unit, rank) a stage-0 workgroup takes, a unit being the
// kThreads * K quarters or chunks the workgroup covers (4 / K units per tile
// of the receive buffer).  Into W planar wire images: blockIdx = (unit,
// rank), so that consecutive workgroups read and write consecutive units of
// one rank.  Into the receive buffer: workgroup (t*W + r) * (4/K) + k takes
// unit k of tile t of rank r, so that consecutive workgroups write
// consecutive bytes of the buffer (the rank-major order writes it at a
// stride of W tiles, which made stage 0 4-9% slower at W=8, 64 MB per rank).
template <bool Recv, int K>
__device__ __forceinline__ void s0_item(int W, uint32_t tile0, uint32_t& unit, int& r) {
  constexpr uint32_t per = 4 / K;               // units per tile
  if constexpr (Recv) {
    const uint32_t tw = blockIdx.x / per;         // (tile - tile0) * W + r
    unit = (tile0 + tw / (uint32_t)W) * per + blockIdx.x % per;
    r = (int)(tw % (uint32_t)W);
  } else {
    unit = blockIdx.x;
    r = blockIdx.y;
  }
}

template <int C, int D, bool Recv, int U>
__global__ __launch_bounds__(kThreads) void k_quantize(InPtrs xs, OutPtrs wires, Geo g, int W) {
  static_assert(kThreads == kTileBlocks && 4 % U == 0, "4 / U workgroups per tile");
  uint32_t unit;
  int r;
  s0_item<Recv, U>(W, g.tile0, unit, r);
  const uint32_t q0 = unit * (kThreads * U) + threadIdx.x;
  u32x4 raw[U];
  // uniform: every quarter of the workgroup holds 8 elements (the path
  // without per-quarter range checks)
  if (8ull * ((uint64_t)unit + 1ull) * (kThreads * U) <= (uint64_t)g.n) {
    load_tile<true, U>(xs.p[r], q0, g.n, raw);
    quantize_tile<C, D, true, Recv, U>(raw, q0, wires.p[r], g);
  } else {
    load_tile<false, U>(xs.p[r], q0, g.n, raw);
    quantize_tile<C, D, false, Recv, U>(raw, q0, wires.p[r], g);
  }
}

// stages 0 and 2 of FP: dst.p[r] <- src.p[r], 16-byte chunks, four per
// lane (a workgroup's 1024 chunks are one tile); Stage selects the store
// policy (and names the two uses apart in profiles); Din != Dout converts
// every element (the cast option: bfloat16 into a binary16 wire at stage 0,
// binary16 back to bfloat16 at stage 2); Recv: the destination is a rank's
// tiles of the receive buffer
template <int Stage, int Din, int Dout, bool Recv, int K = kPerLane>
__global__ __launch_bounds__(kThreads) void k_copy(InPtrs src, OutPtrs dst,
                                                   uint32_t nchunks, uint32_t tstride,
                                                   uint32_t tile0, int W) {
  static_assert(kThreads * kPerLane == kTileBlocks * 4, "stage 0: a workgroup's chunks are one tile");
  constexpr int kS = Stage == 0 ? kStage0 : kStage2;
  // stage 0 (into the receive buffer, or planar) keeps one tile per
  // workgroup; stage 2 (planar) takes K chunks per lane
  static_assert(Stage != 0 || K == kPerLane, "stage 0: one tile per workgroup");
  uint32_t unit;
  int r;
  s0_item<Recv, Stage == 0 ? kPerLane : 4>(W, tile0, unit, r);
  const u32x4* s = reinterpret_cast<const u32x4*>(src.p[r]);
  uint8_t* d = dst.p[r];
  const uint32_t base = unit * (kThreads * K) + threadIdx.x;
  u32x4 q[K];
#pragma unroll
  for (int j = 0; j < K; j++) {
    const uint32_t c = base + j * kThreads;
    q[j] = ld_in<kS>(s + (c < nchunks ? c : 0u));
  }
#pragma unroll
  for (int j = 0; j < K; j++) {
    const uint32_t c = base + j * kThreads;
    if constexpr (Din != Dout) {
#pragma unroll
      for (int k = 0; k < 4; k++)
        q[j][k] = st16x2<Dout>(ld16<Din>(q[j][k] & 0xffffu), ld16<Din>(q[j][k] >> 16));
    }
    if (c < nchunks)
      st_out<kS>(reinterpret_cast<u32x4*>(d + fp_chunk<Recv>(tstride, tile0, c)), q[j]);
  }
}

// ---------------------------------------------------------------------------
// stage 1: one block per lane

// Full: the block holds 32 elements (no partial-block handling)
template <int C, int W, bool Full>
__device__ __forceinline__ void s1_reduce_store(const S1In<C, W>& in, uint8_t* red,
                                                uint32_t blk, const Geo& g) {
  using T = CodecT<C>;
  const uint32_t e0 = blk * kBlock;
  const int L = Full || g.n - e0 >= (uint32_t)kBlock ? kBlock : (int)(g.n - e0);
  // acc = x0 + x1 + ... in rank order.  For W <= 4, 4- and 8-bit codes a
  // word-aligned group of 8 at a time, so that each group's code values are
  // used as soon as they are formed: fewer live registers, higher occupancy.
  // (6-bit groups of 8 start mid-word, and at W = 8 the compiler does better
  // with whole blocks.)
  float acc[kBlock];
#pragma unroll
  for (int r = 0; r < W; r++) {
    if constexpr (T::asym && (T::bits == 4 || T::bits == 6)) {
      // scale and zero straight from their binary16 bits (add_codes_asym)
      const float S0 = h2f_times(in.sh[r], 16777216.0f);
      const float S4 = T::bits == 4 ? h2f_times(in.sh[r], 1048576.0f) : 0.0f;
      if constexpr (T::bits == 6 || W > 4) {
        add_codes_asym<C, kBlock>(acc, in.cw[r], S0, S4, in.zh[r], r == 0);
      } else {
#pragma unroll
        for (int k = 0; k < 4; k++) {
          float a8[8];
#pragma unroll
          for (int i = 0; i < 8; i++) a8[i] = acc[8 * k + i];
          add_codes_asym<C, 8>(a8, in.cw[r] + k, S0, S4, in.zh[r], r == 0);
#pragma unroll
          for (int i = 0; i < 8; i++) acc[8 * k + i] = a8[i];
        }
      }
      continue;
    }
    const float sc = h2f(in.sh[r]) * T::unpack_scale;
    const float zc = T::asym ? h2f(in.zh[r]) : 0.0f;
    if constexpr (T::bits == 6 || W > 4) {
      add_codes<C, kBlock>(acc, in.cw[r], sc, zc, r == 0);
    } else {
#pragma unroll
      for (int k = 0; k < 4; k++) {
        float a8[8];
#pragma unroll
        for (int i = 0; i < 8; i++) a8[i] = acc[8 * k + i];
        add_codes<C, 8>(a8, in.cw[r] + k * (8 * T::bits / 32), sc, zc, r == 0);
#pragma unroll
        for (int i = 0; i < 8; i++) acc[8 * k + i] = a8[i];
      }
    }
  }
  float mx, mn;
  if constexpr (Full) {
    block_max_min(acc, mx, mn);
  } else {
    float gx, gn;
    group_max_min(acc, true, mx, mn);
#pragma unroll
    for (int k = 1; k < 4; k++) {
      group_max_min(acc + 8 * k, 8 * k < L, gx, gn);
      mx = fmaxf(mx, gx);
      mn = fminf(mn, gn);
    }
  }
  const BlockParams<C> p = block_params<C>(mx, mn);
  uint32_t w[T::words];
  quantize_values<C, kBlock>(acc, p, w);
  if (!Full && L < kBlock) {                      // unused slots hold code 0
#pragma unroll
    for (int k = 0; k < T::words; k++) {
      const int first = L * T::bits - 32 * k;     // first unused bit in word k
      w[k] = first <= 0 ? 0u : first >= 32 ? w[k] : w[k] & ((1u << first) - 1u);
    }
  }
  s1_store<C>(red, blk, g, w, p.s, p.z);
}

// one lane per block, TB lanes per workgroup
template <int C, int D, int W, bool Recv, int TB>
__global__ __launch_bounds__(kThreads) void k_stage1(InPtrs wires, uint8_t* red,
                                                     uint32_t blk_lo, uint32_t blk_hi,
                                                     Geo g) {
  const uint32_t blk = blk_lo + blockIdx.x * TB + threadIdx.x;
  // uniform: every block of the workgroup is in range and holds 32 elements
  const uint32_t wg_end = blk_lo + (blockIdx.x + 1) * TB;
  if (wg_end <= blk_hi && (uint64_t)wg_end * kBlock <= (uint64_t)g.n) {
    S1In<C, W> in;
    s1_load<C, W, Recv>(wires, blk, g, in);
    s1_reduce_store<C, W, true>(in, red, blk, g);
    return;
  }
  if (blk >= blk_hi) return;
  S1In<C, W> in;
  s1_load<C, W, Recv>(wires, blk, g, in);
  s1_reduce_store<C, W, false>(in, red, blk, g);
}

// Sum of W raw buffers over 16-byte chunks [c_lo, c_hi): the binary32 sum
// in rank order 0..W-1, rounded once to D, into outs.p[blockIdx.y].  Stage 1
// of the FP codec (one output: the reduced image; Recv: the inputs are the
// ranks' tiles of the receive buffer) and the one-stage allreduce
// (gridDim.y = W: every rank reads all W buffers and writes its own output).
// Stage selects the store policy of the outputs.
template <int D, int W, int Stage, bool Recv>
__global__ __launch_bounds__(kThreads) void k_sum_fp(InPtrs xs, OutPtrs outs,
                                                     uint32_t c_lo, uint32_t c_hi,
                                                     uint32_t tstride, uint32_t tile0) {
  const uint32_t base = c_lo + blockIdx.x * (kThreads * kPerLane) + threadIdx.x;
  u32x4 q[kPerLane][W];
#pragma unroll
  for (int j = 0; j < kPerLane; j++) {
    const uint32_t c = base + j * kThreads;
    const uint32_t off = fp_chunk<Recv>(tstride, tile0, c < c_hi ? c : c_lo);
#pragma unroll
    for (int r = 0; r < W; r++)
      q[j][r] = ld_in<Stage == kStage1 ? kS1Load<W> : kKeep>(
          reinterpret_cast<const u32x4*>(xs.p[r] + off));
  }
  u32x4* out_p = reinterpret_cast<u32x4*>(outs.p[blockIdx.y]);
#pragma unroll
  for (int j = 0; j < kPerLane; j++) {
    const uint32_t c = base + j * kThreads;
    if (c >= c_hi) break;
    uint32_t out[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      float lo = ld16<D>(q[j][0][k] & 0xffffu), hi = ld16<D>(q[j][0][k] >> 16);
#pragma unroll
      for (int r = 1; r < W; r++) {
        lo = lo + ld16<D>(q[j][r][k] & 0xffffu);
        hi = hi + ld16<D>(q[j][r][k] >> 16);
      }
      out[k] = st16x2<D>(lo, hi);
    }
    st_out<Stage>(out_p + c, u32x4{out[0], out[1], out[2], out[3]});
  }
}

// ---------------------------------------------------------------------------
// stage 2 / dequantize: quarter blocks, U per lane

// quarters q0 + 256u (u < U) of the wire -> y; Full: all hold 8 elements
template <int C, int D, bool Full, int U, int Stage = kStage2>
__device__ __forceinline__ void dequant_tile(const uint8_t* wire, uint8_t* y, uint32_t q0,
                                             uint32_t nq, const Geo& g) {
  using T = CodecT<C>;
  using IO = QuarterIO<C>;
  uint32_t w[U][IO::nw];
  float s[U], z[U];
#pragma unroll
  for (int u = 0; u < U; u++) {
    const uint32_t q = Full || q0 + u * kThreads < nq ? q0 + u * kThreads : 0u;  // no branch
    const uint32_t blk = q >> 2;
    IO::load(wire + (size_t)blk * T::block_bytes, q & 3, w[u]);
    s[u] = h2f(ld_u16(wire + g.off_s + (size_t)blk * 2)) * T::unpack_scale;
    z[u] = T::asym ? h2f(ld_u16(wire + g.off_z + (size_t)blk * 2)) : 0.0f;
  }
#pragma unroll
  for (int u = 0; u < U; u++) {
    const uint32_t q = q0 + u * kThreads;
    if (!Full && q >= nq) break;
    float cv[8];
    code_values<C, 8>(w[u], cv);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; i++)
      v[i] = T::asym ? __builtin_fmaf(cv[i], s[u], z[u]) : cv[i] * s[u];
    st_out<Stage>(reinterpret_cast<u32x4*>(y) + q,
                  u32x4{st16x2<D>(v[0], v[1]), st16x2<D>(v[2], v[3]),
                        st16x2<D>(v[4], v[5]), st16x2<D>(v[6], v[7])});
  }
}

template <int C, int D, int U>
__global__ __launch_bounds__(kThreads) void k_dequant(const uint8_t* wire, OutPtrs ys,
                                                      Geo g) {
  const int r = blockIdx.y;
  const uint32_t nq = (g.n + 7) / 8;                // quarters that hold data
  const uint32_t q0 = blockIdx.x * (kThreads * U) + threadIdx.x;
  if (8ull * ((uint64_t)blockIdx.x + 1ull) * (kThreads * U) <= (uint64_t)g.n)
    dequant_tile<C, D, true, U>(wire, ys.p[r], q0, nq, g);
  else
    dequant_tile<C, D, false, U>(wire, ys.p[r], q0, nq, g);
}

// ---------------------------------------------------------------------------
// the whole simulated allreduce in one launch, for buffers small enough that
// three launches cost more than their work.  A block's three stages need no
// other block, so workgroup T takes blocks [64T, 64T+64) of every rank
// through all three with workgroup barriers in between, and no workgroup
// waits for another.  Lane l holds quarter 256T + l (a quad of lanes = one
// block):
//   stage 0  the lane's quarter of every rank, four ranks at a time as the
//            four slots of quantize_core (lane j of the quad derives the
//            scale of rank j's block), written to the rank's tile of the
//            receive buffer;
//   stage 1  the W quarters read back, dequantized and summed in rank
//            order, quantized as one slot into the reduced image;
//   stage 2  the reduced quarter read back, dequantized once and stored to
//            every rank's output (each rank's output is the same function of
//            the same reduced block).
// The arithmetic is that of the three separate kernels, element for element,
// so the outputs and the workspace are theirs.  The wire and reduced images
// are stored through the caches: the same workgroup reads them next.

template <int C, int D, int W, bool Full>
__device__ __forceinline__ void fused_tile(const InPtrs& xs, const OutPtrs& wires, uint8_t* red,
                                           const OutPtrs& ys, uint32_t q, const Geo& g) {
  using T = CodecT<C>;
  using IO = QuarterIO<C>;
  constexpr int U = W < 4 ? W : 4;                 // ranks per quantize_core call
  const uint32_t q_end = 4 * g.nb;
  const uint32_t nq = (g.n + 7) / 8;               // quarters that hold data
  const bool has = Full || q < nq;
  const uint32_t ql = has ? q : 0u;                // stand-in for loads past the data
  const int j = threadIdx.x & 3;

  // stage 0: every rank's quarter is loaded before any is quantized
  u32x4 raw[W];
#pragma unroll
  for (int r = 0; r < W; r++) raw[r] = reinterpret_cast<const u32x4*>(xs.p[r])[ql];
#pragma unroll
  for (int k = 0; k < W / U; k++) {
    float v[U][8];
    uint8_t* wp[U];
    uint32_t qs[U];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const u32x4 x = raw[k * U + u];
      const uint32_t rw[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
      for (int i = 0; i < 4; i++) {
        v[u][2 * i] = ld16<D>(rw[i] & 0xffffu);
        v[u][2 * i + 1] = ld16<D>(rw[i] >> 16);
      }
      wp[u] = wires.p[k * U + u];
      qs[u] = q;
    }
    uint8_t* own = wp[0];
#pragma unroll
    for (int u = 1; u < U; u++)
      if (j % U == u) own = wp[u];
    quantize_core<C, kKeep, Full, U, true>(v, wp, qs, own, q, q_end, g);
  }
  __syncthreads();

  // stage 1: the lane's quarter of the reduced block
  {
    const uint32_t blk = ql >> 2;
    uint32_t w[W][IO::nw];
    float sc[W], zc[W];
    const uint32_t so = At<C, true>::scale(g, blk), zo = At<C, true>::zero(g, blk);
#pragma unroll
    for (int r = 0; r < W; r++) {
      IO::load_recv(wires.p[r], g, blk, ql & 3, w[r]);
      sc[r] = h2f(ld_u16(wires.p[r] + so)) * T::unpack_scale;
      zc[r] = T::asym ? h2f(ld_u16(wires.p[r] + zo)) : 0.0f;
    }
    // acc = x0 + x1 + ... in rank order, as in stage 1's own kernel
    float acc[1][8];
#pragma unroll
    for (int r = 0; r < W; r++) add_codes<C, 8>(acc[0], w[r], sc[r], zc[r], r == 0);
    uint8_t* const rp[1] = {red};
    const uint32_t rq[1] = {q};
    quantize_core<C, kKeep, Full, 1, false>(acc, rp, rq, red, q, q_end, g);
  }
  __syncthreads();

  // stage 2: dequantize the reduced quarter once, store it to every output
  {
    const uint32_t blk = ql >> 2;
    uint32_t w[IO::nw];
    IO::load(red + (size_t)blk * T::block_bytes, ql & 3, w);
    const float sv = h2f(ld_u16(red + g.off_s + (size_t)blk * 2)) * T::unpack_scale;
    const float zv = T::asym ? h2f(ld_u16(red + g.off_z + (size_t)blk * 2)) : 0.0f;
    float cv[8], y[8];
    code_values<C, 8>(w, cv);
#pragma unroll
    for (int i = 0; i < 8; i++) y[i] = T::asym ? __builtin_fmaf(cv[i], sv, zv) : cv[i] * sv;
    const u32x4 out{st16x2<D>(y[0], y[1]), st16x2<D>(y[2], y[3]), st16x2<D>(y[4], y[5]),
                    st16x2<D>(y[6], y[7])};
    if (has) {
#pragma unroll
      for (int r = 0; r < W; r++) st_out<kStage2>(reinterpret_cast<u32x4*>(ys.p[r]) + q, out);
    }
  }
}

template <int C, int D, int W>
__global__ __launch_bounds__(kThreads) void k_fused(InPtrs xs, OutPtrs wires, uint8_t* red,
                                                    OutPtrs ys, Geo g) {
  const uint32_t q = blockIdx.x * kThreads + threadIdx.x;
  // uniform: every quarter of the workgroup holds 8 elements
  if (8ull * ((uint64_t)blockIdx.x + 1ull) * kThreads <= (uint64_t)g.n)
    fused_tile<C, D, W, true>(xs, wires, red, ys, q, g);
  else
    fused_tile<C, D, W, false>(xs, wires, red, ys, q, g);
}

// the FP codec in one launch: copy (converting under the cast option) into
// the receive buffer, sum, copy back; one 16-byte chunk per lane
template <int D, int W>
__global__ __launch_bounds__(kThreads) void k_fused_fp(InPtrs xs, OutPtrs wires, uint8_t* red,
                                                       OutPtrs ys, uint32_t nchunks,
                                                       uint32_t tstride) {
  constexpr int Dw = D == kBF16H ? kF16 : D;      // the wire's element type
  constexpr int Dx = D == kBF16H ? kBF16 : D;     // the buffers' element type
  const uint32_t c = blockIdx.x * kThreads + threadIdx.x;
  const bool has = c < nchunks;
  const uint32_t wo = fp_chunk<true>(tstride, 0u, c);
  if (has) {
#pragma unroll
    for (int r = 0; r < W; r++) {
      u32x4 q = reinterpret_cast<const u32x4*>(xs.p[r])[c];
      if constexpr (Dx != Dw) {
#pragma unroll
        for (int k = 0; k < 4; k++)
          q[k] = st16x2<Dw>(ld16<Dx>(q[k] & 0xffffu), ld16<Dx>(q[k] >> 16));
      }
      *reinterpret_cast<u32x4*>(wires.p[r] + wo) = q;
    }
  }
  __syncthreads();
  if (has) {
    u32x4 q[W];
#pragma unroll
    for (int r = 0; r < W; r++) q[r] = *reinterpret_cast<const u32x4*>(wires.p[r] + wo);
    uint32_t out[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      float lo = ld16<Dw>(q[0][k] & 0xffffu), hi = ld16<Dw>(q[0][k] >> 16);
#pragma unroll
      for (int r = 1; r < W; r++) {
        lo = lo + ld16<Dw>(q[r][k] & 0xffffu);
        hi = hi + ld16<Dw>(q[r][k] >> 16);
      }
      out[k] = st16x2<Dw>(lo, hi);
    }
    reinterpret_cast<u32x4*>(red)[c] = u32x4{out[0], out[1], out[2], out[3]};
  }
  __syncthreads();
  if (has) {
    u32x4 q = reinterpret_cast<const u32x4*>(red)[c];
    if constexpr (Dx != Dw) {
#pragma unroll
      for (int k = 0; k < 4; k++)
        q[k] = st16x2<Dx>(ld16<Dw>(q[k] & 0xffffu), ld16<Dw>(q[k] >> 16));
    }
#pragma unroll
    for (int r = 0; r < W; r++) st_out<kStage2>(reinterpret_cast<u32x4*>(ys.p[r]) + c, q);
  }
}

// ---------------------------------------------------------------------------
// dispatch

// tstride: in the receive buffer, W tiles separate a rank's consecutive
// tiles; tile0: the tile the ranks' base pointers of this launch point at
Geo geo(const Layout& L, int W = 0, bool recv = false, size_t tile0 = 0) {
  return Geo{(uint32_t)L.n, (uint32_t)L.nb, (uint32_t)L.off_s, (uint32_t)L.off_z,
             recv ? (uint32_t)(W * L.tile_bytes) : 0u, (uint32_t)tile0};
}

unsigned groups(size_t items, size_t per_group) {
  return (unsigned)((items + per_group - 1) / per_group);
}

// Tiles of the receive buffer one launch takes: the kernels address a rank's
// tiles by 32-bit offsets from the launch's first tile, so a launch spans at
// most (2^32 - 1) / (W * tile_bytes) - 1 tiles (every workload of up to
// about 1 GiB per rank buffer is one launch).
size_t recv_tiles_per_launch(int W, const Layout& L) {
  const uint64_t stride = (uint64_t)W * L.tile_bytes;
  return (size_t)(0xffffffffull / stride - 1);
}

// the ranks' base pointers at tile t0 of a receive buffer
template <typename P>
P at_tile(const P& base, int W, const Layout& L, size_t t0) {
  P out = base;
  for (int r = 0; r < W; r++) out.p[r] = base.p[r] + t0 * (size_t)W * L.tile_bytes;
  return out;
}

template <int C, int D, int W, bool Recv>
void s1_launch(const InPtrs& wires, uint8_t* red, size_t blk_lo, size_t blk_hi,
               const Layout& L, hipStream_t st) {
  // launches over tile ranges [t0, t1) of the receive buffer (one range for
  // W separate wire images, whose offsets always fit)
  const size_t per = Recv ? recv_tiles_per_launch(W, L) : L.ntiles + 1;
  for (size_t t0 = blk_lo / kTileBlocks; t0 * kTileBlocks < blk_hi; t0 += per) {
    const size_t lo = blk_lo > t0 * kTileBlocks ? blk_lo : t0 * kTileBlocks;
    const size_t hi = blk_hi < (t0 + per) * kTileBlocks ? blk_hi : (t0 + per) * kTileBlocks;
    if (hi <= lo) continue;                       // an owner's empty chunk: no launch
    const InPtrs w = Recv ? at_tile(wires, W, L, t0) : wires;
    const Geo g = geo(L, W, Recv, Recv ? t0 : 0);
    // at W=8, each launch in full rounds (round_cap_lds)
    if constexpr (C == kFP) {
      // block-granular range in 8-element chunks (a partial last block
      // holds fewer than 4 chunks)
      const uint32_t c_lo = (uint32_t)(4 * lo);
      const uint32_t c_hi = (uint32_t)(hi * 4 < L.n / 8 ? hi * 4 : L.n / 8);
      OutPtrs out{};
      out.p[0] = red;
      constexpr auto K = k_sum_fp<D, W, kStage1, Recv>;
      const unsigned ng = groups(c_hi - c_lo, kThreads * kPerLane);
      hipLaunchKernelGGL(K, dim3(ng), dim3(kThreads), W == 8 ? round_cap_lds<K>(kThreads, ng) : 0,
                         st, w, out, c_lo, c_hi, g.tstride, g.tile0);
    } else {
      bool launched = false;
      if constexpr (W == 2) {
        if (s1_lanes_per_workgroup(W, L.nb) == 128) {
          constexpr auto K = k_stage1<C, D, W, Recv, 128>;
          const unsigned ng = groups(hi - lo, 128);
          hipLaunchKernelGGL(K, dim3(ng), dim3(128), 0, st, w, red, (uint32_t)lo, (uint32_t)hi,
                             g);
          launched = true;
        }
      }
      if (!launched) {
        constexpr auto K = k_stage1<C, D, W, Recv, kThreads>;
        const unsigned ng = groups(hi - lo, kThreads);
        hipLaunchKernelGGL(K, dim3(ng), dim3(kThreads), W == 8 ? round_cap_lds<K>(kThreads, ng) : 0,
                           st, w, red, (uint32_t)lo, (uint32_t)hi, g);
      }
    }
  }
}

// stage 1 depends on the buffer type only through the FP wire's element
// type (binary16 under the cast option); the other codecs' wires hold codes
template <int C, int D>
void s1_by_w(int W, const InPtrs& wires, bool recv, uint8_t* red, size_t lo, size_t hi,
             const Layout& L, hipStream_t st) {
  if constexpr (D == kBF16H || (C != kFP && D != kF16)) {
    s1_by_w<C, kF16>(W, wires, recv, red, lo, hi, L, st);
  } else {
    switch (W * 2 + (recv ? 1 : 0)) {
      case 4: s1_launch<C, D, 2, false>(wires, red, lo, hi, L, st); break;
      case 5: s1_launch<C, D, 2, true>(wires, red, lo, hi, L, st); break;
      case 8: s1_launch<C, D, 4, false>(wires, red, lo, hi, L, st); break;
      case 9: s1_launch<C, D, 4, true>(wires, red, lo, hi, L, st); break;
      case 16: s1_launch<C, D, 8, false>(wires, red, lo, hi, L, st); break;
      case 17: s1_launch<C, D, 8, true>(wires, red, lo, hi, L, st); break;
      default: break;
    }
  }
}

template <int C, int D, bool Recv>
void q_launch(int W, const InPtrs& xs, const OutPtrs& wires, const Layout& L, hipStream_t st) {
  // a workgroup quantizes a tile (FP: copies it), or half a tile, of one
  // rank; into the receive buffer over tile ranges [t0, t1) as for stage 1
  const size_t tiles = C == kFP ? groups(L.n / 8, kThreads * kPerLane)
                                : groups(4 * L.nb, kThreads * kPerLane);
  const size_t per = Recv ? recv_tiles_per_launch(W, L) : tiles + 1;
  const int U = C == kFP ? kPerLane : s0_quarters_per_lane(W, L.n, CodecT<C>::bits);
  const size_t wpt = 4 / U;                            // workgroups per tile
  for (size_t t0 = 0; t0 < tiles; t0 += per) {
    const size_t nt = tiles - t0 < per ? tiles - t0 : per;
    const OutPtrs w = Recv ? at_tile(wires, W, L, t0) : wires;
    const Geo g = geo(L, W, Recv, Recv ? t0 : 0);
    const dim3 grid = Recv ? dim3((unsigned)(nt * W * wpt)) : dim3((unsigned)(nt * wpt), W);
    if constexpr (C == kFP) {
      // the FP wire holds the buffer's raw elements (binary16 under the cast)
      constexpr int Dw = D == kBF16H ? kF16 : D;
      constexpr int Din = D == kBF16H ? kBF16 : D;
      hipLaunchKernelGGL((k_copy<0, Din, Dw, Recv>), grid, dim3(kThreads), 0, st, xs, w,
                         (uint32_t)(L.n / 8), g.tstride, g.tile0, W);
    } else if (U == 2) {
      hipLaunchKernelGGL((k_quantize<C, D, Recv, 2>), grid, dim3(kThreads), 0, st, xs, w, g, W);
    } else {
      hipLaunchKernelGGL((k_quantize<C, D, Recv, 4>), grid, dim3(kThreads), 0, st, xs, w, g, W);
    }
  }
}

template <int C, int D>
void q_dispatch(int W, const InPtrs& xs, const OutPtrs& wires, bool recv, const Layout& L,
                hipStream_t st) {
  if (recv)
    q_launch<C, D, true>(W, xs, wires, L, st);
  else
    q_launch<C, D, false>(W, xs, wires, L, st);
}

template <int C, int D>
void dq_dispatch(int W, const uint8_t* wire, const OutPtrs& ys, const Layout& L,
                 hipStream_t st) {
  if constexpr (C == kFP) {
    InPtrs src;
    for (int r = 0; r < kMaxRanks; r++) src.p[r] = wire;
    constexpr int Dw = D == kBF16H ? kF16 : D;
    constexpr int Dout = D == kBF16H ? kBF16 : D;
    if (s2_quarters_per_lane(W, L.n) == 1)
      hipLaunchKernelGGL((k_copy<2, Dw, Dout, false, 1>), dim3(groups(L.n / 8, kThreads), W),
                         dim3(kThreads), 0, st, src, ys, (uint32_t)(L.n / 8), 0u, 0u, W);
    else
      hipLaunchKernelGGL((k_copy<2, Dw, Dout, false, 4>), dim3(groups(L.n / 8, kThreads * 4), W),
                         dim3(kThreads), 0, st, src, ys, (uint32_t)(L.n / 8), 0u, 0u, W);
  } else {
    if (s2_quarters_per_lane(W, L.n) == 1)
      hipLaunchKernelGGL((k_dequant<C, D, 1>), dim3(groups(L.n / 8, kThreads), W),
                         dim3(kThreads), 0, st, wire, ys, geo(L));
    else
      hipLaunchKernelGGL((k_dequant<C, D, 4>), dim3(groups(L.n / 8, kThreads * 4), W),
                         dim3(kThreads), 0, st, wire, ys, geo(L));
  }
}

template <int C, int D, int W>
void fused_launch(const InPtrs& xs, const OutPtrs& wires, uint8_t* red, const OutPtrs& ys,
                  const Layout& L, hipStream_t st) {
  if constexpr (C == kFP) {
    const uint32_t nc = (uint32_t)(L.n / 8);
    hipLaunchKernelGGL((k_fused_fp<D, W>), dim3(groups(nc, kThreads)), dim3(kThreads), 0, st,
                       xs, wires, red, ys, nc, geo(L, W, true).tstride);
  } else {
    // 64 blocks (256 quarters) per workgroup
    hipLaunchKernelGGL((k_fused<C, D, W>), dim3(groups(L.nb, kThreads / 4)), dim3(kThreads),
                       0, st, xs, wires, red, ys, geo(L, W, true));
  }
}

template <int C, int D>
void fused_by_w(int W, const InPtrs& xs, const OutPtrs& wires, uint8_t* red, const OutPtrs& ys,
                const Layout& L, hipStream_t st) {
  switch (W) {
    case 2: fused_launch<C, D, 2>(xs, wires, red, ys, L, st); break;
    case 4: fused_launch<C, D, 4>(xs, wires, red, ys, L, st); break;
    case 8: fused_launch<C, D, 8>(xs, wires, red, ys, L, st); break;
    default: break;
  }
}

// calls FN<codec, dtype>(args...) for the runtime (codec, dtype)
#define QR_BY_DTYPE(C, dtype, FN, ...)                                                  \
  ((dtype) == kBF16H ? FN<C, kBF16H>(__VA_ARGS__)                                       \
                     : (dtype) == kBF16 ? FN<C, kBF16>(__VA_ARGS__) : FN<C, kF16>(__VA_ARGS__))
#define QR_DISPATCH(codec, dtype, FN, ...)                                              \
  do {                                                                                  \
    switch (codec) {                                                                    \
      case kFP: QR_BY_DTYPE(kFP, dtype, FN, __VA_ARGS__); break;                        \
      case kQ8: QR_BY_DTYPE(kQ8, dtype, FN, __VA_ARGS__); break;                        \
      case kQ6: QR_BY_DTYPE(kQ6, dtype, FN, __VA_ARGS__); break;                        \
      case kQ4: QR_BY_DTYPE(kQ4, dtype, FN, __VA_ARGS__); break;                        \
      case kFP8: QR_BY_DTYPE(kFP8, dtype, FN, __VA_ARGS__); break;                      \
      case kQ8A: QR_BY_DTYPE(kQ8A, dtype, FN, __VA_ARGS__); break;                      \
      case kQ6A: QR_BY_DTYPE(kQ6A, dtype, FN, __VA_ARGS__); break;                      \
      case kQ4A: QR_BY_DTYPE(kQ4A, dtype, FN, __VA_ARGS__); break;                      \
      default: break;                                                                   \
    }                                                                                   \
  } while (0)

}  // namespace

hipError_t launch_fused(int codec, int dtype, int W, const InPtrs& xs, const OutPtrs& wires,
                        uint8_t* reduced, const OutPtrs& ys, const Layout& L, hipStream_t st) {
  QR_DISPATCH(codec, dtype, fused_by_w, W, xs, wires, reduced, ys, L, st);
  return hipGetLastError();
}

hipError_t launch_quantize(int codec, int dtype, int W, const InPtrs& xs,
                           const OutPtrs& wires, bool recv, const Layout& L,
                           hipStream_t st) {
  QR_DISPATCH(codec, dtype, q_dispatch, W, xs, wires, recv, L, st);
  return hipGetLastError();
}

hipError_t launch_stage1(int codec, int dtype, int W, const InPtrs& wires, bool recv,
                         uint8_t* reduced, size_t blk_lo, size_t blk_hi,
                         const Layout& L, hipStream_t st) {
  if (blk_hi <= blk_lo) return hipSuccess;
  QR_DISPATCH(codec, dtype, s1_by_w, W, wires, recv, reduced, blk_lo, blk_hi, L, st);
  return hipGetLastError();
}

hipError_t launch_dequantize(int codec, int dtype, int W, const uint8_t* wire,
                             const OutPtrs& ys, const Layout& L, hipStream_t st) {
  QR_DISPATCH(codec, dtype, dq_dispatch, W, wire, ys, L, st);
  return hipGetLastError();
}

template <int D, int W>
void oneshot_launch(const InPtrs& xs, const OutPtrs& ys, size_t n, hipStream_t st) {
  const uint32_t nc = (uint32_t)(n / 8);
  hipLaunchKernelGGL((k_sum_fp<D, W, kStage2, false>), dim3(groups(nc, kThreads * kPerLane), W),
                     dim3(kThreads), 0, st, xs, ys, 0u, nc, 0u, 0u);
}

template <int D>
void oneshot_by_w(int W, const InPtrs& xs, const OutPtrs& ys, size_t n, hipStream_t st) {
  switch (W) {
    case 2: oneshot_launch<D, 2>(xs, ys, n, st); break;
    case 4: oneshot_launch<D, 4>(xs, ys, n, st); break;
    case 8: oneshot_launch<D, 8>(xs, ys, n, st); break;
  }
}

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t scratch_address(void** p) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* a = g_scratch[dev].load(std::memory_order_acquire);
  if (a == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    a = g_scratch[dev].load(std::memory_order_relaxed);
    if (a == nullptr) {
      // each GPU holds its own copy of the array, at its own address
      e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (a == nullptr) return hipErrorInvalidSymbol;
      g_scratch[dev].store(a, std::memory_order_release);
    }
  }
  *p = a;
  return hipSuccess;
}

hipError_t launch_oneshot(int dtype, int W, const InPtrs& xs, const OutPtrs& ys, size_t n,
                          hipStream_t st) {
  if (dtype == kBF16H)
    oneshot_by_w<kBF16H>(W, xs, ys, n, st);
  else if (dtype == kBF16)
    oneshot_by_w<kBF16>(W, xs, ys, n, st);
  else
    oneshot_by_w<kF16>(W, xs, ys, n, st);
  return hipGetLastError();
}

}  // namespace qr
