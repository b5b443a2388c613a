// qr_internal.h -- wire layout and kernel launchers shared by the C ABI
// (qr_api.cpp) and the kernels (qr_kernels.hip).  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qr {

constexpr int kMaxRanks = 8;
// blocks per tile of the receive buffer (one workgroup's blocks in stages 0
// and 1)
constexpr int kTileBlocks = 256;

// Byte layout of one rank's wire image for n elements (see qr.h): codes at
// 0, binary16 scales at the next 256-byte boundary, binary16 zeros
// (asymmetric codecs) at the next 256-byte boundary after the scales.
// The receive buffer holds the same bytes of all W ranks in tiles of
// kTileBlocks blocks: tile t of rank r starts at (t*W + r) * tile_bytes and
// holds the tile's codes, then its scales, then its zeros (FP: the raw data).
struct Layout {
  size_t n = 0;         // elements
  size_t nb = 0;        // 32-element blocks
  size_t nslices = 0;   // 16-element lane slices = 2 * nb
  size_t code_bytes = 0;
  size_t off_s = 0, off_z = 0;
  size_t total = 0;     // qr_wire_bytes
  size_t tile_bytes = 0;  // one rank's tile in the receive buffer
  size_t ntiles = 0;      // ceil(nb / kTileBlocks)
  size_t recv_bytes(int W) const { return ntiles * (size_t)W * tile_bytes; }
};

bool codec_valid(int codec);
Layout make_layout(int codec, size_t n);

struct InPtrs { const uint8_t* p[kMaxRanks]; };
struct OutPtrs { uint8_t* p[kMaxRanks]; };

// Where the stage-0 outputs and stage-1 inputs live: W separate wire images
// (wires.p[r], Recv == false), or one receive buffer (Recv == true; wires.p[r]
// is then the buffer plus r * tile_bytes, the start of rank r's first tile).
// stage 0 for W ranks: wires.p[r] <- quantize(xs.p[r])
hipError_t launch_quantize(int codec, int dtype, int W, const InPtrs& xs,
                           const OutPtrs& wires, bool recv, const Layout& L,
                           hipStream_t st);
// stage 1 over blocks [blk_lo, blk_hi): reduced <- requant(sum_r dequant(wires.p[r]))
hipError_t launch_stage1(int codec, int dtype, int W, const InPtrs& wires, bool recv,
                         uint8_t* reduced, size_t blk_lo, size_t blk_hi,
                         const Layout& L, hipStream_t st);
// stage 2 / dequantize for W outputs: ys.p[r] <- dequant(wire)
hipError_t launch_dequantize(int codec, int dtype, int W, const uint8_t* wire,
                             const OutPtrs& ys, const Layout& L, hipStream_t st);
// the three stages in one launch (each workgroup runs all three for its
// tile of blocks): receive buffer (wires.p[r] as for Recv above) <-
// quantize(xs.p[r]), reduced <- stage 1, ys.p[r] <- dequant(reduced); same
// results and workspace as the three separate launches
hipError_t launch_fused(int codec, int dtype, int W, const InPtrs& xs, const OutPtrs& wires,
                        uint8_t* reduced, const OutPtrs& ys, const Layout& L, hipStream_t st);
// device address of the library's own workspace buffer (QR_SCRATCH_BYTES)
// on the current device; looked up once per device, then cached
hipError_t scratch_address(void** p);
// one-stage allreduce: ys.p[r] <- round(sum of xs.p[0..W-1] in rank order), all r
hipError_t launch_oneshot(int dtype, int W, const InPtrs& xs, const OutPtrs& ys, size_t n,
                          hipStream_t st);

}  // namespace qr
