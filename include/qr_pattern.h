/*
 * qr_pattern.h -- the stage-1 access pattern, a measuring instrument built
 * into its own library (libqr_pattern.so), not part of the allreduce.
 *
 * qrp_stage1_pattern issues the loads and stores of stage 1 read from a
 * receive buffer (qr_reduce_recv over all blocks, include/qr.h): the same
 * grid, lanes, addresses and access widths, with the dequantize, binary32
 * sum and requantize of the two-stage allreduce ("Integrate quick allreduce
 * and select the best allreduce implementation", vLLM PR #18473, PR
 * description item 2) replaced by an XOR of the W ranks' words.  Its time is
 * what the memory system needs for stage 1's bytes in stage 1's pattern:
 * the ceiling a benchmark sets beside the stage-1 kernel.  What it writes is
 * not a reduced image.  qrp_stream times plain reads, writes and copies.
 */
#ifndef QR_PATTERN_H
#define QR_PATTERN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* codec: a qr_codec value; W in {2,4,8}; recv: a receive buffer of
 * qr_recv_bytes(W, codec, n) bytes (device memory, read only); reduced:
 * qr_wire_bytes(codec, n) bytes of device memory, overwritten; stream: a
 * hipStream_t (NULL = the default stream), the launch is enqueued there.
 * n: elements per rank, a positive multiple of 8, at most QR_MAX_BYTES / 2,
 * and small enough that every offset of the receive buffer fits in 32 bits.
 * Returns 0; -1 (nothing launched) for an unsupported codec or W, a null or
 * not 16-byte aligned pointer, or such an n; -6 when the launch fails. */
int qrp_stage1_pattern(int codec, int W, const void* recv, size_t n, void* reduced,
                       void* stream);

/* Plain streams of 16-byte accesses, the memory system's own rates beside
 * which the kernels' access choices were made.  kind: 0 reads `bytes` from
 * src (one 4-byte word per workgroup may be written to dst, which must hold
 * 4 bytes per workgroup: bytes / (4096 * per_lane) rounded up); 1 writes
 * `bytes` to dst; 2 copies bytes / 2 from src to dst.  per_lane: 16-byte
 * accesses per lane, 1 or 4 (a workgroup of 256 lanes covers 4096 * per_lane
 * bytes, access k of lane l at chunk 256k + l of the workgroup's range);
 * nontemporal: 0 through the caches, 1 non-temporal loads (kind 0, 2) or
 * stores (kind 1).  bytes: a positive multiple of 32, at most 2^36.  src,
 * dst: device memory, 16-byte aligned; stream as above.  Returns 0; -1
 * (nothing launched) for other arguments; -6 when the launch fails. */
int qrp_stream(int kind, int per_lane, int nontemporal, const void* src, void* dst,
               size_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QR_PATTERN_H */
