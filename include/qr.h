/*
 * qr.h -- C ABI of the two-stage quantized allreduce for MI355X (gfx950).
 *
 * The method ("Integrate quick allreduce and select the best allreduce
 * implementation", vLLM PR #18473, PR description item 2: a two-stage
 * allreduce whose wire format is f16, fp8, Q8, Q6 or Q4; "Add quickreduce as
 * alternative to custom allreduce", vLLM PR #16804, PR description: int4/int8
 * with symmetric and asymmetric quantization) runs as three stages over W
 * ranks:
 *   stage 0  every rank quantizes its buffer into a wire image;
 *   stage 1  the owner of each chunk of blocks dequantizes the W ranks' wire
 *            blocks, sums them in binary32 in rank order 0..W-1 and
 *            requantizes the sums (reduce-scatter);
 *   stage 2  every rank dequantizes the reduced wire image into its output
 *            (allgather).
 * Here the W ranks are W buffers resident on one GPU; nothing crosses to
 * another device.
 *
 * Numerics (the pages name the formats only; these are the readings taken):
 *   - 32-element blocks; n elements give nb = ceil(n/32) blocks, the last one
 *     possibly partial (8, 16 or 24 elements; its statistics use only those).
 *   - symmetric codecs (Q8, Q6, Q4, FP8): per block mx = max, mn = min,
 *     a = max(|mx|,|mn|); a == 0 gives scale +0 and all codes 0; otherwise
 *     scale s = RU16(mx == mn ? a : a / qmax) (RU16 = least binary16 >= the
 *     binary32 value, saturated at 65504; qmax = 127/31/7, 448 for FP8),
 *     inv = 1/s, t = v*inv, code = clamp(round-half-even(t), -qmax, qmax) as
 *     b-bit two's complement, or the OCP E4M3FN encoding of t (nearest, ties
 *     to even, saturating at 448, sign kept for zero).
 *   - asymmetric codecs (Q8A, Q6A, Q4A): a zero minimum is taken as +0;
 *     zero z = RD16(mn) (greatest binary16 <= mn, saturated at -65504),
 *     d = mx - z; d <= 0 gives scale +0 and codes 0; otherwise
 *     s = RU16(d / qu) (qu = 255/63/15), t = (v - z) * (1/s),
 *     code = clamp(round-half-even(t), 0, qu).
 *   - dequantization: code*s (exact in binary32), plus z for asymmetric (one
 *     rounding); stage 1 adds the W dequantized values in binary32, rank
 *     order, and requantizes the binary32 sums; stage 2 and qr_dequantize
 *     round once to the buffer type (round to nearest even; overflow -> inf).
 *   - FP: the wire image is the raw 16-bit data; stage 1 rounds the binary32
 *     rank-order sum once to the buffer type.
 *
 * Wire image of one rank (n elements): plane 0 = codes, nb * (32*b/8) bytes,
 * code i of a block at bits [b*i, b*i+b) of the block's little-endian
 * bitstring, unused slots of a partial block zero; plane 1 = binary16 scales
 * (2 bytes per block) at the next 256-byte boundary; plane 2 (asymmetric
 * only) = binary16 zeros at the next 256-byte boundary after plane 1.  FP:
 * the 2n raw bytes.  qr_wire_bytes() gives the total.  Padding bytes between
 * planes are left untouched.
 *
 * Conventions for every entry point:
 *   - Buffers are device memory owned by the caller; the library allocates
 *     nothing and keeps no state between calls (qr_allreduce_sim_noalloc
 *     alone uses a buffer of the library's own, described there).  Pointer
 *     arrays (xs, ys, wires) are host arrays of W device pointers, read during
 *     the call only.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls enqueue
 *     their kernels and return without synchronising; results are ready when
 *     the stream reaches that point.
 *   - Arguments are checked on the host before anything is launched; on any
 *     error nothing is written and the call returns a negative QR_ERR_* code,
 *     with a message for qr_last_error().
 *   - n counts 16-bit elements per rank.  It must be > 0, a multiple of 8
 *     (the pages' wrapper requires byte sizes that are multiples of 16:
 *     QuickAllReduce.should_quick_allreduce on the vLLM quick_all_reduce docs
 *     page) and at most QR_MAX_BYTES / 2.
 *   - Every device pointer must be 16-byte aligned.
 *   - Inputs are never modified (the docs page's quick_all_reduce is
 *     out-of-place); input and output buffers must not overlap.
 *   - Calls are thread-safe; calls that share output buffers race.
 */
#ifndef QR_H
#define QR_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element type of the rank buffers.  QR_BF16_VIA_FP16 is the bf16 -> fp16
 * cast option of the vLLM quick_all_reduce docs page (QuickAllReduce.
 * init_quick_all_reduce and quick_all_reduce, VLLM_ROCM_QUICK_REDUCE_CAST_
 * BF16_TO_FP16: bf16 inputs are converted to fp16 and the fp16 kernels run).
 * Reading taken: the buffers hold bfloat16; every input element is rounded
 * to binary16 (nearest even, overflow -> inf), the allreduce then runs
 * exactly as for QR_FP16 buffers holding those values (an FP wire holds
 * binary16), and every binary16 result is rounded to bfloat16 (nearest
 * even).  Inputs beyond the binary16 range are outside the contract for the
 * quantized codecs (they become inf); FP and the one-stage allreduce carry
 * the inf through. */
typedef enum { QR_FP16 = 0, QR_BF16 = 1, QR_BF16_VIA_FP16 = 2 } qr_dtype;

/* wire format; 0..3 follow QuickReduceRegime on the vLLM quick_all_reduce
 * docs page (FP=0, INT8=1, INT6=2, INT4=3; its NONE=4 is rejected here),
 * FP8 and the asymmetric variants (= symmetric | 8) are added. */
typedef enum {
  QR_FP = 0,
  QR_Q8 = 1,
  QR_Q6 = 2,
  QR_Q4 = 3,
  QR_FP8 = 5,
  QR_Q8_ASYM = 9,
  QR_Q6_ASYM = 10,
  QR_Q4_ASYM = 11
} qr_codec;

enum {
  QR_OK = 0,
  QR_ERR_ARG = -1,         /* null pointer, overlapping buffers, bad owner  */
  QR_ERR_UNSUPPORTED = -2, /* W outside what the call takes, unknown dtype  */
                           /* or codec                                      */
  QR_ERR_SIZE = -3,        /* n == 0, n % 8 != 0, or 2n > QR_MAX_BYTES      */
  QR_ERR_ALIGN = -4,       /* a device pointer not 16-byte aligned          */
  QR_ERR_WORKSPACE = -5,   /* workspace smaller than qr_sim_workspace_bytes */
  QR_ERR_HIP = -6          /* a HIP launch failed (text in qr_last_error)   */
};

/* largest rank buffer in bytes (2 GiB; the docs page's qr_max_size) */
#define QR_MAX_BYTES ((size_t)1 << 31)

/* Bytes of one rank's wire image for n elements (0 for an unknown codec). */
size_t qr_wire_bytes(qr_codec codec, size_t n);

/* The receive buffer: the W ranks' wire data as an owner receives them,
 * the stage-0 output and stage-1 input of qr_allreduce_sim.  It holds the
 * bytes of the W wire images in tiles of 256 blocks: tile t of rank r
 * (blocks [256t, 256t+256) of that rank) starts at byte (t*W + r) * T and
 * holds the 256 blocks' codes (256 * 32*b/8 bytes), then their binary16
 * scales (512 bytes), then (asymmetric codecs) their binary16 zeros (512
 * bytes), so T = 256 * (32*b/8 + 2 [+ 2]); FP: the 256 blocks' raw 16-bit
 * data, T = 16384.  The codes are word-major: each block's 32*b/8 code
 * bytes (the planar image's, in order) are cut into words of S bytes (S = 8
 * for 6-bit codes, else 16), and the tile holds word 0 of its 256 blocks,
 * then word 1 of them, and so on (4-bit blocks are one word).  Slots of
 * blocks past the last one are padding, never read or written.  The W tiles
 * of one range of blocks are thus adjacent: stage 1 reads them as one
 * stream instead of W, and each of its load instructions reads one
 * contiguous range (on a real node the senders would write their tiles into
 * the owner's buffer at these offsets).
 * Bytes of the buffer: ceil(ceil(n/32)/256) * W * T (0 for an unknown codec
 * or W outside 1..8). */
size_t qr_recv_bytes(int W, qr_codec codec, size_t n);

/* Workspace qr_allreduce_sim needs: the receive buffer (qr_recv_bytes),
 * then the reduced image at the next 256-byte boundary (0 for an
 * unsupported W or codec). */
size_t qr_sim_workspace_bytes(int W, qr_codec codec, size_t n);

/* Stage 0 for one rank: quantize x (n elements of `dtype`) into `wire`
 * (qr_wire_bytes(codec, n) bytes; plane padding untouched). */
int qr_quantize(qr_codec codec, qr_dtype dtype, const void* x, size_t n,
                void* wire, void* stream);

/* Dequantize one wire image into y (n elements of `dtype`). */
int qr_dequantize(qr_codec codec, qr_dtype dtype, const void* wire, size_t n,
                  void* y, void* stream);

/* Stage 0 for W ranks in one launch: wires[r] = quantize(xs[r]); any W in
 * 1..8 (each rank is quantized on its own). */
int qr_quantize_ranks(qr_codec codec, qr_dtype dtype, int W,
                      const void* const* xs, size_t n, void* const* wires,
                      void* stream);

/* Stage 1: for every block of the chunk owned by `owner` (blocks
 * [owner*bpc, min(nb,(owner+1)*bpc)), bpc = ceil(nb/W)), or of all chunks
 * when owner == -1, dequantize the W wire images' blocks, sum in binary32 in
 * rank order and requantize into reduced_wire (a full-size wire image; only
 * the owned blocks' codes, scales and zeros are written).  For QR_FP the
 * wires are raw buffers and reduced_wire receives the rounded sums.
 * W in {2,4,8}. */
int qr_reduce_stage1(qr_codec codec, qr_dtype dtype, int W,
                     const void* const* wires, size_t n, int owner,
                     void* reduced_wire, void* stream);

/* Stage 0 for W ranks into a receive buffer (qr_recv_bytes(W, codec, n)
 * bytes): the same codes, scales and zeros as qr_quantize_ranks writes, at
 * the receive buffer's offsets.  W in {2,4,8}. */
int qr_quantize_recv(qr_codec codec, qr_dtype dtype, int W,
                     const void* const* xs, size_t n, void* recv, void* stream);

/* Stage 1 from a receive buffer: as qr_reduce_stage1 (the same owner
 * ranges, the same reduced image), reading the W ranks' blocks from `recv`.
 * W in {2,4,8}. */
int qr_reduce_recv(qr_codec codec, qr_dtype dtype, int W, const void* recv,
                   size_t n, int owner, void* reduced_wire, void* stream);

/* Stage 2: every rank r dequantizes reduced_wire into ys[r]; any W in 1..8. */
int qr_gather_stage2(qr_codec codec, qr_dtype dtype, int W,
                     const void* reduced_wire, size_t n, void* const* ys,
                     void* stream);

/* The whole simulated allreduce: ys[r] = stage2(stage1(quantize(xs[0..W-1])))
 * for every r.  `workspace` is caller-owned device memory of at least
 * qr_sim_workspace_bytes(W, codec, n) bytes that must not overlap any x or y;
 * it receives the receive buffer and the reduced image, as qr_quantize_recv
 * and qr_reduce_recv would write them.  Launches on `stream`: for
 * 2n <= 4 MiB, one (each workgroup takes its tile of blocks through all
 * three stages, reading the receive buffer and the reduced image back from
 * the workspace); above, three, the kernels of qr_quantize_recv,
 * qr_reduce_recv and qr_gather_stage2.  Both give the same outputs and
 * workspace contents.  W in {2,4,8}. */
int qr_allreduce_sim(int W, qr_dtype dtype, qr_codec codec,
                     const void* const* xs, void* const* ys, size_t n,
                     void* workspace, size_t ws_bytes, void* stream);

/* The one-stage (one-shot) allreduce without a wire format ("1stage", f16,
 * in PR #18473's description item 2 and its tp2 timing table; the review
 * thread of "Add quickreduce as alternative to custom allreduce", vLLM PR
 * #16804, proposes one shot for small buffers and two shot for large ones):
 * every rank r reads all W buffers and writes
 *     ys[r][i] = round_to_dtype(((x_0[i] + x_1[i]) + ...) + x_{W-1}[i]),
 * the sum taken in binary32 in rank order and rounded once (round to nearest
 * even; overflow -> inf) -- the same values as qr_allreduce_sim with QR_FP.
 * One launch on `stream`; W in {2,4,8}; n, alignment and overlap rules as
 * for every entry point (no workspace). */
int qr_allreduce_oneshot(int W, qr_dtype dtype, const void* const* xs,
                         void* const* ys, size_t n, void* stream);

/* Largest workspace qr_allreduce_sim_noalloc takes from the library's own
 * device buffer (64 MiB per GPU): enough for every W and codec up to 4 MiB
 * per rank buffer, the sizes that run as one launch. */
#define QR_SCRATCH_BYTES ((size_t)64 << 20)

/* qr_allreduce_sim without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The receive buffer and the reduced image
 * (the workspace of qr_allreduce_sim) go to a device buffer of
 * QR_SCRATCH_BYTES that the library holds in every GPU it runs on, from the
 * first call on that GPU until the process ends; the call itself allocates
 * nothing and frees nothing.  The GPU is the current
 * device (hipGetDevice), which `stream` must belong to.  Outputs, launches
 * and argument rules are those of qr_allreduce_sim; additionally the call
 * fails with QR_ERR_WORKSPACE, writing nothing, when
 * qr_sim_workspace_bytes(W, codec, n) > QR_SCRATCH_BYTES.  Every call on one
 * GPU uses the same buffer: calls on that GPU must not overlap in time (on
 * two streams, or from two threads, without ordering between them), or they
 * race on it.  Nothing in the buffer needs to start at zero; it keeps the
 * last call's receive buffer and reduced image. */
int qr_allreduce_sim_noalloc(int W, qr_dtype dtype, qr_codec codec,
                             const void* const* xs, void* const* ys, size_t n,
                             void* stream);

/* Message for the last error returned on this thread ("" if none). */
const char* qr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* QR_H */
