/*
 * fp4q.h -- C ABI of the MI355X (gfx950) FP4 communication-compression library.
 *
 * The operations are those of "FP4Quant: Efficient 4-Bit Communication
 * Compression for Model-Parallel LLM Training" (abstract): a bf16 tensor that a
 * tensor-parallel rank is about to exchange is transformed block by block by a
 * two-level fast Walsh-Hadamard transform, quantised to FP4 with two scales (one
 * per block, one per micro-group of 16) and packed two codes per byte (zot.news
 * digest of the same paper); the receiver dequantises, undoes the transform and
 * sums the payloads of its k peers, the reduce of the tensor-parallel AllReduce
 * (zot.news digest, "Read it as").
 *
 * Tensor: bf16, row-major [rows x row_len], row_len a multiple of 256.  Block b
 * is the flat elements [256 b, 256 b + 256); a block never straddles a row.
 * Payload of a tensor of N = rows * row_len elements, three flat arrays in block
 * order:
 *   codes        N/2 bytes; byte k = code[2k] | code[2k+1] << 4 (E2M1 codes:
 *                sign | 2-bit exponent | 1-bit mantissa, values 0..6)
 *   micro_scales N/16 bytes, OCP E4M3FN, one per 16 consecutive elements
 *   block_scales N/256 fp32, one per block
 * 4.625 bits per element.
 *
 * Conventions for every entry point:
 *   - All buffer pointers are DEVICE pointers; the caller allocates every buffer
 *     and keeps ownership.  The library allocates nothing and keeps no state.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns as soon as the kernel is queued.  Device faults show up
 *     at the caller's next synchronisation.
 *   - Inputs are only read; outputs are fully overwritten.  Inputs and outputs
 *     must not overlap (checked: FP4Q_ERR_ARG).
 *   - Arguments are validated on the host before any HIP call, in this order:
 *     shape (FP4Q_ERR_SHAPE: rows < 0, row_len <= 0, row_len % 256 != 0, or a
 *     byte count that overflows int64), k (FP4Q_ERR_K), flags and out_dtype
 *     (FP4Q_ERR_ARG), then pointers (FP4Q_ERR_NULL), alignment
 *     (FP4Q_ERR_ALIGN), overlap (FP4Q_ERR_ARG).  rows == 0 returns FP4Q_OK
 *     before the pointer checks and launches nothing.
 *   - Alignment: bf16 input, codes, micro_scales and outputs 16 bytes;
 *     block_scales 4 bytes.  (A payload packed into one buffer as codes, then
 *     micro-scales, then block scales meets this when the buffer is 16-byte
 *     aligned: the codes take N/2 bytes, a multiple of 128.)
 *   - A failed launch returns FP4Q_ERR_LAUNCH.
 *   - Inputs must be finite with |x| < 2^118; this is not checked.
 */
#ifndef FP4Q_H
#define FP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { FP4Q_BLOCK = 256, FP4Q_GROUP = 16, FP4Q_MAX_PEERS = 16 };
enum { FP4Q_OUT_F32 = 0, FP4Q_OUT_BF16 = 1 };
/* Skip the Walsh-Hadamard transform on both sides (to measure what it buys). */
enum { FP4Q_FLAG_NO_FWHT = 1u << 0 };

typedef enum {
    FP4Q_OK = 0,
    FP4Q_ERR_NULL = 1,
    FP4Q_ERR_SHAPE = 2,
    FP4Q_ERR_ALIGN = 3,
    FP4Q_ERR_K = 4,
    FP4Q_ERR_ARG = 5,
    FP4Q_ERR_LAUNCH = 6
} fp4q_status;

/* Host-only helper: byte sizes of the three payload arrays for a tensor.
 * Any of the output pointers may be NULL.  Returns FP4Q_OK or FP4Q_ERR_SHAPE. */
int fp4q_payload_bytes(int64_t rows, int64_t row_len, size_t *codes_bytes,
                       size_t *micro_bytes, size_t *block_bytes);

/* Sender side ([FP4Quant] abstract: FWHT, micro-grouped dual-scale FP4
 * quantisation, packing).  Per 256-block: y = H x / 16 (natural-order
 * Walsh-Hadamard, radix-2 stages of stride 1, 2, ..., 128 in fp32);
 * s = max|y| / 2688; per group g of 16: m_g = E4M3(max|y|_g / (6 s)) (round to
 * nearest even, saturating at 448; s == 0 gives m_g = 0); S_g = s * m_g;
 * code_i = E2M1(y_i * (1 / S_g)) (round to nearest even, saturating at 6, sign
 * kept; a zero S_g has reciprocal 0, an overflowing one is clamped to FLT_MAX).
 *   in_bf16       [rows x row_len] bf16 bit patterns
 *   codes         N/2 bytes out;  micro_scales N/16 bytes out;  block_scales N/256 fp32 out */
int fp4q_compress(const uint16_t *in_bf16, int64_t rows, int64_t row_len, uint8_t *codes,
                  uint8_t *micro_scales, float *block_scales, void *stream);

/* fp4q_compress with flags (0 or FP4Q_FLAG_NO_FWHT). */
int fp4q_compress_ex(const uint16_t *in_bf16, int64_t rows, int64_t row_len, uint8_t *codes,
                     uint8_t *micro_scales, float *block_scales, uint32_t flags, void *stream);

/* Receiver side, one payload: yhat_i = E2M1(code_i) * S_g with S_g = s * m_g
 * (fp32, as in compress), then the same transform (H / 16 is its own inverse),
 * same fp32 operation order.  out_f32: [rows x row_len] fp32. */
int fp4q_decompress(const uint8_t *codes, const uint8_t *micro_scales,
                    const float *block_scales, int64_t rows, int64_t row_len, float *out_f32,
                    void *stream);

/* fp4q_decompress with an output type (FP4Q_OUT_F32, or FP4Q_OUT_BF16 rounded to
 * nearest even) and flags (0 or FP4Q_FLAG_NO_FWHT). */
int fp4q_decompress_ex(const uint8_t *codes, const uint8_t *micro_scales,
                       const float *block_scales, int64_t rows, int64_t row_len, void *out,
                       int out_dtype, uint32_t flags, void *stream);

/* Receiver-side reduce of a tensor-parallel AllReduce (zot.news digest, "Read it
 * as"): out = sum over p < k of decompress(payload p), all payloads of the same
 * shape.  `codes`, `micro_scales` and `block_scales` are HOST arrays of k
 * DEVICE pointers (copied into the kernel arguments; the arrays may be freed
 * when the call returns).  1 <= k <= FP4Q_MAX_PEERS.  `out` is overwritten with
 * the sum, fp32 or bf16 (out_dtype).  The sum is taken in fp32 in the transform
 * domain (one inverse transform for all peers), so it matches an exact sum to
 * about 1e-7 of the row's largest summed magnitude (sum over p of |term p|),
 * not bit for bit; that equals 1e-7 of the row's largest result unless the
 * peers' terms cancel. */
int fp4q_decompress_accumulate(int k, const uint8_t *const *codes,
                               const uint8_t *const *micro_scales,
                               const float *const *block_scales, int64_t rows,
                               int64_t row_len, void *out, int out_dtype, void *stream);

/* fp4q_decompress_accumulate with flags (0 or FP4Q_FLAG_NO_FWHT). */
int fp4q_decompress_accumulate_ex(int k, const uint8_t *const *codes,
                                  const uint8_t *const *micro_scales,
                                  const float *const *block_scales, int64_t rows,
                                  int64_t row_len, void *out, int out_dtype, uint32_t flags,
                                  void *stream);

/* Receiver step of a compressed AllReduce done as a reduce-scatter followed by
 * an all-gather (the AllReduce of tensor parallelism, zot.news digest of
 * [FP4Quant], "Read it as"): the k payloads a rank receives for its slice are
 * summed and the sum is quantised again into one payload, ready for the
 * all-gather.  The sum is taken in the transform domain -- each term
 * E2M1(code) * S_g as in decompress, rounded products added in peer order to
 * an accumulator that starts at +0, in fp32 -- and then quantised with the
 * compress steps from the block maximum on; no transform is applied, because
 * decompress + sum + compress would apply the self-inverse H / 16 twice.  The
 * result therefore decompresses (with the same flags as its inputs) to the sum
 * of the k decompressed tensors up to FP4 rounding.
 *   codes, micro_scales, block_scales: HOST arrays of k DEVICE pointers (as in
 *     fp4q_decompress_accumulate), 1 <= k <= FP4Q_MAX_PEERS
 *   out_codes, out_micro, out_block: the new payload (same shape), must not
 *     overlap any input. */
int fp4q_reduce_requantize(int k, const uint8_t *const *codes,
                           const uint8_t *const *micro_scales,
                           const float *const *block_scales, int64_t rows, int64_t row_len,
                           uint8_t *out_codes, uint8_t *out_micro, float *out_block,
                           void *stream);

/* The same step with the rank's own part of the slice added uncompressed (the
 * fused decompress-accumulate, add-local, re-compress of that AllReduce):
 * the accumulator starts at local_bf16 transformed exactly as fp4q_compress
 * transforms its input (as is with FP4Q_FLAG_NO_FWHT, matching payloads
 * compressed with that flag), then the k peers' terms are added as above.
 *   local_bf16  bf16 [rows, row_len], 16-byte aligned, or NULL (then this is
 *     fp4q_reduce_requantize); must not overlap the outputs
 *   k           0 <= k <= FP4Q_MAX_PEERS with a local slice (k = 0 gives
 *     exactly fp4q_compress(local_bf16)), 1 <= k without one
 *   flags       0 or FP4Q_FLAG_NO_FWHT */
int fp4q_reduce_requantize_ex(int k, const uint8_t *const *codes,
                              const uint8_t *const *micro_scales,
                              const float *const *block_scales, const uint16_t *local_bf16,
                              int64_t rows, int64_t row_len, uint8_t *out_codes,
                              uint8_t *out_micro, float *out_block, uint32_t flags,
                              void *stream);

/* MXFP4-style variant: the microscaling FP4 format (blocks of 32, E2M1
 * elements) named on the gist.science page ("Practical FP4 Training for
 * Large-Scale MoE Models on Hopper GPUs", Problemstellung item 2), applied
 * after the same transform in place of the dual scale: every 32 consecutive
 * transformed values y share one power-of-two scale 2^e with
 * e = floor(log2 max|y|) - 2 clamped to [-127, 127] (-127 for a zero group),
 * stored as the E8M0 byte e + 127; element codes are E2M1(y / 2^e) (round to
 * nearest even, saturating, sign kept).  4.25 bits per element.
 *   codes  N/2 bytes (as in fp4q_compress); scales N/32 bytes, 8-byte aligned
 *   flags  0 or FP4Q_FLAG_NO_FWHT */
int fp4q_compress_mx(const uint16_t *in_bf16, int64_t rows, int64_t row_len, uint8_t *codes,
                     uint8_t *scales, uint32_t flags, void *stream);

/* Decode of the MXFP4-style payload: yhat = E2M1(code) * 2^e, then the same
 * transform as fp4q_decompress; output fp32 or bf16 (out_dtype). */
int fp4q_decompress_mx(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t row_len,
                       void *out, int out_dtype, uint32_t flags, void *stream);

/* Static description of a status code; never NULL. */
const char *fp4q_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* FP4Q_H */
