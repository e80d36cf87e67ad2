/*
 * fp4.h -- C ABI of the MI355X (gfx950) FP4 quantize + FP4 GEMM library (libfp4.so).
 *
 * The library implements the data-parallel hot path of fully quantized FP4
 * training of linear layers:
 *   - block-scaled FP4 quantization of training tensors, in the two formats of
 *     Robots Atlas, "FP4", section Components:
 *       NVFP4: 16-element blocks of E2M1 values, an E4M3 scale per block and an
 *              FP32 scale per tensor (two-level scaling, section How it works);
 *       MXFP4: 32-element blocks of E2M1 values, an E8M0 (power-of-two) scale;
 *   - round-to-nearest for the forward pass and stochastic rounding for the
 *     backward and update passes ("FP4 All the Way: Fully Quantized Training of
 *     LLMs", Key points), the random stream being Philox4x32-10 keyed by
 *     (seed, element index);
 *   - the block-wise random-sign Hadamard rotation of operands, 32-wide for
 *     MXFP4 ("Quartet: Native FP4 Training Can Be Optimal for Large Language
 *     Models", Approach) and 16-wide for NVFP4 (Robots Atlas, "FP4", How it
 *     works: random Hadamard transforms among the stabilizers of FP4 training);
 *   - the three linear-layer GEMMs in FP4 with FP32 accumulation (Quartet,
 *     summary; Robots Atlas "FP4", How it works / Execution paradigm):
 *       forward  Y  = X  W^T : A = X  (blocks along K = in-features),
 *                              B = W  (blocks along K)
 *       dgrad    dX = dY W   : A = dY (blocks along out-features),
 *                              B = W quantized along axis ROWS, i.e. W^T
 *       wgrad    dW = dY^T X : A = dY quantized along axis ROWS, i.e. dY^T,
 *                              B = X quantized along axis ROWS, i.e. X^T
 *
 * Conventions (fixed where the pages are silent):
 *   E2M1 code  S|E1E0|M, bias 1; element 2t of a row in the low nibble of byte t.
 *   NVFP4      s_g = amax / 2688 (6 * 448; 1 when amax < 2^-100, so a zero
 *              or vanishingly small tensor quantizes to signed zeros); block byte = E4M3
 *              round-to-nearest-even, saturating at 448, of (amax_b / 6) / s_g;
 *              element v = x * (1 / (sdec * s_g)), the reciprocal rounded once.
 *   MXFP4      block exponent e = the smallest e with 6 * 2^e >= amax_b
 *              (>= -127); byte = e + 127; v = x * 2^-e.
 *   RTN        nearest E2M1 magnitude, ties to even, saturating at 6.
 *   SR         a grid value is kept; else lo < |v| < hi rounds up iff
 *              h + floor(65536 * (|v| - lo) / (hi - lo)) >= 65536, with h the 16-bit draw of
 *              the element: Philox4x32-10, key = seed, counter = (i / 8, 0, 0)
 *              as (lo32, hi32, 0, 0), word (i / 2) % 4, low half for even i;
 *              i = row-major index in the quantized orientation + index_offset.
 *   Hadamard   per B-block along the blocked axis (one rotation per scale
 *              block): negate x_j where bit j of had_signs is set (j < B),
 *              Sylvester FWHT (stages 1, 2, .., B/2, FP32), multiply by
 *              fp32(2^-2.5) (MXFP4, B = 32) or 1/4 (NVFP4, B = 16, exact).
 *              The rotation comes first: the NVFP4 tensor amax is that of the
 *              rotated values (so it depends on the rotation axis). The same
 *              mask must be used for both GEMM operands so the rotation
 *              cancels.
 *
 * Memory and ownership: every pointer argument named "device" is a device
 * pointer the caller allocated (and keeps ownership of); the library never
 * allocates, frees or synchronizes. All work is enqueued in order on the
 * given HIP stream (0 = the null stream). Calls are reentrant.
 *
 * Errors: every call validates its arguments first; on a non-OK status
 * nothing has been enqueued and no output has been touched, except
 * FP4_ERR_HIP, which reports a failed launch (outputs then undefined).
 * Stochastic rounding draws 8 elements' bits from one Philox call, so every
 * call that takes an SR index_offset requires index_offset % 8 == 0
 * (FP4_ERR_ALIGN otherwise).
 * Non-finite inputs are outside the contract: their outputs are unspecified.
 */
#ifndef FP4_H
#define FP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* fp4_stream_t; /* the same type as hipStream_t */

typedef enum fp4_status {
    FP4_OK = 0,
    FP4_ERR_NULL = 1,        /* a required pointer is NULL */
    FP4_ERR_SHAPE = 2,       /* a dimension <= 0, or not a multiple the call requires */
    FP4_ERR_ALIGN = 3,       /* a pointer or leading dimension breaks 16-byte alignment */
    FP4_ERR_UNSUPPORTED = 4, /* a combination the library does not implement */
    FP4_ERR_ARG = 5,         /* an enum value out of range */
    FP4_ERR_HIP = 6,         /* a HIP launch or runtime call failed */
    FP4_ERR_WORKSPACE = 7    /* the workspace is NULL, too small or misaligned */
} fp4_status;

typedef enum fp4_dtype { FP4_DTYPE_F32 = 0, FP4_DTYPE_BF16 = 1 } fp4_dtype;
typedef enum fp4_format { FP4_NVFP4 = 0, FP4_MXFP4 = 1 } fp4_format;
typedef enum fp4_rounding { FP4_RTN = 0, FP4_SR = 1 } fp4_rounding;
/* FP4_AXIS_COLS: blocks run along the contiguous axis C; quantized orientation [R][C].
 * FP4_AXIS_ROWS: blocks run along R; quantized orientation is the transpose [C][R]. */
typedef enum fp4_axis { FP4_AXIS_COLS = 0, FP4_AXIS_ROWS = 1 } fp4_axis;

/* A quantized matrix in its quantized orientation: rows x cols, blocks of B
 * (16 NVFP4, 32 MXFP4) consecutive elements along cols.
 *   codes  device, rows * cols / 2 bytes, row-major [rows][cols/2]
 *   scales device, rows * cols / B bytes, row-major [rows][cols/B]
 *          (E4M3 bytes for NVFP4, E8M0 bytes for MXFP4)
 *   amax   device FP32 scalar: the tensor amax (NVFP4; NULL for MXFP4)
 *   tscale device FP32 scalar: the tensor scale s_g (NVFP4; NULL for MXFP4)
 * codes and scales must be 16-byte aligned. */
typedef struct fp4_tensor {
    uint8_t* codes;
    uint8_t* scales;
    float* amax;
    float* tscale;
    int64_t rows;
    int64_t cols;
    int32_t fmt;        /* fp4_format */
    int32_t had_on;     /* 1: values are in the Hadamard-rotated domain */
    uint32_t had_signs; /* the rotation's sign mask when had_on */
    uint32_t reserved;
} fp4_tensor;

/* Bytes of codes / scales for a quantized rows x cols matrix (0 on bad input). */
size_t fp4_codes_bytes(int64_t rows, int64_t cols);
size_t fp4_scales_bytes(int64_t rows, int64_t cols, int32_t fmt);

/* The Hadamard sign mask of a seed: word 0 of Philox4x32-10 at counter
 * (0, 0, 0, 1) under key = seed (a counter the element stream never uses).
 * Host-only, no device work. */
uint32_t fp4_hadamard_signs(uint64_t seed);

/* Human-readable name of a status. */
const char* fp4_status_str(fp4_status s);

/* Tensor amax: *amax = max |x| over the R x C matrix src (row-major, leading
 * dimension ld elements, FP32 or bf16; device). amax is a device FP32 scalar.
 * The NVFP4 tensor scale depends on it (Robots Atlas "FP4", How it works:
 * the per-tensor FP32 scale). Requires R, C >= 1, C % 8 == 0, ld >= C,
 * ld % 8 == 0, src 16-byte aligned. */
fp4_status fp4_tensor_amax(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                           float* amax, fp4_stream_t stream);

/* The tensor amax of the NVFP4-rotated values: *amax = max |y| where y is src
 * with the 16-wide random-sign Hadamard rotation (mask had_signs, see
 * Conventions) applied to every 16-block along the given axis (COLS: along C;
 * ROWS: down the columns, along R). This is the amax an NVFP4 quantization with
 * had_on uses (Robots Atlas "FP4", How it works: per-tensor scale, random
 * Hadamard transforms); a data-parallel caller reduces it across ranks before
 * quantizing with amax_ready = 1. Same requirements as fp4_tensor_amax, and
 * the rotated dimension a multiple of 16. */
fp4_status fp4_tensor_amax_hadamard16(const void* src, fp4_dtype src_t, int64_t R, int64_t C,
                                      int64_t ld, fp4_axis axis, uint32_t had_signs, float* amax,
                                      fp4_stream_t stream);

/* Quantize the R x C matrix src (row-major, leading dimension ld, FP32 or bf16;
 * device) into *out: block-scaled FP4 with the format of out->fmt (Robots
 * Atlas, "FP4", Components: NVFP4 and MXFP4; How it works: the block scale
 * brings each block into the E2M1 range), round-to-nearest or stochastic
 * ("FP4 All the Way", Key points: round to nearest in the forward pass,
 * stochastic rounding in the backward and update passes), along either axis so
 * that each GEMM operand is blocked along its contraction dimension.
 *   axis         FP4_AXIS_COLS: blocks along C, out is R x C;
 *                FP4_AXIS_ROWS: blocks along R, out is C x R (the transpose).
 *   rnd          FP4_RTN or FP4_SR.
 *   seed, index_offset  the SR stream (ignored for RTN).
 *   amax_ready   NVFP4: 1 if *out->amax already holds the amax of the values
 *                quantized (from fp4_tensor_amax, or fp4_tensor_amax_hadamard16
 *                with this axis and mask when had_on, or an earlier quantize
 *                of the same values); 0 to compute it first. Ignored for MXFP4.
 *   out          caller-filled descriptor: codes, scales, fmt, had_on,
 *                had_signs and, for NVFP4, amax and tscale. The call writes
 *                out->rows and out->cols; *out->tscale receives s_g.
 * Requires: R, C >= 1; the blocked dimension a multiple of B (C for COLS, R
 * for ROWS); C % 8 == 0; ld >= C and ld % 8 == 0; src 16-byte aligned;
 * codes and scales 16-byte aligned; with SR, index_offset % 8 == 0
 * (FP4_ERR_ALIGN). */
fp4_status fp4_quantize(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                        fp4_axis axis, fp4_rounding rnd, uint64_t seed, uint64_t index_offset,
                        int amax_ready, fp4_tensor* out, fp4_stream_t stream);

/* Both orientations of one R x C source from a single read of it, in place
 * of the two quantizations a linear layer's backward pass needs for dY and X
 * (FP4 All the Way, Key points: every GEMM operand blocked along its
 * contraction dimension). Equivalent, bit for bit, to
 *   fp4_quantize(src, ..., FP4_AXIS_COLS, rnd_cols, seed_cols, index_offset_cols, ..., out_cols)
 *   fp4_quantize(src, ..., FP4_AXIS_ROWS, rnd_rows, seed_rows, index_offset_rows, ..., out_rows)
 * with each call's amax_ready set as below.
 *   out_cols     blocks along C: out_cols is R x C.
 *   out_rows     blocks along R: out_rows is C x R (the transpose).
 *   amax_ready   NVFP4 without rotation: 1 if *out_cols->amax already holds the
 *                tensor amax, 0 to compute it first; *out_rows->amax, when it
 *                is another scalar, receives a copy; both tscale scalars
 *                receive s_g.
 *                NVFP4 with had_on in either descriptor: the two orientations'
 *                values have different amaxes, so out_rows->amax and
 *                out_rows->tscale must be scalars of their own (FP4_ERR_NULL if
 *                NULL, FP4_ERR_UNSUPPORTED if shared with out_cols); 1 if each
 *                amax already holds its orientation's amax, 0 to compute both
 *                first; each tscale receives its own s_g.
 * The two descriptors must have the same fmt; had_on and had_signs are each
 * descriptor's own. Requires: R, C >= 1, both multiples of B; C % 8 == 0;
 * ld >= C and ld % 8 == 0; src 16-byte aligned; each orientation's SR
 * index_offset % 8 == 0 (FP4_ERR_ALIGN). Errors as fp4_quantize. */
fp4_status fp4_quantize_dual(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                             fp4_rounding rnd_cols, uint64_t seed_cols, uint64_t index_offset_cols,
                             fp4_rounding rnd_rows, uint64_t seed_rows, uint64_t index_offset_rows,
                             int amax_ready, fp4_tensor* out_cols, fp4_tensor* out_rows,
                             fp4_stream_t stream);

/* One row shard of a tensor split by rows (tokens) across data-parallel ranks
 * ("FP4 All the Way", Key points: the 7B model is trained on 256
 * accelerators; the split over tokens is this library's reading): src holds rows
 * row_offset .. row_offset + R - 1 of a rows_total x C tensor. Quantized as
 * fp4_quantize does, except that every element's stochastic-rounding index is
 * the one it has in the quantization of the whole tensor:
 *   axis COLS: (row_offset + r) * C + c + index_offset
 *   axis ROWS: c * rows_total + row_offset + r + index_offset
 * With the whole tensor's amax (NVFP4: amax_ready = 1 after an all-reduce(max)
 * of the ranks' fp4_tensor_amax, or of fp4_tensor_amax_hadamard16 with the
 * rotation), the shard's codes and scales are exactly rows row_offset ..
 * (COLS) or columns row_offset .. (ROWS) of the whole tensor's quantization.
 * noise: NULL, or the two device doubles of fp4_quantize_noise, accumulated
 * into with this shard's sums (summed across the ranks, they are the whole
 * tensor's, up to the order of FP64 additions).
 * Requires 0 <= row_offset, row_offset + R <= rows_total, rows_total % 8 == 0,
 * and for axis ROWS row_offset % B == 0 (blocks do not straddle shards)
 * (FP4_ERR_SHAPE / FP4_ERR_ALIGN), noise 8-byte aligned (FP4_ERR_ALIGN);
 * otherwise as fp4_quantize. */
fp4_status fp4_quantize_shard(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                              int64_t row_offset, int64_t rows_total, fp4_axis axis, fp4_rounding rnd,
                              uint64_t seed, uint64_t index_offset, int amax_ready, fp4_tensor* out,
                              double* noise, fp4_stream_t stream);

/* fp4_quantize_dual of a row shard (the data-parallel split of
 * fp4_quantize_shard, "FP4 All the Way", Key points), each orientation's
 * stochastic-rounding index that of the whole tensor (as fp4_quantize_shard
 * with axis COLS for out_cols and axis ROWS for out_rows); noise_cols,
 * noise_rows: NULL or the sums of fp4_quantize_dual_noise for either
 * orientation. Requires row_offset % B == 0 and the other conditions of
 * fp4_quantize_shard; otherwise as fp4_quantize_dual. */
fp4_status fp4_quantize_dual_shard(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                                   int64_t row_offset, int64_t rows_total, fp4_rounding rnd_cols,
                                   uint64_t seed_cols, uint64_t index_offset_cols, fp4_rounding rnd_rows,
                                   uint64_t seed_rows, uint64_t index_offset_rows, int amax_ready,
                                   fp4_tensor* out_cols, fp4_tensor* out_rows, double* noise_cols,
                                   double* noise_rows, fp4_stream_t stream);

/* Gradient-noise monitor ("FP4 All the Way", Summary: a threshold relating the
 * gradient norm to the quantization noise marks where quantized training stops
 * paying off). fp4_quantize, plus, in the same pass:
 *   noise[0] += sum x^2           over the values quantized (rotated when had_on)
 *   noise[1] += sum (xhat - x)^2  xhat = the exact value each code and its scales
 *                                 stand for (e2m1 * sdec * s_g, or e2m1 * 2^e)
 * noise: device, two doubles, 8-byte aligned; accumulated into (several calls,
 * e.g. micro-batches or shards, add up; the caller clears it first).
 * sqrt(noise[0] / noise[1]) is the gradient-to-noise norm ratio the threshold
 * is stated on; the threshold itself is the caller's. Each 8-element (COLS) or
 * block (ROWS) partial is formed in FP32 (each difference rounded once, squares
 * accumulated by fma) and added in FP64: relative error below 1e-5 of each sum.
 * The FP64 additions across workgroups are atomic, in no fixed order, so the
 * last bits can differ between runs. Codes, scales and s_g are identical to
 * fp4_quantize's. Requires the squares to be finite in FP32 (|x| < 2^63);
 * otherwise as fp4_quantize (including SR index_offset % 8 == 0), and
 * FP4_ERR_NULL for a NULL noise, FP4_ERR_ALIGN for one not 8-byte aligned. */
fp4_status fp4_quantize_noise(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                              fp4_axis axis, fp4_rounding rnd, uint64_t seed, uint64_t index_offset,
                              int amax_ready, fp4_tensor* out, double* noise, fp4_stream_t stream);

/* fp4_quantize_dual with the noise monitor of fp4_quantize_noise ("FP4 All
 * the Way", Summary: the gradient-noise threshold) on either orientation:
 * noise_cols for out_cols, noise_rows for out_rows (each two
 * device doubles, accumulated into, or NULL to skip; FP4_ERR_NULL if both are
 * NULL). Partials are per block in both orientations. Otherwise as
 * fp4_quantize_dual. */
fp4_status fp4_quantize_dual_noise(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                                   fp4_rounding rnd_cols, uint64_t seed_cols, uint64_t index_offset_cols,
                                   fp4_rounding rnd_rows, uint64_t seed_rows, uint64_t index_offset_rows,
                                   int amax_ready, fp4_tensor* out_cols, fp4_tensor* out_rows,
                                   double* noise_cols, double* noise_rows, fp4_stream_t stream);

/* The monitor's statistic ("FP4 All the Way", Summary: the threshold is stated
 * on the ratio of the gradient norm to the quantization noise norm), computed
 * on the device in stream order from the two sums an fp4_quantize_noise or
 * fp4_quantize_dual_noise call accumulated:
 *   *ratio = sqrt(noise[0] / noise[1])   (FP64; +inf when noise[1] == 0,
 *                                          0 when both are 0)
 * noise: device, two doubles; ratio: device, one double; both 8-byte aligned.
 * Reading the ratio on the host is the caller's (after the stream is
 * synchronized); the threshold itself is the caller's. */
fp4_status fp4_noise_ratio(const double* noise, double* ratio, fp4_stream_t stream);

/* Two-dimensional block quantization (Robots Atlas, "FP4", How it works:
 * two-dimensional quantization among the stabilizers of FP4 training): one
 * scale per B x B block of the R x C source (16 x 16 NVFP4, 32 x 32 MXFP4),
 * from the block's amax by the same rule as a 1-D block, so the matrix and its
 * transpose are one quantization (a weight quantized once serves the forward
 * GEMM, blocked along K, and dgrad, blocked along N).
 *   out     R x C, blocks along C; every row of a block carries its byte.
 *   out_t   C x R, blocks along R: exactly the transpose of out.
 *   rnd     RTN, or SR with element index = row-major position in the R x C
 *           source + index_offset for both outputs (unlike fp4_quantize with
 *           FP4_AXIS_ROWS, whose index follows the transposed orientation).
 *   amax_ready  NVFP4: 1 if *out->amax holds the tensor amax, 0 to compute it;
 *           *out_t->amax, when another scalar, receives a copy; both tscale
 *           scalars receive s_g.
 * Requires: same fmt on both, had_on 0 on both (FP4_ERR_UNSUPPORTED); R and C
 * multiples of B; C % 8 == 0; ld >= C and ld % 8 == 0; src 16-byte aligned;
 * SR index_offset % 8 == 0. Errors as fp4_quantize. */
fp4_status fp4_quantize_2d(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                           fp4_rounding rnd, uint64_t seed, uint64_t index_offset, int amax_ready,
                           fp4_tensor* out, fp4_tensor* out_t, fp4_stream_t stream);

/* Dequantize q to dst (device, q->rows x q->cols row-major, leading dimension
 * ld >= cols, FP32 or bf16): the value each code stands for, its E2M1 value
 * times the block scale (times the tensor scale for NVFP4) (Robots Atlas,
 * "FP4", How it works: two-level scaling; Components: E2M1, E4M3 and E8M0):
 *   NVFP4: (e2m1 * sdec) * s_g, the last product rounded once to FP32;
 *   MXFP4: e2m1 * 2^e (exact); values stay in the rotated domain when had_on.
 * A bf16 output is the FP32 value rounded to nearest even.
 * Requires q->rows, q->cols >= 1, q->cols a multiple of B, ld >= q->cols,
 * ld % 8 == 0, dst and q->codes 16-byte aligned. */
fp4_status fp4_dequantize(const fp4_tensor* q, fp4_dtype dst_t, void* dst, int64_t ld,
                          fp4_stream_t stream);

/* fp4_dequantize, then, when q->had_on, the inverse of the block rotation the
 * quantization applied (Quartet, Approach: block-wise Hadamard rotations;
 * Robots Atlas, "FP4", How it works: random Hadamard transforms), so the
 * values are read back in the tensor's own domain rather than the rotated
 * one. The rotation of a block was y = c H D x (D = diag(+-1) from
 * q->had_signs, H the Sylvester Hadamard matrix, c = 2^-2.5 rounded to FP32
 * for MXFP4's 32-value blocks, 1/4 for NVFP4's 16); its inverse, the
 * transpose D H c, is applied to each block of dequantized values in the
 * quantized orientation: the butterfly stages h = 1, 2, 4, ... (each sum and
 * difference one FP32 operation), the product with c, then the signs. With
 * had_on == 0 the result equals fp4_dequantize's. Requirements and errors as
 * fp4_dequantize. */
fp4_status fp4_dequantize_unrotated(const fp4_tensor* q, fp4_dtype dst_t, void* dst, int64_t ld,
                                    fp4_stream_t stream);

/* GEMM operands. Each operand stands for a rows x K matrix (A: M x K,
 * B: N x K) whose values the GEMM contracts along K. It is either already
 * quantized, or a raw matrix that fp4_gemm quantizes into the caller's
 * workspace first, with the layout, format and rounding flags below (the
 * three linear-layer GEMMs on FP4 operands: "Quartet", one-line summary and
 * Approach; FP4 weights, activations and gradients: "FP4 All the Way", Key
 * points):
 *   FP4_OPERAND_QUANTIZED  q: a quantized tensor blocked along K
 *                          (rows = q->rows, K = q->cols).
 *   FP4_OPERAND_RAW        data: device FP32 or bf16 (dtype), leading
 *                          dimension ld, and
 *                          layout FP4_LAYOUT_N: data is rows x K, K contiguous
 *                                 (quantized with FP4_AXIS_COLS);
 *                          layout FP4_LAYOUT_T: data is K x rows, rows
 *                                 contiguous (quantized with FP4_AXIS_ROWS:
 *                                 e.g. W for dgrad, dY and X for wgrad);
 *                          fmt, rnd, seed, index_offset, had_on, had_signs as
 *                          for fp4_quantize (the element index follows the
 *                          rows x K orientation). NVFP4 takes the tensor amax
 *                          of the values quantized (an amax pass first).
 *                          Requirements are fp4_quantize's for the stored
 *                          matrix (rows x K for N, K x rows for T). */
typedef enum fp4_operand_kind { FP4_OPERAND_QUANTIZED = 0, FP4_OPERAND_RAW = 1 } fp4_operand_kind;
typedef enum fp4_layout { FP4_LAYOUT_N = 0, FP4_LAYOUT_T = 1 } fp4_layout;

typedef struct fp4_operand {
    int32_t kind;            /* fp4_operand_kind */
    int32_t dtype;           /* RAW: fp4_dtype of data */
    const fp4_tensor* q;     /* QUANTIZED */
    const void* data;        /* RAW: device */
    int64_t rows;            /* RAW: M (A) or N (B) */
    int64_t k;               /* RAW: K */
    int64_t ld;              /* RAW: leading dimension of the stored matrix, elements */
    int32_t layout;          /* RAW: fp4_layout */
    int32_t fmt;             /* RAW: fp4_format */
    int32_t rnd;             /* RAW: fp4_rounding */
    int32_t had_on;          /* RAW: 1 to rotate (see Conventions) */
    uint64_t seed;           /* RAW, SR: the stream's seed */
    uint64_t index_offset;   /* RAW, SR: added to the element index; % 8 == 0 */
    uint32_t had_signs;      /* RAW: the rotation's sign mask when had_on */
    uint32_t reserved;
} fp4_operand;

/* Bytes of device workspace fp4_gemm needs for these operands (RAW operands
 * are quantized there first, as every GEMM operand of a fully quantized
 * linear layer is: Quartet, Approach): for each RAW
 * operand, in the order A then B, its codes, its scale bytes and (NVFP4) its
 * two FP32 scalars, each piece starting on a 256-byte boundary. 0 when
 * neither operand is RAW, or when an operand is NULL or its kind, format,
 * rows or K is invalid (fp4_gemm reports which). Host-only. */
size_t fp4_gemm_workspace_bytes(const fp4_operand* A, const fp4_operand* B);

/* Optional workspace beyond fp4_gemm_workspace_bytes(A, B): given at least
 * fp4_gemm_workspace_bytes(A, B) + fp4_gemm_splitk_bytes(A, B) bytes,
 * fp4_gemm splits the output tiles of the last, partial wave of workgroups
 * (one 256 x 256 tile per CU) along K, writes their FP32 partial tiles to
 * this area (placed after the RAW operands' pieces, on a 256-byte boundary)
 * and adds them, in split order, in a second kernel on the stream. This pays
 * when few tiles would keep few CUs busy for a long K: the plan weighs the
 * shorter wave against the partial tiles' traffic, and takes into account
 * that a wave on fewer CUs runs at a higher clock (the chip is power-limited
 * under this load). E.g. 6 tiles of a 520 x 300 x 8192 product split in 4,
 * a 2048 x 2048 x 32768 weight gradient's 64 tiles in 3; the Llama-7B
 * layer's GEMMs do not split. A split product differs from the unsplit one
 * only in the order of its FP32 additions, and is the same on every call
 * for a given shape. 0 when the shape never splits or the operands are
 * invalid. Host-only. */
size_t fp4_gemm_splitk_bytes(const fp4_operand* A, const fp4_operand* B);

/* C[i][j] = alpha * sum_k A_hat[i][k] * B_hat[j][k] with FP32 accumulation
 * (Robots Atlas, "FP4", How it works: FP4 products accumulated in higher
 * precision; "Quartet", one-line summary: forward, dgrad and wgrad all run as
 * FP4 GEMMs), where A_hat, B_hat are the dequantized operands (both blocked
 * along the shared contraction axis K), M = A's rows, N = B's rows, K the
 * operands' common K, alpha = s_gA * s_gB for NVFP4 and 1 for MXFP4. alpha is
 * one FP32 product applied to the FP32 accumulators: for operands whose
 * tensor scales multiply below 2^-126 (both tensor amaxes below about 1e-15)
 * it is subnormal or zero, and the output loses precision or becomes 0.
 *   The three GEMMs of a linear layer: forward Y = X W^T (A = X, B = W, both
 *   layout N); dgrad dX = dY W (A = dY layout N, B = W layout T); wgrad
 *   dW = dY^T X (A = dY layout T, B = X layout T).
 *   MXFP4 runs on the gfx950 block-scaled FP4 MFMA with the E8M0 bytes as its
 *   scale operands. NVFP4 decodes e2m1 * E4M3 exactly into f16 in registers
 *   (at most 6 significant bits, magnitudes in [2^-10, 2688]) and runs the
 *   f16 MFMA.
 * RAW operands are quantized into ws (see fp4_gemm_workspace_bytes) on the
 * stream before the product; ws: device, 256-byte aligned, ws_bytes at least
 * fp4_gemm_workspace_bytes(A, B) (FP4_ERR_WORKSPACE otherwise; ws may be NULL
 * when neither operand is RAW). The workspace holds the quantized operands
 * when the call's work has run. With fp4_gemm_splitk_bytes(A, B) more bytes
 * the last partial wave of output tiles is split along K (see there).
 * C: device, M x N row-major, leading dimension ldc >= N, FP32 or bf16
 * (rounded to nearest even once, after alpha).
 * Requires: same fmt, had_on and had_signs on both operands
 * (FP4_ERR_UNSUPPORTED); the same K, K % 128 == 0; M, N >= 1 (any value);
 * each operand's codes below 2^31 bytes (rows * K / 2); ldc >= N (any value);
 * C aligned to its element size; a QUANTIZED operand's codes and scales
 * 16-byte aligned and, for NVFP4, its tscale set; a RAW operand as above.
 * Validation covers both operands and the workspace before anything is
 * enqueued. */
fp4_status fp4_gemm(const fp4_operand* A, const fp4_operand* B, fp4_dtype out_t, void* C,
                    int64_t ldc, void* ws, size_t ws_bytes, fp4_stream_t stream);

/* The workspace limit of fp4_gemm_noalloc: 128 MiB (both raw NVFP4 operands
 * of a 32768 x 4096 by 11008 x 4096 product take 100.9 MB). */
#define FP4_GEMM_NOALLOC_MAX_BYTES ((size_t)128 << 20)

/* fp4_gemm for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. The
 * same product as fp4_gemm, with RAW operands quantized into a workspace the
 * library owns instead of a caller buffer: a static device array of
 * FP4_GEMM_NOALLOC_MAX_BYTES, one copy on each GPU the library runs on, held
 * until the process ends. Its address on a device is looked up once, on the
 * first call on that device that has a RAW operand (make that call outside
 * graph capture). The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine); the caller still passes C.
 * FP4_ERR_WORKSPACE when fp4_gemm_workspace_bytes(A, B) exceeds
 * FP4_GEMM_NOALLOC_MAX_BYTES (nothing enqueued). Every call on a GPU shares
 * that GPU's array and leaves its quantized operands there: calls with RAW
 * operands that overlap on one GPU (other streams, other threads) race on it,
 * so the caller serializes them. It never splits along K (the array holds
 * only the RAW operands). Otherwise as fp4_gemm. */
fp4_status fp4_gemm_noalloc(const fp4_operand* A, const fp4_operand* B, fp4_dtype out_t, void* C,
                            int64_t ldc, fp4_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* FP4_H */
