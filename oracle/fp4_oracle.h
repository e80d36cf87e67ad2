/*
 * fp4_oracle.h -- plain CPU oracle for block-scaled FP4 quantization.
 *
 * TEST INFRASTRUCTURE ONLY. This library exists so that tests, the smoke
 * check and the CPU-baseline leg of the benchmark can check the GPU library
 * against an independent, slow, obviously correct implementation. The GPU
 * product path never includes, links or calls anything in this directory,
 * and this directory never includes anything from the GPU library.
 *
 * Formats (Robots Atlas, "FP4", section Components):
 *   E2M1 element: 1 sign, 2 exponent, 1 mantissa bit; magnitudes
 *   0, 0.5, 1, 1.5, 2, 3, 4, 6.
 *   NVFP4: 16-element blocks, E4M3 block scale, FP32 per-tensor scale.
 *   MXFP4: 32-element blocks, E8M0 (power-of-two) block scale.
 * Rounding (FP4 All the Way, Key points / Summary): round-to-nearest in the
 *   forward pass, stochastic rounding for backward and update passes.
 * Rotation (Quartet, Approach): block-wise Hadamard rotation.
 *
 * Conventions where the pages are silent are listed in the repository's
 * design notes and restated at each function in fp4_oracle.c.
 */
#ifndef FP4_ORACLE_H
#define FP4_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { O_FMT_NVFP4 = 0, O_FMT_MXFP4 = 1 };
enum { O_RTN = 0, O_SR = 1 };
/* O_AXIS_COLS: blocks run along the contiguous (last) axis; output [R][C].
 * O_AXIS_ROWS: blocks run along the first axis; output is the transpose
 *              orientation [C][R]. */
enum { O_AXIS_COLS = 0, O_AXIS_ROWS = 1 };

/* ---- element and scale codecs ---- */
double   o_e2m1_value(unsigned code4);          /* signed value of a 4-bit code */
unsigned o_e2m1_rtn_mag(float a);               /* a in [0,6] -> magnitude code 0..7 */
unsigned o_e2m1_sr_mag(float a, uint32_t h16);  /* a in [0,6], 16-bit draw -> code 0..7 */
double   o_e4m3_value(unsigned byte);           /* OCP E4M3 "fn" decode; NaN for 0x7F/0xFF */
unsigned o_e4m3_encode(float t);                /* t >= 0: RNE to finite E4M3, saturating */
int      o_e8m0_exponent(float amax_b);         /* smallest e with 6*2^e >= amax_b, in [-127,127] */
double   o_e8m0_value(unsigned byte);           /* 2^(byte-127); NaN for 0xFF */
uint16_t o_f32_to_bf16_rne(float x);            /* round-to-nearest-even, finite inputs */
float    o_bf16_to_f32(uint16_t b);

/* ---- randomness ---- */
void     o_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
uint32_t o_sr_draw16(uint64_t seed, uint64_t index);   /* 16-bit draw of element `index` */
uint32_t o_hadamard_signs(uint64_t seed);

/* ---- rotation ---- */
void     o_fwht32(float x[32], uint32_t signs);        /* signs, Sylvester FWHT, times 2^-2.5 */
void     o_fwht16(float x[16], uint32_t signs);        /* bits 0..15, Sylvester FWHT, times 1/4 */
/* inverses (transposes): FWHT stages, times 2^-2.5 (1/4), then the signs */
void     o_unfwht32(float y[32], uint32_t signs);
void     o_unfwht16(float y[16], uint32_t signs);

/* ---- tensors ---- */
/* max |x| over an R x C matrix with leading dimension ld (elements). */
float    o_tensor_amax(const void* src, int src_bf16, int64_t R, int64_t C, int64_t ld);

/* Quantize an R x C matrix (row-major, leading dimension ld, fp32 or bf16 bits).
 * had_on: every block along the blocked axis is rotated first (MXFP4: 32-wide,
 * o_fwht32; NVFP4: 16-wide, o_fwht16); the NVFP4 tensor amax is then that of
 * the rotated tensor.
 * In the quantized orientation (rows_q x cols_q; [R][C] for COLS, [C][R] for ROWS):
 *   codes  : rows_q * cols_q / 2 bytes, element 2t in the low nibble of byte t
 *   scales : rows_q * cols_q / B bytes (B = 16 NVFP4, 32 MXFP4)
 * NVFP4: if amax_given, amax_in is used as the tensor amax, else it is computed.
 *        *amax_out and *sg_out receive the tensor amax and the FP32 tensor scale.
 * MXFP4: amax_out / sg_out may be NULL and are not written.
 * Returns 0, or a negative number on invalid arguments or non-finite input. */
int o_quantize(const void* src, int src_bf16, int64_t R, int64_t C, int64_t ld,
               int axis, int fmt, int rnd, uint64_t seed, uint64_t index_offset,
               int had_on, uint32_t had_signs, int amax_given, float amax_in,
               uint8_t* codes, uint8_t* scales, float* amax_out, float* sg_out);

/* Dequantize to FP32 exactly as the library contract defines it:
 *   NVFP4: (e2m1 * scale) * tensor_scale, the last product rounded once to FP32;
 *   MXFP4: e2m1 * 2^e (exact). */
/* o_quantize, plus the quantization noise of the result: noise[0] = sum x^2
 * and noise[1] = sum (xhat - x)^2 over the quantized values x (rotated when
 * had_on) and the exact values xhat their codes and scales stand for. */
int o_quantize_noise(const void* src, int src_bf16, int64_t R, int64_t C, int64_t ld,
                     int axis, int fmt, int rnd, uint64_t seed, uint64_t index_offset,
                     int had_on, uint32_t had_signs, int amax_given, float amax_in,
                     uint8_t* codes, uint8_t* scales, float* amax_out, float* sg_out,
                     double noise[2]);
/* Two-dimensional B x B block quantization of an R x C matrix (R, C multiples
 * of B): one scale per square block, element index for SR = row-major [R][C]
 * position + index_offset. codes/scales as o_quantize with axis COLS, and
 * codes_t/scales_t as axis ROWS; the two are transposes of each other. */
int o_quantize_2d(const void* src, int src_bf16, int64_t R, int64_t C, int64_t ld, int fmt, int rnd,
                  uint64_t seed, uint64_t index_offset, int amax_given, float amax_in,
                  uint8_t* codes, uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t,
                  float* amax_out, float* sg_out);
int o_dequantize_f32(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     int fmt, float sg, float* out);
/* Exact dequantized values in FP64 (e2m1 * scale * tensor_scale is exact in FP64). */
int o_dequantize_f64(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     int fmt, float sg, double* out);
/* o_dequantize_f32, then each block of the quantized orientation through the
 * inverse rotation (NVFP4: o_unfwht16, MXFP4: o_unfwht32) with had_signs. */
int o_dequantize_unrotated_f32(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                               int fmt, float sg, uint32_t had_signs, float* out);

int o_num_threads(void);

#ifdef __cplusplus
}
#endif
#endif
