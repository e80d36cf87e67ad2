// fp4_internal.hpp -- launchers shared between the C-ABI layer and the kernel
// translation units of libfp4 (not part of the public interface).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

struct QuantArgs {
  const void* src;
  bool bf16;
  int64_t R, C, ld;      // source matrix, row-major
  bool rows_axis;        // blocks along R (output is the transpose)
  int fmt;               // 0 NVFP4, 1 MXFP4
  bool sr;
  uint64_t seed, offset;
  // SR element index along rows_axis: c * idx_rows + r + offset (0: R). A row
  // shard of a taller tensor passes the tensor's row count and puts its first
  // row in offset, so its draws are those of the whole tensor's quantization.
  int64_t idx_rows;
  bool had_on;
  uint32_t signs;
  uint8_t* codes;
  uint8_t* scales;
  const float* amax;     // NVFP4: device tensor amax (already computed)
  float* tscale;         // NVFP4: receives s_g
  double* noise;         // null, or receives += (sum x^2, sum (xhat - x)^2)
};

// Both orientations of one source (fp4_quantize_dual): *_c blocks along C,
// *_r blocks along R (transposed output).
struct DualArgs {
  const void* src;
  bool bf16;
  int64_t R, C, ld;
  int fmt;
  bool had_c, had_r;               // rotation of each orientation
  bool sr_c, sr_r;
  uint64_t seed_c, offset_c, seed_r, offset_r;
  int64_t idx_rows_r;              // SR index of the *_r orientation: c * idx_rows_r + r (0: R)
  uint32_t signs_c, signs_r;
  uint8_t *codes_c, *scales_c, *codes_r, *scales_r;
  const float* amax_c;             // NVFP4: tensor amax of each orientation's values
  const float* amax_r;             //   (already computed; the same pointer when equal)
  float *tscale_c, *tscale_r;      // NVFP4: receive s_g of each orientation
  float* amax_copy;                // NVFP4: receives a copy of *amax_c, or null
  double *noise_c, *noise_r;       // null, or receive += (sum x^2, sum (xhat - x)^2)
};

// Two-dimensional block quantization (fp4_quantize_2d): codes/scales blocks
// along C ([R][C]), codes_t/scales_t the transpose ([C][R]).
struct Quant2dArgs {
  const void* src;
  bool bf16;
  int64_t R, C, ld;
  int fmt;
  bool sr;
  uint64_t seed, offset;
  uint8_t *codes, *scales, *codes_t, *scales_t;
  const float* amax;               // NVFP4: the tensor amax (already computed)
  float *tscale, *tscale_t;        // NVFP4: receive s_g
  float* amax_copy;                // NVFP4: receives a copy of the amax, or null
};

struct GemmArgs {
  const uint8_t* a_codes;
  const uint8_t* a_scales;
  const uint8_t* b_codes;
  const uint8_t* b_scales;
  const float* a_tscale;  // NVFP4 only
  const float* b_tscale;
  int64_t M, N, K;
  int fmt;
  bool bf16out;
  void* c;
  int64_t ldc;
  // Optional FP32 area of at least fp4i_gemm_split_bytes(M, N, K) bytes, or
  // null: with it, the output tiles of the last partial wave are split along
  // K and their partial sums added by a second kernel.
  float* split_ws;
};

void fp4i_launch_amax(const void* src, bool bf16, int64_t R, int64_t C, int64_t ld, float* amax,
                      hipStream_t s);
// amax of the values rotated 16-wide (NVFP4 Hadamard) along rows (blocks along
// C) or down columns (rows_axis: blocks along R).
void fp4i_launch_amax_rot16(const void* src, bool bf16, int64_t R, int64_t C, int64_t ld,
                            bool rows_axis, uint32_t signs, float* amax, hipStream_t s);
// Both orientations' amaxes of a dual quantization with a rotation on at least
// one side, from one read (R % 16 == 0, C % 16 == 0): amax_c of the values
// blocked along C (rotated along C when had_c), amax_r of those blocked along R
// (rotated along R when had_r).
void fp4i_launch_amax_pair(const void* src, bool bf16, int64_t R, int64_t C, int64_t ld, bool had_c,
                           uint32_t signs_c, bool had_r, uint32_t signs_r, float* amax_c,
                           float* amax_r, hipStream_t s);
void fp4i_launch_quant(const QuantArgs& a, hipStream_t s);
void fp4i_launch_quant_dual(const DualArgs& a, hipStream_t s);
void fp4i_launch_quant_2d(const Quant2dArgs& a, hipStream_t s);
void fp4i_launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* tscale, int fmt,
                         int64_t rows, int64_t cols, bool bf16out, void* dst, int64_t ld,
                         hipStream_t s);
// Dequantize, then the inverse of the block rotation with sign mask `signs`
// (B = 16 for NVFP4, 32 for MXFP4) on every block of each row.
void fp4i_launch_dequant_unrot(const uint8_t* codes, const uint8_t* scales, const float* tscale, int fmt,
                               int64_t rows, int64_t cols, uint32_t signs, bool bf16out, void* dst,
                               int64_t ld, hipStream_t s);
bool fp4i_gemm_fits(int64_t M, int64_t N, int64_t K);
// Bytes of the split-K area the GEMM of this shape can use (0: it never splits).
size_t fp4i_gemm_split_bytes(int64_t M, int64_t N, int64_t K);
// *ratio = sqrt(noise[0] / noise[1]) on the device (the gradient-noise monitor's statistic).
void fp4i_launch_noise_ratio(const double* noise, double* ratio, hipStream_t s);
void fp4i_launch_gemm(const GemmArgs& g, hipStream_t s);
