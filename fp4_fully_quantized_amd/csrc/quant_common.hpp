// quant_common.hpp -- device helpers shared by the quantize kernels (quant.hip,
// quant_dual.hip): the NVFP4 tensor scale, the block scale rules and the
// block-wise random-sign Hadamard rotation.
//
//   NVFP4  s_g = amax/2688; per 16-block byte = E4M3_rne((amax_b/6)/s_g),
//          r = 1/(sdec*s_g)          (Robots Atlas, "FP4", Components)
//   MXFP4  per 32-block e = the smallest e with 6*2^e >= amax_b, r = 2^-e
//   Hadamard  y = c * H_B * D * x on each B-block along the blocked axis, D
//          from bits 0..B-1 of the mask, Sylvester butterfly stages 1, 2, ..,
//          B/2 in FP32, c = 2^-2.5 (B = 32, rounded to FP32) or 1/4 (B = 16,
//          exact) (Quartet, Approach; Robots Atlas, "FP4", How it works).
#pragma once
#include "fp4_device.hpp"

namespace fp4q {

using namespace fp4dev;

constexpr int NV = 0;
constexpr int MX = 1;

// s_g = amax / 2688; 1 for an amax of 0 or below 2^-100 (such a tensor
// quantizes to signed zeros instead of reaching 0/0 or an infinite reciprocal
// through a zero or subnormal s_g).
__device__ __forceinline__ float nv_tensor_scale(float amax) {
  return amax < 0x1p-100f ? 1.0f : amax / 2688.0f;
}

// amax_b / 6 rounded to nearest even in FP32 (m >= 0, finite). From 2^-100
// up, one multiply by RN(1/6) and one fma correction give exactly the IEEE
// quotient: the residual m - 6 q0 is exact (an fma) and zero or a normal
// number there, and the corrected quotient equals the correctly rounded one
// for every such FP32 m (checked over all of them); below 2^-100 the division
// itself. About a third of the division's instructions.
__device__ __forceinline__ float div6(float m) {
  if (m < 0x1p-100f) return m / 6.0f;
  const float r6 = 0x1.555556p-3f;   // RN(1/6)
  const float q0 = m * r6;
  return __builtin_fmaf(__builtin_fmaf(-6.0f, q0, m), r6, q0);
}

// The element multipliers an NVFP4 tensor can use, r(b) = 1 / (E4M3(b) * s_g)
// (0 when the product is 0), for the scale bytes b = 0 .. 127 (127, E4M3's
// NaN, never occurs: the encoder saturates at 448), one IEEE division each,
// written to an LDS table by the first 128 threads. The caller synchronizes
// the workgroup before the table is read.
__device__ __forceinline__ void nv_rcp_table(float* tab, float sg) {
  const int t = threadIdx.x;
  if (t < 128) {
    const float d = e4m3_decode((uint32_t)t) * sg;
    tab[t] = (d == 0.0f) ? 0.0f : 1.0f / d;
  }
}

// Block scale of one block with amax m, the NVFP4 multiplier read from the
// table above (MXFP4 ignores it). Equal to block_scale below.
template <int FMT>
__device__ __forceinline__ uint32_t block_scale_tab(float m, float sg, const float* tab, float& r) {
  if constexpr (FMT == NV) {
    const uint32_t byte = e4m3_encode(div6(m) / sg);
    r = tab[byte];
    return byte;
  } else {
    const int e = e8m0_exponent(m);
    r = pow2_neg(e);
    return (uint32_t)(e + 127);
  }
}

// Block scale of one block with amax m. Returns the scale byte, sets the
// element multiplier r.
template <int FMT>
__device__ __forceinline__ uint32_t block_scale(float m, float sg, float& r) {
  if constexpr (FMT == NV) {
    float q = m / 6.0f;
    q = q / sg;
    uint32_t byte = e4m3_encode(q);
    float d = e4m3_decode(byte) * sg;
    r = (d == 0.0f) ? 0.0f : 1.0f / d;
    return byte;
  } else {
    int e = e8m0_exponent(m);
    r = pow2_neg(e);
    return (uint32_t)(e + 127);
  }
}

// The rotation's normalisation for a B-block.
template <int B>
__device__ __forceinline__ float hadamard_scale() {
  if constexpr (B == 32) return hadamard_norm();
  else return 0.25f;
}

// All butterfly stages and the normalisation on one B-block held by one
// thread whose signs are already applied.
template <int B>
__device__ __forceinline__ void fwht_block(float x[B]) {
#pragma unroll
  for (int h = 1; h < B; h <<= 1) {
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if ((i & h) == 0) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  const float c = hadamard_scale<B>();
#pragma unroll
  for (int i = 0; i < B; ++i) x[i] = x[i] * c;
}

// Signs, all butterfly stages and the normalisation on one B-block held by
// one thread.
template <int B>
__device__ __forceinline__ void hadamard_block(float x[B], uint32_t signs) {
#pragma unroll
  for (int i = 0; i < B; ++i)
    if ((signs >> i) & 1u) x[i] = -x[i];
#pragma unroll
  for (int h = 1; h < B; h <<= 1) {
#pragma unroll
    for (int i = 0; i < B; ++i) {
      if ((i & h) == 0) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  const float c = hadamard_scale<B>();
#pragma unroll
  for (int i = 0; i < B; ++i) x[i] = x[i] * c;
}

// ---- quantization noise (the gradient-noise monitor) ----------------------
// The value a block's scale byte stands for: E4M3 (NVFP4) or 2^(byte - 127).
template <int FMT>
__device__ __forceinline__ float scale_value(uint32_t byte) {
  if constexpr (FMT == NV) return e4m3_decode(byte);
  else return __builtin_ldexpf(1.0f, (int)byte - 127);
}

// Adds sum x^2 and sum (xhat - x)^2 of 8 quantized values to g and e (FP32):
// xhat = e2m1 * bs (* sg for NVFP4) is the value of code nibble i of w; the
// code-scale product is exact, the difference is rounded once (one fma for
// NVFP4), the squares accumulate by fma.
template <int FMT>
__device__ __forceinline__ void noise8(const float x[8], uint32_t w, float bs, float sg, float& g,
                                       float& e) {
  float q[8];
  {
    const auto q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const auto q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const auto q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const auto q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    q[0] = q0[0]; q[1] = q0[1]; q[2] = q1[0]; q[3] = q1[1];
    q[4] = q2[0]; q[5] = q2[1]; q[6] = q3[0]; q[7] = q3[1];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float qs = q[i] * bs;
    const float d = (FMT == NV) ? __builtin_fmaf(qs, sg, -x[i]) : qs - x[i];
    e = __builtin_fmaf(d, d, e);
    g = __builtin_fmaf(x[i], x[i], g);
  }
}

// Grid of a noise-monitored launch over n tiles or tasks: as many workgroups
// of 256 threads as the device runs at once (the kernel's occupancy per CU
// times the CUs), at most n; each workgroup then loops over several tiles.
// Every workgroup ends with two FP64 atomic adds per sum pair on the same two
// addresses, which serialize, so the grid must not be one per tile; and a grid
// beyond what runs at once leaves its last workgroups a whole loop of tiles to
// run alone after the others have finished.
template <typename Kernel>
inline uint32_t noise_grid(Kernel kernel, uint32_t n) {
  int per_cu = 0, dev = 0, cus = 0;
  uint32_t g = 512;  // if the queries fail
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 256, 0) == hipSuccess &&
      hipGetDevice(&dev) == hipSuccess &&
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
      per_cu > 0 && cus > 0)
    g = (uint32_t)per_cu * (uint32_t)cus;
  return n < g ? (n ? n : 1) : g;
}

// Workgroup sum of (g, e), then out[0] += g, out[1] += e. Every thread of the
// workgroup calls it (it synchronizes).
__device__ __forceinline__ void noise_reduce(double g, double e, double* out) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    g += __shfl_xor(g, off, 64);
    e += __shfl_xor(e, off, 64);
  }
  __shared__ double part[4][2];
  if ((threadIdx.x & 63) == 0) {
    part[threadIdx.x >> 6][0] = g;
    part[threadIdx.x >> 6][1] = e;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    atomicAdd(out, (part[0][0] + part[1][0]) + (part[2][0] + part[3][0]));
    atomicAdd(out + 1, (part[0][1] + part[1][1]) + (part[2][1] + part[3][1]));
  }
}

// The dispatcher hands workgroups to the 8 XCDs in turn (workgroup b to XCD
// b % 8), each XCD with its own L2. This maps workgroup b to a tile index so
// that every XCD takes one contiguous range of the n tiles: row-major
// neighbours, whose partial output lines (half-line code runs, 8-byte scale
// runs) complete each other, then meet in one L2 instead of being written
// back as separate partial lines. A bijection on [0, n).
__device__ inline uint32_t xcd_contiguous_tile(uint32_t b, uint32_t n) {
  const uint32_t x = b % 8, l = b / 8, per = n / 8, rem = n % 8;
  return x * per + (x < rem ? x : rem) + l;
}

}  // namespace fp4q
