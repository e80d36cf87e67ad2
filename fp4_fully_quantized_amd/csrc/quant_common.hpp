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

__device__ __forceinline__ float nv_tensor_scale(float amax) {
  return amax == 0.0f ? 1.0f : amax / 2688.0f;
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

}  // namespace fp4q
