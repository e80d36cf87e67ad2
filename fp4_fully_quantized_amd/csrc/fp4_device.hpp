// fp4_device.hpp -- device helpers shared by the gfx950 kernels of libfp4.
//
// Formats (Robots Atlas, "FP4", section Components): E2M1 elements, E4M3
// (NVFP4) and E8M0 (MXFP4) block scales. Conversions use the gfx950 hardware
// converters where their rounding equals the library contract (checked
// element by element against the CPU oracle by the GPU tests):
//   v_cvt_scalef32_pk_fp4_f32  f32 -> E2M1, round-to-nearest-even, saturating
//                              at 6, sign kept (-0 -> 0x8); the scale operand
//                              only contributes its exponent, so 1.0 is passed
//                              and the block scale is applied beforehand;
//   v_cvt_pk_fp8_f32           f32 -> E4M3 (OCP), round-to-nearest-even; the
//                              input is clamped to 448 first (saturation);
//   v_cvt_f32_fp8              E4M3 -> f32;
//   v_cvt_scalef32_pk_f16_fp4  E2M1 -> f16 (exact, scale 1).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4dev {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Loads 8 consecutive elements (bf16 or fp32) starting at p (16-byte aligned).
template <bool BF16>
__device__ __forceinline__ void load8(const void* p, float x[8]) {
  if constexpr (BF16) {
    uint4 w = *reinterpret_cast<const uint4*>(p);
    x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
    x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
    x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
    x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
  } else {
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
  }
}

// Cross-lane exchange inside a quad of lanes (DPP quad_perm).
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// ---- E4M3 ------------------------------------------------------------------
// Round-to-nearest-even, saturating at 448, of t >= 0 (finite).
__device__ __forceinline__ uint32_t e4m3_encode(float t) {
  t = fminf(t, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(t, 0.0f, 0, false) & 0xFFu;
}
__device__ __forceinline__ float e4m3_decode(uint32_t byte) {
  return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0);
}

// ---- E8M0 ------------------------------------------------------------------
// Smallest e with 6 * 2^e >= amax (amax >= 0 finite), clamped to >= -127.
// amax = m * 2^E, m in [1, 2): e = E - 2 if m <= 1.5 else E - 1; zero and
// subnormal amax fall to the clamp.
__device__ __forceinline__ int e8m0_exponent(float amax) {
  uint32_t u = __float_as_uint(amax);
  int E = (int)(u >> 23) - 127;
  uint32_t m = u & 0x7FFFFFu;
  int e = (m <= 0x400000u) ? E - 2 : E - 1;
  if ((u >> 23) == 0) e = -127;
  return e < -127 ? -127 : e;
}
// 2^-e as an FP32 (-e in [-126, 127] for finite inputs: always normal).
__device__ __forceinline__ float pow2_neg(int e) {
  return __uint_as_float((uint32_t)(127 - e) << 23);
}

// ---- E2M1 ------------------------------------------------------------------
// Round-to-nearest-even codes of 8 values (already multiplied by the block's
// reciprocal scale), packed low nibble first.
__device__ __forceinline__ uint32_t e2m1_rtn_pack8(const float v[8]) {
  uint32_t w = 0;
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[0], v[1], 1.0f, 0);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[2], v[3], 1.0f, 1);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[4], v[5], 1.0f, 2);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, v[6], v[7], 1.0f, 3);
  return w;
}

// ---- Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) ----------------------
__device__ __forceinline__ void philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                              uint32_t k0, uint32_t k1, uint32_t out[4]) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    // Three-input XORs as one gfx950 bitop3 each (truth table 0x96 = a ^ b ^ c):
    // written as two XORs the compiler issues two instructions.
    uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

// The draws of elements 8j .. 8j+7 (j = call index = element / 8): word i
// holds element 2i's 16-bit draw in its low half, element 2i+1's in its high half.
__device__ __forceinline__ void sr_draws8(uint64_t seed, uint64_t call, uint32_t w[4]) {
  philox4x32_10((uint32_t)call, (uint32_t)(call >> 32), 0u, 0u, (uint32_t)seed,
                (uint32_t)(seed >> 32), w);
}

// Stochastic rounding of 8 scaled values v with their 16-bit draws: a = |v|
// lies between grid neighbours lo <= a < hi (or is >= 6: code 7); with
// p = (a - lo) / (hi - lo) it rounds up iff h + floor(p * 2^16) >= 2^16; the
// sign is kept (also of zero). That is the rule of the hardware convert
// v_cvt_scalef32_sr_pk_fp4_f32 itself, measured on gfx950: it rounds the first
// value of its pair up iff (R >> 10) + floor(p * 2^22) >= 2^22, R its 32-bit
// random operand (saturating at 6, keeping the sign, also of zero), after
// dividing the value by the scale operand (1 here). With R = h << 16, i.e.
// R >> 10 = 64 h, that is 64 h + floor(p * 2^22) >= 2^22, and since 64 h is a
// multiple of 64, h + floor(p * 2^16) >= 2^16. The second value of the pair
// would use R << 1, not an independent draw, so each value gets its own
// convert and only the first slot's nibble is kept; the destination keeps its
// other bytes, and four byte-selects fill one word for the even elements and
// one for the odd. The second value of each pair is left arbitrary (whatever
// register follows the value), which spares a register move per value: the
// first slot's code does not depend on it (measured: 2^27.6 random values and
// draws, each converted with a zero partner and with a partner of random bits,
// NaN, infinity and denormal encodings included, gave the same first-slot
// code every time), and its nibble is masked off. w[i] holds the draws of
// elements 2i (low half) and 2i+1 (high half).
__device__ __forceinline__ uint32_t e2m1_sr_pack8(const float v[8], const uint32_t w[4]) {
  const float one = 1.0f;
  uint32_t ev = 0, od = 0;
#define FP4_SR_CVT(DST, X, R, SEL)                                                               \
  asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, %3" SEL : "+v"(DST) : "v"(X), "v"(R), "s"(one))
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    // The value in the low half, the high half unspecified (shuffle index -1).
    const v2f ve = {v[2 * i], 0.0f}, vo = {v[2 * i + 1], 0.0f};
    const v2f xe = __builtin_shufflevector(ve, ve, 0, -1);
    const v2f xo = __builtin_shufflevector(vo, vo, 0, -1);
    const uint32_t re = w[i] << 16;           // h_even << 16
    const uint32_t ro = w[i] & 0xFFFF0000u;   // h_odd << 16
    if (i == 0) { FP4_SR_CVT(ev, xe, re, ""); FP4_SR_CVT(od, xo, ro, ""); }
    if (i == 1) { FP4_SR_CVT(ev, xe, re, " op_sel:[0,0,1,0]"); FP4_SR_CVT(od, xo, ro, " op_sel:[0,0,1,0]"); }
    if (i == 2) { FP4_SR_CVT(ev, xe, re, " op_sel:[0,0,0,1]"); FP4_SR_CVT(od, xo, ro, " op_sel:[0,0,0,1]"); }
    if (i == 3) { FP4_SR_CVT(ev, xe, re, " op_sel:[0,0,1,1]"); FP4_SR_CVT(od, xo, ro, " op_sel:[0,0,1,1]"); }
  }
#undef FP4_SR_CVT
  // Even codes sit in the low nibble of each byte of ev, odd ones in od (the
  // high nibbles hold the arbitrary partners' codes).
  return (ev & 0x0F0F0F0Fu) | ((od & 0x0F0F0F0Fu) << 4);
}

// ---- Hadamard --------------------------------------------------------------
// In-register butterfly stages h = 1, 2, 4 over 8 consecutive elements of a
// 32-block (the cross-lane stages 8 and 16 are done by the caller).
__device__ __forceinline__ void fwht8_local(float x[8]) {
#pragma unroll
  for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if ((i & h) == 0) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
}

// fp32(2^-2.5)
__device__ __forceinline__ float hadamard_norm() { return __uint_as_float(0x3E3504F3u); }

}  // namespace fp4dev
