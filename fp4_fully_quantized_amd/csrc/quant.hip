// quant.hip -- tensor amax, block-scaled FP4 quantize (both axes) and dequantize
// for gfx950.
//
// What is computed (Robots Atlas, "FP4", How it works and Components; FP4 All
// the Way, Key points; Quartet, Approach):
//   NVFP4  s_g = amax/2688; per 16-block byte = E4M3_rne((amax_b/6)/s_g),
//          r = 1/(sdec*s_g); codes = E2M1(x*r)
//   MXFP4  optional 32-wide random-sign Hadamard; per 32-block e = the
//          smallest e with 6*2^e >= amax_b; codes = E2M1(x*2^-e)
//   RTN or SR (16-bit Philox4x32-10 draws keyed by seed and element index).
//
// Memory-bound passes: every element is read once from HBM with 16-byte loads
// and written once as a nibble; block scales are one byte per block.
//  * k_amax        wave-strided 16-byte loads, per-lane max, wave and workgroup
//                  reduction, one atomicMax per workgroup on the float bits.
//  * k_quant_cols  blocks along the contiguous axis: each lane owns 8
//                  consecutive elements (one 16-byte bf16 load), a block spans
//                  2 (NVFP4) or 4 (MXFP4) lanes; the block amax and the
//                  Hadamard's cross-lane stages use DPP quad permutes; each
//                  lane stores one dword of 8 codes (256 contiguous bytes per
//                  wave).
//  * k_quant_rows  blocks along rows (the transposed orientation used by dgrad
//                  and wgrad operands): a 256 x 64 tile is loaded with
//                  coalesced 16-byte row loads into LDS (input format), each
//                  thread quantizes one block in each of 2 or 4 adjacent
//                  columns, and the codes leave through an LDS staging area
//                  in whole 128-byte lines.
//  * k_quant_dual  both orientations from one read: a 128 x 128 tile in LDS,
//                  quantized down its columns (staged, as k_quant_rows) and
//                  along its rows (written directly).
//  * k_dequant     8 elements per lane.
#include "fp4_device.hpp"
#include "fp4_internal.hpp"

using namespace fp4dev;

namespace {

constexpr int NV = 0;
constexpr int MX = 1;

__global__ void k_zero1(float* p) { *p = 0.0f; }

// A wave task is a 2048-element segment of one row: each lane issues four
// independent 16-byte (bf16) loads before reducing, to keep enough bytes in
// flight per CU.
template <bool BF16>
__global__ __launch_bounds__(256) void k_amax(const void* __restrict__ src, int64_t C, int64_t ld,
                                               uint32_t spr, uint32_t ntasks, float* amax) {
  constexpr int ES = BF16 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) >> 6;
  const uint32_t nwaves = gridDim.x * 4u;
  float m = 0.0f;
  for (uint32_t t = wave; t < ntasks; t += nwaves) {
    const uint32_t tu = __builtin_amdgcn_readfirstlane(t);
    const uint32_t r = tu / spr;
    const uint32_t seg = tu - r * spr;
    const char* row = static_cast<const char*>(src) + (int64_t)r * ld * ES;
    float x[4][8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t col = (int64_t)seg * 2048 + k * 512 + lane * 8;
      if (col < C) load8<BF16>(row + col * ES, x[k]);
      else
#pragma unroll
        for (int i = 0; i < 8; ++i) x[k][i] = 0.0f;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[k][i]));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float part[4];
  if (lane == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    atomicMax(reinterpret_cast<unsigned int*>(amax), __float_as_uint(b));
  }
}

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

template <int FMT, int RND, bool BF16, bool HAD>
__global__ __launch_bounds__(256) void k_quant_cols(const void* __restrict__ src, int64_t C, int64_t ld,
                                                     uint32_t spr, uint32_t ntasks,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     const float* __restrict__ amax, float* tscale,
                                                     uint64_t seed, uint64_t offset, uint32_t signs) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int B = FMT == NV ? 16 : 32;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) >> 6;
  const uint32_t nwaves = gridDim.x * 4u;
  float sg = 1.0f;
  if constexpr (FMT == NV) {
    sg = nv_tensor_scale(*amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) *tscale = sg;
  }
  const int sub = lane & 3;  // position of this lane's 8 elements inside a 32-block
  for (uint32_t t = wave; t < ntasks; t += nwaves) {
    const uint32_t tu = __builtin_amdgcn_readfirstlane(t);
    const uint32_t r = tu / spr;
    const uint32_t seg = tu - r * spr;
    const int64_t col = (int64_t)seg * 512 + lane * 8;
    const bool active = col < C;
    float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (active) load8<BF16>(static_cast<const char*>(src) + ((int64_t)r * ld + col) * ES, x);
    if constexpr (HAD) {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if ((signs >> (8 * sub + i)) & 1u) x[i] = -x[i];
      fwht8_local(x);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float p = dpp_xor1(x[i]);
        x[i] = (sub & 1) ? p - x[i] : x[i] + p;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float p = dpp_xor2(x[i]);
        x[i] = (sub & 2) ? p - x[i] : x[i] + p;
      }
      const float c = hadamard_norm();
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = x[i] * c;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
    m = fmaxf(m, dpp_xor1(m));
    if constexpr (FMT == MX) m = fmaxf(m, dpp_xor2(m));
    float rcp;
    const uint32_t sbyte = block_scale<FMT>(m, sg, rcp);
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = x[i] * rcp;
    uint32_t w;
    if constexpr (RND == 0) {
      w = e2m1_rtn_pack8(v);
    } else {
      uint32_t h[4];
      sr_draws8(seed, (offset + (uint64_t)r * (uint64_t)C + (uint64_t)col) >> 3, h);
      w = e2m1_sr_pack8(v, h);
    }
    if (active) {
      *reinterpret_cast<uint32_t*>(codes + (int64_t)r * (C / 2) + col / 2) = w;
      if ((lane & (B / 8 - 1)) == 0) scales[(int64_t)r * (C / B) + col / B] = (uint8_t)sbyte;
    }
  }
}

// Full 32-point butterfly (stages 1, 2, 4, 8, 16) on a 32-block held by one thread.
__device__ __forceinline__ void fwht32_local(float x[32]) {
#pragma unroll
  for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      if ((i & h) == 0) {
        float a = x[i], b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
}

// Transposed quantize: blocks along rows (the orientation of the dgrad and
// wgrad operands). A workgroup takes a tile of TR = 256 rows x TC = 64
// columns of the input:
//  1. coalesced 16-byte row loads into LDS, kept in the input format (row
//     pitch padded so the column reads below are free of bank conflicts);
//  2. thread (b, q) quantizes block b (rows b*B .. b*B+B-1) of the NCOL
//     adjacent columns q*NCOL ..: each LDS read brings one row of those NCOL
//     columns, so a block costs B reads for NCOL blocks (NVFP4: 4 columns of
//     16 rows, MXFP4: 2 columns of 32 rows);
//  3. codes and scale bytes are staged in LDS per output row (= input
//     column) and written out in whole 128-byte lines.
template <int FMT, int RND, bool BF16, bool HAD>
__global__ __launch_bounds__(256) void k_quant_rows(const void* __restrict__ src, int64_t R, int64_t C,
                                                     int64_t ld, uint32_t tiles_c,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     const float* __restrict__ amax, float* tscale,
                                                     uint64_t seed, uint64_t offset, uint32_t signs,
                                                     uint32_t scale_words) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int B = FMT == NV ? 16 : 32;
  constexpr int TR = 256, TC = 64;
  constexpr int NB = TR / B;               // blocks per tile column
  constexpr int NCOL = NB * TC / 256;      // adjacent columns per thread
  constexpr int TPB = TC / NCOL;           // threads per block row
  // Row pitch in bytes: the NCOL-column reads are NCOL*ES bytes and aligned to
  // that; one extra read's width of padding puts the block rows that one read
  // instruction touches in disjoint bank ranges.
  constexpr int PITCH = TC * ES + NCOL * ES;
  constexpr int SP = TR / 2 + 4;           // staged code bytes per output row (+ padding)
  __shared__ __attribute__((aligned(16))) uint8_t tile[TR * PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t stage_c[TC * SP];
  __shared__ __attribute__((aligned(16))) uint8_t stage_s[TC * NB];

  float sg = 1.0f;
  if constexpr (FMT == NV) {
    sg = nv_tensor_scale(*amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) *tscale = sg;
  }
  const uint32_t tr = blockIdx.x / tiles_c;
  const uint32_t tc = blockIdx.x - tr * tiles_c;
  const int64_t r0 = (int64_t)tr * TR;
  const int64_t c0 = (int64_t)tc * TC;
  const int tid = threadIdx.x;

  // 1. tile load: TR rows of TC * ES bytes, 16 bytes per load.
  constexpr int CPR = TC * ES / 16;
#pragma unroll
  for (int k = 0; k < TR * CPR / 256; ++k) {
    const int idx = k * 256 + tid;
    const int rr = idx / CPR;
    const int cc = idx % CPR;
    const int64_t col = c0 + cc * (16 / ES);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + rr < R && col < C)
      v = *reinterpret_cast<const uint4*>(static_cast<const char*>(src) + ((r0 + rr) * ld + col) * ES);
    uint32_t* d = reinterpret_cast<uint32_t*>(&tile[rr * PITCH + cc * 16]);
    d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
  }
  __syncthreads();

  // 2. quantize NCOL blocks per thread.
  const int b = tid / TPB;
  const int cl0 = (tid % TPB) * NCOL;
  const int64_t rg = r0 + (int64_t)b * B;
  float x[NCOL][B];
#pragma unroll
  for (int i = 0; i < B; ++i) {
    const uint8_t* p = &tile[(b * B + i) * PITCH + cl0 * ES];
    if constexpr (BF16) {
      if constexpr (NCOL == 4) {
        const uint2 w = *reinterpret_cast<const uint2*>(p);
        x[0][i] = bf16_lo(w.x); x[1][i] = bf16_hi(w.x); x[2][i] = bf16_lo(w.y); x[3][i] = bf16_hi(w.y);
      } else {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
        x[0][i] = bf16_lo(w); x[1][i] = bf16_hi(w);
      }
    } else {
      if constexpr (NCOL == 4) {
        const float4 w = *reinterpret_cast<const float4*>(p);
        x[0][i] = w.x; x[1][i] = w.y; x[2][i] = w.z; x[3][i] = w.w;
      } else {
        const float2 w = *reinterpret_cast<const float2*>(p);
        x[0][i] = w.x; x[1][i] = w.y;
      }
    }
  }
#pragma unroll
  for (int k = 0; k < NCOL; ++k) {
    const int cl = cl0 + k;
    const int64_t cg = c0 + cl;
    float* xk = x[k];
    if constexpr (HAD) {
#pragma unroll
      for (int i = 0; i < 32; ++i)
        if ((signs >> i) & 1u) xk[i] = -xk[i];
      fwht32_local(xk);
      const float hc = hadamard_norm();
#pragma unroll
      for (int i = 0; i < 32; ++i) xk[i] = xk[i] * hc;
    }
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < B; ++i) m = fmaxf(m, fabsf(xk[i]));
    float rcp;
    const uint32_t sbyte = block_scale<FMT>(m, sg, rcp);
    uint32_t* sc = reinterpret_cast<uint32_t*>(&stage_c[cl * SP + b * (B / 2)]);
#pragma unroll
    for (int g = 0; g < B / 8; ++g) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = xk[8 * g + i] * rcp;
      if constexpr (RND == 0) {
        sc[g] = e2m1_rtn_pack8(v);
      } else {
        uint32_t h[4];
        sr_draws8(seed, (offset + (uint64_t)cg * (uint64_t)R + (uint64_t)rg) / 8 + g, h);
        sc[g] = e2m1_sr_pack8(v, h);
      }
    }
    stage_s[cl * NB + b] = (uint8_t)sbyte;
  }
  __syncthreads();

  // 3. write out: output row c0 + cl gets the codes of input rows r0 .. (8-byte
  // pieces, 16 per row) and the scale bytes of its NB blocks.
  const int64_t rows_here = R - r0 < TR ? R - r0 : TR;  // a multiple of B
#pragma unroll
  for (int k = 0; k < TC * 16 / 256; ++k) {
    const int idx = k * 256 + tid;
    const int cl = idx / 16;
    const int seg = idx % 16;
    if (c0 + cl < C && seg * 16 < rows_here) {
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(&stage_c[cl * SP + seg * 8]);
      *reinterpret_cast<uint2*>(codes + (c0 + cl) * (R / 2) + r0 / 2 + seg * 8) = make_uint2(sp[0], sp[1]);
    }
  }
  if (scale_words) {
    // (R / B) % 4 == 0: one 4-byte word per thread covers 4 blocks of a row.
    constexpr int WPR = NB / 4;
    if (tid < TC * WPR) {
      const int cl = tid / WPR;
      const int wd = tid % WPR;
      if (c0 + cl < C && wd * 4 * B < rows_here)
        *reinterpret_cast<uint32_t*>(scales + (c0 + cl) * (R / B) + r0 / B + wd * 4) =
            *reinterpret_cast<const uint32_t*>(&stage_s[cl * NB + wd * 4]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < (TC * NB + 255) / 256; ++k) {
      const int idx = k * 256 + tid;
      const int cl = idx / NB;
      const int bb = idx % NB;
      if (idx < TC * NB && c0 + cl < C && bb * B < rows_here)
        scales[(c0 + cl) * (R / B) + r0 / B + bb] = stage_s[idx];
    }
  }
}

// Both orientations from one read of the source. A workgroup takes a
// 128 x 128 tile into LDS once (input format), then
//  (a) quantizes it with blocks down its columns (the transposed, ROWS
//      orientation), as k_quant_rows does: thread (b, q) handles block b of
//      NCOL adjacent columns; codes and scales are staged in LDS per output
//      row and written out after (b);
//  (b) quantizes it with blocks along its rows (the COLS orientation): thread
//      (row, half) takes 64 consecutive elements of one row (4 NVFP4 or 2
//      MXFP4 blocks) and writes their codes (32 bytes) and scales directly.
// Each orientation has its own rounding mode, SR stream and Hadamard mask;
// the results equal the two separate passes bit for bit.
template <int FMT, int RC, int RR, bool BF16, bool HAD>
__global__ __launch_bounds__(256) void k_quant_dual(
    const void* __restrict__ src, int64_t R, int64_t C, int64_t ld, uint32_t tiles_c,
    uint8_t* __restrict__ codes_c, uint8_t* __restrict__ scales_c,
    uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r,
    const float* __restrict__ amax, float* tscale_c, float* tscale_r, float* amax_r,
    uint64_t seed_c, uint64_t off_c, uint32_t signs_c, uint64_t seed_r, uint64_t off_r,
    uint32_t signs_r, uint32_t scale_words_c, uint32_t scale_words_r) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int B = FMT == NV ? 16 : 32;
  constexpr int T = 128;                  // tile rows = tile columns
  constexpr int NB = T / B;               // blocks per tile column (and per tile row)
  constexpr int NCOL = NB * T / 256;      // (a): adjacent columns per thread
  constexpr int TPB = T / NCOL;           // (a): threads per block row
  constexpr int PITCH = T * ES + 8;       // row pitch in bytes (8-byte reads stay aligned)
  constexpr int SP = T / 2 + 4;           // staged code bytes per output row of (a)
  __shared__ __attribute__((aligned(16))) uint8_t tile[T * PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t stage_c[T * SP];
  __shared__ __attribute__((aligned(16))) uint8_t stage_s[T * NB];

  float sg = 1.0f;
  if constexpr (FMT == NV) {
    const float a = *amax;
    sg = nv_tensor_scale(a);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *tscale_c = sg;
      *tscale_r = sg;
      if (amax_r) *amax_r = a;
    }
  }
  const uint32_t tr = blockIdx.x / tiles_c;
  const uint32_t tc = blockIdx.x - tr * tiles_c;
  const int64_t r0 = (int64_t)tr * T;
  const int64_t c0 = (int64_t)tc * T;
  const int tid = threadIdx.x;

  // 1. tile load, 16 bytes per load.
  constexpr int CPR = T * ES / 16;
#pragma unroll
  for (int k = 0; k < T * CPR / 256; ++k) {
    const int idx = k * 256 + tid;
    const int rr = idx / CPR;
    const int cc = idx % CPR;
    const int64_t col = c0 + cc * (16 / ES);
    uint4 v = make_uint4(0, 0, 0, 0);
    if (r0 + rr < R && col < C)
      v = *reinterpret_cast<const uint4*>(static_cast<const char*>(src) + ((r0 + rr) * ld + col) * ES);
    uint2* d = reinterpret_cast<uint2*>(&tile[rr * PITCH + cc * 16]);
    d[0] = make_uint2(v.x, v.y);
    d[1] = make_uint2(v.z, v.w);
  }
  __syncthreads();

  const int64_t rows_here = R - r0 < T ? R - r0 : T;  // multiples of B
  const int64_t cols_here = C - c0 < T ? C - c0 : T;

  // (a) blocks down the columns: output row c0 + cl, elements r0 ..
  {
    const int b = tid / TPB;
    const int cl0 = (tid % TPB) * NCOL;
    const int64_t rg = r0 + (int64_t)b * B;
    float x[NCOL][B];
#pragma unroll
    for (int i = 0; i < B; ++i) {
      const uint8_t* p = &tile[(b * B + i) * PITCH + cl0 * ES];
      if constexpr (BF16) {
        if constexpr (NCOL == 4) {
          const uint2 w = *reinterpret_cast<const uint2*>(p);
          x[0][i] = bf16_lo(w.x); x[1][i] = bf16_hi(w.x); x[2][i] = bf16_lo(w.y); x[3][i] = bf16_hi(w.y);
        } else {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(p);
          x[0][i] = bf16_lo(w); x[1][i] = bf16_hi(w);
        }
      } else {
#pragma unroll
        for (int k = 0; k < NCOL; k += 2) {
          const float2 w = *reinterpret_cast<const float2*>(p + 4 * k);
          x[k][i] = w.x; x[k + 1][i] = w.y;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < NCOL; ++k) {
      const int cl = cl0 + k;
      const int64_t cg = c0 + cl;
      float* xk = x[k];
      if constexpr (HAD) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if ((signs_r >> i) & 1u) xk[i] = -xk[i];
        fwht32_local(xk);
        const float hc = hadamard_norm();
#pragma unroll
        for (int i = 0; i < 32; ++i) xk[i] = xk[i] * hc;
      }
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < B; ++i) m = fmaxf(m, fabsf(xk[i]));
      float rcp;
      const uint32_t sbyte = block_scale<FMT>(m, sg, rcp);
      uint32_t* sc = reinterpret_cast<uint32_t*>(&stage_c[cl * SP + b * (B / 2)]);
#pragma unroll
      for (int g = 0; g < B / 8; ++g) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = xk[8 * g + i] * rcp;
        if constexpr (RR == 0) {
          sc[g] = e2m1_rtn_pack8(v);
        } else {
          uint32_t h[4];
          sr_draws8(seed_r, (off_r + (uint64_t)cg * (uint64_t)R + (uint64_t)rg) / 8 + g, h);
          sc[g] = e2m1_sr_pack8(v, h);
        }
      }
      stage_s[cl * NB + b] = (uint8_t)sbyte;
    }
  }

  // (b) blocks along the rows: row r0 + row, elements c0 + 64 * half ..
  {
    const int row = tid >> 1;
    const int half = tid & 1;
    const int64_t rgl = r0 + row;
    constexpr int NBT = 64 / B;  // blocks per thread
    uint32_t w[8];
    uint32_t sb[NBT];
#pragma unroll
    for (int bb = 0; bb < NBT; ++bb) {
      float x[B];
      const uint8_t* p = &tile[row * PITCH + (half * 64 + bb * B) * ES];
#pragma unroll
      for (int i = 0; i < B; i += 4) {
        if constexpr (BF16) {
          const uint2 u = *reinterpret_cast<const uint2*>(p + 2 * i);
          x[i] = bf16_lo(u.x); x[i + 1] = bf16_hi(u.x); x[i + 2] = bf16_lo(u.y); x[i + 3] = bf16_hi(u.y);
        } else {
          const float2 a = *reinterpret_cast<const float2*>(p + 4 * i);
          const float2 c = *reinterpret_cast<const float2*>(p + 4 * i + 8);
          x[i] = a.x; x[i + 1] = a.y; x[i + 2] = c.x; x[i + 3] = c.y;
        }
      }
      if constexpr (HAD) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if ((signs_c >> i) & 1u) x[i] = -x[i];
        fwht32_local(x);
        const float hc = hadamard_norm();
#pragma unroll
        for (int i = 0; i < 32; ++i) x[i] = x[i] * hc;
      }
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < B; ++i) m = fmaxf(m, fabsf(x[i]));
      float rcp;
      sb[bb] = block_scale<FMT>(m, sg, rcp);
      const int64_t col0 = c0 + half * 64 + bb * B;
#pragma unroll
      for (int g = 0; g < B / 8; ++g) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = x[8 * g + i] * rcp;
        if constexpr (RC == 0) {
          w[bb * (B / 8) + g] = e2m1_rtn_pack8(v);
        } else {
          uint32_t h[4];
          sr_draws8(seed_c, (off_c + (uint64_t)rgl * (uint64_t)C + (uint64_t)col0) / 8 + g, h);
          w[bb * (B / 8) + g] = e2m1_sr_pack8(v, h);
        }
      }
    }
    if (row < rows_here && half * 64 < cols_here) {
      uint8_t* dst = codes_c + rgl * (C / 2) + (c0 + half * 64) / 2;
      const bool full = half * 64 + 64 <= cols_here;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (full || (half * 64 + 16 * k) < cols_here)
          *reinterpret_cast<uint2*>(dst + 8 * k) = make_uint2(w[2 * k], w[2 * k + 1]);
      uint8_t* sdst = scales_c + rgl * (C / B) + (c0 + half * 64) / B;
      if (scale_words_c && full) {
        if constexpr (NBT == 4) *reinterpret_cast<uint32_t*>(sdst) = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
        else *reinterpret_cast<uint16_t*>(sdst) = (uint16_t)(sb[0] | (sb[1] << 8));
      } else {
#pragma unroll
        for (int bb = 0; bb < NBT; ++bb)
          if (half * 64 + bb * B < cols_here) sdst[bb] = (uint8_t)sb[bb];
      }
    }
  }
  __syncthreads();

  // write out (a): output row c0 + cl gets T/2 code bytes (8-byte pieces) and NB scale bytes.
#pragma unroll
  for (int k = 0; k < T * (T / 16) / 256; ++k) {
    const int idx = k * 256 + tid;
    const int cl = idx / (T / 16);
    const int seg = idx % (T / 16);
    if (cl < cols_here && seg * 16 < rows_here) {
      const uint32_t* sp = reinterpret_cast<const uint32_t*>(&stage_c[cl * SP + seg * 8]);
      *reinterpret_cast<uint2*>(codes_r + (c0 + cl) * (R / 2) + r0 / 2 + seg * 8) = make_uint2(sp[0], sp[1]);
    }
  }
  if (scale_words_r) {
    // (R / B) % 4 == 0: 4-byte words, NB / 4 per output row.
    constexpr int WPR = NB / 4;
    if (tid < T * WPR) {
      const int cl = tid / WPR;
      const int wd = tid % WPR;
      if (cl < cols_here && wd * 4 * B < rows_here)
        *reinterpret_cast<uint32_t*>(scales_r + (c0 + cl) * (R / B) + r0 / B + wd * 4) =
            *reinterpret_cast<const uint32_t*>(&stage_s[cl * NB + wd * 4]);
    }
  } else {
#pragma unroll
    for (int k = 0; k < (T * NB + 255) / 256; ++k) {
      const int idx = k * 256 + tid;
      const int cl = idx / NB;
      const int bb = idx % NB;
      if (idx < T * NB && cl < cols_here && bb * B < rows_here)
        scales_r[(c0 + cl) * (R / B) + r0 / B + bb] = stage_s[idx];
    }
  }
}

template <int FMT, bool BF16OUT>
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* __restrict__ codes,
                                                  const uint8_t* __restrict__ scales,
                                                  const float* __restrict__ tscale, int64_t cols,
                                                  uint32_t spr, uint32_t ntasks, void* dst, int64_t ld) {
  constexpr int B = FMT == NV ? 16 : 32;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) >> 6;
  const uint32_t nwaves = gridDim.x * 4u;
  const float sg = (FMT == NV) ? *tscale : 1.0f;
  for (uint32_t t = wave; t < ntasks; t += nwaves) {
    const uint32_t tu = __builtin_amdgcn_readfirstlane(t);
    const uint32_t r = tu / spr;
    const uint32_t seg = tu - r * spr;
    const int64_t col = (int64_t)seg * 512 + lane * 8;
    if (col >= cols) continue;
    const uint32_t w = *reinterpret_cast<const uint32_t*>(codes + (int64_t)r * (cols / 2) + col / 2);
    const uint32_t sb = scales[(int64_t)r * (cols / B) + col / B];
    float y[8];
    {
      auto q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
      auto q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
      auto q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
      auto q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
      y[0] = q0[0]; y[1] = q0[1]; y[2] = q1[0]; y[3] = q1[1];
      y[4] = q2[0]; y[5] = q2[1]; y[6] = q3[0]; y[7] = q3[1];
    }
    if constexpr (FMT == NV) {
      const float sdec = e4m3_decode(sb);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = (y[i] * sdec) * sg;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] = __builtin_ldexpf(y[i], (int)sb - 127);
    }
    if constexpr (BF16OUT) {
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t a = __float_as_uint(y[2 * i]), b = __float_as_uint(y[2 * i + 1]);
        a = (a + 0x7FFFu + ((a >> 16) & 1u)) >> 16;
        b = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
        o[i] = a | (b << 16);
      }
      *reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst) + (int64_t)r * ld + col) =
          make_uint4(o[0], o[1], o[2], o[3]);
    } else {
      float* d = static_cast<float*>(dst) + (int64_t)r * ld + col;
      reinterpret_cast<float4*>(d)[0] = make_float4(y[0], y[1], y[2], y[3]);
      reinterpret_cast<float4*>(d)[1] = make_float4(y[4], y[5], y[6], y[7]);
    }
  }
}

constexpr uint32_t kMaxGrid = 256 * 16;

uint32_t strided_grid(uint64_t ntasks) {
  uint64_t wgs = (ntasks + 3) / 4;
  return (uint32_t)(wgs < kMaxGrid ? (wgs ? wgs : 1) : kMaxGrid);
}

template <int FMT, int RND, bool BF16, bool HAD>
void launch_cols(const QuantArgs& a, hipStream_t s) {
  const uint32_t spr = (uint32_t)((a.C + 511) / 512);
  const uint32_t ntasks = (uint32_t)(a.R * spr);
  hipLaunchKernelGGL((k_quant_cols<FMT, RND, BF16, HAD>), dim3(strided_grid(ntasks)), dim3(256), 0, s,
                     a.src, a.C, a.ld, spr, ntasks, a.codes, a.scales, a.amax, a.tscale, a.seed,
                     a.offset, a.signs);
}

template <int FMT, int RND, bool BF16, bool HAD>
void launch_rows(const QuantArgs& a, hipStream_t s) {
  constexpr int B = FMT == NV ? 16 : 32;
  const uint32_t tiles_c = (uint32_t)((a.C + 63) / 64);
  const uint32_t tiles_r = (uint32_t)((a.R + 255) / 256);
  const uint32_t scale_words = (a.R / B) % 4 == 0;
  hipLaunchKernelGGL((k_quant_rows<FMT, RND, BF16, HAD>), dim3(tiles_c * tiles_r), dim3(256), 0, s,
                     a.src, a.R, a.C, a.ld, tiles_c, a.codes, a.scales, a.amax, a.tscale, a.seed,
                     a.offset, a.signs, scale_words);
}

template <int FMT, int RND, bool BF16, bool HAD>
void launch_axis(const QuantArgs& a, hipStream_t s) {
  if (a.rows_axis)
    launch_rows<FMT, RND, BF16, HAD>(a, s);
  else
    launch_cols<FMT, RND, BF16, HAD>(a, s);
}

template <int FMT, int RND>
void launch_src(const QuantArgs& a, hipStream_t s) {
  if constexpr (FMT == MX) {
    if (a.had_on) {
      if (a.bf16) launch_axis<FMT, RND, true, true>(a, s);
      else launch_axis<FMT, RND, false, true>(a, s);
      return;
    }
  }
  if (a.bf16) launch_axis<FMT, RND, true, false>(a, s);
  else launch_axis<FMT, RND, false, false>(a, s);
}

template <int FMT, int RC, int RR, bool BF16, bool HAD>
void launch_dual(const DualArgs& a, hipStream_t s) {
  constexpr int B = FMT == NV ? 16 : 32;
  const uint32_t tiles_c = (uint32_t)((a.C + 127) / 128);
  const uint32_t tiles_r = (uint32_t)((a.R + 127) / 128);
  // Scale bytes of a tile go out as words when every row start keeps them aligned.
  const uint32_t words_c = FMT == NV ? (a.C / B) % 4 == 0 : (a.C / B) % 2 == 0;
  const uint32_t words_r = (a.R / B) % 4 == 0;
  hipLaunchKernelGGL((k_quant_dual<FMT, RC, RR, BF16, HAD>), dim3(tiles_c * tiles_r), dim3(256), 0, s,
                     a.src, a.R, a.C, a.ld, tiles_c, a.codes_c, a.scales_c, a.codes_r, a.scales_r,
                     a.amax, a.tscale_c, a.tscale_r, a.amax_r, a.seed_c, a.offset_c, a.signs_c,
                     a.seed_r, a.offset_r, a.signs_r, words_c, words_r);
}

template <int FMT, bool BF16, bool HAD>
void launch_dual_rnd(const DualArgs& a, hipStream_t s) {
  if (a.sr_c) {
    if (a.sr_r) launch_dual<FMT, 1, 1, BF16, HAD>(a, s);
    else launch_dual<FMT, 1, 0, BF16, HAD>(a, s);
  } else {
    if (a.sr_r) launch_dual<FMT, 0, 1, BF16, HAD>(a, s);
    else launch_dual<FMT, 0, 0, BF16, HAD>(a, s);
  }
}

}  // namespace

void fp4i_launch_quant_dual(const DualArgs& a, hipStream_t s) {
  if (a.fmt == NV) {
    if (a.bf16) launch_dual_rnd<NV, true, false>(a, s);
    else launch_dual_rnd<NV, false, false>(a, s);
  } else if (a.had_on) {
    if (a.bf16) launch_dual_rnd<MX, true, true>(a, s);
    else launch_dual_rnd<MX, false, true>(a, s);
  } else {
    if (a.bf16) launch_dual_rnd<MX, true, false>(a, s);
    else launch_dual_rnd<MX, false, false>(a, s);
  }
}

void fp4i_launch_amax(const void* src, bool bf16, int64_t R, int64_t C, int64_t ld, float* amax,
                      hipStream_t s) {
  hipLaunchKernelGGL(k_zero1, dim3(1), dim3(1), 0, s, amax);
  const uint32_t spr = (uint32_t)((C + 2047) / 2048);
  const uint32_t ntasks = (uint32_t)(R * spr);
  if (bf16)
    hipLaunchKernelGGL(k_amax<true>, dim3(strided_grid(ntasks)), dim3(256), 0, s, src, C, ld, spr,
                       ntasks, amax);
  else
    hipLaunchKernelGGL(k_amax<false>, dim3(strided_grid(ntasks)), dim3(256), 0, s, src, C, ld, spr,
                       ntasks, amax);
}

void fp4i_launch_quant(const QuantArgs& a, hipStream_t s) {
  if (a.fmt == NV) {
    if (a.sr) launch_src<NV, 1>(a, s);
    else launch_src<NV, 0>(a, s);
  } else {
    if (a.sr) launch_src<MX, 1>(a, s);
    else launch_src<MX, 0>(a, s);
  }
}

void fp4i_launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* tscale, int fmt,
                         int64_t rows, int64_t cols, bool bf16out, void* dst, int64_t ld,
                         hipStream_t s) {
  const uint32_t spr = (uint32_t)((cols + 511) / 512);
  const uint32_t ntasks = (uint32_t)(rows * spr);
  const dim3 g(strided_grid(ntasks)), b(256);
  if (fmt == NV) {
    if (bf16out) hipLaunchKernelGGL((k_dequant<NV, true>), g, b, 0, s, codes, scales, tscale, cols, spr, ntasks, dst, ld);
    else hipLaunchKernelGGL((k_dequant<NV, false>), g, b, 0, s, codes, scales, tscale, cols, spr, ntasks, dst, ld);
  } else {
    if (bf16out) hipLaunchKernelGGL((k_dequant<MX, true>), g, b, 0, s, codes, scales, tscale, cols, spr, ntasks, dst, ld);
    else hipLaunchKernelGGL((k_dequant<MX, false>), g, b, 0, s, codes, scales, tscale, cols, spr, ntasks, dst, ld);
  }
}
