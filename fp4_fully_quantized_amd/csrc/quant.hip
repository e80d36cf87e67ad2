// quant.hip -- tensor amax, block-scaled FP4 quantize (both axes) and dequantize
// for gfx950.
//
// What is computed (Robots Atlas, "FP4", How it works and Components; FP4 All
// the Way, Key points; Quartet, Approach):
//   NVFP4  s_g = amax/2688; per 16-block byte = E4M3_rne((amax_b/6)/s_g),
//          r = 1/(sdec*s_g); codes = E2M1(x*r)
//   MXFP4  per 32-block e = the smallest e with 6*2^e >= amax_b;
//          codes = E2M1(x*2^-e)
//   optional random-sign Hadamard rotation of each block first (32-wide for
//   MXFP4, 16-wide for NVFP4, whose tensor amax is then the rotated values')
//   RTN or SR (16-bit Philox4x32-10 draws keyed by seed and element index).
//
// Memory-bound passes: every element is read once from HBM with 16-byte loads
// and written once as a nibble; block scales are one byte per block.
//  * k_amax        wave-strided 16-byte loads, per-lane max, wave and workgroup
//                  reduction, an atomicMax on the float bits by each
//                  workgroup whose max exceeds the value read there;
//                  optionally of the 16-wide rotated values along rows (pairs
//                  of lanes hold a block: one DPP butterfly stage).
//  * k_amax_rot_rows  the same for the rotation down columns: each lane reads
//                  16 rows x 8 columns and rotates each column in registers.
//  * k_quant_cols  blocks along the contiguous axis: each lane owns one whole
//                  block (16 or 32 consecutive elements, 2-8 16-byte loads),
//                  so the rotation's stages, the block amax and the block
//                  scale run in registers without cross-lane traffic; each
//                  lane stores its block's codes (8 or 16 bytes) and scale.
//  * k_quant_rows  blocks along rows (the transposed orientation used by dgrad
//                  and wgrad operands): a 256 x 64 tile is loaded with
//                  coalesced 16-byte row loads into LDS (input format), each
//                  thread quantizes one block in each of 2 or 4 adjacent
//                  columns, and the codes leave through an LDS staging area
//                  in whole 128-byte lines.
//  * k_dequant     8 elements per lane.
//  * k_dequant_unrot  one block per lane, then the inverse block rotation.
// Both orientations from one read are in quant_dual.hip.
#include "fp4_internal.hpp"
#include "quant_common.hpp"

using namespace fp4q;

namespace {

__global__ void k_zero1(float* p) { *p = 0.0f; }

// The monitor's ratio ||g|| / ||Q(g) - g|| from its two FP64 sums.
__global__ void k_noise_ratio(const double* __restrict__ noise, double* __restrict__ ratio) {
  const double g = noise[0], e = noise[1];
  *ratio = e > 0.0 ? sqrt(g / e) : (g > 0.0 ? __builtin_inf() : 0.0);
}

// The 16-wide rotation of 8 elements per lane, lanes 2j and 2j+1 holding one
// block (elements 0..7 and 8..15): signs, stages 1, 2, 4 in registers, stage
// 8 across the lane pair, times 1/4. Every lane of the wave must take part.
__device__ __forceinline__ void hadamard16_lane_pair(float x[8], uint32_t signs, int upper) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    if ((signs >> (8 * upper + i)) & 1u) x[i] = -x[i];
  fwht8_local(x);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = dpp_xor1(x[i]);
    x[i] = upper ? p - x[i] : x[i] + p;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = x[i] * 0.25f;
}

// Wave and workgroup max of m >= 0, then at most one atomicMax per workgroup
// on the float bits (monotone for non-negative floats). The value at *amax
// only grows, so a workgroup whose max does not exceed a value read from it
// has nothing to add: reading first skips nearly all of the same-address
// atomics, which the L2 serializes (with one per workgroup they set a floor
// of about 30 us under every amax pass).
__device__ __forceinline__ void amax_reduce(float m, float* amax) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float part[4];
  if (lane == 0) part[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float b = fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]));
    unsigned int* const a = reinterpret_cast<unsigned int*>(amax);
    if (__float_as_uint(b) > __atomic_load_n(a, __ATOMIC_RELAXED)) atomicMax(a, __float_as_uint(b));
  }
}

// A wave task is a 2048-element segment of one row: each lane issues four
// independent 16-byte (bf16) loads before reducing, to keep enough bytes in
// flight per CU. ROT: the amax of the values rotated 16-wide along the row
// (C % 16 == 0, so both lanes of a block are in or out of range together).
template <bool BF16, bool ROT>
__global__ __launch_bounds__(256) void k_amax(const void* __restrict__ src, int64_t C, int64_t ld,
                                               uint32_t spr, uint32_t ntasks, uint32_t signs,
                                               float* amax) {
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
    if constexpr (ROT) {
#pragma unroll
      for (int k = 0; k < 4; ++k) hadamard16_lane_pair(x[k], signs, lane & 1);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
#pragma unroll
      for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[k][i]));
  }
  amax_reduce(m, amax);
}

// Tensor amax of a contiguous source (ld == C): one flat grid-strided pass
// over its 16-byte pieces with four nontemporal loads in flight per lane, the
// maximum taken on the magnitude bits (|x| of a finite float, bf16 or fp32,
// orders as its bit pattern with the sign cleared, an unsigned integer): bf16
// pairs by a packed 16-bit unsigned max, fp32 by a 32-bit one; exact.
template <bool BF16>
__global__ __launch_bounds__(256) void k_amax_flat(const v4u* __restrict__ src, uint64_t n16, float* amax) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const uint32_t mag = BF16 ? 0x7FFF7FFFu : 0x7FFFFFFFu;
  uint32_t m0 = 0, m1 = 0;
  typedef unsigned short v2us __attribute__((ext_vector_type(2)));
  v2us p0 = {0, 0}, p1 = {0, 0};
  auto take = [&](v4u v) {
    if constexpr (BF16) {
      p0 = __builtin_elementwise_max(p0, __builtin_bit_cast(v2us, v.x & mag));
      p1 = __builtin_elementwise_max(p1, __builtin_bit_cast(v2us, v.y & mag));
      p0 = __builtin_elementwise_max(p0, __builtin_bit_cast(v2us, v.z & mag));
      p1 = __builtin_elementwise_max(p1, __builtin_bit_cast(v2us, v.w & mag));
    } else {
      m0 = max(m0, max(v.x & mag, v.y & mag));
      m1 = max(m1, max(v.z & mag, v.w & mag));
    }
  };
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4u x0 = __builtin_nontemporal_load(src + i);
    const v4u x1 = __builtin_nontemporal_load(src + i + stride);
    const v4u x2 = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4u x3 = __builtin_nontemporal_load(src + i + 3 * stride);
    take(x0);
    take(x1);
    take(x2);
    take(x3);
  }
  for (; i < n16; i += stride) take(__builtin_nontemporal_load(src + i));
  float m;
  if constexpr (BF16) {
    const v2us q = __builtin_elementwise_max(p0, p1);
    m = __uint_as_float((uint32_t)max(q.x, q.y) << 16);
  } else {
    m = __uint_as_float(max(m0, m1));
  }
  amax_reduce(m, amax);
}

// The amax of the values rotated 16-wide down the columns (R % 16 == 0). A
// wave task is a band of 16 rows by 512 columns: each lane loads 16 rows of
// its 8 columns (coalesced 16-byte loads, 1 KiB per row per wave for bf16)
// and rotates each column in registers.
template <bool BF16>
__global__ __launch_bounds__(256) void k_amax_rot_rows(const void* __restrict__ src, int64_t C,
                                                        int64_t ld, uint32_t spr, uint32_t ntasks,
                                                        uint32_t signs, float* amax) {
  constexpr int ES = BF16 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) >> 6;
  const uint32_t nwaves = gridDim.x * 4u;
  float m = 0.0f;
  for (uint32_t t = wave; t < ntasks; t += nwaves) {
    const uint32_t tu = __builtin_amdgcn_readfirstlane(t);
    const uint32_t band = tu / spr;
    const uint32_t seg = tu - band * spr;
    const int64_t col = (int64_t)seg * 512 + lane * 8;
    if (col < C) {
      const char* base = static_cast<const char*>(src) + ((int64_t)band * 16 * ld + col) * ES;
      float x[16][8];
#pragma unroll
      for (int i = 0; i < 16; ++i) load8<BF16>(base + (int64_t)i * ld * ES, x[i]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = x[i][j];
        hadamard_block<16>(v, signs);
#pragma unroll
        for (int i = 0; i < 16; ++i) m = fmaxf(m, fabsf(v[i]));
      }
    }
  }
  amax_reduce(m, amax);
}


// Blocks along the contiguous axis: every lane owns one whole block (16 or 32
// consecutive elements of a row), a wave 64 consecutive blocks of one row (a
// task). The lane loads its block with 16-byte loads (a wave reads one
// contiguous 2 or 4 KiB run of bf16), applies the rotation's signs while the
// values are still packed (one XOR flips two bf16 elements), runs every
// butterfly stage and the block amax in registers, derives the block scale
// once per block, and stores its codes (8 or 16 bytes) and its scale byte.
template <int FMT, int RND, bool BF16, bool HAD, bool MON>
__global__ __launch_bounds__(256) void k_quant_cols(const void* __restrict__ src, int64_t C, int64_t ld,
                                                     uint32_t spr, uint32_t ntasks,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     const float* __restrict__ amax, float* tscale,
                                                     uint64_t seed, uint64_t offset, uint32_t signs,
                                                     double* noise) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int B = FMT == NV ? 16 : 32;
  constexpr int LOADS = B * ES / 16;   // 16-byte loads per block
  const int lane = threadIdx.x & 63;
  double ng = 0.0, ne = 0.0;
  const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) >> 6;
  const uint32_t nwaves = gridDim.x * 4u;
  float sg = 1.0f;
  __shared__ float rtab[128];   // NVFP4 element multipliers per scale byte
  if constexpr (FMT == NV) {
    sg = nv_tensor_scale(*amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) *tscale = sg;
    nv_rcp_table(rtab, sg);
    __syncthreads();
  }
  for (uint32_t t = wave; t < ntasks; t += nwaves) {
    const uint32_t tu = __builtin_amdgcn_readfirstlane(t);
    const uint32_t r = tu / spr;
    const uint32_t seg = tu - r * spr;
    const int64_t col = ((int64_t)seg * 64 + lane) * B;   // first element of this lane's block
    if (col >= C) continue;
    const char* p = static_cast<const char*>(src) + ((int64_t)r * ld + col) * ES;
    float x[B];
#pragma unroll
    for (int k = 0; k < LOADS; ++k) {
      uint4 w = reinterpret_cast<const uint4*>(p)[k];
      if constexpr (BF16) {
        uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 8 * k + 2 * j;   // element of u[j]'s low half
          if constexpr (HAD)             // negate x_e, x_e+1 where the mask says so
            u[j] ^= (((signs >> e) & 1u) << 15) | (((signs >> (e + 1)) & 1u) << 31);
          x[e] = bf16_lo(u[j]);
          x[e + 1] = bf16_hi(u[j]);
        }
      } else {
        uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * k + j;
          if constexpr (HAD) u[j] ^= ((signs >> e) & 1u) << 31;
          x[e] = __uint_as_float(u[j]);
        }
      }
    }
    if constexpr (HAD) fwht_block<B>(x);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < B; ++i) m = fmaxf(m, fabsf(x[i]));
    float rcp;
    const uint32_t sbyte = block_scale_tab<FMT>(m, sg, rtab, rcp);
    uint32_t w[B / 8];
#pragma unroll
    for (int g = 0; g < B / 8; ++g) {
      float v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = x[8 * g + i] * rcp;
      if constexpr (RND == 0) {
        w[g] = e2m1_rtn_pack8(v);
      } else {
        uint32_t h[4];
        sr_draws8(seed, (offset + (uint64_t)r * (uint64_t)C + (uint64_t)col) / 8 + g, h);
        w[g] = e2m1_sr_pack8(v, h);
      }
    }
    uint8_t* dst = codes + (int64_t)r * (C / 2) + col / 2;
    if constexpr (B == 16) *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
    else *reinterpret_cast<uint4*>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    scales[(int64_t)r * (C / B) + col / B] = (uint8_t)sbyte;
    if constexpr (MON) {
      float g = 0.0f, e = 0.0f;
      const float bs = scale_value<FMT>(sbyte);
#pragma unroll
      for (int k = 0; k < B / 8; ++k) noise8<FMT>(x + 8 * k, w[k], bs, sg, g, e);
      ng += (double)g;
      ne += (double)e;
    }
  }
  if constexpr (MON) noise_reduce(ng, ne, noise);
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
template <int FMT, int RND, bool BF16, bool HAD, bool MON>
__global__ __launch_bounds__(256) void k_quant_rows(const void* __restrict__ src, int64_t R, int64_t C,
                                                     int64_t ld, uint32_t tiles_c, uint32_t ntiles,
                                                     uint8_t* __restrict__ codes,
                                                     uint8_t* __restrict__ scales,
                                                     const float* __restrict__ amax, float* tscale,
                                                     uint64_t seed, uint64_t offset, uint64_t idx_rows,
                                                     uint32_t signs, uint32_t scale_words, double* noise) {
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
  __shared__ float rtab[128];   // NVFP4 element multipliers (published by the tile load's barrier)
  if constexpr (FMT == NV) {
    sg = nv_tensor_scale(*amax);
    if (blockIdx.x == 0 && threadIdx.x == 0) *tscale = sg;
    nv_rcp_table(rtab, sg);
  }
  double ng = 0.0, ne = 0.0;  // quantization noise, when asked for
  // One tile per workgroup; with the noise monitor (MON) a capped grid loops
  // over the tiles.
  const uint32_t n_it = MON ? (ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x : 1u;
  for (uint32_t it = 0; it < n_it; ++it) {
    const uint32_t ti = blockIdx.x + it * gridDim.x;
    const uint32_t tr = ti / tiles_c;
    const uint32_t tc = ti - tr * tiles_c;
    const int64_t r0 = (int64_t)tr * TR;
    const int64_t c0 = (int64_t)tc * TC;
    // With the monitor's tile loop, the thread index through an opaque move in
    // each iteration: otherwise the compiler hoists the thread-dependent
    // addresses out of the loop and keeps them live across it. (Without the
    // loop the plain index lets it use what it knows of the index's range.)
    int tid = threadIdx.x;
    if constexpr (MON) asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"((int)threadIdx.x));

    // 1. tile load: TR rows of TC * ES bytes, 16 bytes per load; only edge
    //    tiles check bounds.
    constexpr int CPR = TC * ES / 16;
    if (r0 + TR <= R && c0 + TC <= C) {
#pragma unroll
      for (int k = 0; k < TR * CPR / 256; ++k) {
        const int idx = k * 256 + tid;
        const int rr = idx / CPR;
        const int cc = idx % CPR;
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const char*>(src) +
                                                        ((r0 + rr) * ld + c0 + cc * (16 / ES)) * ES);
        uint32_t* d = reinterpret_cast<uint32_t*>(&tile[rr * PITCH + cc * 16]);
        d[0] = v.x; d[1] = v.y; d[2] = v.z; d[3] = v.w;
      }
    } else {
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
      if constexpr (HAD) hadamard_block<B>(xk, signs);
      float m = 0.0f;
#pragma unroll
      for (int i = 0; i < B; ++i) m = fmaxf(m, fabsf(xk[i]));
      float rcp;
      const uint32_t sbyte = block_scale_tab<FMT>(m, sg, rtab, rcp);
      uint32_t* sc = reinterpret_cast<uint32_t*>(&stage_c[cl * SP + b * (B / 2)]);
      float bg = 0.0f, be = 0.0f;
      const float bs = MON ? scale_value<FMT>(sbyte) : 0.0f;
#pragma unroll
      for (int g = 0; g < B / 8; ++g) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = xk[8 * g + i] * rcp;
        uint32_t cw;
        if constexpr (RND == 0) {
          cw = e2m1_rtn_pack8(v);
        } else {
          uint32_t h[4];
          sr_draws8(seed, (offset + (uint64_t)cg * idx_rows + (uint64_t)rg) / 8 + g, h);
          cw = e2m1_sr_pack8(v, h);
        }
        sc[g] = cw;
        if constexpr (MON) noise8<FMT>(xk + 8 * g, cw, bs, sg, bg, be);
      }
      stage_s[cl * NB + b] = (uint8_t)sbyte;
      ng += (double)bg;
      ne += (double)be;
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
    if constexpr (MON) __syncthreads();  // the next tile reuses the LDS buffers
  }
  if constexpr (MON) noise_reduce(ng, ne, noise);
}

// Both orientations' tensor amaxes from one read, for a dual quantization with
// a rotation on at least one side (R % 16 == 0, C % 16 == 0): the values
// blocked along C (rotated 16-wide along the row when HC) and the values
// blocked along R (rotated 16-wide down the column when HR). A wave task is a
// band of 16 rows by 512 columns, each lane holding 16 rows of 8 columns: a
// row's 16-block sits in a lane pair, a column's in one lane.
template <bool BF16, bool HC, bool HR>
__global__ __launch_bounds__(256) void k_amax_pair(const void* __restrict__ src, int64_t C, int64_t ld,
                                                    uint32_t spr, uint32_t ntasks, uint32_t signs_c,
                                                    uint32_t signs_r, float* amax_c, float* amax_r) {
  constexpr int ES = BF16 ? 2 : 4;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = (blockIdx.x * 256u + threadIdx.x) >> 6;
  const uint32_t nwaves = gridDim.x * 4u;
  float mc = 0.0f, mr = 0.0f;
  for (uint32_t t = wave; t < ntasks; t += nwaves) {
    const uint32_t tu = __builtin_amdgcn_readfirstlane(t);
    const uint32_t band = tu / spr;
    const uint32_t seg = tu - band * spr;
    const int64_t col = (int64_t)seg * 512 + lane * 8;
    const char* base = static_cast<const char*>(src) + ((int64_t)band * 16 * ld + col) * ES;
    float x[16][8];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (col < C) load8<BF16>(base + (int64_t)i * ld * ES, x[i]);
      else
#pragma unroll
        for (int j = 0; j < 8; ++j) x[i][j] = 0.0f;
    }
    // blocks along C (all lanes take part in the lane-pair exchange)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float w[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) w[j] = x[i][j];
      if constexpr (HC) hadamard16_lane_pair(w, signs_c, lane & 1);
#pragma unroll
      for (int j = 0; j < 8; ++j) mc = fmaxf(mc, fabsf(w[j]));
    }
    // blocks along R
    if constexpr (HR) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float v[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = x[i][j];
        hadamard_block<16>(v, signs_r);
#pragma unroll
        for (int i = 0; i < 16; ++i) mr = fmaxf(mr, fabsf(v[i]));
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) mr = fmaxf(mr, fabsf(x[i][j]));
    }
  }
  amax_reduce(mc, amax_c);
  __syncthreads();
  amax_reduce(mr, amax_r);
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

// Dequantize and undo the quantization's block rotation: one block per lane
// (16 or 32 values), decoded as k_dequant does, then the FWHT stages and the
// normalisation (fwht_block) and the signs: D H c, the transpose of the
// rotation c H D.
template <int FMT, bool BF16OUT>
__global__ __launch_bounds__(256) void k_dequant_unrot(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        const float* __restrict__ tscale, int64_t cols,
                                                        uint64_t nblocks, uint32_t signs, void* dst,
                                                        int64_t ld) {
  constexpr int B = FMT == NV ? 16 : 32;
  const int64_t bpr = cols / B;
  const float sg = (FMT == NV) ? *tscale : 1.0f;
  for (uint64_t blk = (uint64_t)blockIdx.x * 256u + threadIdx.x; blk < nblocks;
       blk += (uint64_t)gridDim.x * 256u) {
    const int64_t r = (int64_t)(blk / (uint64_t)bpr);
    const int64_t cb = (int64_t)blk - r * bpr;
    const uint8_t* cp = codes + r * (cols / 2) + cb * (B / 2);
    uint32_t w[B / 8];
    if constexpr (B == 16) {
      const uint2 v = *reinterpret_cast<const uint2*>(cp);
      w[0] = v.x; w[1] = v.y;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(cp);
      w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    }
    const uint32_t sb = scales[r * bpr + cb];
    float x[B];
#pragma unroll
    for (int g = 0; g < B / 8; ++g) {
      const auto q0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[g], 1.0f, 0);
      const auto q1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[g], 1.0f, 1);
      const auto q2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[g], 1.0f, 2);
      const auto q3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[g], 1.0f, 3);
      x[8 * g + 0] = q0[0]; x[8 * g + 1] = q0[1]; x[8 * g + 2] = q1[0]; x[8 * g + 3] = q1[1];
      x[8 * g + 4] = q2[0]; x[8 * g + 5] = q2[1]; x[8 * g + 6] = q3[0]; x[8 * g + 7] = q3[1];
    }
    if constexpr (FMT == NV) {
      const float sdec = e4m3_decode(sb);
#pragma unroll
      for (int i = 0; i < B; ++i) x[i] = (x[i] * sdec) * sg;
    } else {
#pragma unroll
      for (int i = 0; i < B; ++i) x[i] = __builtin_ldexpf(x[i], (int)sb - 127);
    }
    fwht_block<B>(x);
#pragma unroll
    for (int i = 0; i < B; ++i)
      if ((signs >> i) & 1u) x[i] = -x[i];
    if constexpr (BF16OUT) {
      uint32_t o[B / 2];
#pragma unroll
      for (int i = 0; i < B / 2; ++i) {
        uint32_t a = __float_as_uint(x[2 * i]), b = __float_as_uint(x[2 * i + 1]);
        a = (a + 0x7FFFu + ((a >> 16) & 1u)) >> 16;
        b = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
        o[i] = a | (b << 16);
      }
      uint4* d = reinterpret_cast<uint4*>(static_cast<uint16_t*>(dst) + r * ld + cb * B);
#pragma unroll
      for (int i = 0; i < B / 8; ++i) d[i] = make_uint4(o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]);
    } else {
      float4* d = reinterpret_cast<float4*>(static_cast<float*>(dst) + r * ld + cb * B);
#pragma unroll
      for (int i = 0; i < B / 4; ++i) d[i] = make_float4(x[4 * i], x[4 * i + 1], x[4 * i + 2], x[4 * i + 3]);
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
  // A task is 64 blocks of one row (one block per lane).
  const int64_t per_task = 64 * (FMT == NV ? 16 : 32);
  const uint32_t spr = (uint32_t)((a.C + per_task - 1) / per_task);
  const uint32_t ntasks = (uint32_t)(a.R * spr);
  uint32_t grid = strided_grid(ntasks);
  if (a.noise) grid = noise_grid(k_quant_cols<FMT, RND, BF16, HAD, true>, grid);
  if (a.noise)
    hipLaunchKernelGGL((k_quant_cols<FMT, RND, BF16, HAD, true>), dim3(grid), dim3(256), 0, s,
                       a.src, a.C, a.ld, spr, ntasks, a.codes, a.scales, a.amax, a.tscale, a.seed,
                       a.offset, a.signs, a.noise);
  else
    hipLaunchKernelGGL((k_quant_cols<FMT, RND, BF16, HAD, false>), dim3(grid), dim3(256), 0, s,
                       a.src, a.C, a.ld, spr, ntasks, a.codes, a.scales, a.amax, a.tscale, a.seed,
                       a.offset, a.signs, nullptr);
}

template <int FMT, int RND, bool BF16, bool HAD, bool MON>
void launch_rows_mon(const QuantArgs& a, hipStream_t s) {
  constexpr int B = FMT == NV ? 16 : 32;
  const uint32_t tiles_c = (uint32_t)((a.C + 63) / 64);
  const uint32_t tiles_r = (uint32_t)((a.R + 255) / 256);
  const uint32_t scale_words = (a.R / B) % 4 == 0;
  const uint32_t ntiles = tiles_c * tiles_r;
  const uint32_t grid = MON ? noise_grid(k_quant_rows<FMT, RND, BF16, HAD, MON>, ntiles) : ntiles;
  hipLaunchKernelGGL((k_quant_rows<FMT, RND, BF16, HAD, MON>), dim3(grid), dim3(256), 0, s, a.src, a.R,
                     a.C, a.ld, tiles_c, ntiles, a.codes, a.scales, a.amax, a.tscale, a.seed, a.offset,
                     (uint64_t)(a.idx_rows ? a.idx_rows : a.R), a.signs, scale_words, a.noise);
}

template <int FMT, int RND, bool BF16, bool HAD>
void launch_rows(const QuantArgs& a, hipStream_t s) {
  if (a.noise) launch_rows_mon<FMT, RND, BF16, HAD, true>(a, s);
  else launch_rows_mon<FMT, RND, BF16, HAD, false>(a, s);
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
  if (a.had_on) {
    if (a.bf16) launch_axis<FMT, RND, true, true>(a, s);
    else launch_axis<FMT, RND, false, true>(a, s);
  } else {
    if (a.bf16) launch_axis<FMT, RND, true, false>(a, s);
    else launch_axis<FMT, RND, false, false>(a, s);
  }
}

}  // namespace


void fp4i_launch_amax(const void* src, bool bf16, int64_t R, int64_t C, int64_t ld, float* amax,
                      hipStream_t s) {
  hipLaunchKernelGGL(k_zero1, dim3(1), dim3(1), 0, s, amax);
  if (ld == C) {
    // Contiguous: one flat pass (16-byte pieces; C % 8 == 0 makes R * C * ES a
    // multiple of 16). At most 512 workgroups (two per CU), each looping over
    // many pieces: every workgroup ends with a read (and possibly an atomic)
    // of the one amax word, which the L2 serializes, and larger grids measured
    // slower (Llama-7B X: 44 us at 512 workgroups, 48 at 1024, 73 at 8192; dY
    // 110, 132, 142 us), while 512 already keeps 6.1-6.6 TB/s of reads in
    // flight.
    const uint64_t n16 = (uint64_t)R * (uint64_t)C * (bf16 ? 2u : 4u) / 16u;
    const uint64_t want = (n16 + 256 * 4 - 1) / (256 * 4);
    const dim3 g((uint32_t)(want < 512 ? (want ? want : 1) : 512)), b(256);
    if (bf16) hipLaunchKernelGGL(k_amax_flat<true>, g, b, 0, s, static_cast<const v4u*>(src), n16, amax);
    else hipLaunchKernelGGL(k_amax_flat<false>, g, b, 0, s, static_cast<const v4u*>(src), n16, amax);
    return;
  }
  const uint32_t spr = (uint32_t)((C + 2047) / 2048);
  const uint32_t ntasks = (uint32_t)(R * spr);
  const dim3 g(strided_grid(ntasks)), b(256);
  if (bf16)
    hipLaunchKernelGGL((k_amax<true, false>), g, b, 0, s, src, C, ld, spr, ntasks, 0u, amax);
  else
    hipLaunchKernelGGL((k_amax<false, false>), g, b, 0, s, src, C, ld, spr, ntasks, 0u, amax);
}

void fp4i_launch_amax_rot16(const void* src, bool bf16, int64_t R, int64_t C, int64_t ld,
                            bool rows_axis, uint32_t signs, float* amax, hipStream_t s) {
  hipLaunchKernelGGL(k_zero1, dim3(1), dim3(1), 0, s, amax);
  if (rows_axis) {
    const uint32_t spr = (uint32_t)((C + 511) / 512);
    const uint32_t ntasks = (uint32_t)(R / 16 * spr);
    const dim3 g(strided_grid(ntasks)), b(256);
    if (bf16)
      hipLaunchKernelGGL((k_amax_rot_rows<true>), g, b, 0, s, src, C, ld, spr, ntasks, signs, amax);
    else
      hipLaunchKernelGGL((k_amax_rot_rows<false>), g, b, 0, s, src, C, ld, spr, ntasks, signs, amax);
  } else {
    const uint32_t spr = (uint32_t)((C + 2047) / 2048);
    const uint32_t ntasks = (uint32_t)(R * spr);
    const dim3 g(strided_grid(ntasks)), b(256);
    if (bf16)
      hipLaunchKernelGGL((k_amax<true, true>), g, b, 0, s, src, C, ld, spr, ntasks, signs, amax);
    else
      hipLaunchKernelGGL((k_amax<false, true>), g, b, 0, s, src, C, ld, spr, ntasks, signs, amax);
  }
}

void fp4i_launch_amax_pair(const void* src, bool bf16, int64_t R, int64_t C, int64_t ld, bool had_c,
                           uint32_t signs_c, bool had_r, uint32_t signs_r, float* amax_c,
                           float* amax_r, hipStream_t s) {
  hipLaunchKernelGGL(k_zero1, dim3(1), dim3(1), 0, s, amax_c);
  hipLaunchKernelGGL(k_zero1, dim3(1), dim3(1), 0, s, amax_r);
  const uint32_t spr = (uint32_t)((C + 511) / 512);
  const uint32_t ntasks = (uint32_t)(R / 16 * spr);
  const dim3 g(strided_grid(ntasks)), b(256);
#define FP4_AMAX_PAIR(BF, HC, HR)                                                                 \
  hipLaunchKernelGGL((k_amax_pair<BF, HC, HR>), g, b, 0, s, src, C, ld, spr, ntasks, signs_c, signs_r, \
                     amax_c, amax_r)
  if (bf16) {
    if (had_c && had_r) FP4_AMAX_PAIR(true, true, true);
    else if (had_c) FP4_AMAX_PAIR(true, true, false);
    else FP4_AMAX_PAIR(true, false, true);
  } else {
    if (had_c && had_r) FP4_AMAX_PAIR(false, true, true);
    else if (had_c) FP4_AMAX_PAIR(false, true, false);
    else FP4_AMAX_PAIR(false, false, true);
  }
#undef FP4_AMAX_PAIR
}

void fp4i_launch_noise_ratio(const double* noise, double* ratio, hipStream_t s) {
  hipLaunchKernelGGL(k_noise_ratio, dim3(1), dim3(1), 0, s, noise, ratio);
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

void fp4i_launch_dequant_unrot(const uint8_t* codes, const uint8_t* scales, const float* tscale, int fmt,
                               int64_t rows, int64_t cols, uint32_t signs, bool bf16out, void* dst,
                               int64_t ld, hipStream_t s) {
  const uint64_t nblocks = (uint64_t)rows * (uint64_t)(cols / (fmt == NV ? 16 : 32));
  const uint64_t wgs = (nblocks + 255) / 256;
  const dim3 g((uint32_t)(wgs < 8192 ? wgs : 8192)), b(256);
  if (fmt == NV) {
    if (bf16out) hipLaunchKernelGGL((k_dequant_unrot<NV, true>), g, b, 0, s, codes, scales, tscale, cols, nblocks, signs, dst, ld);
    else hipLaunchKernelGGL((k_dequant_unrot<NV, false>), g, b, 0, s, codes, scales, tscale, cols, nblocks, signs, dst, ld);
  } else {
    if (bf16out) hipLaunchKernelGGL((k_dequant_unrot<MX, true>), g, b, 0, s, codes, scales, tscale, cols, nblocks, signs, dst, ld);
    else hipLaunchKernelGGL((k_dequant_unrot<MX, false>), g, b, 0, s, codes, scales, tscale, cols, nblocks, signs, dst, ld);
  }
}
