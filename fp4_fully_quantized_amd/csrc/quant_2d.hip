// quant_2d.hip -- two-dimensional block quantization for gfx950 (Robots Atlas,
// "FP4", How it works: two-dimensional quantization): one scale per B x B
// block (16 x 16 NVFP4, 32 x 32 MXFP4), so that a weight matrix and its
// transpose are one quantization (the forward GEMM reads W blocked along K,
// dgrad reads the same values blocked along N).
//
// A workgroup takes a 128 x 128 tile of the source into LDS once, then
//  1. the block amaxes: NBT x NBT blocks, 256 / NBLK threads per block each
//     scanning 64 elements in LDS, a shuffle reduction, and the block's scale
//     byte and element multiplier into LDS;
//  2. thread (row, half) encodes 64 consecutive elements of one row with their
//     blocks' multipliers (RTN, or SR with the row-major element index),
//     writes the row-major codes and scale bytes directly, and leaves one code
//     per byte in a transposed LDS array;
//  3. the transposed output is packed from that array (two rows per byte) and
//     written in 8-byte pieces, with the blocks' bytes as its scales.
#include "fp4_internal.hpp"
#include "quant_common.hpp"

using namespace fp4q;

namespace {

template <int FMT, int RND, bool BF16>
__global__ __launch_bounds__(256) void k_quant_2d(
    const void* __restrict__ src, int64_t R, int64_t C, int64_t ld, uint32_t tiles_c,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, const float* __restrict__ amax, float* tscale, float* tscale_t,
    float* amax_copy, uint64_t seed, uint64_t offset, uint32_t scale_words_c, uint32_t scale_words_t) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int B = FMT == NV ? 16 : 32;
  constexpr int T = 128;                  // tile rows = tile columns
  constexpr int NBT = T / B;              // blocks per tile side
  constexpr int NBLK = NBT * NBT;         // blocks per tile
  constexpr int TPK = 256 / NBLK;         // threads per block in the amax step (4 or 16)
  constexpr int RPT = B / TPK;            // rows per thread in the amax step (4 or 2)
  constexpr int PITCH = T * ES + 16;      // source row pitch in LDS (bytes)
  constexpr int TP = T + 16;              // transposed code array pitch (bytes)
  __shared__ __attribute__((aligned(16))) uint8_t tile[T * PITCH];
  __shared__ __attribute__((aligned(16))) uint8_t tcodes[T * TP];
  __shared__ float blk_r[NBLK];
  __shared__ uint8_t blk_s[NBLK];

  float sg = 1.0f;
  if constexpr (FMT == NV) {
    const float a = *amax;
    sg = nv_tensor_scale(a);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *tscale = sg;
      *tscale_t = sg;
      if (amax_copy) *amax_copy = a;
    }
  }
  const uint32_t ti = xcd_contiguous_tile(blockIdx.x, gridDim.x);
  const uint32_t tr = ti / tiles_c;
  const uint32_t tc = ti - tr * tiles_c;
  const int64_t r0 = (int64_t)tr * T;
  const int64_t c0 = (int64_t)tc * T;
  const int tid = threadIdx.x;

  // 0. tile load, 16 bytes per load (zeros outside the matrix).
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
    *reinterpret_cast<uint4*>(&tile[rr * PITCH + cc * 16]) = v;
  }
  __syncthreads();

  const int64_t rows_here = R - r0 < T ? R - r0 : T;  // multiples of B
  const int64_t cols_here = C - c0 < T ? C - c0 : T;

  // 1. block amaxes -> scale bytes and element multipliers.
  {
    const int blk = tid / TPK;
    const int part = tid % TPK;
    const int br = blk / NBT, bc = blk % NBT;
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const uint8_t* p = &tile[(br * B + part * RPT + i) * PITCH + bc * B * ES];
#pragma unroll
      for (int j = 0; j < B * ES / 16; ++j) {
        const uint4 w = *reinterpret_cast<const uint4*>(p + 16 * j);
        if constexpr (BF16) {
          const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int k = 0; k < 4; ++k) m = fmaxf(m, fmaxf(fabsf(bf16_lo(u[k])), fabsf(bf16_hi(u[k]))));
        } else {
          m = fmaxf(m, fmaxf(fmaxf(fabsf(__uint_as_float(w.x)), fabsf(__uint_as_float(w.y))),
                             fmaxf(fabsf(__uint_as_float(w.z)), fabsf(__uint_as_float(w.w)))));
        }
      }
    }
#pragma unroll
    for (int off = 1; off < TPK; off <<= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    if (part == 0) {
      float rcp;
      blk_s[blk] = (uint8_t)block_scale<FMT>(m, sg, rcp);
      blk_r[blk] = rcp;
    }
  }
  __syncthreads();

  // 2. rows: row r0 + row, elements c0 + 64 * half .. + 63.
  {
    const int row = tid >> 1;
    const int half = tid & 1;
    const int64_t rgl = r0 + row;
    constexpr int NBR = 64 / B;  // blocks per thread
    uint32_t w[8];
    uint32_t sb[NBR];
#pragma unroll
    for (int bb = 0; bb < NBR; ++bb) {
      const int cl0 = half * 64 + bb * B;
      const int blk = (row / B) * NBT + cl0 / B;
      const float rcp = blk_r[blk];
      sb[bb] = blk_s[blk];
      const uint8_t* p = &tile[row * PITCH + cl0 * ES];
#pragma unroll
      for (int g = 0; g < B / 8; ++g) {
        float x[8];
        if constexpr (BF16) {
          const uint4 u = *reinterpret_cast<const uint4*>(p + 16 * g);
          x[0] = bf16_lo(u.x); x[1] = bf16_hi(u.x); x[2] = bf16_lo(u.y); x[3] = bf16_hi(u.y);
          x[4] = bf16_lo(u.z); x[5] = bf16_hi(u.z); x[6] = bf16_lo(u.w); x[7] = bf16_hi(u.w);
        } else {
          const float4 a = *reinterpret_cast<const float4*>(p + 32 * g);
          const float4 b = *reinterpret_cast<const float4*>(p + 32 * g + 16);
          x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
          x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        }
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = x[i] * rcp;
        uint32_t cw;
        if constexpr (RND == 0) {
          cw = e2m1_rtn_pack8(v);
        } else {
          uint32_t h[4];
          sr_draws8(seed, (offset + (uint64_t)rgl * (uint64_t)C + (uint64_t)(c0 + cl0 + 8 * g)) / 8, h);
          cw = e2m1_sr_pack8(v, h);
        }
        w[bb * (B / 8) + g] = cw;
#pragma unroll
        for (int i = 0; i < 8; ++i) tcodes[(cl0 + 8 * g + i) * TP + row] = (uint8_t)((cw >> (4 * i)) & 15u);
      }
    }
    if (row < rows_here && half * 64 < cols_here) {
      uint8_t* dst = codes + rgl * (C / 2) + (c0 + half * 64) / 2;
      const bool full = half * 64 + 64 <= cols_here;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (full || (half * 64 + 16 * k) < cols_here)
          *reinterpret_cast<uint2*>(dst + 8 * k) = make_uint2(w[2 * k], w[2 * k + 1]);
      uint8_t* sdst = scales + rgl * (C / B) + (c0 + half * 64) / B;
      if (scale_words_c && full) {
        if constexpr (NBR == 4) *reinterpret_cast<uint32_t*>(sdst) = sb[0] | (sb[1] << 8) | (sb[2] << 16) | (sb[3] << 24);
        else *reinterpret_cast<uint16_t*>(sdst) = (uint16_t)(sb[0] | (sb[1] << 8));
      } else {
#pragma unroll
        for (int bb = 0; bb < NBR; ++bb)
          if (half * 64 + bb * B < cols_here) sdst[bb] = (uint8_t)sb[bb];
      }
    }
  }
  __syncthreads();

  // 3. transposed output: row c0 + cl holds rows r0 .. of column cl, two per byte.
#pragma unroll
  for (int k = 0; k < T * (T / 16) / 256; ++k) {
    const int idx = k * 256 + tid;
    const int cl = idx / (T / 16);
    const int seg = idx % (T / 16);  // 16 source rows -> 8 bytes
    if (cl < cols_here && seg * 16 < rows_here) {
      const uint4 b = *reinterpret_cast<const uint4*>(&tcodes[cl * TP + seg * 16]);
      // bytes hold one code each: pack byte pairs (2i, 2i + 1) into one byte.
      const uint32_t u[4] = {b.x, b.y, b.z, b.w};
      uint32_t o[2] = {0u, 0u};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t lo = (u[q] & 0x0Fu) | ((u[q] >> 4) & 0xF0u);          // bytes 0, 1
        const uint32_t hi = ((u[q] >> 16) & 0x0Fu) | ((u[q] >> 20) & 0xF0u);  // bytes 2, 3
        o[q >> 1] |= (lo | (hi << 8)) << (16 * (q & 1));
      }
      *reinterpret_cast<uint2*>(codes_t + (c0 + cl) * (R / 2) + r0 / 2 + seg * 8) = make_uint2(o[0], o[1]);
    }
  }
  if (tid < T) {
    const int cl = tid;
    if (cl < cols_here) {
      uint8_t* sdst = scales_t + (c0 + cl) * (R / B) + r0 / B;
      const int bc = cl / B;
      if (scale_words_t && rows_here == T) {
        if constexpr (NBT == 8) {
          uint32_t a = 0, b = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            a |= (uint32_t)blk_s[i * NBT + bc] << (8 * i);
            b |= (uint32_t)blk_s[(i + 4) * NBT + bc] << (8 * i);
          }
          *reinterpret_cast<uint2*>(sdst) = make_uint2(a, b);
        } else {
          uint32_t a = 0;
#pragma unroll
          for (int i = 0; i < NBT; ++i) a |= (uint32_t)blk_s[i * NBT + bc] << (8 * i);
          *reinterpret_cast<uint32_t*>(sdst) = a;
        }
      } else {
#pragma unroll
        for (int i = 0; i < NBT; ++i)
          if (i * B < rows_here) sdst[i] = blk_s[i * NBT + bc];
      }
    }
  }
}

template <int FMT, int RND, bool BF16>
void launch_2d(const Quant2dArgs& a, hipStream_t s) {
  constexpr int B = FMT == NV ? 16 : 32;
  constexpr int NBT = 128 / B;
  const uint32_t tiles_c = (uint32_t)((a.C + 127) / 128);
  const uint32_t tiles_r = (uint32_t)((a.R + 127) / 128);
  // Scale bytes go out as words when every row start keeps them aligned.
  const uint32_t words_c = FMT == NV ? (a.C / B) % 4 == 0 : (a.C / B) % 2 == 0;
  const uint32_t words_t = (a.R / B) % NBT == 0;
  hipLaunchKernelGGL((k_quant_2d<FMT, RND, BF16>), dim3(tiles_c * tiles_r), dim3(256), 0, s, a.src, a.R,
                     a.C, a.ld, tiles_c, a.codes, a.scales, a.codes_t, a.scales_t, a.amax, a.tscale,
                     a.tscale_t, a.amax_copy, a.seed, a.offset, words_c, words_t);
}

template <int FMT>
void launch_2d_fmt(const Quant2dArgs& a, hipStream_t s) {
  if (a.sr) {
    if (a.bf16) launch_2d<FMT, 1, true>(a, s);
    else launch_2d<FMT, 1, false>(a, s);
  } else {
    if (a.bf16) launch_2d<FMT, 0, true>(a, s);
    else launch_2d<FMT, 0, false>(a, s);
  }
}

}  // namespace

void fp4i_launch_quant_2d(const Quant2dArgs& a, hipStream_t s) {
  if (a.fmt == NV) launch_2d_fmt<NV>(a, s);
  else launch_2d_fmt<MX>(a, s);
}
