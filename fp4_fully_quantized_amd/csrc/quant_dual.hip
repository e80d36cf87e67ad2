// quant_dual.hip -- both orientations of a tensor's block-scaled FP4
// quantization from one read (FP4 All the Way, Key points: the forward GEMM
// takes X and W with blocks along the reduction axis K, the backward GEMMs take
// them, and dY, with blocks along the other axis).
#include "fp4_internal.hpp"
#include "quant_common.hpp"

using namespace fp4q;

namespace {

// Both orientations from one read of the source. A workgroup takes a
// 128 x 128 tile into LDS once (input format), then
//  (b) quantizes it with blocks along its rows (the COLS orientation): thread
//      (row, half) takes 64 consecutive elements of one row (4 NVFP4 or 2
//      MXFP4 blocks) and writes their codes (32 bytes) and scales directly;
//  (a) quantizes it with blocks down its columns (the transposed, ROWS
//      orientation), as k_quant_rows does: thread (b, q) handles block b of
//      NCOL adjacent columns; codes and scales are staged in LDS (over the
//      tile, which is no longer read) per output row and written out last.
// Each orientation has its own rounding mode, SR stream, rotation (on or off,
// and its mask) and, for NVFP4, tensor amax (the rotated values' amax differs
// per rotation axis); the results equal the two separate passes bit for bit.
template <int FMT, int RC, int RR, bool BF16, bool HC, bool HR, bool MON>
__device__ __forceinline__ void quant_dual_body(
    const void* __restrict__ src, int64_t R, int64_t C, int64_t ld, uint32_t tiles_c, uint32_t ntiles,
    uint8_t* __restrict__ codes_c, uint8_t* __restrict__ scales_c,
    uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r,
    const float* __restrict__ amax_c, const float* __restrict__ amax_r, float* tscale_c,
    float* tscale_r, float* amax_copy,
    uint64_t seed_c, uint64_t off_c, uint32_t signs_c, uint64_t seed_r, uint64_t off_r,
    uint64_t idx_rows, uint32_t signs_r, uint32_t scale_words_c, uint32_t scale_words_r, double* noise_c,
    double* noise_r) {
  constexpr int ES = BF16 ? 2 : 4;
  constexpr int B = FMT == NV ? 16 : 32;
  constexpr int T = 128;                  // tile rows = tile columns
  constexpr int NB = T / B;               // blocks per tile column (and per tile row)
  constexpr int NCOL = NB * T / 256;      // (a): adjacent columns per thread
  constexpr int TPB = T / NCOL;           // (a): threads per block row
  constexpr int PITCH = T * ES + 8;       // row pitch in bytes (8-byte reads stay aligned)
  constexpr int SP = T / 2 + 4;           // staged code bytes per output row of (a)
  __shared__ __attribute__((aligned(16))) uint8_t tile[T * PITCH];
  // (a)'s staged codes and scales reuse the tile once every thread has read
  // its part of it: 33 KB of LDS per workgroup (bf16), four per CU.
  static_assert(T * SP + T * NB <= T * PITCH && (T * SP) % 16 == 0, "staging fits in the tile");
  uint8_t* const stage_c = tile;
  uint8_t* const stage_s = tile + T * SP;
  // NVFP4 element multipliers of each orientation (the tile load's barrier
  // publishes them).
  __shared__ float rtab[FMT == NV ? 2 : 1][128];

  float sg_c = 1.0f, sg_r = 1.0f;
  if constexpr (FMT == NV) {
    const float ac = *amax_c;
    const float ar = *amax_r;
    sg_c = nv_tensor_scale(ac);
    sg_r = nv_tensor_scale(ar);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      *tscale_c = sg_c;
      *tscale_r = sg_r;
      if (amax_copy) *amax_copy = ac;
    }
    nv_rcp_table(rtab[0], sg_c);
    nv_rcp_table(rtab[FMT == NV ? 1 : 0], sg_r);
  }
  double ngc = 0.0, nec = 0.0, ngr = 0.0, ner = 0.0;  // quantization noise, when asked for
  // One tile per workgroup; with the noise monitor (MON) a capped grid loops
  // over the tiles: workgroup b takes tiles b, b + grid, ...
  constexpr int CPR = T * ES / 16;        // 16-byte pieces per tile row
  constexpr int NLD = T * CPR / 256;      // 16-byte loads per thread and tile
  const uint32_t n_it = MON ? (ntiles - blockIdx.x + gridDim.x - 1) / gridDim.x : 1u;
  const uint32_t t_first = MON ? blockIdx.x : xcd_contiguous_tile(blockIdx.x, ntiles);
  const uint32_t t_step = MON ? gridDim.x : 0u;
  // With the monitor the thread index is taken afresh in each iteration
  // through an opaque move, so that nothing derived from it is hoisted out of
  // the tile loop and held in registers across it: the monitored kernels
  // needed 155-168 registers and scratch that way, 100-121 and none this way.
  // (The single-tile kernels keep the plain index, whose known range makes
  // their address arithmetic cheaper: 1915 against 2212 VALU instructions in
  // the dY kernel.)
  const int tid0 = threadIdx.x;
  auto opaque_tid = [&]() {
    int t;
    asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(tid0));
    return t;
  };
  uint4 pre[NLD];
  // Tile ti's source into pre (16 bytes per load; only edge tiles check bounds).
  auto load_tile = [&](uint32_t ti, int tid) {
    const uint32_t tr = ti / tiles_c;
    const int64_t r0 = (int64_t)tr * T;
    const int64_t c0 = (int64_t)(ti - tr * tiles_c) * T;
    if (r0 + T <= R && c0 + T <= C) {
#pragma unroll
      for (int k = 0; k < NLD; ++k) {
        const int idx = k * 256 + tid;
        const int rr = idx / CPR;
        const int cc = idx % CPR;
        pre[k] = *reinterpret_cast<const uint4*>(static_cast<const char*>(src) +
                                                 ((r0 + rr) * ld + c0 + cc * (16 / ES)) * ES);
      }
    } else {
#pragma unroll
      for (int k = 0; k < NLD; ++k) {
        const int idx = k * 256 + tid;
        const int rr = idx / CPR;
        const int cc = idx % CPR;
        const int64_t col = c0 + cc * (16 / ES);
        pre[k] = make_uint4(0, 0, 0, 0);
        if (r0 + rr < R && col < C)
          pre[k] = *reinterpret_cast<const uint4*>(static_cast<const char*>(src) + ((r0 + rr) * ld + col) * ES);
      }
    }
  };
#pragma unroll 1
  for (uint32_t it = 0; it < n_it; ++it) {
    const uint32_t ti = t_first + it * t_step;
    const uint32_t tr = ti / tiles_c;
    const uint32_t tc = ti - tr * tiles_c;
    const int64_t r0 = (int64_t)tr * T;
    const int64_t c0 = (int64_t)tc * T;
    const int tid = MON ? opaque_tid() : tid0;   // (one iteration without the monitor)

    // 1. the tile into LDS
    load_tile(ti, tid);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int idx = k * 256 + tid;
      uint2* d = reinterpret_cast<uint2*>(&tile[(idx / CPR) * PITCH + (idx % CPR) * 16]);
      d[0] = make_uint2(pre[k].x, pre[k].y);
      d[1] = make_uint2(pre[k].z, pre[k].w);
    }
    __syncthreads();

    const int64_t rows_here = R - r0 < T ? R - r0 : T;  // multiples of B
    const int64_t cols_here = C - c0 < T ? C - c0 : T;


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
        if constexpr (HC) hadamard_block<B>(x, signs_c);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < B; ++i) m = fmaxf(m, fabsf(x[i]));
        float rcp;
        sb[bb] = block_scale_tab<FMT>(m, sg_c, rtab[0], rcp);
        const int64_t col0 = c0 + half * 64 + bb * B;
        float bg = 0.0f, be = 0.0f;
        const float bs = (MON && noise_c) ? scale_value<FMT>(sb[bb]) : 0.0f;
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
          if (MON && noise_c) noise8<FMT>(x + 8 * g, w[bb * (B / 8) + g], bs, sg_c, bg, be);
        }
        ngc += (double)bg;
        nec += (double)be;
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
      // The staging below overwrites the tile: every thread has read its
      // part of it ((b) before, its own columns just now) past this barrier.
      __syncthreads();
#pragma unroll
      for (int k = 0; k < NCOL; ++k) {
        const int cl = cl0 + k;
        const int64_t cg = c0 + cl;
        float* xk = x[k];
        if constexpr (HR) hadamard_block<B>(xk, signs_r);
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < B; ++i) m = fmaxf(m, fabsf(xk[i]));
        float rcp;
        const uint32_t sbyte = block_scale_tab<FMT>(m, sg_r, rtab[FMT == NV ? 1 : 0], rcp);
        uint32_t* sc = reinterpret_cast<uint32_t*>(&stage_c[cl * SP + b * (B / 2)]);
        float bg = 0.0f, be = 0.0f;
        const float bs = (MON && noise_r) ? scale_value<FMT>(sbyte) : 0.0f;
#pragma unroll
        for (int g = 0; g < B / 8; ++g) {
          float v[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) v[i] = xk[8 * g + i] * rcp;
          uint32_t cw;
          if constexpr (RR == 0) {
            cw = e2m1_rtn_pack8(v);
          } else {
            uint32_t h[4];
            sr_draws8(seed_r, (off_r + (uint64_t)cg * idx_rows + (uint64_t)rg) / 8 + g, h);
            cw = e2m1_sr_pack8(v, h);
          }
          sc[g] = cw;
          if (MON && noise_r) noise8<FMT>(xk + 8 * g, cw, bs, sg_r, bg, be);
        }
        stage_s[cl * NB + b] = (uint8_t)sbyte;
        ngr += (double)bg;
        ner += (double)be;
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
    __syncthreads();  // the next tile reuses the LDS buffers
  }
  if constexpr (MON) {
    if (noise_c) noise_reduce(ngc, nec, noise_c);
    if (noise_c && noise_r) __syncthreads();
    if (noise_r) noise_reduce(ngr, ner, noise_r);
  }
}

// The kernels. The NVFP4 bf16 noise-monitored variants ask for 4 waves per
// SIMD (at most 128 registers), so that as many workgroups run on each CU as
// their LDS allows (4); the others need about 100 registers, or their LDS
// (fp32 input) allows only 2 workgroups per CU anyway.
template <int FMT, int RC, int RR, bool BF16, bool HC, bool HR, bool MON>
__global__ __launch_bounds__(256) void k_quant_dual(
    const void* __restrict__ src, int64_t R, int64_t C, int64_t ld, uint32_t tiles_c, uint32_t ntiles,
    uint8_t* __restrict__ codes_c, uint8_t* __restrict__ scales_c,
    uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r,
    const float* __restrict__ amax_c, const float* __restrict__ amax_r, float* tscale_c,
    float* tscale_r, float* amax_copy,
    uint64_t seed_c, uint64_t off_c, uint32_t signs_c, uint64_t seed_r, uint64_t off_r,
    uint64_t idx_rows, uint32_t signs_r, uint32_t scale_words_c, uint32_t scale_words_r, double* noise_c,
    double* noise_r) {
  quant_dual_body<FMT, RC, RR, BF16, HC, HR, MON>(src, R, C, ld, tiles_c, ntiles, codes_c, scales_c, codes_r, scales_r,
                                                  amax_c, amax_r, tscale_c, tscale_r, amax_copy, seed_c, off_c,
                                                  signs_c, seed_r, off_r, idx_rows, signs_r, scale_words_c, scale_words_r,
                                                  noise_c, noise_r);
}
template <int FMT, int RC, int RR, bool BF16, bool HC, bool HR, bool MON>
__global__ __launch_bounds__(256, 4) void k_quant_dual_w4(
    const void* __restrict__ src, int64_t R, int64_t C, int64_t ld, uint32_t tiles_c, uint32_t ntiles,
    uint8_t* __restrict__ codes_c, uint8_t* __restrict__ scales_c,
    uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r,
    const float* __restrict__ amax_c, const float* __restrict__ amax_r, float* tscale_c,
    float* tscale_r, float* amax_copy,
    uint64_t seed_c, uint64_t off_c, uint32_t signs_c, uint64_t seed_r, uint64_t off_r,
    uint64_t idx_rows, uint32_t signs_r, uint32_t scale_words_c, uint32_t scale_words_r, double* noise_c,
    double* noise_r) {
  quant_dual_body<FMT, RC, RR, BF16, HC, HR, MON>(src, R, C, ld, tiles_c, ntiles, codes_c, scales_c, codes_r, scales_r,
                                                  amax_c, amax_r, tscale_c, tscale_r, amax_copy, seed_c, off_c,
                                                  signs_c, seed_r, off_r, idx_rows, signs_r, scale_words_c, scale_words_r,
                                                  noise_c, noise_r);
}

template <int FMT, int RC, int RR, bool BF16, bool HC, bool HR, bool MON>
void launch_dual(const DualArgs& a, hipStream_t s) {
  constexpr int B = FMT == NV ? 16 : 32;
  const uint32_t tiles_c = (uint32_t)((a.C + 127) / 128);
  const uint32_t tiles_r = (uint32_t)((a.R + 127) / 128);
  // Scale bytes of a tile go out as words when every row start keeps them aligned.
  const uint32_t words_c = FMT == NV ? (a.C / B) % 4 == 0 : (a.C / B) % 2 == 0;
  const uint32_t words_r = (a.R / B) % 4 == 0;
  const uint32_t ntiles = tiles_c * tiles_r;
  const auto kernel = [] {
    if constexpr (MON && FMT == NV && BF16) return k_quant_dual_w4<FMT, RC, RR, BF16, HC, HR, MON>;
    else return k_quant_dual<FMT, RC, RR, BF16, HC, HR, MON>;
  }();
  const uint32_t grid = MON ? noise_grid(kernel, ntiles) : ntiles;
  hipLaunchKernelGGL(kernel, dim3(grid), dim3(256), 0,
                     s, a.src, a.R, a.C, a.ld, tiles_c, ntiles, a.codes_c, a.scales_c, a.codes_r, a.scales_r,
                     a.amax_c, a.amax_r, a.tscale_c, a.tscale_r, a.amax_copy, a.seed_c, a.offset_c,
                     a.signs_c, a.seed_r, a.offset_r, (uint64_t)(a.idx_rows_r ? a.idx_rows_r : a.R), a.signs_r,
                     words_c, words_r, a.noise_c,
                     a.noise_r);
}

template <int FMT, bool BF16, bool HC, bool HR, bool MON>
void launch_dual_rnd(const DualArgs& a, hipStream_t s) {
  if (a.sr_c) {
    if (a.sr_r) launch_dual<FMT, 1, 1, BF16, HC, HR, MON>(a, s);
    else launch_dual<FMT, 1, 0, BF16, HC, HR, MON>(a, s);
  } else {
    if (a.sr_r) launch_dual<FMT, 0, 1, BF16, HC, HR, MON>(a, s);
    else launch_dual<FMT, 0, 0, BF16, HC, HR, MON>(a, s);
  }
}

template <int FMT, bool BF16, bool HC, bool HR>
void launch_dual_mon(const DualArgs& a, hipStream_t s) {
  if (a.noise_c || a.noise_r) launch_dual_rnd<FMT, BF16, HC, HR, true>(a, s);
  else launch_dual_rnd<FMT, BF16, HC, HR, false>(a, s);
}

template <int FMT, bool BF16>
void launch_dual_had(const DualArgs& a, hipStream_t s) {
  if (a.had_c) {
    if (a.had_r) launch_dual_mon<FMT, BF16, true, true>(a, s);
    else launch_dual_mon<FMT, BF16, true, false>(a, s);
  } else {
    if (a.had_r) launch_dual_mon<FMT, BF16, false, true>(a, s);
    else launch_dual_mon<FMT, BF16, false, false>(a, s);
  }
}

}  // namespace

void fp4i_launch_quant_dual(const DualArgs& a, hipStream_t s) {
  if (a.fmt == NV) {
    if (a.bf16) launch_dual_had<NV, true>(a, s);
    else launch_dual_had<NV, false>(a, s);
  } else {
    if (a.bf16) launch_dual_had<MX, true>(a, s);
    else launch_dual_had<MX, false>(a, s);
  }
}
