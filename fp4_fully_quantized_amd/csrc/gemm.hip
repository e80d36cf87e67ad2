// gemm.hip -- FP4 x FP4 GEMMs with FP32 accumulation on gfx950 MFMA.
//
// C[i][j] = alpha * sum_k A_hat[i][k] * B_hat[j][k]: the three linear-layer
// GEMMs of fully quantized training run this one contraction, each operand
// blocked along the shared axis K (Quartet, one-line summary: all three
// linear-layer GEMMs in FP4; Robots Atlas, "FP4", How it works: FP4 operands,
// higher-precision accumulation).
//
// MXFP4: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands FP4 (format 4).
//   Lane l of an operand holds row l%32 and the 32 consecutive K values of one
//   MX block (16 bytes, low nibble first); its E8M0 byte is that lane's scale
//   operand, so the hardware applies 2^(eA+eB) per block exactly.
// NVFP4: the E4M3 scale is not a power of two and covers 16 values, finer
//   than the MFMA's 32-value scale granularity. Each operand value
//   e2m1 * sdec has at most 6 significant bits and lies in [2^-10, 2688], so
//   it is exact in f16: codes are decoded with v_cvt_scalef32_pk_f16_fp4
//   (scale 1), multiplied by sdec with v_pk_mul_f16 (exact), and fed to
//   v_mfma_f32_32x32x16_f16. alpha = s_gA * s_gB is applied in the epilogue.
//
// Tiling: 256 threads = 4 waves (2 x 2), workgroup tile BM x BN, K tile of 128
// values (64 bytes of codes per row), double-buffered in LDS with the 16-byte
// chunks of each row XOR-swizzled against bank conflicts. Global loads of the
// next K tile are issued before the MFMAs of the current one.
#include "fp4_device.hpp"
#include "fp4_internal.hpp"

using namespace fp4dev;

namespace {

constexpr int NV = 0;
constexpr int MX = 1;
constexpr int BK = 128;   // K values per tile
constexpr int ROWB = 64;  // code bytes per row per tile

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 3; }

template <int FMT, int BM, int BN, bool BF16OUT>
__global__ __launch_bounds__(256) void k_gemm(const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
                                               const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs,
                                               const float* __restrict__ a_ts, const float* __restrict__ b_ts,
                                               int64_t M, int64_t N, int64_t K, uint32_t tiles_n,
                                               void* __restrict__ cout, int64_t ldc) {
  constexpr int SCB = FMT == NV ? 8 : 4;  // scale bytes per row per tile
  constexpr int WM = BM / 2, WN = BN / 2;
  constexpr int FM = WM / 32, FN = WN / 32;
  constexpr int CHUNKS = (BM + BN) * 4;           // 16-byte chunks per tile
  constexpr int CPT = CHUNKS / 256;               // chunks per thread
  constexpr int SROWS_PT = (BM + BN) / 256;       // scale rows per thread
  static_assert(CHUNKS % 256 == 0 && (BM + BN) % 256 == 0, "tile");

  __shared__ __attribute__((aligned(16))) uint8_t lds_c[2][(BM + BN) * ROWB];
  __shared__ __attribute__((aligned(16))) uint8_t lds_s[2][(BM + BN) * SCB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t tm = blockIdx.x / tiles_n;
  const uint32_t tn = blockIdx.x - tm * tiles_n;
  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t kb_row = K / 2;                       // code bytes per operand row
  const int64_t ks_row = K / (FMT == NV ? 16 : 32);   // scale bytes per operand row
  const int nk = (int)(K / BK);

  // Per-thread global sources (rows clamped into range; clamped rows are never stored).
  const uint8_t* gsrc[CPT];
  int ldst[CPT];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int q = tid + 256 * j;
    const int row = q >> 2, c = q & 3;
    int64_t grow;
    const uint8_t* base;
    if (row < BM) {
      grow = m0 + row; if (grow >= M) grow = M - 1;
      base = ac + grow * kb_row;
    } else {
      grow = n0 + (row - BM); if (grow >= N) grow = N - 1;
      base = bc + grow * kb_row;
    }
    gsrc[j] = base + c * 16;
    ldst[j] = row * ROWB + ((c ^ swz(row)) * 16);
  }
  const uint8_t* ssrc[SROWS_PT];
  int sdst[SROWS_PT];
#pragma unroll
  for (int j = 0; j < SROWS_PT; ++j) {
    const int row = tid + 256 * j;
    int64_t grow;
    const uint8_t* base;
    if (row < BM) {
      grow = m0 + row; if (grow >= M) grow = M - 1;
      base = as + grow * ks_row;
    } else {
      grow = n0 + (row - BM); if (grow >= N) grow = N - 1;
      base = bs + grow * ks_row;
    }
    ssrc[j] = base;
    sdst[j] = row * SCB;
  }

  uint4 creg[CPT];
  uint2 sreg[SROWS_PT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) creg[j] = *reinterpret_cast<const uint4*>(gsrc[j] + (int64_t)kt * ROWB);
#pragma unroll
    for (int j = 0; j < SROWS_PT; ++j) {
      if constexpr (SCB == 8) sreg[j] = *reinterpret_cast<const uint2*>(ssrc[j] + (int64_t)kt * SCB);
      else sreg[j].x = *reinterpret_cast<const uint32_t*>(ssrc[j] + (int64_t)kt * SCB);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) *reinterpret_cast<uint4*>(&lds_c[buf][ldst[j]]) = creg[j];
#pragma unroll
    for (int j = 0; j < SROWS_PT; ++j) {
      if constexpr (SCB == 8) *reinterpret_cast<uint2*>(&lds_s[buf][sdst[j]]) = sreg[j];
      else *reinterpret_cast<uint32_t*>(&lds_s[buf][sdst[j]]) = sreg[j].x;
    }
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int g = lane >> 5;   // K half of the MFMA operand this lane supplies
  const int lr = lane & 31;  // operand row inside a 32-row fragment

  gload(0);
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) gload(kt + 1);
    const uint8_t* Ac = lds_c[buf];
    const uint8_t* Bc = lds_c[buf] + BM * ROWB;
    const uint8_t* Asc = lds_s[buf];
    const uint8_t* Bsc = lds_s[buf] + BM * SCB;
    if constexpr (FMT == MX) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int chunk = 2 * s + g;
        v8i a[FM], b[FN];
        int sa[FM], sb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * WM + i * 32 + lr;
          uint4 v = *reinterpret_cast<const uint4*>(Ac + row * ROWB + ((chunk ^ swz(row)) * 16));
          a[i] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
          sa[i] = Asc[row * SCB + chunk];
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn * WN + j * 32 + lr;
          uint4 v = *reinterpret_cast<const uint4*>(Bc + row * ROWB + ((chunk ^ swz(row)) * 16));
          b[j] = (v8i){(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
          sb[j] = Bsc[row * SCB + chunk];
        }
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[i], b[j], acc[i][j], 4, 4, 0,
                                                                          sa[i], 0, sb[j]);
      }
    } else {
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2) {
        const int chunk = g + 2 * c2;
        uint4 av[FM], bv[FN];
        uint32_t asb[FM], bsb[FN];
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const int row = wm * WM + i * 32 + lr;
          av[i] = *reinterpret_cast<const uint4*>(Ac + row * ROWB + ((chunk ^ swz(row)) * 16));
          asb[i] = *reinterpret_cast<const uint16_t*>(Asc + row * SCB + 2 * chunk);
        }
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int row = wn * WN + j * 32 + lr;
          bv[j] = *reinterpret_cast<const uint4*>(Bc + row * ROWB + ((chunk ^ swz(row)) * 16));
          bsb[j] = *reinterpret_cast<const uint16_t*>(Bsc + row * SCB + 2 * chunk);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v8h a[FM], b[FN];
#pragma unroll
          for (int i = 0; i < FM; ++i) {
            const uint32_t w = s == 0 ? av[i].x : s == 1 ? av[i].y : s == 2 ? av[i].z : av[i].w;
            const _Float16 sd = (_Float16)e4m3_decode((asb[i] >> (8 * (s >> 1))) & 0xFFu);
            const v2h sd2 = {sd, sd};
            v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sd2;
            v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sd2;
            v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sd2;
            v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sd2;
            a[i] = (v8h){h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
          }
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const uint32_t w = s == 0 ? bv[j].x : s == 1 ? bv[j].y : s == 2 ? bv[j].z : bv[j].w;
            const _Float16 sd = (_Float16)e4m3_decode((bsb[j] >> (8 * (s >> 1))) & 0xFFu);
            const v2h sd2 = {sd, sd};
            v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sd2;
            v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sd2;
            v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sd2;
            v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sd2;
            b[j] = (v8h){h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
          }
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
      }
    }
    if (kt + 1 < nk) lstore(buf ^ 1);
    __syncthreads();
  }

  float alpha = 1.0f;
  if constexpr (FMT == NV) alpha = (*a_ts) * (*b_ts);

  // Epilogue. Lane l of a 32x32 fragment holds column l%32 and rows
  // 8*(r/4) + 4*(l/32) + r%4, r = 0..15.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t col = n0 + wn * WN + j * 32 + lr;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * WM + i * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
        if (row >= M) continue;
        float y = acc[i][j][r];
        if constexpr (FMT == NV) y = y * alpha;
        if constexpr (BF16OUT) {
          uint32_t u = __float_as_uint(y);
          u = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
          static_cast<uint16_t*>(cout)[row * ldc + col] = (uint16_t)u;
        } else {
          static_cast<float*>(cout)[row * ldc + col] = y;
        }
      }
    }
  }
}

template <int FMT, int BM, int BN>
void launch(const GemmArgs& g, hipStream_t s) {
  const uint32_t tiles_m = (uint32_t)((g.M + BM - 1) / BM);
  const uint32_t tiles_n = (uint32_t)((g.N + BN - 1) / BN);
  const dim3 grid(tiles_m * tiles_n), block(256);
  if (g.bf16out)
    hipLaunchKernelGGL((k_gemm<FMT, BM, BN, true>), grid, block, 0, s, g.a_codes, g.a_scales, g.b_codes,
                       g.b_scales, g.a_tscale, g.b_tscale, g.M, g.N, g.K, tiles_n, g.c, g.ldc);
  else
    hipLaunchKernelGGL((k_gemm<FMT, BM, BN, false>), grid, block, 0, s, g.a_codes, g.a_scales, g.b_codes,
                       g.b_scales, g.a_tscale, g.b_tscale, g.M, g.N, g.K, tiles_n, g.c, g.ldc);
}

}  // namespace

void fp4i_launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.fmt == NV) launch<NV, 128, 128>(g, s);
  else launch<MX, 128, 128>(g, s);
}
