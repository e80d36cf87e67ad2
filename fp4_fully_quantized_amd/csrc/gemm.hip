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
//   v_mfma_f32_32x32x16_f16; the decode of the next substep's operands is
//   interleaved with the current substep's MFMAs. alpha = s_gA * s_gB is
//   applied in the epilogue.
//   For the f16 MFMA the K order inside an instruction is free as long as A
//   and B agree: lane half g of substep s carries K values 32g + 8s .. +7 of a
//   64-value group, so each lane reads 16 contiguous bytes per group.
//
// Tiling: 256 threads = 4 waves (2 x 2), workgroup tile 256 x 256 (each wave
// owns 128 x 128 = 4 x 4 MFMA fragments, accumulators in AGPRs; the MXFP4
// whole tiles at K tile 256 run k_gemm_mx8: 8 waves of 128 x 64, two per
// SIMD, since that kernel is bound by LDS and barrier waits, not VALU), K tile BK
// (256 values when K allows, else 128). Global loads are buffer loads (the
// descriptor's size bound turns rows past M or N into zeros), issued one K
// tile ahead into VGPRs and written to the other half of a double-buffered
// LDS tile after the current tile's MFMAs. In LDS the 16-byte chunks of each
// row are XOR-swizzled by (row / 2) so that the 32 rows read by one ds_read_b128
// hit distinct banks; the block-scale bytes are permuted on the way in so that
// each lane fetches the scales of all its substeps with one LDS read (MXFP4:
// the MFMA's op_sel picks the substep's byte). Operand fragments of the next
// substep are read while the current substep's MFMAs run. Workgroups are mapped
// to tiles so that the ones resident on one XCD (dispatch is round-robin over
// the 8 XCDs) cover a compact group of tile rows and share operand panels in
// that XCD's L2. The MFMAs take the B fragment first, so each lane's
// accumulator holds four consecutive columns of one output row; after the K
// loop each wave stages its outputs through the idle LDS tiles, 32 rows at a
// time, and every store instruction writes whole rows in 16-byte pieces.
//
// Split-K (optional, with caller workspace): when the tiles do not fill the
// last wave of workgroups and K is long enough to pay for it (split_plan), the
// whole tiles run first, then the remaining tiles as pieces over K ranges
// that write FP32 partial tiles, which k_split_reduce adds in piece order.
#include "fp4_device.hpp"
#include "fp4_internal.hpp"

#include <algorithm>
#include <type_traits>

using namespace fp4dev;

namespace {

constexpr int NV = 0;
constexpr int MX = 1;
constexpr int NXCD = 8;
constexpr int BM = 256, BN = 256;
constexpr int WM = 128, WN = 128;
constexpr int FM = 4, FN = 4;
constexpr uint32_t kRsrcWord3 = 0x00020000u;
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedValu = 0x002;
constexpr int kSchedMfma = 0x008;
constexpr int kSchedVmemRead = 0x020;
constexpr int kSchedDsRead = 0x100;
constexpr int kSchedDsWrite = 0x200;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, (int)kRsrcWord3);
}
// off: the lane's byte offset; soff: a part common to the workgroup (held in
// the instruction's scalar offset, so it costs no vector add per load).
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, (int)soff, 0));
}
__device__ __forceinline__ uint2 bload8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t soff = 0) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, (int)soff, 0));
}

// Scaled FP4 MFMA; S selects the byte of the lanes' scale words (op_sel).
template <int S>
__device__ __forceinline__ v16f mfma_mx(const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, S, sa, S, sb);
}
__device__ __forceinline__ v16f mfma_mx_sel(int s, const v8i& a, const v8i& b, const v16f& c, int sa, int sb) {
  return s == 0 ? mfma_mx<0>(a, b, c, sa, sb)
       : s == 1 ? mfma_mx<1>(a, b, c, sa, sb)
       : s == 2 ? mfma_mx<2>(a, b, c, sa, sb)
                : mfma_mx<3>(a, b, c, sa, sb);
}

// Output tile t (in the grouped order) -> tile row and column: groups of
// group_m tile rows, column-major inside a group, so that the workgroups one
// XCD runs at a time share A and B panels in that XCD's L2.
__device__ __forceinline__ void tile_coords(uint32_t t, uint32_t tiles_m, uint32_t tiles_n, uint32_t group_m,
                                            uint32_t& tm, uint32_t& tn) {
  const uint32_t per_group = group_m * tiles_n;
  const uint32_t grp = t / per_group;
  const uint32_t first_m = grp * group_m;
  const uint32_t gsize = min(group_m, tiles_m - first_m);
  const uint32_t in_grp = t - grp * per_group;
  tm = first_m + in_grp % gsize;
  tn = in_grp / gsize;
}

template <int FMT, int BK>
struct Cfg {
  static constexpr int ROWB = BK / 2;               // code bytes per row per K tile
  static constexpr int CPR = ROWB / 16;             // 16-byte chunks per row
  static constexpr int SB = FMT == NV ? 16 : 32;    // elements per scale byte
  static constexpr int SCB = BK / SB;               // scale bytes per row per K tile
  static constexpr int ROWS = BM + BN;
  static constexpr int CODE_LOADS = ROWS * CPR / 256;   // 16-byte loads per thread
  static constexpr int RPL = 256 / CPR;                 // rows covered by one load round
  static constexpr int SCALE_LOADS = ROWS * SCB / 16 / 256 > 0 ? ROWS * SCB / 16 / 256 : 1;
  static constexpr int LDS_CODES = ROWS * ROWB;
  static constexpr int LDS_SCALES = ROWS * SCB;
};

// Scale bytes of one row permuted so that lane half g finds the bytes of all
// its substeps contiguous (see the file comment).
template <int FMT, int BK>
__device__ __forceinline__ uint4 permute_scales(uint4 v) {
  if constexpr (FMT == NV && BK == 256) {
    // 16 blocks; half g uses blocks {2g,2g+1, 2g+4,2g+5, 2g+8,2g+9, 2g+12,2g+13}
    return make_uint4(__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x05040100u),
                      __builtin_amdgcn_perm(v.y, v.x, 0x07060302u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u));
  } else if constexpr (FMT == NV) {
    // 8 blocks in v.x, v.y; half g uses {2g, 2g+1, 2g+4, 2g+5}
    return make_uint4(__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.y, v.x, 0x07060302u), 0, 0);
  } else if constexpr (BK == 256) {
    // 8 blocks in v.x, v.y; half g uses {g, g+2, g+4, g+6}
    return make_uint4(__builtin_amdgcn_perm(v.y, v.x, 0x06040200u), __builtin_amdgcn_perm(v.y, v.x, 0x07050301u), 0, 0);
  } else {
    // 4 blocks in v.x; half g uses {g, g+2}
    return make_uint4(__builtin_amdgcn_perm(0u, v.x, 0x03010200u), 0, 0, 0);
  }
}

// SPLIT = false: whole output tiles 0 .. nfull-1. SPLIT = true: the pieces of
// the split tiles nfull .. nfull+ntail-1, each a range of K, whose FP32
// partial tiles go to `part` (added by k_split_reduce).
template <int FMT, int BK, bool BF16OUT, bool SPLIT>
__global__ __launch_bounds__(256, 1) void k_gemm(const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
                                                  const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs,
                                                  const float* __restrict__ a_ts, const float* __restrict__ b_ts,
                                                  uint32_t M, uint32_t N, uint32_t K, uint32_t tiles_m,
                                                  uint32_t tiles_n, uint32_t group_m, uint32_t nfull,
                                                  uint32_t ntail, uint32_t split, float* __restrict__ part,
                                                  void* __restrict__ cout, int64_t ldc, uint32_t vec_ok) {
  using C = Cfg<FMT, BK>;
  // One LDS array: the double-buffered code and scale tiles of the K loop,
  // reused afterwards to stage the output tile for row-contiguous stores.
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (C::LDS_CODES + C::LDS_SCALES)];
  uint8_t (*lds_c)[C::LDS_CODES] = reinterpret_cast<uint8_t (*)[C::LDS_CODES]>(lds);
  uint8_t (*lds_s)[C::LDS_SCALES] = reinterpret_cast<uint8_t (*)[C::LDS_SCALES]>(lds + 2 * C::LDS_CODES);

  // ---- work of this workgroup. Dispatch goes round robin over the 8 XCDs
  // and the grid (of each split piece) is a multiple of 8 workgroups, so each
  // XCD takes one contiguous range of the tiles.
  const int nk_all = (int)(K / BK);
  uint32_t t, tt = 0, sidx = 0;
  int kb = 0, nk = nk_all;
  if constexpr (!SPLIT) {
    const uint32_t gfull = (nfull + NXCD - 1) / NXCD * NXCD;
    t = (blockIdx.x % NXCD) * (gfull / NXCD) + blockIdx.x / NXCD;
    if (t >= nfull) return;
  } else {
    const uint32_t gtail = (ntail + NXCD - 1) / NXCD * NXCD;
    const uint32_t u = blockIdx.x;
    sidx = u / gtail;
    const uint32_t v = u - sidx * gtail;
    tt = (v % NXCD) * (gtail / NXCD) + v / NXCD;
    if (tt >= ntail) return;
    t = nfull + tt;
    kb = (int)(sidx * (uint32_t)nk_all / split);
    nk = (int)((sidx + 1) * (uint32_t)nk_all / split) - kb;
  }
  uint32_t tm, tn;
  tile_coords(t, tiles_m, tiles_n, group_m, tm, tn);
  const uint32_t m0 = tm * BM, n0 = tn * BN;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint32_t kb_row = K / 2;
  const uint32_t ks_row = K / C::SB;

  const __amdgpu_buffer_rsrc_t ra = make_rsrc(ac, M * kb_row);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(bc, N * kb_row);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(as, M * ks_row);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(bs, N * ks_row);

  // Code loads: load j covers tile rows RPL*j + tid/CPR, chunk tid%CPR.
  const int lrow = tid / C::CPR, lchk = tid % C::CPR;
  const uint32_t goff_a = (m0 + lrow) * kb_row + lchk * 16;
  const uint32_t goff_b = (n0 + lrow) * kb_row + lchk * 16;
  const int lds_w = lrow * C::ROWB + ((lchk ^ ((lrow >> 1) & (C::CPR - 1))) * 16);
  constexpr int JA = BM / C::RPL;   // loads that cover A rows
  // Scale loads: one row per thread (A rows, then B rows).
  const uint32_t soff_a = (m0 + tid) * ks_row;
  const uint32_t soff_b = (n0 + tid) * ks_row;

  uint4 creg[C::CODE_LOADS];
  uint4 sreg[2];
  // Staging of one K tile: code load j (16 bytes) and the two scale rows.
  // kt counts the K tiles of this workgroup's range (from kb).
  auto gload_code = [&](int j, int kt) {
    const uint32_t kc = (uint32_t)(kb + kt) * C::ROWB;
    if (j < JA) creg[j] = bload16(ra, goff_a, (uint32_t)(j * C::RPL) * kb_row + kc);
    else creg[j] = bload16(rb, goff_b, (uint32_t)((j - JA) * C::RPL) * kb_row + kc);
  };
  auto gload_scales = [&](int kt) {
    const uint32_t ks = (uint32_t)(kb + kt) * C::SCB;
    if constexpr (C::SCB == 16) {
      sreg[0] = bload16(rsa, soff_a, ks);
      sreg[1] = bload16(rsb, soff_b, ks);
    } else if constexpr (C::SCB == 8) {
      uint2 x = bload8(rsa, soff_a, ks), y = bload8(rsb, soff_b, ks);
      sreg[0] = make_uint4(x.x, x.y, 0, 0);
      sreg[1] = make_uint4(y.x, y.y, 0, 0);
    } else {
      sreg[0] = make_uint4(__builtin_amdgcn_raw_buffer_load_b32(rsa, (int)soff_a, (int)ks, 0), 0, 0, 0);
      sreg[1] = make_uint4(__builtin_amdgcn_raw_buffer_load_b32(rsb, (int)soff_b, (int)ks, 0), 0, 0, 0);
    }
  };
  auto lstore_code = [&](int j, int buf) {
    *reinterpret_cast<uint4*>(&lds_c[buf][lds_w + j * C::RPL * C::ROWB]) = creg[j];
  };
  auto lstore_scales = [&](int buf) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint8_t* p = &lds_s[buf][(tid + 256 * h) * C::SCB];
      const uint4 v = permute_scales<FMT, BK>(sreg[h]);
      if constexpr (C::SCB == 16) *reinterpret_cast<uint4*>(p) = v;
      else if constexpr (C::SCB == 8) *reinterpret_cast<uint2*>(p) = make_uint2(v.x, v.y);
      else *reinterpret_cast<uint32_t*>(p) = v.x;
    }
  };
  // Write the staged tile to LDS buffer `buf` piece by piece, each piece
  // followed by the global load of the same piece of tile `kt_next`.
  auto stage = [&](int j, int buf, int kt_next) {
    lstore_code(j, buf);
    gload_code(j, kt_next);
  };
  auto stage_scales = [&](int buf, int kt_next) {
    lstore_scales(buf);
    gload_scales(kt_next);
  };

  v16f acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int g = lane >> 5;   // which half of the MFMA operand's K this lane supplies
  const int lr = lane & 31;  // operand row inside a 32-row fragment
  // LDS rows of this lane's fragments (A rows, then B rows).
  int arow[FM], brow[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) arow[i] = wm * WM + i * 32 + lr;
#pragma unroll
  for (int j = 0; j < FN; ++j) brow[j] = BM + wn * WN + j * 32 + lr;
  // Fragment f (A fragments 0 .. FM-1, then B) at chunk 2k + g. Every row
  // this lane reads is lr plus a multiple of 32, so its swizzle key
  // (row / 2) % CPR is the lane's own and the chunk's swizzled position,
  // 16 ((2k + g) ^ key) = 32k ^ T, is shared by all its fragments, which then
  // differ by constants (immediate offsets of the LDS reads).
  const int T = (g ^ ((lr >> 1) & (C::CPR - 1))) * 16;
  const int a_lane = (wm * WM + lr) * C::ROWB, b_lane = (BM + wn * WN + lr) * C::ROWB;
  auto frag = [&](const uint8_t* L, int f, int k) {
    const int sw = T ^ (32 * k);
    return f < FM ? *reinterpret_cast<const uint4*>(L + a_lane + sw + f * 32 * C::ROWB)
                  : *reinterpret_cast<const uint4*>(L + b_lane + sw + (f - FM) * 32 * C::ROWB);
  };

  // Pipeline: tile 0 in LDS buffer 0 and tile 1 in the staging registers
  // before the loop. Iteration kt computes tile kt from buffer kt&1 while it
  // writes tile kt+1 from the registers into the other buffer and loads tile
  // kt+2 into the registers (clamped at the last tile: the extra loads and
  // writes are never read). One barrier per iteration, placed before the last
  // group of MFMAs, whose operand reads were issued before it; after it the
  // first operands of tile kt+1 are read while those MFMAs run.
#pragma unroll
  for (int j = 0; j < C::CODE_LOADS; ++j) gload_code(j, 0);
  gload_scales(0);
#pragma unroll
  for (int j = 0; j < C::CODE_LOADS; ++j) stage(j, 0, nk > 1 ? 1 : 0);
  stage_scales(0, nk > 1 ? 1 : 0);
  __syncthreads();

  if constexpr (FMT == MX) {
    constexpr int NS = BK / 64;                          // substeps (one K=64 MFMA each)
    constexpr int PER = (C::CODE_LOADS + NS - 2) / (NS - 1);  // staging pieces per substep
    uint32_t sa[FM], sb[FN];
    uint4 a[2][FM], b[2][FN];
    auto read_scales = [&](const uint8_t* S) {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        if constexpr (NS == 4) sa[i] = *reinterpret_cast<const uint32_t*>(S + arow[i] * C::SCB + 4 * g);
        else sa[i] = *reinterpret_cast<const uint16_t*>(S + arow[i] * C::SCB + 2 * g);
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        if constexpr (NS == 4) sb[j] = *reinterpret_cast<const uint32_t*>(S + brow[j] * C::SCB + 4 * g);
        else sb[j] = *reinterpret_cast<const uint16_t*>(S + brow[j] * C::SCB + 2 * g);
      }
    };
    auto read_frags = [&](const uint8_t* L, int s, int dst) {
#pragma unroll
      for (int i = 0; i < FM; ++i) a[dst][i] = frag(L, i, s);
#pragma unroll
      for (int j = 0; j < FN; ++j) b[dst][j] = frag(L, FM + j, s);
    };
    read_scales(lds_s[0]);
    read_frags(lds_c[0], 0, 0);
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      const int kn = kt + 2 < nk ? kt + 2 : nk - 1;
      uint32_t sa_keep[FM], sb_keep[FN];  // scales of tile kt while tile kt+1's are read
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int cur = s & 1;
        if (s == NS - 1) {
          __syncthreads();
          // first operands of tile kt+1 (its buffer is complete after the barrier)
#pragma unroll
          for (int i = 0; i < FM; ++i) sa_keep[i] = sa[i];
#pragma unroll
          for (int j = 0; j < FN; ++j) sb_keep[j] = sb[j];
          read_scales(lds_s[buf ^ 1]);
          read_frags(lds_c[buf ^ 1], 0, cur ^ 1);
        } else {
          read_frags(lds_c[buf], s + 1, cur ^ 1);
#pragma unroll
          for (int q = 0; q < PER; ++q)
            if (s * PER + q < C::CODE_LOADS) stage(s * PER + q, buf ^ 1, kn);
          if (s == NS - 2) stage_scales(buf ^ 1, kn);
        }
        const uint32_t* SA = (s == NS - 1) ? sa_keep : sa;
        const uint32_t* SB = (s == NS - 1) ? sb_keep : sb;
#pragma unroll
        for (int i = 0; i < FM; ++i) {
          const v8i av = {(int)a[cur][i].x, (int)a[cur][i].y, (int)a[cur][i].z, (int)a[cur][i].w, 0, 0, 0, 0};
#pragma unroll
          for (int j = 0; j < FN; ++j) {
            const v8i bv = {(int)b[cur][j].x, (int)b[cur][j].y, (int)b[cur][j].z, (int)b[cur][j].w, 0, 0, 0, 0};
            acc[i][j] = mfma_mx_sel(s, bv, av, acc[i][j], (int)SB[j], (int)SA[i]);
          }
        }
        // Instruction order for the scheduler: the next substep's LDS reads
        // first, then the MFMAs with the staging writes and global loads
        // threaded between them, so LDS and memory latency run under MFMAs.
        if (s < NS - 1) {
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, FM + FN, 0);
#pragma unroll
          for (int q = 0; q < PER; ++q) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, FM * FN - 2 * PER > 0 ? FM * FN - 2 * PER : 0, 0);
        } else {
          __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * (FM + FN), 0);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, FM * FN, 0);
        }
      }
    }
  } else {
    // Chunk pair c2 of a K tile = 64 K values = 4 substeps of K = 16. The
    // operands of substep t + 1 are decoded (e2m1 -> f16, times the block's
    // E4M3 scale) while the 16 MFMAs of substep t run, a few VALU after each
    // MFMA, so the decode issues under the matrix pipe instead of in bursts
    // between MFMAs.
    constexpr int NC = BK / 64;                          // chunk pairs; each is 4 substeps of K=16
    constexpr int PER = (C::CODE_LOADS + NC - 2) / (NC - 1);
    uint32_t sw[FM + FN][2];                             // scale words of the tile (A frags, then B)
    uint4 raw[2][FM + FN];
    auto read_scales = [&](const uint8_t* S) {
#pragma unroll
      for (int f = 0; f < FM + FN; ++f) {
        const int row = f < FM ? arow[f] : brow[f - FM];
        if constexpr (NC == 4) {
          const uint2 v = *reinterpret_cast<const uint2*>(S + row * C::SCB + 8 * g);
          sw[f][0] = v.x; sw[f][1] = v.y;
        } else {
          sw[f][0] = *reinterpret_cast<const uint32_t*>(S + row * C::SCB + 4 * g);
          sw[f][1] = 0;
        }
      }
    };
    auto read_raw = [&](const uint8_t* L, int c2, int dst) {
#pragma unroll
      for (int f = 0; f < FM + FN; ++f) raw[dst][f] = frag(L, f, c2);
    };
    // The two E4M3 scales of chunk pair c2 (blocks 2c, 2c+1 of chunk c) as one
    // exact f16 pair per fragment; the multiplies broadcast one half.
    auto scales_of = [&](int c2, v2h* sd) {
#pragma unroll
      for (int f = 0; f < FM + FN; ++f)
        sd[f] = (c2 & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw[f][c2 >> 1], 1.0f, true)
                         : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sw[f][c2 >> 1], 1.0f, false);
    };
    auto decode = [&](const uint4* R, const v2h* sd, int s, v8h* op) {
#pragma unroll
      for (int f = 0; f < FM + FN; ++f) {
        const uint32_t w = s == 0 ? R[f].x : s == 1 ? R[f].y : s == 2 ? R[f].z : R[f].w;
        const v2h sd2 = (s >> 1) ? sd[f].yy : sd[f].xx;
        const v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * sd2;
        const v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * sd2;
        const v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * sd2;
        const v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * sd2;
        op[f] = (v8h){h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
      }
    };
    read_scales(lds_s[0]);
    read_raw(lds_c[0], 0, 0);
    v2h sdc[FM + FN];
    v8h op[FM + FN];
    scales_of(0, sdc);
    decode(raw[0], sdc, 0, op);
    for (int kt = 0; kt < nk; ++kt) {
      const int buf = kt & 1;
      const int kn = kt + 2 < nk ? kt + 2 : nk - 1;
#pragma unroll
      for (int c2 = 0; c2 < NC; ++c2) {
        const int cur = c2 & 1;
        if (c2 == NC - 1) {
          __syncthreads();
          // first operands and the scales of tile kt+1 (its buffer is complete after the barrier)
          read_scales(lds_s[buf ^ 1]);
          read_raw(lds_c[buf ^ 1], 0, cur ^ 1);
        } else {
          read_raw(lds_c[buf], c2 + 1, cur ^ 1);
#pragma unroll
          for (int q = 0; q < PER; ++q)
            if (c2 * PER + q < C::CODE_LOADS) stage(c2 * PER + q, buf ^ 1, kn);
          if (c2 == NC - 2) stage_scales(buf ^ 1, kn);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v8h opn[FM + FN];
          if (s < 3) {
            decode(raw[cur], sdc, s + 1, opn);
          } else {
            // first substep of the next chunk pair (or of tile kt+1)
            v2h sdn[FM + FN];
            scales_of(c2 == NC - 1 ? 0 : c2 + 1, sdn);
            decode(raw[cur ^ 1], sdn, 0, opn);
#pragma unroll
            for (int f = 0; f < FM + FN; ++f) sdc[f] = sdn[f];
          }
#pragma unroll
          for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(op[FM + j], op[i], acc[i][j], 0, 0, 0);
          // The next substep's decode (64 VALU: 8 fragments x 4 converts + 4
          // multiplies) in groups of five after the MFMAs, so it is done by the
          // 13th MFMA and the last ones leave room for the LDS and memory work
          // (groups of 4 and 6 measured slower, 3 much slower). The chunk
          // pair's LDS reads (the next chunk pair's fragments; after the K
          // tile's barrier also the next tile's scales) go one after each MFMA
          // of its first substep, and the staging of the next K tile (an LDS
          // write and a global load) after every other MFMA of its second:
          // placed by the compiler, the reads came late in the chunk pair, each
          // followed at once by a wait for it, and the staging as one burst.
#pragma unroll
          for (int m = 0; m < FM * FN; ++m) {
            __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
            if (s == 0) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
            if (s == 1 && (m & 1) == 0) {
              __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
              __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
            }
            __builtin_amdgcn_sched_group_barrier(kSchedValu, 5, 0);
          }
#pragma unroll
          for (int f = 0; f < FM + FN; ++f) op[f] = opn[f];
        }
        // One scheduling region per chunk pair (128 groups): as one region, the
        // K tile's 512 groups took the scheduler over ten minutes to place.
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }

  // Epilogue. The MFMAs take the B fragment as their first operand, so the
  // accumulator of fragments (i, j) is the transposed product: lane l holds
  // output row i*32 + l%32 (of the wave's 128 rows) and columns j*32 + 8*(r/4)
  // + 4*(l/32) + r%4, r = 0..15: four consecutive columns of one row per group
  // of four r. bf16 outputs are rounded to nearest even. `out` is the output
  // (or the FP32 partial tile), `rows`/`cols` the bounds of its valid part.
  auto epilogue = [&](auto bf16_tag, uint8_t* out, int64_t ld, uint32_t r0, uint32_t c0, uint32_t rows,
                      uint32_t cols, float alpha, bool interior) {
    constexpr bool OBF = decltype(bf16_tag)::value;
    constexpr int ES = OBF ? 2 : 4;  // output element bytes
    const uint32_t row0 = r0 + wm * WM;  // first output row / column of this wave
    const uint32_t col0 = c0 + wn * WN;
    auto out_at = [&](uint32_t row, uint32_t col) { return out + ((int64_t)row * ld + col) * ES; };
    if (interior) {
      // Interior tile: staged through LDS, 32 rows of the wave at a time, so
      // that every store instruction writes whole rows in 16-byte pieces
      // (non-temporal: the output is not read again by this kernel). The row
      // pitch of 132 outputs (4 of padding) keeps the LDS writes and reads free
      // of bank conflicts.
      constexpr int PITCH = 132 * ES;
      static_assert(4 * 32 * PITCH <= 2 * (C::LDS_CODES + C::LDS_SCALES), "output staging exceeds the LDS tiles");
      __syncthreads();  // every wave is done with the K loop's LDS tiles
      uint8_t* stage = lds + wave * 32 * PITCH;
#pragma unroll
      for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            v4f y = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            if constexpr (FMT == NV) y = y * alpha;
            uint8_t* d = stage + lr * PITCH + (j * 32 + 8 * q + 4 * g) * ES;
            if constexpr (OBF) {
              const v2bf lo = __builtin_convertvector((v2f){y[0], y[1]}, v2bf);
              const v2bf hi = __builtin_convertvector((v2f){y[2], y[3]}, v2bf);
              *reinterpret_cast<uint2*>(d) = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
            } else {
              *reinterpret_cast<v4f*>(d) = y;
            }
          }
        }
        // Read back 16 bytes per lane: a row of 128 outputs is 128 * ES / 16
        // lanes. All of the 32 rows' LDS reads go out before the first store
        // (the scheduling barrier keeps the compiler from pairing each read
        // with its store, which made every store wait for its own read's
        // round trip).
        constexpr int LPR = 128 * ES / 16;  // lanes per row
        constexpr int RPS = 64 / LPR;       // rows per store instruction
        constexpr int NST = 32 / RPS;       // store instructions per 32 rows
        uint4 v[NST];
#pragma unroll
        for (int k = 0; k < NST; ++k) {
          const int rr = k * RPS + lane / LPR;
          const int cc = (lane % LPR) * (16 / ES);
          v[k] = *reinterpret_cast<const uint4*>(stage + rr * PITCH + cc * ES);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < NST; ++k) {
          const int rr = k * RPS + lane / LPR;
          const int cc = (lane % LPR) * (16 / ES);
          __builtin_nontemporal_store(__builtin_bit_cast(v4u, v[k]), reinterpret_cast<v4u*>(out_at(row0 + i * 32 + rr, col0 + cc)));
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const uint32_t row = row0 + i * 32 + lr;
        if (row >= rows) continue;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t col = col0 + j * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
            if (col >= cols) continue;
            float y = acc[i][j][r];
            if constexpr (FMT == NV) y = y * alpha;
            if constexpr (OBF) {
              const v2bf b = __builtin_convertvector((v2f){y, y}, v2bf);
              *reinterpret_cast<uint16_t*>(out_at(row, col)) = __builtin_bit_cast(uint16_t, b[0]);
            } else {
              *reinterpret_cast<float*>(out_at(row, col)) = y;
            }
          }
        }
      }
    }
  };
  if constexpr (SPLIT) {
    // FP32 partial tile, row-major 256 x 256, unscaled (the reduction applies alpha).
    float* P = part + ((size_t)tt * split + sidx) * (BM * BN);
    epilogue(std::integral_constant<bool, false>{}, reinterpret_cast<uint8_t*>(P), BN, 0, 0, BM, BN, 1.0f, true);
  } else {
    float alpha = 1.0f;
    if constexpr (FMT == NV) alpha = (*a_ts) * (*b_ts);
    epilogue(std::integral_constant<bool, BF16OUT>{}, static_cast<uint8_t*>(cout), ldc, m0, n0, M, N, alpha,
             vec_ok && m0 + BM <= M && n0 + BN <= N);
  }
}

// MXFP4, K tile 256, whole output tiles: 512 threads = 8 waves, two per SIMD.
// Wave (wm, wn), wm = wave / 4, wn = wave % 4, owns 128 x 64 outputs (4 x 2
// fragments, 128 accumulators, so two waves fit a SIMD's registers), and one
// wave's barrier and LDS waits overlap the other's MFMAs. The staging, LDS
// layout, pipeline and epilogue are k_gemm's, for 512 threads.
template <bool BF16OUT>
__global__ __launch_bounds__(512, 1) void k_gemm_mx8(const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
                                                      const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs,
                                                      uint32_t M, uint32_t N, uint32_t K, uint32_t tiles_m,
                                                      uint32_t tiles_n, uint32_t group_m, uint32_t nfull,
                                                      void* __restrict__ cout, int64_t ldc, uint32_t vec_ok) {
  constexpr int ROWB = 128, CPR = 8, SCB = 8, NS = 4;
  constexpr int ROWS = BM + BN;                  // 512 staged rows per K tile
  constexpr int LDS_CODES = ROWS * ROWB, LDS_SCALES = ROWS * SCB;
  constexpr int NT = 512;
  constexpr int RPL = NT / CPR;                  // rows per load round (64)
  constexpr int CODE_LOADS = ROWS / RPL;         // 8 per thread
  constexpr int JA = BM / RPL;                   // loads that cover A rows (4)
  constexpr int PER = (CODE_LOADS + NS - 2) / (NS - 1);  // staging pieces per substep (3)
  constexpr int WM8 = 128, WN8 = 64, FM8 = 4, FN8 = 2;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * (LDS_CODES + LDS_SCALES)];
  uint8_t (*lds_c)[LDS_CODES] = reinterpret_cast<uint8_t (*)[LDS_CODES]>(lds);
  uint8_t (*lds_s)[LDS_SCALES] = reinterpret_cast<uint8_t (*)[LDS_SCALES]>(lds + 2 * LDS_CODES);

  const uint32_t gfull = (nfull + NXCD - 1) / NXCD * NXCD;
  const uint32_t t = (blockIdx.x % NXCD) * (gfull / NXCD) + blockIdx.x / NXCD;
  if (t >= nfull) return;
  uint32_t tm, tn;
  tile_coords(t, tiles_m, tiles_n, group_m, tm, tn);
  const uint32_t m0 = tm * BM, n0 = tn * BN;
  const int nk = (int)(K / 256);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: the scale rows' descriptor is scalar
  const int wm = wave >> 2, wn = wave & 3;
  const int g = lane >> 5;
  const int lr = lane & 31;
  const uint32_t kb_row = K / 2;
  const uint32_t ks_row = K / 32;
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(ac, M * kb_row);
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(bc, N * kb_row);
  const __amdgpu_buffer_rsrc_t rsa = make_rsrc(as, M * ks_row);
  const __amdgpu_buffer_rsrc_t rsb = make_rsrc(bs, N * ks_row);

  // Code loads: load j covers tile rows RPL*j + tid/CPR (A rows, then B), chunk tid%CPR.
  const int lrow = tid / CPR, lchk = tid % CPR;
  const uint32_t goff_a = (m0 + lrow) * kb_row + lchk * 16;
  const uint32_t goff_b = (n0 + lrow) * kb_row + lchk * 16;
  const int lds_w = lrow * ROWB + ((lchk ^ ((lrow >> 1) & (CPR - 1))) * 16);
  // Scale loads: one row per thread (A rows for tid < 256, then B rows).
  const bool srow_a = wave < BM / 64;
  const uint32_t soff = srow_a ? (m0 + tid) * ks_row : (n0 + tid - BM) * ks_row;
  const __amdgpu_buffer_rsrc_t rs = srow_a ? rsa : rsb;

  uint4 creg[CODE_LOADS];
  uint2 sreg;
  auto gload_code = [&](int j, int kt) {
    const uint32_t kc = (uint32_t)kt * ROWB;
    if (j < JA) creg[j] = bload16(ra, goff_a, (uint32_t)(j * RPL) * kb_row + kc);
    else creg[j] = bload16(rb, goff_b, (uint32_t)((j - JA) * RPL) * kb_row + kc);
  };
  auto gload_scales = [&](int kt) { sreg = bload8(rs, soff, (uint32_t)kt * SCB); };
  auto stage = [&](int j, int buf, int kt_next) {
    *reinterpret_cast<uint4*>(&lds_c[buf][lds_w + j * RPL * ROWB]) = creg[j];
    gload_code(j, kt_next);
  };
  auto stage_scales = [&](int buf, int kt_next) {
    *reinterpret_cast<uint2*>(&lds_s[buf][tid * SCB]) =
        make_uint2(__builtin_amdgcn_perm(sreg.y, sreg.x, 0x06040200u), __builtin_amdgcn_perm(sreg.y, sreg.x, 0x07050301u));
    gload_scales(kt_next);
  };

  v16f acc[FM8][FN8];
#pragma unroll
  for (int i = 0; i < FM8; ++i)
#pragma unroll
    for (int j = 0; j < FN8; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Fragment reads as k_gemm's: every row a lane reads is lr plus a multiple
  // of 32, so one swizzled chunk position serves all its fragments.
  const int T = (g ^ ((lr >> 1) & (CPR - 1))) * 16;
  const int a_lane = (wm * WM8 + lr) * ROWB, b_lane = (BM + wn * WN8 + lr) * ROWB;
  auto frag = [&](const uint8_t* L, int f, int k) {
    const int sw = T ^ (32 * k);
    return f < FM8 ? *reinterpret_cast<const uint4*>(L + a_lane + sw + f * 32 * ROWB)
                   : *reinterpret_cast<const uint4*>(L + b_lane + sw + (f - FM8) * 32 * ROWB);
  };
  const int arow0 = wm * WM8 + lr, brow0 = BM + wn * WN8 + lr;
  uint32_t sa[FM8], sb[FN8];
  uint4 a[2][FM8], b[2][FN8];
  auto read_scales = [&](const uint8_t* S) {
#pragma unroll
    for (int i = 0; i < FM8; ++i) sa[i] = *reinterpret_cast<const uint32_t*>(S + (arow0 + 32 * i) * SCB + 4 * g);
#pragma unroll
    for (int j = 0; j < FN8; ++j) sb[j] = *reinterpret_cast<const uint32_t*>(S + (brow0 + 32 * j) * SCB + 4 * g);
  };
  auto read_frags = [&](const uint8_t* L, int s, int dst) {
#pragma unroll
    for (int i = 0; i < FM8; ++i) a[dst][i] = frag(L, i, s);
#pragma unroll
    for (int j = 0; j < FN8; ++j) b[dst][j] = frag(L, FM8 + j, s);
  };

#pragma unroll
  for (int j = 0; j < CODE_LOADS; ++j) gload_code(j, 0);
  gload_scales(0);
#pragma unroll
  for (int j = 0; j < CODE_LOADS; ++j) stage(j, 0, nk > 1 ? 1 : 0);
  stage_scales(0, nk > 1 ? 1 : 0);
  __syncthreads();

  read_scales(lds_s[0]);
  read_frags(lds_c[0], 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    const int kn = kt + 2 < nk ? kt + 2 : nk - 1;
    uint32_t sa_keep[FM8], sb_keep[FN8];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int cur = s & 1;
      if (s == NS - 1) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < FM8; ++i) sa_keep[i] = sa[i];
#pragma unroll
        for (int j = 0; j < FN8; ++j) sb_keep[j] = sb[j];
        read_scales(lds_s[buf ^ 1]);
        read_frags(lds_c[buf ^ 1], 0, cur ^ 1);
      } else {
        read_frags(lds_c[buf], s + 1, cur ^ 1);
#pragma unroll
        for (int q = 0; q < PER; ++q)
          if (s * PER + q < CODE_LOADS) stage(s * PER + q, buf ^ 1, kn);
        if (s == NS - 2) stage_scales(buf ^ 1, kn);
      }
      const uint32_t* SA = (s == NS - 1) ? sa_keep : sa;
      const uint32_t* SB = (s == NS - 1) ? sb_keep : sb;
#pragma unroll
      for (int i = 0; i < FM8; ++i) {
        const v8i av = {(int)a[cur][i].x, (int)a[cur][i].y, (int)a[cur][i].z, (int)a[cur][i].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < FN8; ++j) {
          const v8i bv = {(int)b[cur][j].x, (int)b[cur][j].y, (int)b[cur][j].z, (int)b[cur][j].w, 0, 0, 0, 0};
          acc[i][j] = mfma_mx_sel(s, bv, av, acc[i][j], (int)SB[j], (int)SA[i]);
        }
      }
      if (s < NS - 1) {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, FM8 + FN8, 0);
#pragma unroll
        for (int q = 0; q < PER; ++q) {
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedDsWrite, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
          __builtin_amdgcn_sched_group_barrier(kSchedVmemRead, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, FM8 * FN8 - 2 * PER > 0 ? FM8 * FN8 - 2 * PER : 0, 0);
      } else {
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * (FM8 + FN8), 0);
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, FM8 * FN8, 0);
      }
    }
  }

  // Epilogue: lane l of fragment (i, j) holds output row 32 i + l % 32 of the
  // wave's 128 and columns 32 j + 8 (r / 4) + 4 (l / 32) + r % 4 of its 64.
  constexpr int ES = BF16OUT ? 2 : 4;
  const uint32_t row0 = m0 + wm * WM8, col0 = n0 + wn * WN8;
  auto out_at = [&](uint32_t row, uint32_t col) {
    return static_cast<uint8_t*>(cout) + ((int64_t)row * ldc + col) * ES;
  };
  if (vec_ok && m0 + BM <= M && n0 + BN <= N) {
    constexpr int PITCH = 68 * ES;
    static_assert(8 * 32 * PITCH <= 2 * (LDS_CODES + LDS_SCALES), "output staging exceeds the LDS tiles");
    __syncthreads();
    uint8_t* stg = lds + wave * 32 * PITCH;
#pragma unroll
    for (int i = 0; i < FM8; ++i) {
#pragma unroll
      for (int j = 0; j < FN8; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const v4f y = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
          uint8_t* d = stg + lr * PITCH + (j * 32 + 8 * q + 4 * g) * ES;
          if constexpr (BF16OUT) {
            const v2bf lo = __builtin_convertvector((v2f){y[0], y[1]}, v2bf);
            const v2bf hi = __builtin_convertvector((v2f){y[2], y[3]}, v2bf);
            *reinterpret_cast<uint2*>(d) = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
          } else {
            *reinterpret_cast<v4f*>(d) = y;
          }
        }
      }
      constexpr int LPR = 64 * ES / 16;   // lanes per 64-output row
      constexpr int RPS = 64 / LPR;       // rows per store instruction
      constexpr int NST = 32 / RPS;       // store instructions per 32 rows
      uint4 v[NST];                       // all LDS reads before the stores, as in k_gemm
#pragma unroll
      for (int k = 0; k < NST; ++k) {
        const int rr = k * RPS + lane / LPR;
        const int cc = (lane % LPR) * (16 / ES);
        v[k] = *reinterpret_cast<const uint4*>(stg + rr * PITCH + cc * ES);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < NST; ++k) {
        const int rr = k * RPS + lane / LPR;
        const int cc = (lane % LPR) * (16 / ES);
        __builtin_nontemporal_store(__builtin_bit_cast(v4u, v[k]), reinterpret_cast<v4u*>(out_at(row0 + i * 32 + rr, col0 + cc)));
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < FM8; ++i) {
      const uint32_t row = row0 + i * 32 + lr;
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < FN8; ++j) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t col = col0 + j * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
          if (col >= N) continue;
          const float y = acc[i][j][r];
          if constexpr (BF16OUT) {
            const v2bf bb = __builtin_convertvector((v2f){y, y}, v2bf);
            *reinterpret_cast<uint16_t*>(out_at(row, col)) = __builtin_bit_cast(uint16_t, bb[0]);
          } else {
            *reinterpret_cast<float*>(out_at(row, col)) = y;
          }
        }
      }
    }
  }
}

// Sum of the `split` FP32 partial tiles of each split output tile, in split
// order, times alpha (NVFP4: s_gA * s_gB), converted and stored. Workgroup
// (tile tt, 32-row slab): lane c of a row holds its columns 4c .. 4c+3, so
// every load and store instruction covers whole 1 KB partial rows.
template <int FMT, bool BF16OUT>
__global__ __launch_bounds__(256) void k_split_reduce(const float* __restrict__ part, uint32_t nfull,
                                                      uint32_t split, uint32_t tiles_m, uint32_t tiles_n,
                                                      uint32_t group_m, const float* __restrict__ a_ts,
                                                      const float* __restrict__ b_ts, uint32_t M, uint32_t N,
                                                      void* __restrict__ cout, int64_t ldc, uint32_t vec_ok) {
  const uint32_t tt = blockIdx.x / (BM / 32);
  const uint32_t slab = blockIdx.x % (BM / 32);
  uint32_t tm, tn;
  tile_coords(nfull + tt, tiles_m, tiles_n, group_m, tm, tn);
  float alpha = 1.0f;
  if constexpr (FMT == NV) alpha = (*a_ts) * (*b_ts);
  const int c4 = threadIdx.x % 64;
  const uint32_t col = tn * BN + 4 * c4;
  const float* P = part + (size_t)tt * split * (BM * BN);
  constexpr int ES = BF16OUT ? 2 : 4;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int r = (int)slab * 32 + k * 4 + (int)threadIdx.x / 64;
    const uint32_t row = tm * BM + r;
    v4f y = __builtin_nontemporal_load(reinterpret_cast<const v4f*>(P + r * BN + 4 * c4));
    for (uint32_t sp = 1; sp < split; ++sp)
      y += __builtin_nontemporal_load(reinterpret_cast<const v4f*>(P + (size_t)sp * (BM * BN) + r * BN + 4 * c4));
    if constexpr (FMT == NV) y = y * alpha;
    if (row >= M) continue;
    uint8_t* d = static_cast<uint8_t*>(cout) + ((int64_t)row * ldc + col) * ES;
    if (vec_ok && col + 4 <= N) {
      if constexpr (BF16OUT) {
        const v2bf lo = __builtin_convertvector((v2f){y[0], y[1]}, v2bf);
        const v2bf hi = __builtin_convertvector((v2f){y[2], y[3]}, v2bf);
        *reinterpret_cast<uint2*>(d) = make_uint2(__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi));
      } else {
        *reinterpret_cast<v4f*>(d) = y;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (col + e >= N) break;
        if constexpr (BF16OUT) {
          const v2bf b = __builtin_convertvector((v2f){y[e], y[e]}, v2bf);
          *reinterpret_cast<uint16_t*>(d + e * ES) = __builtin_bit_cast(uint16_t, b[0]);
        } else {
          *reinterpret_cast<float*>(d + e * ES) = y[e];
        }
      }
    }
  }
}

// How the output tiles are cut: tiles whole, and the tiles of the last,
// partial wave (one workgroup per CU: the LDS tiles take most of a CU's LDS)
// split along K when that shortens the wave enough to pay for the partial
// sums. The chip is power-limited under this load: with all 256 CUs busy it
// holds about 1.7 GHz, with fewer the clock rises towards 2.4 GHz, so a wave
// of n tiles takes max(n / 256, 1.7 / 2.4) of a full wave's time (the
// Llama-7B wgrad's last wave of 176 tiles runs nearly as fast as a split of
// it would, measured). Splitting in S pieces costs writing and re-reading
// S + 1 tiles of FP32 per split tile (at about 5 TB/s) and a second launch,
// against a tile time of about 2 us per 256-deep K tile (the faster, MXFP4,
// kernel). kPlanCUs is the CU count of the gfx950 parts (MI350X, MI355X).
constexpr uint32_t kPlanCUs = 256;
struct SplitPlan {
  uint32_t tiles_m, tiles_n, nfull, ntail, split;
};
double wave_time(uint32_t n) { return std::max((double)n / kPlanCUs, 1.7 / 2.4); }
SplitPlan split_plan(int64_t M, int64_t N, int64_t K) {
  SplitPlan p;
  p.tiles_m = (uint32_t)((M + BM - 1) / BM);
  p.tiles_n = (uint32_t)((N + BN - 1) / BN);
  const uint32_t tiles = p.tiles_m * p.tiles_n;
  p.nfull = tiles;
  p.ntail = 0;
  p.split = 1;
  const int bk = K % 256 == 0 ? 256 : 128;
  const int64_t nk = K / bk;
  const uint32_t tail = tiles % kPlanCUs;
  if (tail == 0) return p;
  const double tile_us = (double)nk * 2.0 * bk / 256;
  double best = wave_time(tail);
  for (uint32_t sp = 2; sp <= 8 && nk / sp >= 8; ++sp) {
    const uint32_t units = tail * sp;
    const uint32_t waves = (units + kPlanCUs - 1) / kPlanCUs;
    const double t = ((waves - 1) + wave_time(units - (waves - 1) * kPlanCUs)) / sp;
    const double extra_us = (double)(sp + 1) * tail * (BM * BN * 4) / 5e6 + 5.0;
    const double cost = t + extra_us / tile_us + 0.005 * sp;
    if (cost < best) {
      best = cost;
      p.split = sp;
    }
  }
  if (p.split > 1) {
    p.ntail = tail;
    p.nfull = tiles - tail;
  }
  return p;
}

template <int FMT, int BK>
void launch(const GemmArgs& g, hipStream_t s) {
  SplitPlan p = split_plan(g.M, g.N, g.K);
  if (!g.split_ws) {
    p.nfull += p.ntail;
    p.ntail = 0;
    p.split = 1;
  }
  const uint32_t group_m = 8;
  const dim3 block(256);
  // Interior tiles store 16-byte pieces of output rows: the base address and
  // every row start must be 16-byte aligned.
  const int64_t es = g.bf16out ? 2 : 4;
  const uint32_t vec_ok = (g.ldc * es) % 16 == 0 && reinterpret_cast<uintptr_t>(g.c) % 16 == 0;
  float* part = p.ntail ? g.split_ws : nullptr;
  if (p.nfull && FMT == MX && BK == 256) {
    const dim3 grid((p.nfull + NXCD - 1) / NXCD * NXCD);
    if (g.bf16out)
      hipLaunchKernelGGL((k_gemm_mx8<true>), grid, dim3(512), 0, s, g.a_codes, g.a_scales, g.b_codes, g.b_scales,
                         (uint32_t)g.M, (uint32_t)g.N, (uint32_t)g.K, p.tiles_m, p.tiles_n, group_m, p.nfull, g.c,
                         g.ldc, vec_ok);
    else
      hipLaunchKernelGGL((k_gemm_mx8<false>), grid, dim3(512), 0, s, g.a_codes, g.a_scales, g.b_codes, g.b_scales,
                         (uint32_t)g.M, (uint32_t)g.N, (uint32_t)g.K, p.tiles_m, p.tiles_n, group_m, p.nfull, g.c,
                         g.ldc, vec_ok);
  } else if (p.nfull) {
    const dim3 grid((p.nfull + NXCD - 1) / NXCD * NXCD);
    if (g.bf16out)
      hipLaunchKernelGGL((k_gemm<FMT, BK, true, false>), grid, block, 0, s, g.a_codes, g.a_scales, g.b_codes,
                         g.b_scales, g.a_tscale, g.b_tscale, (uint32_t)g.M, (uint32_t)g.N, (uint32_t)g.K,
                         p.tiles_m, p.tiles_n, group_m, p.nfull, p.ntail, p.split, part, g.c, g.ldc, vec_ok);
    else
      hipLaunchKernelGGL((k_gemm<FMT, BK, false, false>), grid, block, 0, s, g.a_codes, g.a_scales, g.b_codes,
                         g.b_scales, g.a_tscale, g.b_tscale, (uint32_t)g.M, (uint32_t)g.N, (uint32_t)g.K,
                         p.tiles_m, p.tiles_n, group_m, p.nfull, p.ntail, p.split, part, g.c, g.ldc, vec_ok);
  }
  if (p.ntail) {
    // The split pieces after the whole tiles (a partial wave of whole tiles
    // is exactly what the split replaces), then their sum.
    const dim3 grid(p.split * ((p.ntail + NXCD - 1) / NXCD * NXCD));
    hipLaunchKernelGGL((k_gemm<FMT, BK, false, true>), grid, block, 0, s, g.a_codes, g.a_scales, g.b_codes,
                       g.b_scales, g.a_tscale, g.b_tscale, (uint32_t)g.M, (uint32_t)g.N, (uint32_t)g.K,
                       p.tiles_m, p.tiles_n, group_m, p.nfull, p.ntail, p.split, part, g.c, g.ldc, vec_ok);
  }
  if (!p.ntail) return;
  const dim3 rgrid(p.ntail * (BM / 32));
  if (g.bf16out)
    hipLaunchKernelGGL((k_split_reduce<FMT, true>), rgrid, block, 0, s, part, p.nfull, p.split, p.tiles_m,
                       p.tiles_n, group_m, g.a_tscale, g.b_tscale, (uint32_t)g.M, (uint32_t)g.N, g.c, g.ldc,
                       vec_ok);
  else
    hipLaunchKernelGGL((k_split_reduce<FMT, false>), rgrid, block, 0, s, part, p.nfull, p.split, p.tiles_m,
                       p.tiles_n, group_m, g.a_tscale, g.b_tscale, (uint32_t)g.M, (uint32_t)g.N, g.c, g.ldc,
                       vec_ok);
}

}  // namespace

size_t fp4i_gemm_split_bytes(int64_t M, int64_t N, int64_t K) {
  const SplitPlan p = split_plan(M, N, K);
  return (size_t)p.ntail * p.split * (BM * BN) * sizeof(float);
}

bool fp4i_gemm_fits(int64_t M, int64_t N, int64_t K) {
  // Buffer offsets are 32-bit: each operand's codes must stay below 2^31 bytes.
  return M * (K / 2) < (int64_t(1) << 31) && N * (K / 2) < (int64_t(1) << 31);
}

void fp4i_launch_gemm(const GemmArgs& g, hipStream_t s) {
  const bool k256 = g.K % 256 == 0;
  if (g.fmt == NV) {
    if (k256) launch<NV, 256>(g, s);
    else launch<NV, 128>(g, s);
  } else {
    if (k256) launch<MX, 256>(g, s);
    else launch<MX, 128>(g, s);
  }
}
