// abi.cpp -- the C ABI of libfp4 (declared in include/fp4.h): argument
// validation, then kernel launches on the caller's stream. Nothing is
// launched when validation fails; the library never allocates or synchronizes.
#include "fp4.h"

#include <hip/hip_runtime.h>

#include <mutex>

#include "fp4_internal.hpp"

#include <cstdint>

// Workspace of fp4_gemm_noalloc: a device array each GPU holds from the
// library's load until the process ends. Host code never uses this name as a
// device address (on the host it is a stand-in); it uses the address
// hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) uint8_t scratch[FP4_GEMM_NOALLOC_MAX_BYTES];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
int block_of(int32_t fmt) { return fmt == FP4_NVFP4 ? 16 : 32; }
bool valid_fmt(int32_t fmt) { return fmt == FP4_NVFP4 || fmt == FP4_MXFP4; }
bool valid_dtype(int d) { return d == FP4_DTYPE_F32 || d == FP4_DTYPE_BF16; }

fp4_status hip_status() {
  return hipGetLastError() == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

// Work counts are kept in 32 bits inside the kernels.
bool fits_tasks(int64_t R, int64_t C) {
  const int64_t spr = (C + 511) / 512;
  return R <= (int64_t)0xFFFFFFFF / (spr > 0 ? spr : 1);
}

fp4_status check_matrix(const void* src, int dt, int64_t R, int64_t C, int64_t ld) {
  if (!src) return FP4_ERR_NULL;
  if (!valid_dtype(dt)) return FP4_ERR_ARG;
  if (R <= 0 || C <= 0 || C % 8 != 0 || ld < C) return FP4_ERR_SHAPE;
  if (!aligned16(src) || ld % 8 != 0) return FP4_ERR_ALIGN;
  if (!fits_tasks(R, C)) return FP4_ERR_SHAPE;
  return FP4_OK;
}

bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

// Every check of a single-orientation quantization, before anything is enqueued.
fp4_status check_quant(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld, fp4_axis axis,
                       fp4_rounding rnd, uint64_t index_offset, const fp4_tensor* out) {
  if (!out) return FP4_ERR_NULL;
  fp4_status st = check_matrix(src, src_t, R, C, ld);
  if (st != FP4_OK) return st;
  if (axis != FP4_AXIS_COLS && axis != FP4_AXIS_ROWS) return FP4_ERR_ARG;
  if (rnd != FP4_RTN && rnd != FP4_SR) return FP4_ERR_ARG;
  if (!valid_fmt(out->fmt)) return FP4_ERR_ARG;
  if (!out->codes || !out->scales) return FP4_ERR_NULL;
  if (!aligned16(out->codes) || !aligned16(out->scales)) return FP4_ERR_ALIGN;
  const bool nv = out->fmt == FP4_NVFP4;
  if (nv && (!out->amax || !out->tscale)) return FP4_ERR_NULL;
  const int B = block_of(out->fmt);
  const int64_t blocked = axis == FP4_AXIS_ROWS ? R : C;
  if (blocked % B != 0) return FP4_ERR_SHAPE;
  if (rnd == FP4_SR && index_offset % 8 != 0) return FP4_ERR_ALIGN;
  if (axis == FP4_AXIS_ROWS && (R + 255) / 256 * ((C + 63) / 64) > 0x7FFFFFFF)
    return FP4_ERR_SHAPE;
  return FP4_OK;
}

// Enqueue a quantization that check_quant accepted.
// idx_rows: the row count of the ROWS orientation's SR index (0: R).
fp4_status launch_quant(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld, fp4_axis axis,
                        fp4_rounding rnd, uint64_t seed, uint64_t index_offset, int amax_ready,
                        fp4_tensor* out, double* noise, hipStream_t s, int64_t idx_rows = 0) {
  const bool nv = out->fmt == FP4_NVFP4;
  if (nv && !amax_ready) {
    if (out->had_on)
      fp4i_launch_amax_rot16(src, src_t == FP4_DTYPE_BF16, R, C, ld, axis == FP4_AXIS_ROWS,
                             out->had_signs, out->amax, s);
    else
      fp4i_launch_amax(src, src_t == FP4_DTYPE_BF16, R, C, ld, out->amax, s);
    const fp4_status st = hip_status();
    if (st != FP4_OK) return st;
  }
  QuantArgs a;
  a.src = src;
  a.bf16 = src_t == FP4_DTYPE_BF16;
  a.R = R;
  a.C = C;
  a.ld = ld;
  a.rows_axis = axis == FP4_AXIS_ROWS;
  a.fmt = out->fmt;
  a.sr = rnd == FP4_SR;
  a.seed = seed;
  a.offset = index_offset;
  a.idx_rows = idx_rows;
  a.had_on = out->had_on != 0;
  a.signs = out->had_signs;
  a.codes = out->codes;
  a.scales = out->scales;
  a.amax = out->amax;
  a.tscale = out->tscale;
  a.noise = noise;
  fp4i_launch_quant(a, s);
  out->rows = a.rows_axis ? C : R;
  out->cols = a.rows_axis ? R : C;
  return hip_status();
}

fp4_status quantize_impl(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                         fp4_axis axis, fp4_rounding rnd, uint64_t seed, uint64_t index_offset,
                         int amax_ready, fp4_tensor* out, double* noise, fp4_stream_t stream) {
  const fp4_status st = check_quant(src, src_t, R, C, ld, axis, rnd, index_offset, out);
  if (st != FP4_OK) return st;
  return launch_quant(src, src_t, R, C, ld, axis, rnd, seed, index_offset, amax_ready, out, noise,
                      reinterpret_cast<hipStream_t>(stream));
}

// A row shard (rows row_offset .. row_offset + R - 1 of a rows_total-row
// tensor): every check that depends on where the shard lies. Blocks along
// rows (axis ROWS, or the dual's second orientation) must not straddle
// shards; the ROWS index c * rows_total + row must keep 8-element Philox
// calls aligned.
fp4_status check_shard(int64_t R, int64_t C, int64_t row_offset, int64_t rows_total, bool blocks_along_rows,
                       int B) {
  if (row_offset < 0 || rows_total <= 0 || R <= 0 || C <= 0) return FP4_ERR_SHAPE;
  if (row_offset > rows_total || R > rows_total - row_offset) return FP4_ERR_SHAPE;
  if (rows_total > INT64_MAX / C) return FP4_ERR_SHAPE;
  if (rows_total % 8 != 0) return FP4_ERR_ALIGN;
  if (blocks_along_rows && row_offset % B != 0) return FP4_ERR_ALIGN;
  return FP4_OK;
}

// ---------------------------------------------------------------- GEMM operands
constexpr size_t kWsAlign = 256;
size_t round_up(size_t n) { return (n + kWsAlign - 1) / kWsAlign * kWsAlign; }

// The matrix a GEMM operand stands for (rows x K, blocked along K), and for a
// RAW operand the quantization that produces it.
struct OperandView {
  int64_t rows = 0, k = 0;
  int32_t fmt = 0, had_on = 0;
  uint32_t had_signs = 0;
  bool raw = false;
  fp4_tensor q{};       // the quantized operand (for RAW: carved from the workspace)
  size_t ws_bytes = 0;  // RAW: workspace this operand takes
};

// Workspace pieces of a RAW operand: codes, scales, then (NVFP4) amax and
// tscale, each on a 256-byte boundary.
size_t raw_ws_bytes(int64_t rows, int64_t k, int32_t fmt) {
  size_t n = round_up((size_t)rows * (size_t)(k / 2)) + round_up((size_t)rows * (size_t)(k / block_of(fmt)));
  if (fmt == FP4_NVFP4) n += kWsAlign;
  return n;
}

// Shape, kind and format of an operand (what fp4_gemm_workspace_bytes needs).
fp4_status view_operand(const fp4_operand* op, OperandView* v) {
  if (!op) return FP4_ERR_NULL;
  if (op->kind == FP4_OPERAND_QUANTIZED) {
    if (!op->q) return FP4_ERR_NULL;
    if (!valid_fmt(op->q->fmt)) return FP4_ERR_ARG;
    v->raw = false;
    v->q = *op->q;
    v->rows = op->q->rows;
    v->k = op->q->cols;
    v->fmt = op->q->fmt;
    v->had_on = op->q->had_on != 0;
    v->had_signs = op->q->had_signs;
    return FP4_OK;
  }
  if (op->kind != FP4_OPERAND_RAW) return FP4_ERR_ARG;
  if (!valid_fmt(op->fmt)) return FP4_ERR_ARG;
  if (op->rows <= 0 || op->k <= 0 || op->k % block_of(op->fmt) != 0) return FP4_ERR_SHAPE;
  v->raw = true;
  v->rows = op->rows;
  v->k = op->k;
  v->fmt = op->fmt;
  v->had_on = op->had_on != 0;
  v->had_signs = op->had_signs;
  v->ws_bytes = raw_ws_bytes(op->rows, op->k, op->fmt);
  return FP4_OK;
}

// Source matrix of a RAW operand as fp4_quantize sees it: N stores rows x K
// (blocks along C), T stores K x rows (blocks along R).
struct RawSource {
  int64_t R, C;
  fp4_axis axis;
};
RawSource raw_source(const fp4_operand* op) {
  if (op->layout == FP4_LAYOUT_T) return {op->k, op->rows, FP4_AXIS_ROWS};
  return {op->rows, op->k, FP4_AXIS_COLS};
}

// Point v->q at the operand's workspace pieces starting at base.
void carve_raw(OperandView* v, uint8_t* base) {
  const size_t nc = round_up((size_t)v->rows * (size_t)(v->k / 2));
  const size_t ns = round_up((size_t)v->rows * (size_t)(v->k / block_of(v->fmt)));
  v->q = fp4_tensor{};
  v->q.codes = base;
  v->q.scales = base + nc;
  if (v->fmt == FP4_NVFP4) {
    v->q.amax = reinterpret_cast<float*>(base + nc + ns);
    v->q.tscale = reinterpret_cast<float*>(base + nc + ns + 4);
  }
  v->q.rows = v->rows;
  v->q.cols = v->k;
  v->q.fmt = v->fmt;
  v->q.had_on = v->had_on;
  v->q.had_signs = v->had_signs;
}

// Every check of a RAW operand's quantization (v->q already carved).
fp4_status check_raw(const fp4_operand* op, const OperandView& v) {
  if (op->layout != FP4_LAYOUT_N && op->layout != FP4_LAYOUT_T) return FP4_ERR_ARG;
  const RawSource rs = raw_source(op);
  return check_quant(op->data, (fp4_dtype)op->dtype, rs.R, rs.C, op->ld, rs.axis, (fp4_rounding)op->rnd,
                     op->index_offset, &v.q);
}

// The GEMM proper on two quantized operands blocked along K.
fp4_status check_gemm_pair(const fp4_tensor* A, const fp4_tensor* B, fp4_dtype out_t, const void* C,
                           int64_t ldc) {
  if (!valid_dtype(out_t)) return FP4_ERR_ARG;
  if (!A->codes || !A->scales || !B->codes || !B->scales) return FP4_ERR_NULL;
  if (A->fmt != B->fmt) return FP4_ERR_UNSUPPORTED;
  if ((A->had_on != 0) != (B->had_on != 0)) return FP4_ERR_UNSUPPORTED;
  if (A->had_on && A->had_signs != B->had_signs) return FP4_ERR_UNSUPPORTED;
  if (A->fmt == FP4_NVFP4 && (!A->tscale || !B->tscale)) return FP4_ERR_NULL;
  if (A->rows <= 0 || B->rows <= 0 || A->cols <= 0 || A->cols != B->cols || A->cols % 128 != 0)
    return FP4_ERR_SHAPE;
  if (!fp4i_gemm_fits(A->rows, B->rows, A->cols)) return FP4_ERR_SHAPE;
  if (ldc < B->rows) return FP4_ERR_SHAPE;
  if (!aligned16(A->codes) || !aligned16(B->codes) || !aligned16(A->scales) || !aligned16(B->scales))
    return FP4_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(C) & (out_t == FP4_DTYPE_F32 ? 3u : 1u)) != 0) return FP4_ERR_ALIGN;
  return FP4_OK;
}

void launch_gemm_pair(const fp4_tensor* A, const fp4_tensor* B, fp4_dtype out_t, void* C, int64_t ldc,
                      float* split_ws, hipStream_t s) {
  GemmArgs g;
  g.a_codes = A->codes;
  g.a_scales = A->scales;
  g.b_codes = B->codes;
  g.b_scales = B->scales;
  g.a_tscale = A->tscale;
  g.b_tscale = B->tscale;
  g.M = A->rows;
  g.N = B->rows;
  g.K = A->cols;
  g.fmt = A->fmt;
  g.bf16out = out_t == FP4_DTYPE_BF16;
  g.c = C;
  g.ldc = ldc;
  g.split_ws = split_ws;
  fp4i_launch_gemm(g, s);
}

fp4_status quantize_dual_impl(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                              fp4_rounding rnd_cols, uint64_t seed_cols, uint64_t index_offset_cols,
                              fp4_rounding rnd_rows, uint64_t seed_rows, uint64_t index_offset_rows,
                              int amax_ready, fp4_tensor* out_cols, fp4_tensor* out_rows,
                              double* noise_cols, double* noise_rows, fp4_stream_t stream,
                              int64_t idx_rows = 0) {
  if (!out_cols || !out_rows) return FP4_ERR_NULL;
  fp4_status st = check_matrix(src, src_t, R, C, ld);
  if (st != FP4_OK) return st;
  if ((rnd_cols != FP4_RTN && rnd_cols != FP4_SR) || (rnd_rows != FP4_RTN && rnd_rows != FP4_SR))
    return FP4_ERR_ARG;
  if (!valid_fmt(out_cols->fmt) || !valid_fmt(out_rows->fmt)) return FP4_ERR_ARG;
  if (out_cols->fmt != out_rows->fmt) return FP4_ERR_UNSUPPORTED;
  for (const fp4_tensor* o : {out_cols, out_rows}) {
    if (!o->codes || !o->scales) return FP4_ERR_NULL;
    if (!aligned16(o->codes) || !aligned16(o->scales)) return FP4_ERR_ALIGN;
  }
  const bool nv = out_cols->fmt == FP4_NVFP4;
  const bool had_c = out_cols->had_on != 0, had_r = out_rows->had_on != 0;
  // NVFP4 with a rotation: the two orientations' values have different amaxes,
  // each kept in its own descriptor.
  const bool two_amax = nv && (had_c || had_r);
  if (nv && (!out_cols->amax || !out_cols->tscale || !out_rows->tscale)) return FP4_ERR_NULL;
  if (two_amax && !out_rows->amax) return FP4_ERR_NULL;
  if (two_amax && (out_rows->amax == out_cols->amax || out_rows->tscale == out_cols->tscale))
    return FP4_ERR_UNSUPPORTED;
  const int B = block_of(out_cols->fmt);
  if (R % B != 0 || C % B != 0) return FP4_ERR_SHAPE;
  if ((rnd_cols == FP4_SR && index_offset_cols % 8 != 0) || (rnd_rows == FP4_SR && index_offset_rows % 8 != 0))
    return FP4_ERR_ALIGN;
  if ((R + 127) / 128 * ((C + 127) / 128) > 0x7FFFFFFF) return FP4_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (nv && !amax_ready) {
    const bool bf = src_t == FP4_DTYPE_BF16;
    if (two_amax)
      fp4i_launch_amax_pair(src, bf, R, C, ld, had_c, out_cols->had_signs, had_r, out_rows->had_signs,
                            out_cols->amax, out_rows->amax, s);
    else
      fp4i_launch_amax(src, bf, R, C, ld, out_cols->amax, s);
    st = hip_status();
    if (st != FP4_OK) return st;
  }
  DualArgs a;
  a.src = src;
  a.bf16 = src_t == FP4_DTYPE_BF16;
  a.R = R;
  a.C = C;
  a.ld = ld;
  a.fmt = out_cols->fmt;
  a.had_c = had_c;
  a.had_r = had_r;
  a.sr_c = rnd_cols == FP4_SR;
  a.sr_r = rnd_rows == FP4_SR;
  a.seed_c = seed_cols;
  a.offset_c = index_offset_cols;
  a.seed_r = seed_rows;
  a.offset_r = index_offset_rows;
  a.idx_rows_r = idx_rows;
  a.signs_c = out_cols->had_signs;
  a.signs_r = out_rows->had_signs;
  a.codes_c = out_cols->codes;
  a.scales_c = out_cols->scales;
  a.codes_r = out_rows->codes;
  a.scales_r = out_rows->scales;
  a.amax_c = out_cols->amax;
  a.amax_r = two_amax ? out_rows->amax : out_cols->amax;
  a.tscale_c = out_cols->tscale;
  a.tscale_r = out_rows->tscale;
  a.amax_copy = (nv && !two_amax && out_rows->amax && out_rows->amax != out_cols->amax)
                    ? out_rows->amax : nullptr;
  a.noise_c = noise_cols;
  a.noise_r = noise_rows;
  fp4i_launch_quant_dual(a, s);
  out_cols->rows = R;
  out_cols->cols = C;
  out_rows->rows = C;
  out_rows->cols = R;
  return hip_status();
}

// Bytes of the optional split-K area (after the RAW pieces) for a valid pair.
size_t splitk_bytes(const OperandView& va, const OperandView& vb) {
  if (va.fmt != vb.fmt || va.k != vb.k || va.k <= 0 || va.k % 128 != 0) return 0;
  if (!fp4i_gemm_fits(va.rows, vb.rows, va.k)) return 0;
  return round_up(fp4i_gemm_split_bytes(va.rows, vb.rows, va.k));
}

// The product, with RAW operands quantized into ws first; with allow_split and
// room in ws after the RAW pieces, the last partial wave of output tiles is
// split along K.
fp4_status gemm_impl(const fp4_operand* A, const fp4_operand* B, fp4_dtype out_t, void* C, int64_t ldc,
                     void* ws, size_t ws_bytes, bool allow_split, fp4_stream_t stream) {
  if (!C) return FP4_ERR_NULL;
  OperandView va, vb;
  fp4_status st = view_operand(A, &va);
  if (st != FP4_OK) return st;
  st = view_operand(B, &vb);
  if (st != FP4_OK) return st;
  // Format, rotation and K agreement first: a RAW operand's K must suit the
  // product before its workspace is sized.
  if (va.fmt != vb.fmt) return FP4_ERR_UNSUPPORTED;
  if (va.had_on != vb.had_on || (va.had_on && va.had_signs != vb.had_signs)) return FP4_ERR_UNSUPPORTED;
  if (va.k != vb.k || va.k <= 0 || va.k % 128 != 0 || va.rows <= 0 || vb.rows <= 0) return FP4_ERR_SHAPE;
  if (!fp4i_gemm_fits(va.rows, vb.rows, va.k)) return FP4_ERR_SHAPE;
  const size_t need = va.ws_bytes + vb.ws_bytes;
  if (need > 0) {
    if (!ws || ws_bytes < need || (reinterpret_cast<uintptr_t>(ws) % kWsAlign) != 0) return FP4_ERR_WORKSPACE;
    uint8_t* base = static_cast<uint8_t*>(ws);
    if (va.raw) carve_raw(&va, base);
    if (vb.raw) carve_raw(&vb, base + va.ws_bytes);
    if (va.raw && (st = check_raw(A, va)) != FP4_OK) return st;
    if (vb.raw && (st = check_raw(B, vb)) != FP4_OK) return st;
  }
  st = check_gemm_pair(&va.q, &vb.q, out_t, C, ldc);
  if (st != FP4_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  for (int i = 0; i < 2; ++i) {
    const fp4_operand* op = i == 0 ? A : B;
    OperandView* v = i == 0 ? &va : &vb;
    if (!v->raw) continue;
    const RawSource rs = raw_source(op);
    st = launch_quant(op->data, (fp4_dtype)op->dtype, rs.R, rs.C, op->ld, rs.axis, (fp4_rounding)op->rnd,
                      op->seed, op->index_offset, 0, &v->q, nullptr, s);
    if (st != FP4_OK) return st;
  }
  float* split_ws = nullptr;
  const size_t opt = allow_split ? splitk_bytes(va, vb) : 0;
  if (opt > 0 && ws && (reinterpret_cast<uintptr_t>(ws) % kWsAlign) == 0 && ws_bytes >= need + opt)
    split_ws = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + need);
  launch_gemm_pair(&va.q, &vb.q, out_t, C, ldc, split_ws, s);
  return hip_status();
}

// Every check of a dequantization (both entry points).
fp4_status check_dequant(const fp4_tensor* q, fp4_dtype dst_t, const void* dst, int64_t ld) {
  if (!q || !dst) return FP4_ERR_NULL;
  if (!valid_dtype(dst_t) || !valid_fmt(q->fmt)) return FP4_ERR_ARG;
  if (!q->codes || !q->scales) return FP4_ERR_NULL;
  if (q->fmt == FP4_NVFP4 && !q->tscale) return FP4_ERR_NULL;
  if (q->rows <= 0 || q->cols <= 0 || q->cols % block_of(q->fmt) != 0 || ld < q->cols)
    return FP4_ERR_SHAPE;
  if (!fits_tasks(q->rows, q->cols)) return FP4_ERR_SHAPE;
  if (!aligned16(dst) || ld % 8 != 0 || !aligned16(q->codes)) return FP4_ERR_ALIGN;
  return FP4_OK;
}

// The address of `scratch` on each device, looked up once per device with
// that device current (each GPU holds its own copy at its own address).
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];

fp4_status scratch_on_current_device(void** p) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FP4_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return FP4_ERR_UNSUPPORTED;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) == hipSuccess) g_scratch_ptr[dev] = ptr;
    else (void)hipGetLastError();
  });
  if (!g_scratch_ptr[dev]) return FP4_ERR_HIP;
  *p = g_scratch_ptr[dev];
  return FP4_OK;
}

}  // namespace

extern "C" {

size_t fp4_codes_bytes(int64_t rows, int64_t cols) {
  if (rows <= 0 || cols <= 0 || cols % 2 != 0) return 0;
  return (size_t)rows * (size_t)(cols / 2);
}

size_t fp4_scales_bytes(int64_t rows, int64_t cols, int32_t fmt) {
  if (rows <= 0 || cols <= 0 || !valid_fmt(fmt) || cols % block_of(fmt) != 0) return 0;
  return (size_t)rows * (size_t)(cols / block_of(fmt));
}

uint32_t fp4_hadamard_signs(uint64_t seed) {
  // Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11) at counter (0, 0, 0, 1), word 0.
  uint32_t c0 = 0, c1 = 0, c2 = 0, c3 = 1;
  uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

const char* fp4_status_str(fp4_status s) {
  switch (s) {
    case FP4_OK: return "ok";
    case FP4_ERR_NULL: return "null pointer";
    case FP4_ERR_SHAPE: return "bad shape";
    case FP4_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case FP4_ERR_UNSUPPORTED: return "unsupported combination";
    case FP4_ERR_ARG: return "bad enum argument";
    case FP4_ERR_HIP: return "HIP launch or runtime error";
    case FP4_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
  }
  return "unknown status";
}

fp4_status fp4_tensor_amax(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                           float* amax, fp4_stream_t stream) {
  fp4_status st = check_matrix(src, src_t, R, C, ld);
  if (st != FP4_OK) return st;
  if (!amax) return FP4_ERR_NULL;
  fp4i_launch_amax(src, src_t == FP4_DTYPE_BF16, R, C, ld, amax, reinterpret_cast<hipStream_t>(stream));
  return hip_status();
}

fp4_status fp4_tensor_amax_hadamard16(const void* src, fp4_dtype src_t, int64_t R, int64_t C,
                                      int64_t ld, fp4_axis axis, uint32_t had_signs, float* amax,
                                      fp4_stream_t stream) {
  fp4_status st = check_matrix(src, src_t, R, C, ld);
  if (st != FP4_OK) return st;
  if (!amax) return FP4_ERR_NULL;
  if (axis != FP4_AXIS_COLS && axis != FP4_AXIS_ROWS) return FP4_ERR_ARG;
  if ((axis == FP4_AXIS_ROWS ? R : C) % 16 != 0) return FP4_ERR_SHAPE;
  fp4i_launch_amax_rot16(src, src_t == FP4_DTYPE_BF16, R, C, ld, axis == FP4_AXIS_ROWS, had_signs,
                         amax, reinterpret_cast<hipStream_t>(stream));
  return hip_status();
}

fp4_status fp4_quantize(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                        fp4_axis axis, fp4_rounding rnd, uint64_t seed, uint64_t index_offset,
                        int amax_ready, fp4_tensor* out, fp4_stream_t stream) {
  return quantize_impl(src, src_t, R, C, ld, axis, rnd, seed, index_offset, amax_ready, out, nullptr,
                       stream);
}

fp4_status fp4_quantize_shard(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                              int64_t row_offset, int64_t rows_total, fp4_axis axis, fp4_rounding rnd,
                              uint64_t seed, uint64_t index_offset, int amax_ready, fp4_tensor* out,
                              double* noise, fp4_stream_t stream) {
  if (!out) return FP4_ERR_NULL;
  if (!valid_fmt(out->fmt)) return FP4_ERR_ARG;
  if (!aligned8(noise)) return FP4_ERR_ALIGN;
  if (axis != FP4_AXIS_COLS && axis != FP4_AXIS_ROWS) return FP4_ERR_ARG;
  fp4_status st = check_shard(R, C, row_offset, rows_total, axis == FP4_AXIS_ROWS, block_of(out->fmt));
  if (st != FP4_OK) return st;
  // COLS: (row_offset + r) * C + c; ROWS: c * rows_total + row_offset + r.
  const uint64_t off = index_offset + (axis == FP4_AXIS_COLS ? (uint64_t)row_offset * (uint64_t)C
                                                             : (uint64_t)row_offset);
  st = check_quant(src, src_t, R, C, ld, axis, rnd, off, out);
  if (st != FP4_OK) return st;
  return launch_quant(src, src_t, R, C, ld, axis, rnd, seed, off, amax_ready, out, noise,
                      reinterpret_cast<hipStream_t>(stream), rows_total);
}

fp4_status fp4_quantize_dual_shard(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                                   int64_t row_offset, int64_t rows_total, fp4_rounding rnd_cols,
                                   uint64_t seed_cols, uint64_t index_offset_cols, fp4_rounding rnd_rows,
                                   uint64_t seed_rows, uint64_t index_offset_rows, int amax_ready,
                                   fp4_tensor* out_cols, fp4_tensor* out_rows, double* noise_cols,
                                   double* noise_rows, fp4_stream_t stream) {
  if (!out_cols) return FP4_ERR_NULL;
  if (!valid_fmt(out_cols->fmt)) return FP4_ERR_ARG;
  if (!aligned8(noise_cols) || !aligned8(noise_rows)) return FP4_ERR_ALIGN;
  const fp4_status st = check_shard(R, C, row_offset, rows_total, true, block_of(out_cols->fmt));
  if (st != FP4_OK) return st;
  return quantize_dual_impl(src, src_t, R, C, ld, rnd_cols, seed_cols,
                            index_offset_cols + (uint64_t)row_offset * (uint64_t)C, rnd_rows, seed_rows,
                            index_offset_rows + (uint64_t)row_offset, amax_ready, out_cols, out_rows, noise_cols,
                            noise_rows, stream, rows_total);
}

fp4_status fp4_quantize_noise(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                              fp4_axis axis, fp4_rounding rnd, uint64_t seed, uint64_t index_offset,
                              int amax_ready, fp4_tensor* out, double* noise, fp4_stream_t stream) {
  if (!noise) return FP4_ERR_NULL;
  if (!aligned8(noise)) return FP4_ERR_ALIGN;
  return quantize_impl(src, src_t, R, C, ld, axis, rnd, seed, index_offset, amax_ready, out, noise,
                       stream);
}

fp4_status fp4_quantize_dual(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                             fp4_rounding rnd_cols, uint64_t seed_cols, uint64_t index_offset_cols,
                             fp4_rounding rnd_rows, uint64_t seed_rows, uint64_t index_offset_rows,
                             int amax_ready, fp4_tensor* out_cols, fp4_tensor* out_rows,
                             fp4_stream_t stream) {
  return quantize_dual_impl(src, src_t, R, C, ld, rnd_cols, seed_cols, index_offset_cols, rnd_rows,
                            seed_rows, index_offset_rows, amax_ready, out_cols, out_rows, nullptr,
                            nullptr, stream);
}

fp4_status fp4_quantize_dual_noise(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                                   fp4_rounding rnd_cols, uint64_t seed_cols, uint64_t index_offset_cols,
                                   fp4_rounding rnd_rows, uint64_t seed_rows, uint64_t index_offset_rows,
                                   int amax_ready, fp4_tensor* out_cols, fp4_tensor* out_rows,
                                   double* noise_cols, double* noise_rows, fp4_stream_t stream) {
  if (!noise_cols && !noise_rows) return FP4_ERR_NULL;
  if (!aligned8(noise_cols) || !aligned8(noise_rows)) return FP4_ERR_ALIGN;
  return quantize_dual_impl(src, src_t, R, C, ld, rnd_cols, seed_cols, index_offset_cols, rnd_rows,
                            seed_rows, index_offset_rows, amax_ready, out_cols, out_rows, noise_cols,
                            noise_rows, stream);
}

fp4_status fp4_quantize_2d(const void* src, fp4_dtype src_t, int64_t R, int64_t C, int64_t ld,
                           fp4_rounding rnd, uint64_t seed, uint64_t index_offset, int amax_ready,
                           fp4_tensor* out, fp4_tensor* out_t, fp4_stream_t stream) {
  if (!out || !out_t) return FP4_ERR_NULL;
  fp4_status st = check_matrix(src, src_t, R, C, ld);
  if (st != FP4_OK) return st;
  if (rnd != FP4_RTN && rnd != FP4_SR) return FP4_ERR_ARG;
  if (!valid_fmt(out->fmt) || !valid_fmt(out_t->fmt)) return FP4_ERR_ARG;
  if (out->fmt != out_t->fmt) return FP4_ERR_UNSUPPORTED;
  if (out->had_on || out_t->had_on) return FP4_ERR_UNSUPPORTED;
  for (const fp4_tensor* o : {out, out_t}) {
    if (!o->codes || !o->scales) return FP4_ERR_NULL;
    if (!aligned16(o->codes) || !aligned16(o->scales)) return FP4_ERR_ALIGN;
  }
  const bool nv = out->fmt == FP4_NVFP4;
  if (nv && (!out->amax || !out->tscale || !out_t->tscale)) return FP4_ERR_NULL;
  const int B = block_of(out->fmt);
  if (R % B != 0 || C % B != 0) return FP4_ERR_SHAPE;
  if (rnd == FP4_SR && index_offset % 8 != 0) return FP4_ERR_ALIGN;
  if ((R + 127) / 128 * ((C + 127) / 128) > 0x7FFFFFFF) return FP4_ERR_SHAPE;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (nv && !amax_ready) {
    fp4i_launch_amax(src, src_t == FP4_DTYPE_BF16, R, C, ld, out->amax, s);
    st = hip_status();
    if (st != FP4_OK) return st;
  }
  Quant2dArgs a;
  a.src = src;
  a.bf16 = src_t == FP4_DTYPE_BF16;
  a.R = R;
  a.C = C;
  a.ld = ld;
  a.fmt = out->fmt;
  a.sr = rnd == FP4_SR;
  a.seed = seed;
  a.offset = index_offset;
  a.codes = out->codes;
  a.scales = out->scales;
  a.codes_t = out_t->codes;
  a.scales_t = out_t->scales;
  a.amax = out->amax;
  a.tscale = out->tscale;
  a.tscale_t = out_t->tscale;
  a.amax_copy = (nv && out_t->amax && out_t->amax != out->amax) ? out_t->amax : nullptr;
  fp4i_launch_quant_2d(a, s);
  out->rows = R;
  out->cols = C;
  out_t->rows = C;
  out_t->cols = R;
  return hip_status();
}

fp4_status fp4_dequantize_unrotated(const fp4_tensor* q, fp4_dtype dst_t, void* dst, int64_t ld,
                                    fp4_stream_t stream) {
  const fp4_status st = check_dequant(q, dst_t, dst, ld);
  if (st != FP4_OK) return st;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (q->had_on)
    fp4i_launch_dequant_unrot(q->codes, q->scales, q->tscale, q->fmt, q->rows, q->cols, q->had_signs,
                              dst_t == FP4_DTYPE_BF16, dst, ld, s);
  else
    fp4i_launch_dequant(q->codes, q->scales, q->tscale, q->fmt, q->rows, q->cols,
                        dst_t == FP4_DTYPE_BF16, dst, ld, s);
  return hip_status();
}

fp4_status fp4_dequantize(const fp4_tensor* q, fp4_dtype dst_t, void* dst, int64_t ld,
                          fp4_stream_t stream) {
  const fp4_status st = check_dequant(q, dst_t, dst, ld);
  if (st != FP4_OK) return st;
  fp4i_launch_dequant(q->codes, q->scales, q->tscale, q->fmt, q->rows, q->cols,
                      dst_t == FP4_DTYPE_BF16, dst, ld, reinterpret_cast<hipStream_t>(stream));
  return hip_status();
}

size_t fp4_gemm_workspace_bytes(const fp4_operand* A, const fp4_operand* B) {
  OperandView va, vb;
  if (view_operand(A, &va) != FP4_OK || view_operand(B, &vb) != FP4_OK) return 0;
  return va.ws_bytes + vb.ws_bytes;
}

size_t fp4_gemm_splitk_bytes(const fp4_operand* A, const fp4_operand* B) {
  OperandView va, vb;
  if (view_operand(A, &va) != FP4_OK || view_operand(B, &vb) != FP4_OK) return 0;
  return splitk_bytes(va, vb);
}

fp4_status fp4_gemm(const fp4_operand* A, const fp4_operand* B, fp4_dtype out_t, void* C,
                    int64_t ldc, void* ws, size_t ws_bytes, fp4_stream_t stream) {
  return gemm_impl(A, B, out_t, C, ldc, ws, ws_bytes, true, stream);
}

fp4_status fp4_gemm_noalloc(const fp4_operand* A, const fp4_operand* B, fp4_dtype out_t, void* C,
                            int64_t ldc, fp4_stream_t stream) {
  if (!C) return FP4_ERR_NULL;
  OperandView va, vb;
  fp4_status st = view_operand(A, &va);
  if (st != FP4_OK) return st;
  st = view_operand(B, &vb);
  if (st != FP4_OK) return st;
  const size_t need = va.ws_bytes + vb.ws_bytes;
  if (need > FP4_GEMM_NOALLOC_MAX_BYTES) return FP4_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_on_current_device(&ws);
    if (st != FP4_OK) return st;
  }
  return gemm_impl(A, B, out_t, C, ldc, ws, need > 0 ? FP4_GEMM_NOALLOC_MAX_BYTES : 0, false, stream);
}

fp4_status fp4_noise_ratio(const double* noise, double* ratio, fp4_stream_t stream) {
  if (!noise || !ratio) return FP4_ERR_NULL;
  if (!aligned8(noise) || !aligned8(ratio)) return FP4_ERR_ALIGN;
  fp4i_launch_noise_ratio(noise, ratio, reinterpret_cast<hipStream_t>(stream));
  return hip_status();
}

}  // extern "C"
