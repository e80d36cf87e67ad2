"""Thin Python binding of libfp4.so (include/fp4.h), the gfx950 FP4 quantize +
FP4 GEMM library.

Argument marshalling only: every step of the path runs in the library's HIP
kernels. PyTorch supplies device memory and the stream. Importing this module
does not load the library; the first call does, and raises if it is missing
(build it with ``python -m fp4_fully_quantized_amd.build``).
"""
from __future__ import annotations

import ctypes
import os

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libfp4.so")

FP4_OK = 0
FP4_DTYPE_F32, FP4_DTYPE_BF16 = 0, 1
FP4_NVFP4, FP4_MXFP4 = 0, 1
FP4_RTN, FP4_SR = 0, 1
FP4_AXIS_COLS, FP4_AXIS_ROWS = 0, 1
FP4_OPERAND_QUANTIZED, FP4_OPERAND_RAW = 0, 1
FP4_LAYOUT_N, FP4_LAYOUT_T = 0, 1
FP4_ERR_WORKSPACE = 7
BLOCK = {FP4_NVFP4: 16, FP4_MXFP4: 32}

EXPORTS = ["fp4_codes_bytes", "fp4_scales_bytes", "fp4_hadamard_signs", "fp4_status_str",
           "fp4_tensor_amax", "fp4_tensor_amax_hadamard16", "fp4_quantize", "fp4_quantize_dual",
           "fp4_quantize_shard", "fp4_quantize_dual_shard", "fp4_quantize_noise", "fp4_quantize_dual_noise", "fp4_noise_ratio", "fp4_quantize_2d",
           "fp4_dequantize", "fp4_dequantize_unrotated", "fp4_gemm_workspace_bytes", "fp4_gemm_splitk_bytes", "fp4_gemm",
           "fp4_gemm_noalloc"]
# The allocation-free GEMM's workspace limit (FP4_GEMM_NOALLOC_MAX_BYTES).
FP4_GEMM_NOALLOC_MAX_BYTES = 128 << 20


class Fp4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {fp4_status_str(status)} (status {status})")
        self.status = status


class fp4_tensor(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("amax", ctypes.c_void_p), ("tscale", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("cols", ctypes.c_int64),
                ("fmt", ctypes.c_int32), ("had_on", ctypes.c_int32),
                ("had_signs", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


class fp4_operand(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("q", ctypes.POINTER(fp4_tensor)), ("data", ctypes.c_void_p),
                ("rows", ctypes.c_int64), ("k", ctypes.c_int64), ("ld", ctypes.c_int64),
                ("layout", ctypes.c_int32), ("fmt", ctypes.c_int32), ("rnd", ctypes.c_int32),
                ("had_on", ctypes.c_int32), ("seed", ctypes.c_uint64), ("index_offset", ctypes.c_uint64),
                ("had_signs", ctypes.c_uint32), ("reserved", ctypes.c_uint32)]


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run python -m fp4_fully_quantized_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        c = ctypes
        L.fp4_codes_bytes.restype = c.c_size_t
        L.fp4_codes_bytes.argtypes = [c.c_int64, c.c_int64]
        L.fp4_scales_bytes.restype = c.c_size_t
        L.fp4_scales_bytes.argtypes = [c.c_int64, c.c_int64, c.c_int32]
        L.fp4_hadamard_signs.restype = c.c_uint32
        L.fp4_hadamard_signs.argtypes = [c.c_uint64]
        L.fp4_status_str.restype = c.c_char_p
        L.fp4_status_str.argtypes = [c.c_int]
        L.fp4_tensor_amax.restype = c.c_int
        L.fp4_tensor_amax.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_int64,
                                      c.c_void_p, c.c_void_p]
        L.fp4_tensor_amax_hadamard16.restype = c.c_int
        L.fp4_tensor_amax_hadamard16.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_int64,
                                                 c.c_int, c.c_uint32, c.c_void_p, c.c_void_p]
        L.fp4_quantize.restype = c.c_int
        L.fp4_quantize.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_int64, c.c_int,
                                   c.c_int, c.c_uint64, c.c_uint64, c.c_int,
                                   c.POINTER(fp4_tensor), c.c_void_p]
        L.fp4_quantize_dual.restype = c.c_int
        L.fp4_quantize_dual.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_int64,
                                        c.c_int, c.c_uint64, c.c_uint64, c.c_int, c.c_uint64, c.c_uint64,
                                        c.c_int, c.POINTER(fp4_tensor), c.POINTER(fp4_tensor), c.c_void_p]
        L.fp4_quantize_shard.restype = c.c_int
        L.fp4_quantize_shard.argtypes = (L.fp4_quantize.argtypes[:5] + [c.c_int64, c.c_int64]
                                         + L.fp4_quantize.argtypes[5:-1] + [c.c_void_p, c.c_void_p])
        L.fp4_quantize_dual_shard.restype = c.c_int
        L.fp4_quantize_dual_shard.argtypes = (L.fp4_quantize_dual.argtypes[:5] + [c.c_int64, c.c_int64]
                                              + L.fp4_quantize_dual.argtypes[5:-1]
                                              + [c.c_void_p, c.c_void_p, c.c_void_p])
        L.fp4_quantize_noise.restype = c.c_int
        L.fp4_quantize_noise.argtypes = L.fp4_quantize.argtypes[:-1] + [c.c_void_p, c.c_void_p]
        L.fp4_quantize_dual_noise.restype = c.c_int
        L.fp4_quantize_dual_noise.argtypes = L.fp4_quantize_dual.argtypes[:-1] + [c.c_void_p, c.c_void_p,
                                                                                  c.c_void_p]
        L.fp4_quantize_2d.restype = c.c_int
        L.fp4_quantize_2d.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_int64, c.c_int,
                                      c.c_uint64, c.c_uint64, c.c_int, c.POINTER(fp4_tensor),
                                      c.POINTER(fp4_tensor), c.c_void_p]
        L.fp4_dequantize.restype = c.c_int
        L.fp4_dequantize_unrotated.restype = c.c_int
        L.fp4_dequantize_unrotated.argtypes = [c.POINTER(fp4_tensor), c.c_int, c.c_void_p, c.c_int64,
                                               c.c_void_p]
        L.fp4_dequantize.argtypes = [c.POINTER(fp4_tensor), c.c_int, c.c_void_p, c.c_int64,
                                     c.c_void_p]
        L.fp4_noise_ratio.restype = c.c_int
        L.fp4_noise_ratio.argtypes = [c.c_void_p, c.c_void_p, c.c_void_p]
        L.fp4_gemm_workspace_bytes.restype = c.c_size_t
        L.fp4_gemm_workspace_bytes.argtypes = [c.POINTER(fp4_operand), c.POINTER(fp4_operand)]
        L.fp4_gemm_splitk_bytes.restype = c.c_size_t
        L.fp4_gemm_splitk_bytes.argtypes = [c.POINTER(fp4_operand), c.POINTER(fp4_operand)]
        L.fp4_gemm.restype = c.c_int
        L.fp4_gemm.argtypes = [c.POINTER(fp4_operand), c.POINTER(fp4_operand), c.c_int, c.c_void_p,
                               c.c_int64, c.c_void_p, c.c_size_t, c.c_void_p]
        L.fp4_gemm_noalloc.restype = c.c_int
        L.fp4_gemm_noalloc.argtypes = [c.POINTER(fp4_operand), c.POINTER(fp4_operand), c.c_int, c.c_void_p,
                                       c.c_int64, c.c_void_p]
        _lib = L
    return _lib


# ---------------------------------------------------------------- raw ABI calls
def fp4_codes_bytes(rows: int, cols: int) -> int:
    return lib().fp4_codes_bytes(rows, cols)


def fp4_scales_bytes(rows: int, cols: int, fmt: int) -> int:
    return lib().fp4_scales_bytes(rows, cols, fmt)


def fp4_hadamard_signs(seed: int) -> int:
    return lib().fp4_hadamard_signs(seed)


def fp4_status_str(status: int) -> str:
    return lib().fp4_status_str(status).decode()


def _check(status: int, what: str) -> None:
    if status != FP4_OK:
        raise Fp4Error(status, what)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return FP4_DTYPE_BF16
    if t.dtype == torch.float32:
        return FP4_DTYPE_F32
    raise TypeError(f"FP4 library takes float32 or bfloat16 tensors, got {t.dtype}")


# ---------------------------------------------------------------- argument checks
# The library checks shapes, alignment and enums, but it sees raw pointers: it
# cannot tell a host pointer, a tensor that is too small or a transposed view
# from a good one. These checks run before every call that passes tensors.
def _check_device(t, name: str, device=None):
    if not getattr(t, "is_cuda", False):
        raise ValueError(f"{name} must be a tensor on a GPU (got device {getattr(t, 'device', None)})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the other arguments on {device}")


def _check_matrix(t, name: str, device=None):
    """A 2-D float32/bfloat16 device matrix, row-major with unit column stride."""
    _check_device(t, name, device)
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    _dtype_code(t)
    if t.stride(1) != 1 and t.shape[1] > 1:
        raise ValueError(f"{name} must be row-major with unit column stride")
    if t.shape[0] > 1 and t.stride(0) < t.shape[1]:
        raise ValueError(f"{name} rows overlap (stride {t.stride(0)} < {t.shape[1]} columns)")


def _check_scalar(t, name: str, dtype, count: int, device):
    import torch
    _check_device(t, name, device)
    if t.dtype != dtype or t.numel() < count or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} device tensor of at least {count} element(s)")
    del torch


def _check_qtensor(q, name: str, device=None):
    """The QTensor's buffers exist on the device and hold rows x cols codes and scales."""
    import torch
    if not isinstance(q, QTensor):
        raise TypeError(f"{name} must be a QTensor")
    device = device or q.codes.device
    for part, t, need in (("codes", q.codes, fp4_codes_bytes(q.rows, q.cols)),
                          ("scales", q.scales, fp4_scales_bytes(q.rows, q.cols, q.fmt))):
        _check_device(t, f"{name}.{part}", device)
        if t.dtype != torch.uint8 or not t.is_contiguous():
            raise ValueError(f"{name}.{part} must be a contiguous uint8 tensor")
        if need == 0 or t.numel() < need:
            raise ValueError(f"{name}.{part} holds {t.numel()} bytes, {q.rows} x {q.cols} needs {need}")
    if q.fmt == FP4_NVFP4:
        _check_scalar(q.amax, f"{name}.amax", torch.float32, 1, device)
        _check_scalar(q.tscale, f"{name}.tscale", torch.float32, 1, device)


def _check_quant_out(src, out, axis: int, name: str = "out"):
    """The output QTensor has the quantized orientation of src."""
    R, C = src.shape
    want = (C, R) if axis == FP4_AXIS_ROWS else (R, C)
    if (out.rows, out.cols) != want:
        raise ValueError(f"{name} is {out.rows} x {out.cols}; quantizing a {R} x {C} source along "
                         f"{'rows' if axis == FP4_AXIS_ROWS else 'cols'} needs {want[0]} x {want[1]}")
    _check_qtensor(out, name, src.device)


# ---------------------------------------------------------------- tensors
class QTensor:
    """A quantized matrix (quantized orientation rows x cols) held in torch
    device tensors, and its fp4_tensor descriptor."""

    def __init__(self, rows: int, cols: int, fmt: int, device="cuda", had_signs: int | None = None):
        import torch
        B = BLOCK[fmt]
        if cols % B:
            raise ValueError(f"cols={cols} is not a multiple of the block size {B}")
        self.rows, self.cols, self.fmt = rows, cols, fmt
        self.codes = torch.empty((rows, cols // 2), dtype=torch.uint8, device=device)
        self.scales = torch.empty((rows, cols // B), dtype=torch.uint8, device=device)
        if fmt == FP4_NVFP4:
            self.amax = torch.zeros(1, dtype=torch.float32, device=device)
            self.tscale = torch.zeros(1, dtype=torch.float32, device=device)
        else:
            self.amax = self.tscale = None
        self.had_on = had_signs is not None
        self.had_signs = int(had_signs or 0)

    def desc(self) -> fp4_tensor:
        d = fp4_tensor()
        d.codes = self.codes.data_ptr()
        d.scales = self.scales.data_ptr()
        d.amax = self.amax.data_ptr() if self.amax is not None else None
        d.tscale = self.tscale.data_ptr() if self.tscale is not None else None
        d.rows, d.cols = self.rows, self.cols
        d.fmt = self.fmt
        d.had_on = int(self.had_on)
        d.had_signs = self.had_signs
        return d


def fp4_tensor_amax(src, amax, stream=None) -> None:
    import torch
    _check_matrix(src, "src")
    _check_scalar(amax, "amax", torch.float32, 1, src.device)
    R, C = src.shape
    _check(lib().fp4_tensor_amax(src.data_ptr(), _dtype_code(src), R, C, src.stride(0),
                                 amax.data_ptr(), _stream(stream)), "fp4_tensor_amax")


def fp4_tensor_amax_hadamard16(src, axis: int, had_signs: int, amax, stream=None) -> None:
    import torch
    _check_matrix(src, "src")
    _check_scalar(amax, "amax", torch.float32, 1, src.device)
    R, C = src.shape
    _check(lib().fp4_tensor_amax_hadamard16(src.data_ptr(), _dtype_code(src), R, C, src.stride(0),
                                            axis, had_signs, amax.data_ptr(), _stream(stream)),
           "fp4_tensor_amax_hadamard16")


def fp4_quantize(src, axis: int, rnd: int, seed: int, index_offset: int, amax_ready: bool,
                 out: QTensor, stream=None) -> None:
    _check_matrix(src, "src")
    _check_quant_out(src, out, axis)
    R, C = src.shape
    d = out.desc()
    _check(lib().fp4_quantize(src.data_ptr(), _dtype_code(src), R, C, src.stride(0), axis, rnd,
                              seed, index_offset, int(bool(amax_ready)), ctypes.byref(d),
                              _stream(stream)), "fp4_quantize")
    out.rows, out.cols = d.rows, d.cols


def fp4_quantize_dual(src, rnd_cols: int, seed_cols: int, index_offset_cols: int, rnd_rows: int,
                      seed_rows: int, index_offset_rows: int, amax_ready: bool, out_cols: QTensor,
                      out_rows: QTensor, stream=None) -> None:
    _check_matrix(src, "src")
    _check_quant_out(src, out_cols, FP4_AXIS_COLS, "out_cols")
    _check_quant_out(src, out_rows, FP4_AXIS_ROWS, "out_rows")
    R, C = src.shape
    dc, dr = out_cols.desc(), out_rows.desc()
    _check(lib().fp4_quantize_dual(src.data_ptr(), _dtype_code(src), R, C, src.stride(0), rnd_cols,
                                   seed_cols, index_offset_cols, rnd_rows, seed_rows, index_offset_rows,
                                   int(bool(amax_ready)), ctypes.byref(dc), ctypes.byref(dr),
                                   _stream(stream)), "fp4_quantize_dual")
    out_cols.rows, out_cols.cols = dc.rows, dc.cols
    out_rows.rows, out_rows.cols = dr.rows, dr.cols


def fp4_quantize_shard(src, row_offset: int, rows_total: int, axis: int, rnd: int, seed: int,
                       index_offset: int, amax_ready: bool, out: QTensor, noise=None, stream=None) -> None:
    """fp4_quantize of rows row_offset .. of a rows_total-row tensor, with the
    whole tensor's stochastic-rounding indices (noise: None, or the float64
    device tensor of 2 sums of fp4_quantize_noise)."""
    import torch
    _check_matrix(src, "src")
    _check_quant_out(src, out, axis)
    if noise is not None:
        _check_scalar(noise, "noise", torch.float64, 2, src.device)
    R, C = src.shape
    d = out.desc()
    _check(lib().fp4_quantize_shard(src.data_ptr(), _dtype_code(src), R, C, src.stride(0), row_offset,
                                    rows_total, axis, rnd, seed, index_offset, int(bool(amax_ready)),
                                    ctypes.byref(d), _ptr(noise), _stream(stream)), "fp4_quantize_shard")
    out.rows, out.cols = d.rows, d.cols


def fp4_quantize_dual_shard(src, row_offset: int, rows_total: int, rnd_cols: int, seed_cols: int,
                            index_offset_cols: int, rnd_rows: int, seed_rows: int, index_offset_rows: int,
                            amax_ready: bool, out_cols: QTensor, out_rows: QTensor, noise_cols=None,
                            noise_rows=None, stream=None) -> None:
    """fp4_quantize_dual of a row shard, with the whole tensor's stochastic-rounding indices."""
    import torch
    _check_matrix(src, "src")
    _check_quant_out(src, out_cols, FP4_AXIS_COLS, "out_cols")
    _check_quant_out(src, out_rows, FP4_AXIS_ROWS, "out_rows")
    for nm, t in (("noise_cols", noise_cols), ("noise_rows", noise_rows)):
        if t is not None:
            _check_scalar(t, nm, torch.float64, 2, src.device)
    R, C = src.shape
    dc, dr = out_cols.desc(), out_rows.desc()
    _check(lib().fp4_quantize_dual_shard(src.data_ptr(), _dtype_code(src), R, C, src.stride(0), row_offset,
                                         rows_total, rnd_cols, seed_cols, index_offset_cols, rnd_rows,
                                         seed_rows, index_offset_rows, int(bool(amax_ready)), ctypes.byref(dc),
                                         ctypes.byref(dr), _ptr(noise_cols), _ptr(noise_rows), _stream(stream)),
           "fp4_quantize_dual_shard")
    out_cols.rows, out_cols.cols = dc.rows, dc.cols
    out_rows.rows, out_rows.cols = dr.rows, dr.cols


def _ptr(t):
    return None if t is None else t.data_ptr()


def fp4_quantize_noise(src, axis: int, rnd: int, seed: int, index_offset: int, amax_ready: bool,
                       out: QTensor, noise, stream=None) -> None:
    """fp4_quantize plus noise[0] += sum x^2, noise[1] += sum (xhat - x)^2
    (noise: a float64 device tensor of 2 elements)."""
    import torch
    _check_matrix(src, "src")
    _check_quant_out(src, out, axis)
    _check_scalar(noise, "noise", torch.float64, 2, src.device)
    R, C = src.shape
    d = out.desc()
    _check(lib().fp4_quantize_noise(src.data_ptr(), _dtype_code(src), R, C, src.stride(0), axis, rnd,
                                    seed, index_offset, int(bool(amax_ready)), ctypes.byref(d),
                                    _ptr(noise), _stream(stream)), "fp4_quantize_noise")
    out.rows, out.cols = d.rows, d.cols


def fp4_quantize_dual_noise(src, rnd_cols: int, seed_cols: int, index_offset_cols: int, rnd_rows: int,
                            seed_rows: int, index_offset_rows: int, amax_ready: bool, out_cols: QTensor,
                            out_rows: QTensor, noise_cols=None, noise_rows=None, stream=None) -> None:
    import torch
    _check_matrix(src, "src")
    _check_quant_out(src, out_cols, FP4_AXIS_COLS, "out_cols")
    _check_quant_out(src, out_rows, FP4_AXIS_ROWS, "out_rows")
    for nm, t in (("noise_cols", noise_cols), ("noise_rows", noise_rows)):
        if t is not None:
            _check_scalar(t, nm, torch.float64, 2, src.device)
    R, C = src.shape
    dc, dr = out_cols.desc(), out_rows.desc()
    _check(lib().fp4_quantize_dual_noise(src.data_ptr(), _dtype_code(src), R, C, src.stride(0),
                                         rnd_cols, seed_cols, index_offset_cols, rnd_rows, seed_rows,
                                         index_offset_rows, int(bool(amax_ready)), ctypes.byref(dc),
                                         ctypes.byref(dr), _ptr(noise_cols), _ptr(noise_rows),
                                         _stream(stream)), "fp4_quantize_dual_noise")
    out_cols.rows, out_cols.cols = dc.rows, dc.cols
    out_rows.rows, out_rows.cols = dr.rows, dr.cols


def fp4_quantize_2d(src, rnd: int, seed: int, index_offset: int, amax_ready: bool, out: QTensor,
                    out_t: QTensor, stream=None) -> None:
    _check_matrix(src, "src")
    _check_quant_out(src, out, FP4_AXIS_COLS, "out")
    _check_quant_out(src, out_t, FP4_AXIS_ROWS, "out_t")
    R, C = src.shape
    d, dt = out.desc(), out_t.desc()
    _check(lib().fp4_quantize_2d(src.data_ptr(), _dtype_code(src), R, C, src.stride(0), rnd, seed,
                                 index_offset, int(bool(amax_ready)), ctypes.byref(d), ctypes.byref(dt),
                                 _stream(stream)), "fp4_quantize_2d")
    out.rows, out.cols = d.rows, d.cols
    out_t.rows, out_t.cols = dt.rows, dt.cols


def quantize_2d(src, fmt: int = FP4_NVFP4, rnd: int = FP4_RTN, seed: int = 0, index_offset: int = 0,
                amax_from: QTensor | None = None, stream=None):
    """Allocate both QTensors and quantize src with B x B blocks. Returns
    (q [R, C] blocked along C, q_t [C, R] blocked along R), one quantization
    sharing the tensor amax (NVFP4)."""
    R, C = src.shape
    q = QTensor(R, C, fmt, device=src.device)
    qt = QTensor(C, R, fmt, device=src.device)
    ready = False
    if amax_from is not None and fmt == FP4_NVFP4:
        q.amax = amax_from.amax
        ready = True
    if fmt == FP4_NVFP4:
        qt.amax = q.amax
    fp4_quantize_2d(src, rnd, seed, index_offset, ready, q, qt, stream)
    return q, qt


def fp4_noise_ratio(noise, ratio, stream=None) -> None:
    """ratio[0] = sqrt(noise[0] / noise[1]), computed by the library on the
    device in stream order (noise: 2 float64, ratio: 1 float64, device)."""
    import torch
    _check_scalar(noise, "noise", torch.float64, 2, None)
    _check_scalar(ratio, "ratio", torch.float64, 1, noise.device)
    _check(lib().fp4_noise_ratio(noise.data_ptr(), ratio.data_ptr(), _stream(stream)), "fp4_noise_ratio")


def noise_ratio(noise, stream=None):
    """The monitor's ratio ||g|| / ||Q(g) - g|| as a 1-element float64 device
    tensor (fp4_noise_ratio into a new tensor)."""
    import torch
    ratio = torch.empty(1, dtype=torch.float64, device=noise.device)
    fp4_noise_ratio(noise, ratio, stream)
    return ratio


def fp4_dequantize(q: QTensor, dst, stream=None) -> None:
    _dequantize("fp4_dequantize", q, dst, stream)


def fp4_dequantize_unrotated(q: QTensor, dst, stream=None) -> None:
    """fp4_dequantize, then the inverse of the quantization's block rotation
    (when q.had_on): the values in the tensor's own domain."""
    _dequantize("fp4_dequantize_unrotated", q, dst, stream)


def _dequantize(name, q, dst, stream):
    _check_qtensor(q, "q")
    _check_matrix(dst, "dst", q.codes.device)
    if tuple(dst.shape) != (q.rows, q.cols):
        raise ValueError(f"dst is {tuple(dst.shape)}, q is {q.rows} x {q.cols}")
    d = q.desc()
    _check(getattr(lib(), name)(ctypes.byref(d), _dtype_code(dst), dst.data_ptr(), dst.stride(0),
                                _stream(stream)), name)


class RawOperand:
    """A GEMM operand that fp4_gemm quantizes into its workspace first: the
    rows x K matrix `data` (layout N: data is rows x K) or its transpose
    (layout T: data is K x rows), with the format, rounding, SR stream and
    rotation of fp4_quantize."""

    def __init__(self, data, layout: int = FP4_LAYOUT_N, fmt: int = FP4_NVFP4, rnd: int = FP4_RTN,
                 seed: int = 0, index_offset: int = 0, had_signs: int | None = None):
        _check_matrix(data, "data")
        if layout not in (FP4_LAYOUT_N, FP4_LAYOUT_T):
            raise ValueError(f"layout must be FP4_LAYOUT_N or FP4_LAYOUT_T, got {layout}")
        self.data, self.layout, self.fmt, self.rnd = data, layout, fmt, rnd
        self.seed, self.index_offset = seed, index_offset
        self.had_on = had_signs is not None
        self.had_signs = int(had_signs or 0)
        R, C = data.shape
        self.rows, self.k = (C, R) if layout == FP4_LAYOUT_T else (R, C)

    @property
    def device(self):
        return self.data.device

    def operand(self) -> fp4_operand:
        o = fp4_operand()
        o.kind = FP4_OPERAND_RAW
        o.dtype = _dtype_code(self.data)
        o.data = self.data.data_ptr()
        o.rows, o.k, o.ld = self.rows, self.k, self.data.stride(0)
        o.layout, o.fmt, o.rnd = self.layout, self.fmt, self.rnd
        o.had_on, o.had_signs = int(self.had_on), self.had_signs
        o.seed, o.index_offset = self.seed, self.index_offset
        return o


def _operand(x, name: str):
    """(fp4_operand, keep-alive) for a QTensor or a RawOperand."""
    if isinstance(x, RawOperand):
        return x.operand(), None
    _check_qtensor(x, name)
    d = x.desc()
    o = fp4_operand()
    o.kind = FP4_OPERAND_QUANTIZED
    o.q = ctypes.pointer(d)
    return o, d


def _operand_device(x):
    return x.device if isinstance(x, RawOperand) else x.codes.device


def fp4_gemm_workspace_bytes(A, B) -> int:
    oa, ka = _operand(A, "A")
    ob, kb = _operand(B, "B")
    return lib().fp4_gemm_workspace_bytes(ctypes.byref(oa), ctypes.byref(ob))


def fp4_gemm_splitk_bytes(A, B) -> int:
    oa, ka = _operand(A, "A")
    ob, kb = _operand(B, "B")
    return lib().fp4_gemm_splitk_bytes(ctypes.byref(oa), ctypes.byref(ob))


def fp4_gemm(A, B, C, ws=None, stream=None) -> None:
    """C = A_hat B_hat^T (FP32 accumulation). A and B are QTensors blocked
    along K or RawOperands (quantized into `ws`, a uint8 device tensor of at
    least fp4_gemm_workspace_bytes(A, B) bytes; with fp4_gemm_splitk_bytes(A, B)
    more, the last partial wave of output tiles is split along K)."""
    import torch
    dev = _operand_device(A)
    if _operand_device(B) != dev:
        raise ValueError(f"A is on {dev}, B on {_operand_device(B)}")
    oa, ka = _operand(A, "A")
    ob, kb = _operand(B, "B")
    _check_matrix(C, "C", dev)
    if tuple(C.shape) != (A.rows, B.rows):
        raise ValueError(f"C is {tuple(C.shape)}, the product is {A.rows} x {B.rows}")
    ws_ptr, ws_bytes = None, 0
    if ws is not None:
        _check_device(ws, "ws", dev)
        if ws.dtype != torch.uint8 or not ws.is_contiguous():
            raise ValueError("ws must be a contiguous uint8 device tensor")
        ws_ptr, ws_bytes = ws.data_ptr(), ws.numel()
    _check(lib().fp4_gemm(ctypes.byref(oa), ctypes.byref(ob), _dtype_code(C), C.data_ptr(), C.stride(0),
                          ws_ptr, ws_bytes, _stream(stream)), "fp4_gemm")


def fp4_gemm_noalloc(A, B, C, stream=None) -> None:
    """fp4_gemm with the library's own static workspace (for callers that
    cannot allocate): RAW operands are quantized there. Calls with RAW
    operands that overlap on one GPU race on that workspace."""
    dev = _operand_device(A)
    if _operand_device(B) != dev:
        raise ValueError(f"A is on {dev}, B on {_operand_device(B)}")
    oa, ka = _operand(A, "A")
    ob, kb = _operand(B, "B")
    _check_matrix(C, "C", dev)
    if tuple(C.shape) != (A.rows, B.rows):
        raise ValueError(f"C is {tuple(C.shape)}, the product is {A.rows} x {B.rows}")
    _check(lib().fp4_gemm_noalloc(ctypes.byref(oa), ctypes.byref(ob), _dtype_code(C), C.data_ptr(),
                                  C.stride(0), _stream(stream)), "fp4_gemm_noalloc")


# ---------------------------------------------------------------- conveniences
def quantize(src, axis: int = FP4_AXIS_COLS, fmt: int = FP4_NVFP4, rnd: int = FP4_RTN,
             seed: int = 0, index_offset: int = 0, had_signs: int | None = None,
             amax_from: QTensor | None = None, noise=None, stream=None) -> QTensor:
    """Allocate a QTensor and quantize src into it. `amax_from`: reuse the
    tensor amax already computed for the same tensor (NVFP4). `noise`: a float64
    device tensor of 2 elements that the quantization noise sums are added to."""
    R, C = src.shape
    rows, cols = (C, R) if axis == FP4_AXIS_ROWS else (R, C)
    q = QTensor(rows, cols, fmt, device=src.device, had_signs=had_signs)
    ready = False
    if amax_from is not None and fmt == FP4_NVFP4:
        q.amax = amax_from.amax
        ready = True
    if noise is None:
        fp4_quantize(src, axis, rnd, seed, index_offset, ready, q, stream)
    else:
        fp4_quantize_noise(src, axis, rnd, seed, index_offset, ready, q, noise, stream)
    return q


def quantize_dual(src, fmt: int = FP4_NVFP4, rnd_cols: int = FP4_RTN, seed_cols: int = 0,
                  index_offset_cols: int = 0, rnd_rows: int = FP4_SR, seed_rows: int = 0,
                  index_offset_rows: int = 0, had_signs_cols: int | None = None,
                  had_signs_rows: int | None = None, amax_from: QTensor | None = None,
                  noise_cols=None, noise_rows=None, stream=None):
    """Allocate both QTensors and quantize src along C and along R in one
    read. Returns (q_cols [R, C], q_rows [C, R]). NVFP4 without rotation: they
    share the tensor amax (`amax_from`: a QTensor whose amax to reuse). NVFP4
    with a rotation on either side: each keeps its own amax (`amax_from`: a
    pair of QTensors, for the cols and the rows orientation)."""
    R, C = src.shape
    qc = QTensor(R, C, fmt, device=src.device, had_signs=had_signs_cols)
    qr = QTensor(C, R, fmt, device=src.device, had_signs=had_signs_rows)
    ready = False
    two = fmt == FP4_NVFP4 and (qc.had_on or qr.had_on)
    if amax_from is not None and fmt == FP4_NVFP4:
        if two:
            qc.amax, qr.amax = amax_from[0].amax, amax_from[1].amax
        else:
            qc.amax = amax_from.amax
        ready = True
    if fmt == FP4_NVFP4 and not two:
        qr.amax = qc.amax
    if noise_cols is None and noise_rows is None:
        fp4_quantize_dual(src, rnd_cols, seed_cols, index_offset_cols, rnd_rows, seed_rows,
                          index_offset_rows, ready, qc, qr, stream)
    else:
        fp4_quantize_dual_noise(src, rnd_cols, seed_cols, index_offset_cols, rnd_rows, seed_rows,
                                index_offset_rows, ready, qc, qr, noise_cols, noise_rows, stream)
    return qc, qr


def dequantize(q: QTensor, dtype=None, stream=None, unrotate=False):
    """Allocate the output and run fp4_dequantize (fp4_dequantize_unrotated
    with unrotate=True)."""
    import torch
    dst = torch.empty((q.rows, q.cols), dtype=dtype or torch.float32, device=q.codes.device)
    (fp4_dequantize_unrotated if unrotate else fp4_dequantize)(q, dst, stream)
    return dst


def gemm(A, B, dtype=None, out=None, ws=None, stream=None):
    """Allocate the output (and, when none is given, the workspace: the RAW
    operands' and the split-K area) and run fp4_gemm."""
    import torch
    dev = _operand_device(A)
    if out is None:
        out = torch.empty((A.rows, B.rows), dtype=dtype or torch.float32, device=dev)
    if ws is None:
        n = fp4_gemm_workspace_bytes(A, B) + fp4_gemm_splitk_bytes(A, B)
        if n:
            ws = torch.empty(n, dtype=torch.uint8, device=dev)
    fp4_gemm(A, B, out, ws, stream)
    return out
