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
BLOCK = {FP4_NVFP4: 16, FP4_MXFP4: 32}

EXPORTS = ["fp4_codes_bytes", "fp4_scales_bytes", "fp4_hadamard_signs", "fp4_status_str",
           "fp4_tensor_amax", "fp4_tensor_amax_hadamard16", "fp4_quantize", "fp4_quantize_dual",
           "fp4_quantize_noise", "fp4_quantize_dual_noise", "fp4_quantize_2d", "fp4_dequantize",
           "fp4_gemm"]


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
        L.fp4_dequantize.argtypes = [c.POINTER(fp4_tensor), c.c_int, c.c_void_p, c.c_int64,
                                     c.c_void_p]
        L.fp4_gemm.restype = c.c_int
        L.fp4_gemm.argtypes = [c.POINTER(fp4_tensor), c.POINTER(fp4_tensor), c.c_int, c.c_void_p,
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
    R, C = src.shape
    _check(lib().fp4_tensor_amax(src.data_ptr(), _dtype_code(src), R, C, src.stride(0),
                                 amax.data_ptr(), _stream(stream)), "fp4_tensor_amax")


def fp4_tensor_amax_hadamard16(src, axis: int, had_signs: int, amax, stream=None) -> None:
    R, C = src.shape
    _check(lib().fp4_tensor_amax_hadamard16(src.data_ptr(), _dtype_code(src), R, C, src.stride(0),
                                            axis, had_signs, amax.data_ptr(), _stream(stream)),
           "fp4_tensor_amax_hadamard16")


def fp4_quantize(src, axis: int, rnd: int, seed: int, index_offset: int, amax_ready: bool,
                 out: QTensor, stream=None) -> None:
    R, C = src.shape
    if src.stride(1) != 1:
        raise ValueError("src must be row-major with unit column stride")
    d = out.desc()
    _check(lib().fp4_quantize(src.data_ptr(), _dtype_code(src), R, C, src.stride(0), axis, rnd,
                              seed, index_offset, int(bool(amax_ready)), ctypes.byref(d),
                              _stream(stream)), "fp4_quantize")
    out.rows, out.cols = d.rows, d.cols


def fp4_quantize_dual(src, rnd_cols: int, seed_cols: int, index_offset_cols: int, rnd_rows: int,
                      seed_rows: int, index_offset_rows: int, amax_ready: bool, out_cols: QTensor,
                      out_rows: QTensor, stream=None) -> None:
    R, C = src.shape
    if src.stride(1) != 1:
        raise ValueError("src must be row-major with unit column stride")
    dc, dr = out_cols.desc(), out_rows.desc()
    _check(lib().fp4_quantize_dual(src.data_ptr(), _dtype_code(src), R, C, src.stride(0), rnd_cols,
                                   seed_cols, index_offset_cols, rnd_rows, seed_rows, index_offset_rows,
                                   int(bool(amax_ready)), ctypes.byref(dc), ctypes.byref(dr),
                                   _stream(stream)), "fp4_quantize_dual")
    out_cols.rows, out_cols.cols = dc.rows, dc.cols
    out_rows.rows, out_rows.cols = dr.rows, dr.cols


def _ptr(t):
    return None if t is None else t.data_ptr()


def fp4_quantize_noise(src, axis: int, rnd: int, seed: int, index_offset: int, amax_ready: bool,
                       out: QTensor, noise, stream=None) -> None:
    """fp4_quantize plus noise[0] += sum x^2, noise[1] += sum (xhat - x)^2
    (noise: a float64 device tensor of 2 elements)."""
    R, C = src.shape
    if src.stride(1) != 1:
        raise ValueError("src must be row-major with unit column stride")
    d = out.desc()
    _check(lib().fp4_quantize_noise(src.data_ptr(), _dtype_code(src), R, C, src.stride(0), axis, rnd,
                                    seed, index_offset, int(bool(amax_ready)), ctypes.byref(d),
                                    _ptr(noise), _stream(stream)), "fp4_quantize_noise")
    out.rows, out.cols = d.rows, d.cols


def fp4_quantize_dual_noise(src, rnd_cols: int, seed_cols: int, index_offset_cols: int, rnd_rows: int,
                            seed_rows: int, index_offset_rows: int, amax_ready: bool, out_cols: QTensor,
                            out_rows: QTensor, noise_cols=None, noise_rows=None, stream=None) -> None:
    R, C = src.shape
    if src.stride(1) != 1:
        raise ValueError("src must be row-major with unit column stride")
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
    R, C = src.shape
    if src.stride(1) != 1:
        raise ValueError("src must be row-major with unit column stride")
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


def noise_ratio(noise) -> float:
    """||g|| / ||Q(g) - g|| from a monitor's two sums (host read-out)."""
    g, e = (float(v) for v in noise.cpu())
    return float("inf") if e == 0.0 else (g / e) ** 0.5


def fp4_dequantize(q: QTensor, dst, stream=None) -> None:
    d = q.desc()
    _check(lib().fp4_dequantize(ctypes.byref(d), _dtype_code(dst), dst.data_ptr(), dst.stride(0),
                                _stream(stream)), "fp4_dequantize")


def fp4_gemm(A: QTensor, B: QTensor, C, stream=None) -> None:
    da, db = A.desc(), B.desc()
    _check(lib().fp4_gemm(ctypes.byref(da), ctypes.byref(db), _dtype_code(C), C.data_ptr(),
                          C.stride(0), _stream(stream)), "fp4_gemm")


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


def dequantize(q: QTensor, dtype=None, stream=None):
    import torch
    dst = torch.empty((q.rows, q.cols), dtype=dtype or torch.float32, device=q.codes.device)
    fp4_dequantize(q, dst, stream)
    return dst


def gemm(A: QTensor, B: QTensor, dtype=None, out=None, stream=None):
    import torch
    if out is None:
        out = torch.empty((A.rows, B.rows), dtype=dtype or torch.float32, device=A.codes.device)
    fp4_gemm(A, B, out, stream)
    return out
