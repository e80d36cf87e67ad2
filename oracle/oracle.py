"""Python face of the CPU oracle.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
CPU-baseline leg of the benchmark. The GPU product path never imports it.

Quantization, dequantization and the codecs run in the plain C library
``liboracle.so`` built from ``fp4_oracle.c`` beside this file. The GEMM
reference is the definition of the product of two block-scaled FP4 matrices:
dequantize both operands exactly (every dequantized value is a dyadic number
exact in FP64) and take their FP64 matrix product (Robots Atlas, "FP4", How it
works and Execution paradigm: FP4 operands, products accumulated in higher
precision; Quartet, one-line summary: all three linear-layer GEMMs in FP4).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

FMT_NVFP4, FMT_MXFP4 = 0, 1
RTN, SR = 0, 1
AXIS_COLS, AXIS_ROWS = 0, 1
BLOCK = {FMT_NVFP4: 16, FMT_MXFP4: 32}

_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with the Makefile beside this file."""
    if force or not os.path.exists(_LIB_PATH):
        subprocess.run(["make", "-s", "-B" if force else "-s", "-C", _HERE], check=True)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB_PATH)
        c = ctypes
        L.o_e2m1_value.restype = c.c_double
        L.o_e2m1_value.argtypes = [c.c_uint]
        L.o_e2m1_rtn_mag.restype = c.c_uint
        L.o_e2m1_rtn_mag.argtypes = [c.c_float]
        L.o_e2m1_sr_mag.restype = c.c_uint
        L.o_e2m1_sr_mag.argtypes = [c.c_float, c.c_uint32]
        L.o_e4m3_value.restype = c.c_double
        L.o_e4m3_value.argtypes = [c.c_uint]
        L.o_e4m3_encode.restype = c.c_uint
        L.o_e4m3_encode.argtypes = [c.c_float]
        L.o_e8m0_exponent.restype = c.c_int
        L.o_e8m0_exponent.argtypes = [c.c_float]
        L.o_e8m0_value.restype = c.c_double
        L.o_e8m0_value.argtypes = [c.c_uint]
        L.o_f32_to_bf16_rne.restype = c.c_uint16
        L.o_f32_to_bf16_rne.argtypes = [c.c_float]
        L.o_philox4x32_10.restype = None
        L.o_philox4x32_10.argtypes = [c.POINTER(c.c_uint32), c.POINTER(c.c_uint32),
                                      c.POINTER(c.c_uint32)]
        L.o_sr_draw16.restype = c.c_uint32
        L.o_sr_draw16.argtypes = [c.c_uint64, c.c_uint64]
        L.o_hadamard_signs.restype = c.c_uint32
        L.o_hadamard_signs.argtypes = [c.c_uint64]
        L.o_fwht32.restype = None
        L.o_fwht32.argtypes = [c.POINTER(c.c_float), c.c_uint32]
        L.o_fwht16.restype = None
        L.o_fwht16.argtypes = [c.POINTER(c.c_float), c.c_uint32]
        L.o_unfwht32.restype = None
        L.o_unfwht32.argtypes = [c.POINTER(c.c_float), c.c_uint32]
        L.o_unfwht16.restype = None
        L.o_unfwht16.argtypes = [c.POINTER(c.c_float), c.c_uint32]
        L.o_tensor_amax.restype = c.c_float
        L.o_tensor_amax.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_int64]
        L.o_quantize.restype = c.c_int
        L.o_quantize.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_int64,
                                 c.c_int, c.c_int, c.c_int, c.c_uint64, c.c_uint64,
                                 c.c_int, c.c_uint32, c.c_int, c.c_float,
                                 c.c_void_p, c.c_void_p, c.POINTER(c.c_float),
                                 c.POINTER(c.c_float)]
        L.o_quantize_noise.restype = c.c_int
        L.o_quantize_noise.argtypes = L.o_quantize.argtypes + [c.c_void_p]
        L.o_quantize_2d.restype = c.c_int
        L.o_quantize_2d.argtypes = [c.c_void_p, c.c_int, c.c_int64, c.c_int64, c.c_int64, c.c_int, c.c_int,
                                    c.c_uint64, c.c_uint64, c.c_int, c.c_float, c.c_void_p, c.c_void_p,
                                    c.c_void_p, c.c_void_p, c.POINTER(c.c_float), c.POINTER(c.c_float)]
        L.o_dequantize_f32.restype = c.c_int
        L.o_dequantize_f32.argtypes = [c.c_void_p, c.c_void_p, c.c_int64, c.c_int64, c.c_int,
                                       c.c_float, c.c_void_p]
        L.o_dequantize_f64.restype = c.c_int
        L.o_dequantize_f64.argtypes = [c.c_void_p, c.c_void_p, c.c_int64, c.c_int64, c.c_int,
                                       c.c_float, c.c_void_p]
        L.o_dequantize_unrotated_f32.restype = c.c_int
        L.o_dequantize_unrotated_f32.argtypes = [c.c_void_p, c.c_void_p, c.c_int64, c.c_int64, c.c_int,
                                                 c.c_float, c.c_uint32, c.c_void_p]
        L.o_num_threads.restype = c.c_int
        _lib = L
    return _lib


# ---------------------------------------------------------------- scalars
def e2m1_value(code: int) -> float:
    return lib().o_e2m1_value(code)


def e2m1_rtn_mag(a: float) -> int:
    return lib().o_e2m1_rtn_mag(a)


def e2m1_sr_mag(a: float, h16: int) -> int:
    return lib().o_e2m1_sr_mag(a, h16)


def e4m3_value(b: int) -> float:
    return lib().o_e4m3_value(b)


def e4m3_encode(t: float) -> int:
    return lib().o_e4m3_encode(t)


def e8m0_exponent(amax: float) -> int:
    return lib().o_e8m0_exponent(amax)


def e8m0_value(b: int) -> float:
    return lib().o_e8m0_value(b)


def f32_to_bf16_rne(x: float) -> int:
    return lib().o_f32_to_bf16_rne(x)


def philox4x32_10(ctr, key):
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    lib().o_philox4x32_10(c, k, o)
    return [int(v) for v in o]


def sr_draw16(seed: int, index: int) -> int:
    return lib().o_sr_draw16(seed, index)


def hadamard_signs(seed: int) -> int:
    return lib().o_hadamard_signs(seed)


def fwht32(x, signs: int) -> np.ndarray:
    buf = np.ascontiguousarray(np.asarray(x, dtype=np.float32).copy())
    assert buf.shape == (32,)
    lib().o_fwht32(buf.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), signs)
    return buf


def fwht16(x, signs: int) -> np.ndarray:
    buf = np.ascontiguousarray(np.asarray(x, dtype=np.float32).copy())
    assert buf.shape == (16,)
    lib().o_fwht16(buf.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), signs)
    return buf


def unfwht32(y, signs: int) -> np.ndarray:
    """The inverse (transpose) of fwht32: FWHT stages, times 2^-2.5, then the signs."""
    buf = np.ascontiguousarray(np.asarray(y, dtype=np.float32).copy())
    assert buf.shape == (32,)
    lib().o_unfwht32(buf.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), signs)
    return buf


def unfwht16(y, signs: int) -> np.ndarray:
    """The inverse of fwht16: FWHT stages, times 1/4, then the signs."""
    buf = np.ascontiguousarray(np.asarray(y, dtype=np.float32).copy())
    assert buf.shape == (16,)
    lib().o_unfwht16(buf.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), signs)
    return buf


def num_threads() -> int:
    return lib().o_num_threads()


# ---------------------------------------------------------------- tensors
def _src(x: np.ndarray):
    """(pointer-able contiguous array, is_bf16). bf16 tensors travel as uint16 bits."""
    if x.dtype == np.uint16:
        return np.ascontiguousarray(x), 1
    if x.dtype == np.float32:
        return np.ascontiguousarray(x), 0
    raise TypeError(f"oracle takes float32 or bf16 bits (uint16), got {x.dtype}")


def tensor_amax(x: np.ndarray) -> float:
    a, bf = _src(x)
    R, C = a.shape
    return float(lib().o_tensor_amax(a.ctypes.data, bf, R, C, C))


def quantize(x: np.ndarray, axis: int = AXIS_COLS, fmt: int = FMT_NVFP4, rnd: int = RTN,
             seed: int = 0, index_offset: int = 0, had_on: bool = False, had_signs: int = 0,
             amax: float | None = None, noise: bool = False) -> dict:
    """Quantize a 2-D float32 (or bf16-bits uint16) matrix. Returns codes, scales
    (uint8, quantized orientation), and for NVFP4 the tensor amax and scale.
    noise: also return "noise" = [sum x^2, sum (xhat - x)^2] (FP64) over the
    quantized values x and the exact values xhat of their codes."""
    a, bf = _src(x)
    R, C = a.shape
    B = BLOCK[fmt]
    rows_q, cols_q = (C, R) if axis == AXIS_ROWS else (R, C)
    codes = np.zeros((rows_q, cols_q // 2), dtype=np.uint8)
    scales = np.zeros((rows_q, cols_q // B), dtype=np.uint8)
    am = ctypes.c_float(0.0)
    sg = ctypes.c_float(1.0)
    args = (a.ctypes.data, bf, R, C, C, axis, fmt, rnd, seed, index_offset,
            int(bool(had_on)), had_signs, int(amax is not None),
            float(amax or 0.0), codes.ctypes.data, scales.ctypes.data,
            ctypes.byref(am), ctypes.byref(sg))
    nz = np.zeros(2, dtype=np.float64)
    if noise:
        rc = lib().o_quantize_noise(*args, nz.ctypes.data)
    else:
        rc = lib().o_quantize(*args)
    if rc != 0:
        raise ValueError(f"oracle quantize rejected its input (rc={rc})")
    out = {"codes": codes, "scales": scales, "fmt": fmt, "rows": rows_q, "cols": cols_q}
    if fmt == FMT_NVFP4:
        out["amax"] = float(am.value)
        out["sg"] = float(sg.value)
    else:
        out["amax"] = None
        out["sg"] = 1.0
    if noise:
        out["noise"] = nz
    return out


def noise_ratio(sums) -> float:
    """The gradient-noise monitor's statistic ("FP4 All the Way", Summary: the
    threshold relates the gradient norm to the quantization noise norm): the
    ratio of the two norms, sqrt(sum x^2 / sum (xhat - x)^2), from the FP64 sums
    `quantize(..., noise=True)` returns. No noise gives +inf (0 when the
    tensor is 0 too)."""
    g, e = float(sums[0]), float(sums[1])
    if e > 0.0:
        return (g / e) ** 0.5
    return float("inf") if g > 0.0 else 0.0


def quantize_2d(x: np.ndarray, fmt: int = FMT_NVFP4, rnd: int = RTN, seed: int = 0,
                index_offset: int = 0, amax: float | None = None):
    """Two-dimensional B x B block quantization. Returns (q, q_t): the [R, C]
    quantization (blocks along C) and its transpose [C, R] (blocks along R),
    both in the layout of quantize()."""
    a, bf = _src(x)
    R, C = a.shape
    B = BLOCK[fmt]
    codes = np.zeros((R, C // 2), dtype=np.uint8)
    scales = np.zeros((R, C // B), dtype=np.uint8)
    codes_t = np.zeros((C, R // 2), dtype=np.uint8)
    scales_t = np.zeros((C, R // B), dtype=np.uint8)
    am = ctypes.c_float(0.0)
    sg = ctypes.c_float(1.0)
    rc = lib().o_quantize_2d(a.ctypes.data, bf, R, C, C, fmt, rnd, seed, index_offset,
                             int(amax is not None), float(amax or 0.0), codes.ctypes.data,
                             scales.ctypes.data, codes_t.ctypes.data, scales_t.ctypes.data,
                             ctypes.byref(am), ctypes.byref(sg))
    if rc != 0:
        raise ValueError(f"oracle quantize_2d rejected its input (rc={rc})")
    out = []
    for cd, scl, rows, cols in ((codes, scales, R, C), (codes_t, scales_t, C, R)):
        q = {"codes": cd, "scales": scl, "fmt": fmt, "rows": rows, "cols": cols}
        if fmt == FMT_NVFP4:
            q["amax"], q["sg"] = float(am.value), float(sg.value)
        else:
            q["amax"], q["sg"] = None, 1.0
        out.append(q)
    return out[0], out[1]


def dequantize_f32(q: dict) -> np.ndarray:
    out = np.zeros((q["rows"], q["cols"]), dtype=np.float32)
    rc = lib().o_dequantize_f32(np.ascontiguousarray(q["codes"]).ctypes.data,
                                np.ascontiguousarray(q["scales"]).ctypes.data,
                                q["rows"], q["cols"], q["fmt"], q["sg"], out.ctypes.data)
    assert rc == 0
    return out


def dequantize_unrotated_f32(q: dict, had_signs: int) -> np.ndarray:
    """dequantize_f32 followed by the inverse of the quantization's block
    rotation (16-wide for NVFP4, 32-wide for MXFP4) with the same sign mask:
    the values read back in the tensor's own domain (quantized orientation)."""
    out = np.zeros((q["rows"], q["cols"]), dtype=np.float32)
    rc = lib().o_dequantize_unrotated_f32(np.ascontiguousarray(q["codes"]).ctypes.data,
                                          np.ascontiguousarray(q["scales"]).ctypes.data,
                                          q["rows"], q["cols"], q["fmt"], q["sg"], had_signs,
                                          out.ctypes.data)
    assert rc == 0
    return out


def dequantize_f64(q: dict) -> np.ndarray:
    out = np.zeros((q["rows"], q["cols"]), dtype=np.float64)
    rc = lib().o_dequantize_f64(np.ascontiguousarray(q["codes"]).ctypes.data,
                                np.ascontiguousarray(q["scales"]).ctypes.data,
                                q["rows"], q["cols"], q["fmt"], q["sg"], out.ctypes.data)
    assert rc == 0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even FP32 -> bf16 bits (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------- GEMM
def gemm_ref(qa: dict, qb: dict, rows: np.ndarray | None = None):
    """FP64 product C = A_hat * B_hat^T of two quantized operands blocked along
    the shared contraction axis, and S = |A_hat| * |B_hat|^T (the sum of
    |a_k b_k| that bounds the accumulation error). `rows` selects A rows."""
    if qa["fmt"] != qb["fmt"] or qa["cols"] != qb["cols"]:
        raise ValueError("operands must share format and contraction length")
    A = dequantize_f64(qa)
    Bm = dequantize_f64(qb)
    if rows is not None:
        A = A[rows]
    ref = A @ Bm.T
    S = np.abs(A) @ np.abs(Bm).T
    return ref, S


def gemm_tolerance(ref: np.ndarray, S: np.ndarray, out_dtype: str) -> np.ndarray:
    """Per-element bound: 1e-5 * sum|a_k b_k| for FP32 output; a bf16 output
    also carries its own rounding, 2^-8 |ref|."""
    tol = 1e-5 * S
    if out_dtype == "bf16":
        tol = tol + np.abs(ref) * 2.0 ** -8
    return tol


def gemm_check(y: np.ndarray, ref: np.ndarray, S: np.ndarray, out_dtype: str):
    """Returns (ok, worst error as a fraction of the bound)."""
    y = np.asarray(y, dtype=np.float64)
    err = np.abs(y - ref)
    tol = gemm_tolerance(ref, S, out_dtype)
    zero = tol == 0
    ok_zero = bool(np.all(y[zero] == 0.0))
    frac = np.where(zero, 0.0, err / np.where(zero, 1.0, tol))
    worst = float(frac.max()) if frac.size else 0.0
    return bool(ok_zero and worst <= 1.0), worst
