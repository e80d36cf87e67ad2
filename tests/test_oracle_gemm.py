"""Pins of the oracle's GEMM reference and tolerance check.

The reference is the definition: the FP64 product of the exactly dequantized
operands (Robots Atlas, "FP4", How it works: FP4 operands, higher-precision
accumulation). It is pinned against exact rational arithmetic and integer
special cases.
"""
from fractions import Fraction

import numpy as np
import torch

E2M1 = [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def _rational_operand(q):
    """Exact dequantized values as Fractions, decoded independently of the
    oracle: E2M1 from the grid the pages print, E4M3 through PyTorch's
    float8_e4m3fn, E8M0 as 2^(byte-127)."""
    B = 16 if q["fmt"] == 0 else 32
    codes = q["codes"]
    rows, cols = q["rows"], q["cols"]
    e4m3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    out = []
    for r in range(rows):
        row = []
        for c in range(cols):
            byte = int(codes[r, c // 2])
            code = (byte >> (4 * (c % 2))) & 15
            val = Fraction(E2M1[code & 7]) * (-1 if code & 8 else 1)
            sb = int(q["scales"][r, c // B])
            if q["fmt"] == 0:
                val *= Fraction(float(e4m3[sb])) * Fraction(q["sg"])
            else:
                val *= Fraction(2) ** (sb - 127)
            row.append(val)
        out.append(row)
    return out


def test_reference_matches_exact_rational_product(orc):
    rng = np.random.default_rng(0)
    for fmt, (M, N, K) in [(0, (8, 8, 128)), (1, (8, 8, 128)), (0, (4, 4, 256))]:
        A = (rng.standard_normal((M, K)) * np.exp(rng.uniform(-3, 3, (M, 1)))).astype(np.float32)
        Bm = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
        qa, qb = orc.quantize(A, fmt=fmt), orc.quantize(Bm, fmt=fmt)
        ref, S = orc.gemm_ref(qa, qb)
        Ar, Br = _rational_operand(qa), _rational_operand(qb)
        for i in range(M):
            for j in range(N):
                exact = sum(a * b for a, b in zip(Ar[i], Br[j]))
                sabs = sum(abs(a * b) for a, b in zip(Ar[i], Br[j]))
                assert abs(Fraction(ref[i, j]) - exact) <= Fraction(1, 10 ** 12) * sabs
                assert abs(Fraction(S[i, j]) - sabs) <= Fraction(1, 10 ** 12) * sabs


def test_unit_scales_reduce_to_an_integer_matmul(orc):
    # codes in {0, +1, -1} (0x0, 0x2, 0xA) with every block scale 1.0 (E4M3
    # 0x38, tensor scale 1) give an integer matrix product.
    rng = np.random.default_rng(1)
    M, N, K = 16, 24, 256
    pick = np.array([0x0, 0x2, 0xA], dtype=np.uint8)
    ia = rng.integers(0, 3, (M, K))
    ib = rng.integers(0, 3, (N, K))

    def mk(idx, rows):
        c = pick[idx]
        return {"codes": (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8),
                "scales": np.full((rows, K // 16), 0x38, dtype=np.uint8),
                "fmt": 0, "rows": rows, "cols": K, "sg": 1.0}

    ival = np.array([0, 1, -1])
    ref, S = orc.gemm_ref(mk(ia, M), mk(ib, N))
    assert np.array_equal(ref, (ival[ia] @ ival[ib].T).astype(np.float64))
    assert np.array_equal(S, (np.abs(ival[ia]) @ np.abs(ival[ib]).T).astype(np.float64))


def test_tolerance_check_accepts_and_rejects(orc):
    rng = np.random.default_rng(2)
    A = rng.standard_normal((32, 256)).astype(np.float32)
    Bm = rng.standard_normal((48, 256)).astype(np.float32)
    ref, S = orc.gemm_ref(orc.quantize(A), orc.quantize(Bm))
    ok, worst = orc.gemm_check(ref + 0.5e-5 * S, ref, S, "fp32")
    assert ok and 0.49 < worst < 0.51
    ok, _ = orc.gemm_check(ref + 2e-5 * S, ref, S, "fp32")
    assert not ok
    # a dropped term (one k missing) is caught
    qa, qb = orc.quantize(A), orc.quantize(Bm)
    Ad, Bd = orc.dequantize_f64(qa), orc.dequantize_f64(qb)
    dropped = Ad[:, 1:] @ Bd[:, 1:].T
    ok, _ = orc.gemm_check(dropped, ref, S, "fp32")
    assert not ok
    # bf16 output carries its own rounding
    y16 = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert orc.gemm_check(y16, ref, S, "bf16")[0]
    assert not orc.gemm_check(y16, ref, S, "fp32")[0]


def test_zero_rows_need_exact_zero(orc):
    A = np.zeros((16, 128), dtype=np.float32)
    Bm = np.ones((16, 128), dtype=np.float32)
    ref, S = orc.gemm_ref(orc.quantize(A), orc.quantize(Bm))
    assert orc.gemm_check(np.zeros_like(ref), ref, S, "fp32")[0]
    assert not orc.gemm_check(np.full_like(ref, 1e-30), ref, S, "fp32")[0]
