"""Pins of the oracle's scalar codecs, random stream and rotation.

Each test checks the oracle against something other than itself: the grid the
pages print, hand-derived fixtures, an independent library (PyTorch's float8
casts, ATen's Philox engine, SciPy's Hadamard matrix), published known-answer
vectors, or a differently derived algorithm.
"""
import math
import os
import struct
import subprocess
import tempfile

import numpy as np
import pytest
import torch

from golden_io import fields, rows


def f32(x):
    return struct.unpack("<f", struct.pack("<f", x))[0]


def f32_bits(x):
    return struct.unpack("<I", struct.pack("<f", x))[0]


def bits_f32(u):
    return struct.unpack("<f", struct.pack("<I", u))[0]


# ------------------------------------------------------------------ E2M1
def test_e2m1_grid_is_the_pages_grid(orc):
    # Robots Atlas, "FP4", Components / E2M1 format: 0, 0.5, 1, 1.5, 2, 3, 4, 6
    assert [orc.e2m1_value(c) for c in range(8)] == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert [orc.e2m1_value(8 | c) for c in range(8)] == [-0.0, -0.5, -1, -1.5, -2, -3, -4, -6]
    assert math.copysign(1.0, orc.e2m1_value(8)) == -1.0


def test_e2m1_rtn_midpoints_fixture(orc):
    for a, code, val in rows("e2m1_rtn_ties.txt"):
        assert orc.e2m1_rtn_mag(float(a)) == int(code), a
        assert orc.e2m1_value(int(code)) == float(val)


def _rtn_by_mantissa_rounding(a):
    """Independent derivation: E2M1 has one mantissa bit, so for a >= 1 round
    the fp32 significand to 1 bit (round half to even via integer carry); below
    1 the spacing is 0.5 (numpy rint is half-to-even)."""
    if a < 1.0:
        return float(np.rint(np.float32(a) * np.float32(2))) / 2.0
    u = f32_bits(a)
    u = (u + 0x1FFFFF + ((u >> 22) & 1)) & 0xFFC00000
    return min(bits_f32(u), 6.0)


def test_e2m1_rtn_matches_mantissa_rounding(orc):
    vals = set()
    for e in range(-12, 3):                    # binades 2^-12 .. 2^2 (covers (0, 6])
        for m in range(0, 1 << 23, 1 << 12):   # 2048 significands per binade
            v = bits_f32(((e + 127) << 23) | m)
            if v <= 6.0:
                vals.add(v)
    for mid in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
        u = f32_bits(mid)
        vals.update({mid, bits_f32(u - 1), bits_f32(u + 1)})
    vals.update({0.0, 6.0})
    for a in sorted(vals):
        got = orc.e2m1_value(orc.e2m1_rtn_mag(a))
        assert got == _rtn_by_mantissa_rounding(a), a


# ------------------------------------------------------------------ E4M3
def test_e4m3_decode_matches_torch(orc):
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()
    for b in range(256):
        v = orc.e4m3_value(b)
        if math.isnan(t[b]):
            assert math.isnan(v), b
        else:
            assert v == float(t[b]), b
    assert orc.e4m3_value(0x7E) == 448.0          # largest finite value


def _e4m3_sweep():
    vals = set()
    for e in range(-20, 9):
        for m in range(0, 1 << 23, 1 << 14):
            v = bits_f32(((e + 127) << 23) | m)
            if v <= 464.0:
                vals.add(v)
    # every midpoint between neighbouring E4M3 values, and one ulp either side
    pos = sorted({float(v) for v in torch.arange(0x7F, dtype=torch.uint8)
                  .view(torch.float8_e4m3fn).float().numpy()})
    for lo, hi in zip(pos, pos[1:]):
        mid = f32((lo + hi) / 2)
        u = f32_bits(mid)
        vals.update({mid, bits_f32(u - 1), bits_f32(u + 1)})
    vals.update({0.0, 448.0, 464.0})
    return sorted(vals)


def test_e4m3_encode_matches_torch_cast(orc):
    # PyTorch's float8_e4m3fn cast rounds to nearest even and agrees with a
    # saturating encoder on [0, 464] (above 464 it gives NaN, which the
    # block-scale rule never asks for).
    vals = _e4m3_sweep()
    ref = torch.tensor(vals, dtype=torch.float32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for v, r in zip(vals, ref):
        assert orc.e4m3_encode(v) == int(r), v


def test_e4m3_encode_saturates(orc):
    for v in (448.0, 449.0, 463.99, 464.0, 465.0, 1e6, 3.0e38):
        assert orc.e4m3_encode(v) == 0x7E


# ------------------------------------------------------------------ E8M0
def test_e8m0_decode_matches_torch(orc):
    t = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().numpy()
    for b in range(255):
        assert orc.e8m0_value(b) == float(t[b]) or (b == 0 and orc.e8m0_value(0) == 2.0 ** -127)
    assert math.isnan(orc.e8m0_value(255))


def test_e8m0_exponent_integer_form(orc):
    # Independent derivation of the round-up rule: write amax = m * 2^E with
    # m in [1, 2). Then 6 * 2^e >= amax holds first at e = E - 2 when m <= 1.5
    # and at e = E - 1 otherwise; clamp below at -127.
    rng = np.random.default_rng(5)
    vals = list(np.float32(rng.uniform(0.5, 2.0, 4000)) * np.float32(2.0) **
                rng.integers(-140, 120, 4000).astype(np.float32))
    for E in range(-126, 127):
        for m in (1.0, 1.5, f32(1.5 + 2 ** -22), 1.25, f32(2 - 2 ** -23)):
            vals.append(f32(m * 2.0 ** E))
    vals += [0.0, 1e-45, 6.0, 3.0, f32(3.0 + 2 ** -21), 3.4e38]
    for a in vals:
        a = float(np.float32(a))
        if a == 0.0 or not np.isfinite(a):
            exp = -127
        else:
            m, E = math.frexp(a)      # a = m * 2^E, m in [0.5, 1)
            m, E = m * 2, E - 1       # m in [1, 2)
            exp = E - 2 if m <= 1.5 else E - 1
            exp = max(exp, -127)
        assert orc.e8m0_exponent(a) == exp, a


# ------------------------------------------------------------------ bf16
def test_bf16_rounding_matches_torch(orc):
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.standard_normal(5000).astype(np.float32) * 10.0 **
                        rng.integers(-30, 30, 5000).astype(np.float32),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -9], dtype=np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    for v, r in zip(x, ref):
        assert orc.f32_to_bf16_rne(float(v)) == int(r)


# ------------------------------------------------------------------ Philox
def test_philox_known_answer_vectors(orc):
    for r in rows("philox4x32_10_kat.txt"):
        v = [int(t, 16) for t in r]
        assert orc.philox4x32_10(v[0:4], v[4:6]) == v[6:10]


ATEN_DRIVER = r"""
#include <ATen/core/PhiloxRNGEngine.h>
#include <cstdio>
#include <cstdint>
int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llx %llx %llx", &seed, &sub, &off) == 3) {
    at::philox_engine e(seed, sub, off);
    unsigned a = e(), b = e(), c = e(), d = e();
    std::printf("%08x %08x %08x %08x\n", a, b, c, d);
  }
}
"""


@pytest.fixture(scope="module")
def aten_philox():
    """ATen's header-only Philox4x32-10 engine, compiled here with g++ (a
    library run, not a retype): a function mapping (seed, subsequence, offset)
    triples to the four output words of the engine's first block. ATen's engine
    uses key = seed and counter = (offset lo/hi, subsequence lo/hi)."""
    inc = os.path.join(os.path.dirname(torch.__file__), "include")
    if not os.path.exists(os.path.join(inc, "ATen", "core", "PhiloxRNGEngine.h")):
        pytest.skip("ATen headers not installed")
    d = tempfile.mkdtemp()
    src = os.path.join(d, "drv.cpp")
    exe = os.path.join(d, "drv")
    with open(src, "w") as f:
        f.write(ATEN_DRIVER)
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", inc, src, "-o", exe], check=True)

    def run(triples):
        inp = "\n".join(f"{int(s):x} {int(u):x} {int(o):x}" for s, u, o in triples)
        out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
        return [[int(t, 16) for t in line.split()] for line in out.strip().split("\n")]

    yield run
    os.remove(exe)
    os.remove(src)
    os.rmdir(d)


def test_philox_matches_aten_engine(orc, aten_philox):
    rng = np.random.default_rng(11)
    cases = rng.integers(0, 2 ** 63, size=(4000, 3), dtype=np.uint64) * np.uint64(2) + \
        rng.integers(0, 2, size=(4000, 3), dtype=np.uint64)
    out = aten_philox(cases)
    for (s, u, o), words in zip(cases, out):
        s, u, o = int(s), int(u), int(o)
        ctr = [o & 0xFFFFFFFF, o >> 32, u & 0xFFFFFFFF, u >> 32]
        key = [s & 0xFFFFFFFF, s >> 32]
        assert orc.philox4x32_10(ctr, key) == words


def test_sr_stream_layout_from_known_answer_vector(orc):
    # Seed 0, elements 0..7: the eight 16-bit halves of the published first
    # known-answer block, in little-endian order (derivation in the fixture).
    for seed, i, draw in rows("sr_stream_layout.txt"):
        assert orc.sr_draw16(int(seed), int(i)) == int(draw, 16), (seed, i)


def test_sr_stream_layout_matches_aten_engine(orc, aten_philox):
    # Element i's draw is half number i % 8 (little-endian) of the 16-byte
    # output block of ATen's engine at offset i / 8 (subsequence 0), for seeds
    # with both key words set and for indices whose block counter needs its
    # high word (i / 8 >= 2^32).
    rng = np.random.default_rng(12)
    seeds = [0, 1, 0x1234_5678_9ABC_DEF0, (2 << 8) | 3] + \
        [int(v) for v in rng.integers(0, 2 ** 63, size=4, dtype=np.uint64)]
    bases = [0, 8, 4096 * 8 + 8, (1 << 35) - 8, (1 << 35), (3 << 40) + 16] + \
        [int(v) * 8 for v in rng.integers(0, 2 ** 58, size=6, dtype=np.uint64)]
    triples = [(s, 0, b >> 3) for s in seeds for b in bases]
    blocks = aten_philox(triples)
    for (s, _, call), words in zip(triples, blocks):
        halves = np.frombuffer(np.array(words, dtype="<u4").tobytes(), dtype="<u2")
        for j in range(8):
            assert orc.sr_draw16(s, call * 8 + j) == int(halves[j]), (hex(s), call, j)


def test_sr_draws_are_uniform_and_distinct_per_seed(orc):
    n = 1 << 15
    d0 = np.array([orc.sr_draw16(7, i) for i in range(n)])
    d1 = np.array([orc.sr_draw16(8, i) for i in range(n)])
    assert d0.min() >= 0 and d0.max() < 65536
    counts = np.bincount(d0 >> 12, minlength=16)         # 16 bins, chi-square
    chi2 = (((counts - n / 16) ** 2) / (n / 16)).sum()
    assert chi2 < 50.0                                    # 15 dof: p ~ 1e-5
    assert np.mean(d0 == d1) < 0.001
    assert abs(np.corrcoef(d0[:-1], d0[1:])[0, 1]) < 0.03


# ------------------------------------------------------------------ stochastic rounding
def test_sr_decision_fixture(orc):
    for a, h, code in rows("sr_decisions.txt"):
        assert orc.e2m1_sr_mag(f32(float(a)), int(h)) == int(code), (a, h)


def test_sr_support_and_fixed_points(orc):
    grid = [orc.e2m1_value(c) for c in range(8)]
    for a in [0.1, 0.3, 0.6, 0.9, 1.2, 1.6, 1.9, 2.2, 2.7, 3.3, 3.9, 4.4, 5.5, 5.99]:
        a = f32(a)
        lo = max(g for g in grid if g <= a)
        hi = min(g for g in grid if g > a)
        for h in (0, 1, 12345, 32768, 65534, 65535):
            assert grid[orc.e2m1_sr_mag(a, h)] in (lo, hi)
    for c, g in enumerate(grid):
        for h in (0, 32768, 65535):
            assert orc.e2m1_sr_mag(g, h) == c


def test_sr_is_unbiased(orc):
    # Over N draws of the element stream the mean of the rounded value equals
    # a within 5 standard errors, plus the 2^-16 resolution of the draw (of
    # the grid step between a's neighbours: below 2^-16 of a step, as for
    # 1e-6, the value never rounds up).
    n = 40000
    grid = [orc.e2m1_value(c) for c in range(8)]
    for a in [0.25, 0.1, 0.75, 1.1, 1.75, 2.5, 3.3, 5.0, 5.99, 1e-6]:
        a = f32(a)
        vals = np.array([orc.e2m1_value(orc.e2m1_sr_mag(a, orc.sr_draw16(3, i)))
                         for i in range(n)])
        sd = max(vals.std(), 1e-12)
        step = min(g for g in grid if g > a) - max(g for g in grid if g <= a)
        assert abs(vals.mean() - a) <= 5 * sd / math.sqrt(n) + step * 2 ** -16 + 1e-12, a


# ------------------------------------------------------------------ Hadamard
def test_rotation_constant():
    c = np.float32(2.0 ** -2.5)
    assert f32_bits(float(c)) == 0x3E3504F3


def test_fwht_is_sylvester_hadamard(orc):
    from scipy.linalg import hadamard
    H = hadamard(32)                               # Sylvester construction
    assert np.array_equal(H @ H.T, 32 * np.eye(32, dtype=H.dtype))
    c = np.float32(2.0 ** -2.5)
    rng = np.random.default_rng(2)
    for trial in range(200):
        signs = int(rng.integers(0, 2 ** 32))
        x = rng.integers(-(2 ** 18), 2 ** 18, 32).astype(np.int64)
        D = np.array([-1 if (signs >> j) & 1 else 1 for j in range(32)], dtype=np.int64)
        exact = H @ (D * x)                        # integer, |.| < 2^23: exact in fp32
        expect = exact.astype(np.float32) * c      # one rounding
        got = orc.fwht32(x.astype(np.float32), signs)
        assert np.array_equal(got, expect), trial


def test_fwht_orthonormal_and_invertible(orc):
    from scipy.linalg import hadamard
    H = hadamard(32).astype(np.float64)
    rng = np.random.default_rng(3)
    for _ in range(100):
        signs = int(rng.integers(0, 2 ** 32))
        x = rng.standard_normal(32).astype(np.float32)
        y = orc.fwht32(x, signs).astype(np.float64)
        D = np.array([-1.0 if (signs >> j) & 1 else 1.0 for j in range(32)])
        ref = (H @ (D * x.astype(np.float64))) * 2.0 ** -2.5
        assert np.max(np.abs(y - ref)) <= 6 * 2.0 ** -24 * np.linalg.norm(x)
        assert abs(np.linalg.norm(y) - np.linalg.norm(x)) <= 1e-5 * np.linalg.norm(x)
        back = D * (H.T @ y) * 2.0 ** -2.5          # inverse: D H^T c
        assert np.max(np.abs(back - x)) <= 1e-5 * np.linalg.norm(x)


def test_fwht16_is_sylvester_hadamard(orc):
    from scipy.linalg import hadamard
    H = hadamard(16)
    assert np.array_equal(H @ H.T, 16 * np.eye(16, dtype=H.dtype))
    rng = np.random.default_rng(4)
    for trial in range(200):
        signs = int(rng.integers(0, 2 ** 32))
        x = rng.integers(-(2 ** 19), 2 ** 19, 16).astype(np.int64)
        D = np.array([-1 if (signs >> j) & 1 else 1 for j in range(16)], dtype=np.int64)
        exact = H @ (D * x)                        # integer, |.| < 2^23: exact in fp32
        expect = exact.astype(np.float32) * np.float32(0.25)   # exact
        got = orc.fwht16(x.astype(np.float32), signs)
        assert np.array_equal(got, expect), trial
        # only bits 0..15 of the mask act
        assert np.array_equal(orc.fwht16(x.astype(np.float32), signs & 0xFFFF), got)


def test_fwht16_inverse_is_exact(orc):
    # (1/4) H16 is its own inverse; with integer x every step is exact, so
    # undoing the rotation (H16 / 4, then the signs) gives x back bit for bit.
    rng = np.random.default_rng(5)
    for _ in range(100):
        signs = int(rng.integers(0, 2 ** 16))
        x = rng.integers(-(2 ** 12), 2 ** 12, 16).astype(np.float32)
        y = orc.fwht16(x, signs)
        back = orc.fwht16(y, 0)
        D = np.array([-1.0 if (signs >> j) & 1 else 1.0 for j in range(16)], dtype=np.float32)
        assert np.array_equal(back * D, x)
        assert np.isclose(np.linalg.norm(y.astype(np.float64)), np.linalg.norm(x.astype(np.float64)),
                          rtol=1e-12)



def test_unfwht_is_the_transposed_rotation(orc):
    """unfwht = D H c, the transpose of c H D: on integer inputs every
    butterfly is exact, so the result is the integer product H y, rounded once
    by the product with c, then signed (a dropped sign, a wrong stage or the
    signs applied before H fail this)."""
    from scipy.linalg import hadamard
    c = np.float32(2.0 ** -2.5)
    for n, fn, k in ((32, orc.unfwht32, c), (16, orc.unfwht16, np.float32(0.25))):
        H = hadamard(n).astype(np.int64)
        rng = np.random.default_rng(40 + n)
        for trial in range(200):
            signs = int(rng.integers(0, 2 ** 32))
            y = rng.integers(-(2 ** 18), 2 ** 18, n).astype(np.int64)
            D = np.array([-1 if (signs >> j) & 1 else 1 for j in range(n)], dtype=np.float32)
            expect = (H @ y).astype(np.float32) * k * D
            assert np.array_equal(fn(y.astype(np.float32), signs), expect), (n, trial)


def test_unfwht_undoes_the_rotation(orc):
    rng = np.random.default_rng(42)
    for _ in range(100):
        signs = int(rng.integers(0, 2 ** 32))
        x = rng.standard_normal(32).astype(np.float32)
        back = orc.unfwht32(orc.fwht32(x, signs), signs).astype(np.float64)
        # two FP32 transforms of a norm-preserving map (c rounded to FP32)
        assert np.max(np.abs(back - x)) <= 1e-5 * np.linalg.norm(x.astype(np.float64))
        x16 = rng.integers(-(2 ** 12), 2 ** 12, 16).astype(np.float32)
        assert np.array_equal(orc.unfwht16(orc.fwht16(x16, signs), signs), x16)   # exact


def test_dequantize_unrotated(orc):
    """Read back in the source's domain: each block is the inverse rotation of
    the plain dequantization's block, and the result approximates the source
    as closely as the rotated dequantization approximates the rotated source
    (an orthonormal map keeps the error's norm)."""
    rng = np.random.default_rng(43)
    x = rng.standard_normal((48, 256)).astype(np.float32)
    for fmt, B, fn, fwd in ((1, 32, orc.unfwht32, orc.fwht32), (0, 16, orc.unfwht16, orc.fwht16)):
        signs = orc.hadamard_signs(11)
        q = orc.quantize(x, fmt=fmt, had_on=True, had_signs=signs)
        rot = orc.dequantize_f32(q)
        got = orc.dequantize_unrotated_f32(q, signs)
        for r in (0, 17, 47):
            for c0 in range(0, 256, B):
                assert np.array_equal(got[r, c0:c0 + B], fn(rot[r, c0:c0 + B], signs))
        xr = np.stack([np.concatenate([fwd(x[r, c0:c0 + B], signs) for c0 in range(0, 256, B)])
                       for r in range(48)]).astype(np.float64)
        e_rot = np.linalg.norm(rot.astype(np.float64) - xr)
        e_src = np.linalg.norm(got.astype(np.float64) - x.astype(np.float64))
        assert abs(e_src - e_rot) <= 1e-4 * np.linalg.norm(x.astype(np.float64)), (fmt, e_src, e_rot)

def test_hadamard_mask_is_a_separate_philox_counter(orc):
    # word 0 of counter (0,0,0,1), which the element stream (c2 = c3 = 0) never uses
    for seed in (0, 1, 3, 2 ** 40 + 5):
        w = orc.philox4x32_10([0, 0, 0, 1], [seed & 0xFFFFFFFF, seed >> 32])[0]
        assert orc.hadamard_signs(seed) == w
