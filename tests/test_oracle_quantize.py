"""Pins of the oracle's tensor quantizer and dequantizer.

Hand-derived worked examples (tests/golden/), invariants that follow from the
format definitions (Robots Atlas, "FP4", Components and How it works), the
statistics of stochastic rounding (FP4 All the Way, Key points), and exact
special cases.
"""
import math

import numpy as np
import pytest

from golden_io import fields


def unpack(codes):
    lo = codes & 0x0F
    hi = codes >> 4
    return np.stack([lo, hi], axis=-1).reshape(codes.shape[0], -1)


def load_worked(name, nblk, B):
    f = fields(name)
    x = np.zeros((1, nblk * B), dtype=np.float32)
    c = np.zeros(nblk * B, dtype=np.uint8)
    for b in range(nblk):
        xs = [float(v) for v in f[f"x{b}"]]
        cs = [int(v, 16) for v in f[f"c{b}"]]
        x[0, b * B:b * B + len(xs)] = xs
        c[b * B:b * B + len(cs)] = cs
    return f, x, c


def test_nvfp4_worked_example(orc):
    f, x, c = load_worked("nvfp4_worked.txt", 7, 16)
    q = orc.quantize(x, fmt=orc.FMT_NVFP4)
    assert q["amax"] == float(f["amax"][0]) and q["sg"] == float(f["sg"][0])
    assert list(q["scales"][0]) == [int(v, 16) for v in f["scales"]]
    assert list(unpack(q["codes"])[0]) == list(c)
    assert list(q["codes"][0, 8:16]) == [int(v, 16) for v in f["packed1"]]


def test_mxfp4_worked_example(orc):
    f, x, c = load_worked("mxfp4_worked.txt", 4, 32)
    q = orc.quantize(x, fmt=orc.FMT_MXFP4)
    assert list(q["scales"][0]) == [int(v, 16) for v in f["scales"]]
    assert list(unpack(q["codes"])[0]) == list(c)


def test_mxfp4_hadamard_worked_example(orc):
    f, x, c = load_worked("mxfp4_hadamard_worked.txt", 2, 32)
    q = orc.quantize(x, fmt=orc.FMT_MXFP4, had_on=True, had_signs=int(f["mask"][0], 16))
    assert list(q["scales"][0]) == [int(v, 16) for v in f["scales"]]
    assert list(unpack(q["codes"])[0]) == list(c)


def test_nvfp4_hadamard_worked_example(orc):
    f, x, c = load_worked("nvfp4_hadamard_worked.txt", 2, 16)
    q = orc.quantize(x, fmt=orc.FMT_NVFP4, had_on=True, had_signs=int(f["mask"][0], 16))
    assert q["amax"] == float(f["amax"][0])
    assert q["sg"] == float(np.float32(2.0) / np.float32(2688.0))
    assert list(q["scales"][0]) == [int(v, 16) for v in f["scales"]]
    assert list(unpack(q["codes"])[0]) == list(c)


def _rotate_blocks(x, B, signs):
    """(H_B D) applied to every B-block of each row, exactly, in integers."""
    from scipy.linalg import hadamard
    H = hadamard(B).astype(np.int64)
    D = np.array([-1 if (signs >> j) & 1 else 1 for j in range(B)], dtype=np.int64)
    R, C = x.shape
    blocks = x.astype(np.int64).reshape(R, C // B, B) * D
    return (blocks @ H.T).reshape(R, C)


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("rnd", [0, 1])
def test_nvfp4_hadamard_is_quantization_of_the_rotated_tensor(orc, axis, rnd):
    # Integer inputs with |H x| < 2^24: the rotation is exact in FP32, so the
    # rotated tensor is known without the oracle's butterfly; quantizing it
    # without rotation must give the same codes, scales and tensor scale.
    rng = np.random.default_rng(21)
    x = rng.integers(-1000, 1001, (48, 96)).astype(np.int64)
    x[5, 7] = 40000                                 # an outlier the rotation spreads
    signs = 0xA5C3F00F
    if axis == orc.AXIS_COLS:
        y = _rotate_blocks(x, 16, signs)
    else:
        y = _rotate_blocks(x.T, 16, signs).T
    yf = (y.astype(np.float64) * 0.25).astype(np.float32)
    assert np.array_equal(yf.astype(np.float64), y * 0.25)
    a = orc.quantize(x.astype(np.float32), axis=axis, fmt=orc.FMT_NVFP4, rnd=rnd, seed=3,
                     had_on=True, had_signs=signs)
    b = orc.quantize(np.ascontiguousarray(yf), axis=axis, fmt=orc.FMT_NVFP4, rnd=rnd, seed=3)
    assert a["amax"] == float(np.abs(yf).max()) != float(np.abs(x).max())
    assert a["sg"] == b["sg"]
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


def _randn(shape, seed, outliers=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    if outliers:
        cols = rng.permutation(shape[1])[: max(1, shape[1] // 100)]
        x[:, cols] *= 20
    return x


@pytest.mark.parametrize("fmt", [0, 1])
def test_amax_element_lands_on_the_top_of_the_grid(orc, fmt):
    # NVFP4 with a normal E4M3 scale: the block maximum maps to within 2^-4
    # (relative) of 6, so it rounds to 6. MXFP4 (round-up power of two): the
    # maximum maps into (3, 6], so it rounds to 3, 4 or 6.
    x = _randn((64, 512), 1, outliers=True)
    q = orc.quantize(x, fmt=fmt)
    B = 16 if fmt == 0 else 32
    mags = unpack(q["codes"]) & 7
    xb = np.abs(x).reshape(64, -1, B)
    arg = xb.argmax(axis=2)
    top = np.take_along_axis(mags.reshape(64, -1, B), arg[..., None], axis=2)[..., 0]
    if fmt == 0:
        normal = (q["scales"] >> 3) & 15 != 0
        assert np.all(top[normal] == 7)
    else:
        assert np.all(np.isin(top, [5, 6, 7]))


@pytest.mark.parametrize("fmt", [0, 1])
def test_rtn_error_bound(orc, fmt):
    # |x - x_hat| <= half the local grid step times the block's scale for
    # values inside the grid range (plus fp32 rounding of x * r).
    x = _randn((32, 256), 2, outliers=True)
    q = orc.quantize(x, fmt=fmt)
    deq = orc.dequantize_f64(q)
    B = 16 if fmt == 0 else 32
    s = np.repeat(q["scales"].astype(np.int64), B, axis=1)
    if fmt == 0:
        d = np.array([orc.e4m3_value(int(v)) for v in range(256)])[s] * q["sg"]
    else:
        d = 2.0 ** (s - 127)
    v = np.abs(x / d)
    step = np.select([v < 2, v < 4], [0.5, 1.0], 2.0)
    inside = v <= 6.0
    err = np.abs(x - deq)
    assert np.all(err[inside] <= 0.5 * step[inside] * d[inside] * (1 + 1e-6) + 1e-30)
    if fmt == 0:      # clipped values (NVFP4 only, |v| <= 6.4) err by at most 0.4 d
        assert np.all(err[~inside] <= 0.4 * d[~inside] * (1 + 1e-6))
    else:
        assert np.all(inside)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("k", [-95, -7, 3, 11])
def test_power_of_two_scale_invariance(orc, fmt, k):
    x = _randn((16, 256), 3)
    q0 = orc.quantize(x, fmt=fmt)
    q1 = orc.quantize(x * np.float32(2.0 ** k), fmt=fmt)
    assert np.array_equal(q0["codes"], q1["codes"])
    if fmt == 0:
        assert np.array_equal(q0["scales"], q1["scales"])
        assert q1["sg"] == q0["sg"] * 2.0 ** k
    else:
        assert np.array_equal(q0["scales"].astype(int) + k, q1["scales"].astype(int))


@pytest.mark.parametrize("fmt,rnd,had", [(0, 0, 0), (0, 1, 0), (0, 0, 1), (0, 1, 1), (1, 0, 0), (1, 1, 1)])
def test_rows_axis_equals_cols_axis_of_the_transpose(orc, fmt, rnd, had):
    x = _randn((96, 64), 4)
    a = orc.quantize(x, axis=orc.AXIS_ROWS, fmt=fmt, rnd=rnd, seed=9, had_on=had,
                     had_signs=0x1234567)
    b = orc.quantize(np.ascontiguousarray(x.T), axis=orc.AXIS_COLS, fmt=fmt, rnd=rnd,
                     seed=9, had_on=had, had_signs=0x1234567)
    assert np.array_equal(a["codes"], b["codes"]) and np.array_equal(a["scales"], b["scales"])


@pytest.mark.parametrize("rnd", [0, 1])
def test_vanishing_tensor_quantizes_to_signed_zeros(orc, rnd):
    # NVFP4 amax below 2^-100: s_g = 1, every block byte 0, every code a signed zero
    x = _randn((32, 64), 18) * np.float32(1e-32)
    assert np.abs(x).max() < 2.0 ** -100
    q = orc.quantize(x, fmt=0, rnd=rnd, seed=2)
    assert q["sg"] == 1.0 and q["amax"] == float(np.abs(x).max())
    assert (q["scales"] == 0).all()
    u = unpack(q["codes"])
    assert np.array_equal(u, np.where(np.signbit(x), 8, 0))
    # just above the floor the tensor is quantized as usual (power-of-two invariance)
    y = _randn((32, 64), 18)
    k = -100 - int(np.floor(np.log2(np.abs(y).max())))
    q0, q1 = orc.quantize(y, fmt=0), orc.quantize(y * np.float32(2.0 ** k), fmt=0)
    assert q1["amax"] >= 2.0 ** -100
    assert np.array_equal(q0["codes"], q1["codes"]) and np.array_equal(q0["scales"], q1["scales"])


def test_bf16_input_equals_its_fp32_value(orc):
    x = _randn((32, 128), 5)
    bits = orc.f32_to_bf16_bits(x)
    a = orc.quantize(bits, fmt=0, rnd=1, seed=3)
    b = orc.quantize(orc.bf16_bits_to_f32(bits), fmt=0, rnd=1, seed=3)
    assert np.array_equal(a["codes"], b["codes"]) and a["sg"] == b["sg"]


def test_given_amax_equals_computed_amax(orc):
    x = _randn((32, 128), 6)
    a = orc.quantize(x, fmt=0)
    b = orc.quantize(x, fmt=0, amax=float(np.abs(x).max()))
    assert np.array_equal(a["codes"], b["codes"]) and a["sg"] == b["sg"]
    assert a["amax"] == float(np.abs(x).max())
    assert a["sg"] == float(np.float32(np.abs(x).max()) / np.float32(2688.0))


def test_zero_tensor(orc):
    x = np.zeros((16, 64), dtype=np.float32)
    q = orc.quantize(x, fmt=0)
    assert q["amax"] == 0.0 and q["sg"] == 1.0
    assert not q["codes"].any() and not q["scales"].any()
    m = orc.quantize(x, fmt=1)
    assert not m["codes"].any() and np.all(m["scales"] == 0)


def test_non_finite_input_is_rejected(orc):
    x = np.ones((16, 64), dtype=np.float32)
    x[3, 5] = np.inf
    with pytest.raises(ValueError):
        orc.quantize(x)
    x[3, 5] = np.nan
    with pytest.raises(ValueError):
        orc.quantize(x, fmt=1)


def test_mxfp4_requantize_is_idempotent(orc):
    x = _randn((32, 256), 7, outliers=True)
    d1 = orc.dequantize_f32(orc.quantize(x, fmt=1))
    d2 = orc.dequantize_f32(orc.quantize(d1, fmt=1))
    assert np.array_equal(d1, d2)


def test_dequantize_f32_is_one_rounding_of_the_exact_value(orc):
    x = _randn((32, 256), 8, outliers=True)
    for fmt in (0, 1):
        q = orc.quantize(x, fmt=fmt)
        assert np.array_equal(orc.dequantize_f32(q), orc.dequantize_f64(q).astype(np.float32))


@pytest.mark.parametrize("fmt", [0, 1])
def test_sr_tensor_is_unbiased(orc, fmt):
    # Over independent seeds, each element rounds up (to the upper grid
    # neighbour of v = x * r) with probability p = (v - lo) / (hi - lo): the
    # count of ups is Binomial(n, p) up to the 2^-16 resolution of the draw.
    x = _randn((8, 64), 9)
    n = 400
    B = 16 if fmt == 0 else 32
    q = orc.quantize(x, fmt=fmt)
    s = np.repeat(q["scales"].astype(np.int64), B, axis=1)
    if fmt == 0:
        d = (np.array([orc.e4m3_value(int(v)) for v in range(256)])[s] * q["sg"]).astype(np.float32)
        r = np.where(d == 0, np.float32(0), np.float32(1) / d)
    else:
        r = (2.0 ** (127 - s)).astype(np.float32)
    v = np.abs(x * r)                                     # fp32, as the quantizer computes it
    grid = np.array([orc.e2m1_value(c) for c in range(8)])
    inside = v < 6.0
    lo_i = np.clip(np.searchsorted(grid, v, side="right") - 1, 0, 6)
    lo, hi = grid[lo_i], grid[lo_i + 1]
    p = np.where(inside, (v - lo) / (hi - lo), 0.0)
    ups = np.zeros(x.shape)
    for sd in range(n):
        mags = unpack(orc.quantize(x, fmt=fmt, rnd=orc.SR, seed=1000 + sd)["codes"]) & 7
        ups += grid[mags] == hi
    k, mu = ups[inside], n * p[inside]
    var = n * p[inside] * (1 - p[inside])
    assert np.all(np.abs(k - mu) <= 5 * np.sqrt(var) + 1.0)
    assert abs((k - mu).sum()) <= 5 * math.sqrt(var.sum()) + 1.0


def test_sr_index_offset_shifts_the_stream(orc):
    x = _randn((4, 64), 10)
    full = orc.quantize(np.vstack([x, x]), fmt=1, rnd=orc.SR, seed=4)
    second = orc.quantize(x, fmt=1, rnd=orc.SR, seed=4, index_offset=4 * 64)
    assert np.array_equal(full["codes"][4:], second["codes"])


# ------------------------------------------------------------ quantization noise
def test_noise_worked_examples(orc):
    f = fields("quant_noise_worked.txt")
    for fmt, key, B in ((1, "mx", 32), (0, "nv", 16)):
        x = np.zeros((1, B), dtype=np.float32)
        vals = [float(v) for v in f[f"{key}_x"]]
        x[0, :len(vals)] = vals
        q = orc.quantize(x, fmt=fmt, noise=True)
        assert q["noise"][0] == float(f[f"{key}_g2"][0])
        assert q["noise"][1] == float(f[f"{key}_e2"][0])


def test_noise_zero_tensor_and_grid_values(orc):
    q = orc.quantize(np.zeros((16, 64), dtype=np.float32), fmt=0, noise=True)
    assert list(q["noise"]) == [0.0, 0.0]
    # MXFP4 blocks whose values sit on the grid (amax 6 * 2^k): no noise
    rng = np.random.default_rng(8)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float32)
    x = rng.choice(grid, size=(8, 64)) * rng.choice([-1.0, 1.0], size=(8, 64)).astype(np.float32)
    x[:, ::32] = 6.0
    x *= np.float32(2.0 ** -3)
    q = orc.quantize(x, fmt=1, rnd=1, seed=3, noise=True)
    assert q["noise"][1] == 0.0
    assert q["noise"][0] == float(np.sum(x.astype(np.float64) ** 2))


@pytest.mark.parametrize("fmt", [0, 1])
def test_noise_matches_the_dequantizer(orc, fmt):
    # The noise sum equals sum (dequantize_f64 - x)^2 taken with numpy from the
    # separately pinned dequantizer; the signal sum equals numpy's sum of squares.
    x = _randn((64, 256), 12, outliers=True)
    for rnd in (0, 1):
        q = orc.quantize(x, fmt=fmt, rnd=rnd, seed=5, noise=True)
        x64 = x.astype(np.float64)
        e2 = float(np.sum((orc.dequantize_f64(q) - x64) ** 2))
        assert np.isclose(q["noise"][1], e2, rtol=1e-12, atol=0)
        assert np.isclose(q["noise"][0], float(np.sum(x64 ** 2)), rtol=1e-12, atol=0)
        assert 0 < q["noise"][1] < q["noise"][0]


def test_noise_of_rotated_values_keeps_the_signal_norm(orc):
    # the rotation is orthonormal: sum y^2 = sum x^2 up to FP32 rounding
    x = _randn((32, 256), 13, outliers=True)
    for fmt, signs in ((0, 0xBEEF), (1, 0x12345678)):
        q = orc.quantize(x, fmt=fmt, had_on=True, had_signs=signs, noise=True)
        g = float(np.sum(x.astype(np.float64) ** 2))
        assert abs(q["noise"][0] - g) <= 1e-6 * g


def test_sr_noise_has_the_bernoulli_expectation(orc):
    # MXFP4 with SR: an element a (scaled) between grid neighbours lo < a < hi
    # rounds up with probability p = (a - lo)/(hi - lo), so its squared error
    # has mean (hi - a)(a - lo) * s^2 and variance p(1-p)((hi-a)^2-(a-lo)^2)^2 s^4.
    # Averaged over seeds the oracle's noise sum must match the closed form.
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    x = _randn((4, 64), 14)
    q0 = orc.quantize(x, fmt=1)
    s = 2.0 ** (q0["scales"].astype(np.float64) - 127)          # per block
    sc = np.repeat(s, 32, axis=1)
    a = np.abs(x.astype(np.float64)) / sc
    hi_i = np.searchsorted(grid, a, side="left")
    on = grid[np.minimum(hi_i, 7)] == a
    lo = grid[np.maximum(hi_i - 1, 0)]
    hi = grid[np.minimum(hi_i, 7)]
    mean = np.where(on, 0.0, (hi - a) * (a - lo)) * sc ** 2
    p = np.where(on, 0.0, (a - lo) / np.where(hi > lo, hi - lo, 1.0))
    var = p * (1 - p) * (((hi - a) ** 2 - (a - lo) ** 2) * sc ** 2) ** 2
    n = 400
    e2 = np.array([orc.quantize(x, fmt=1, rnd=1, seed=1000 + k, noise=True)["noise"][1] for k in range(n)])
    assert abs(e2.mean() - mean.sum()) <= 4.5 * np.sqrt(var.sum() / n) + 1e-12


# ------------------------------------------------------ 2-D block quantization
def test_2d_worked_example(orc):
    f = fields("nvfp4_2d_worked.txt")
    x = np.ones((16, 32), dtype=np.float32)
    x[:, 16:] = 0.5
    x[3, 5], x[10, 20] = 6.0, 3.0
    q, qt = orc.quantize_2d(x)
    want_row = [int(v, 16) for v in f["scales_row"]]
    assert all(list(r) == want_row for r in q["scales"])
    assert [list(r) for r in qt["scales"]] == [[want_row[0]]] * 16 + [[want_row[1]]] * 16
    u = unpack(q["codes"])
    at = [int(v) for v in f["code7_at"]]
    want = np.full((16, 32), 2)
    want[at[0], at[1]] = want[at[2], at[3]] = 7
    assert np.array_equal(u, want)
    assert orc.quantize(x)["scales"][0, 0] == int(f["scale_1d_row0"][0], 16)


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rnd", [0, 1])
def test_2d_outputs_are_transposes(orc, fmt, rnd):
    x = _randn((96, 128), 15, outliers=True)
    q, qt = orc.quantize_2d(x, fmt=fmt, rnd=rnd, seed=7, index_offset=64)
    assert np.array_equal(unpack(qt["codes"]), unpack(q["codes"]).T)
    B = 16 if fmt == 0 else 32
    s_full = np.repeat(q["scales"], B, axis=1)               # [R][C]: each element's block byte
    st_full = np.repeat(qt["scales"], B, axis=1)             # [C][R]
    assert np.array_equal(st_full, s_full.T)
    # one byte per square block
    blocks = s_full.reshape(96 // B, B, 128 // B, B)
    assert (blocks == blocks[:, :1, :, :1]).all()


@pytest.mark.parametrize("fmt", [0, 1])
def test_2d_reduces_to_1d_when_every_row_and_column_holds_the_block_amax(orc, fmt):
    # Put each block's amax on its diagonal: every row and every column of the
    # block then has the block amax as its own 1-D block amax, so the 2-D
    # scales equal the 1-D ones and the codes equal the 1-D quantizations along
    # either axis (RTN; SR along rows, where both use the row-major index).
    B = 16 if fmt == 0 else 32
    x = _randn((2 * B, 3 * B), 16)
    for br in range(2):
        for bc in range(3):
            blk = x[br * B:(br + 1) * B, bc * B:(bc + 1) * B]
            m = np.abs(blk).max() * np.float32(1.5)
            idx = np.arange(B)
            blk[idx, idx] = m * np.where(idx % 2 == 0, 1, -1)
    for rnd in (0, 1):
        q, qt = orc.quantize_2d(x, fmt=fmt, rnd=rnd, seed=9)
        a = orc.quantize(x, axis=orc.AXIS_COLS, fmt=fmt, rnd=rnd, seed=9)
        assert np.array_equal(q["codes"], a["codes"]) and np.array_equal(q["scales"], a["scales"])
        if rnd == 0:
            b = orc.quantize(x, axis=orc.AXIS_ROWS, fmt=fmt)
            assert np.array_equal(qt["codes"], b["codes"]) and np.array_equal(qt["scales"], b["scales"])
        if fmt == 0:
            assert q["sg"] == a["sg"]


def test_2d_error_bound(orc):
    # RTN with a block scale covering the block: |xhat - x| <= half the largest
    # grid step (1 for E2M1) times the block's decoded scale, for every element
    x = _randn((64, 64), 17, outliers=True)
    q, _ = orc.quantize_2d(x)
    xhat = orc.dequantize_f64(q)
    sdec = np.array([[orc.e4m3_value(int(b)) for b in row] for row in q["scales"]])
    bound = np.repeat(sdec, 16, axis=1) * q["sg"] * 1.0 * (1 + 2.0 ** -20)
    assert (np.abs(xhat - x.astype(np.float64)) <= bound).all()


def test_noise_ratio_from_the_sums(orc):
    # The statistic is a ratio of norms: |g| = 3 and |Q(g) - g| = 0.5 give 6.
    assert orc.noise_ratio([9.0, 0.25]) == 6.0
    assert orc.noise_ratio([2.0, 0.0]) == float("inf")
    assert orc.noise_ratio([0.0, 0.0]) == 0.0
    # A tensor on the E2M1 grid quantizes without noise (MXFP4, one block whose
    # amax is 6 so the scale is 1): infinite ratio.
    x = np.array([[0.5, 1, 1.5, 2, 3, 4, 6, -6] * 4], dtype=np.float32)
    q = orc.quantize(x, fmt=orc.FMT_MXFP4, noise=True)
    assert q["noise"][1] == 0.0 and orc.noise_ratio(q["noise"]) == float("inf")
    # Halving the quantization step (all values scaled by 2^k change nothing):
    # the ratio is scale invariant.
    rng = np.random.default_rng(3)
    y = rng.standard_normal((64, 64)).astype(np.float32)
    r1 = orc.noise_ratio(orc.quantize(y, noise=True)["noise"])
    r2 = orc.noise_ratio(orc.quantize(y * np.float32(8), noise=True)["noise"])
    assert abs(r1 - r2) <= 1e-12 * r1
