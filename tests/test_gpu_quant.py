"""GPU parity of amax, quantize (both axes, both formats, RTN/SR, Hadamard)
and dequantize against the CPU oracle: bit-exact codes, scale bytes, tensor
amax and tensor scale."""
import numpy as np
import pytest

from gpu_util import assert_same_quant, q_from_oracle, q_to_host, say, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp4_fully_quantized_amd as m
    m.lib()          # raises if the HIP library is not built
    return m


def _mixed(shape, seed, bf16=True):
    """Heavy-tailed data with outlier columns and the degenerate cases of the
    block-scale rules: an all-zero block and row, signed zeros, values tiny
    enough to underflow the E4M3 scale, and a huge block."""
    rng = np.random.default_rng(seed)
    R, C = shape
    x = rng.standard_t(3, size=shape).astype(np.float32)
    x[:, rng.permutation(C)[: max(1, C // 100)]] *= 20
    x[0, :32] = 0.0
    x[1, :] = 0.0
    x[2, 0:32:2] = -0.0
    x[3, 32:64] *= 1e-6
    x[4, 64:96] *= 300.0
    x[5 % R, :] = rng.choice([0.25, 0.75, 1.25, -2.5, 5.0, 6.0, 0.0], size=C).astype(np.float32)
    if bf16:
        from oracle.oracle import f32_to_bf16_bits
        return f32_to_bf16_bits(x)
    return x


CASES = []
for fmt in (0, 1):
    for rnd in (0, 1):
        for axis in (0, 1):
            for had in (False, True):
                for bf16 in (True, False):
                    CASES.append((fmt, rnd, axis, had, bf16))


@pytest.mark.parametrize("fmt,rnd,axis,had,bf16", CASES)
@pytest.mark.parametrize("shape", [(96, 1056), (256, 256), (32, 64)])
def test_quantize_matches_oracle(fp4, orc, fmt, rnd, axis, had, bf16, shape):
    say("quantize", shape, "fmt", fmt, "rnd", rnd, "axis", axis, "had", had, "bf16", bf16)
    xh = _mixed(shape, 7 + shape[0], bf16)
    signs = orc.hadamard_signs(5) if had else 0
    want = orc.quantize(xh, axis=axis, fmt=fmt, rnd=rnd, seed=11, index_offset=64,
                        had_on=had, had_signs=signs)
    x = to_device(xh)
    q = fp4.quantize(x, axis=axis, fmt=fmt, rnd=rnd, seed=11, index_offset=64,
                     had_signs=signs if had else None)
    assert_same_quant(q_to_host(q), want, "quantize")


def test_amax_ready_reuses_the_given_amax(fp4, orc):
    import torch
    xh = _mixed((64, 512), 3)
    x = to_device(xh)
    a = fp4.quantize(x, axis=0)
    b = fp4.quantize(x, axis=1, rnd=1, seed=2, amax_from=a)
    want = orc.quantize(xh, axis=1, rnd=1, seed=2)
    assert_same_quant(q_to_host(b), want, "rows with amax reuse")
    amax = torch.zeros(1, dtype=torch.float32, device="cuda")
    fp4.fp4_tensor_amax(x, amax)
    assert float(amax.cpu()[0]) == orc.tensor_amax(xh)


AMAX_H16 = [((96, 1056), True), ((256, 256), False), ((32, 2064), True), ((4112, 48), True)]


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("shape,bf16", AMAX_H16)
def test_amax_hadamard16_matches_oracle(fp4, orc, axis, shape, bf16):
    """The amax of the 16-wide rotated values, along either axis, on shapes
    with ragged wave segments (C not a multiple of 512 or 2048)."""
    import torch
    say("amax hadamard16", shape, "axis", axis, "bf16", bf16)
    xh = _mixed(shape, 41 + shape[0], bf16)
    signs = orc.hadamard_signs(12)
    want = orc.quantize(xh, axis=axis, fmt=0, had_on=True, had_signs=signs)["amax"]
    amax = torch.full((1,), 7.0, dtype=torch.float32, device="cuda")
    fp4.fp4_tensor_amax_hadamard16(to_device(xh), axis, signs, amax)
    assert float(amax.cpu()[0]) == want
    assert want != orc.tensor_amax(xh)           # the rotation changes the amax here


def test_nvfp4_hadamard_with_a_given_amax(fp4, orc):
    """amax_ready: a rotated quantization takes the amax of the rotated values
    from the dedicated call (as a data-parallel caller would after reducing it)."""
    import torch
    xh = _mixed((256, 512), 43)
    x = to_device(xh)
    signs = orc.hadamard_signs(13)
    q = fp4.QTensor(512, 256, 0, had_signs=signs)
    fp4.fp4_tensor_amax_hadamard16(x, 1, signs, q.amax)
    fp4.fp4_quantize(x, 1, 1, 4, 0, True, q)
    want = orc.quantize(xh, axis=1, rnd=1, seed=4, had_on=True, had_signs=signs)
    assert_same_quant(q_to_host(q), want, "rows, rotated, given amax")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("kind", ["cols", "rows", "dual", "2d"])
def test_strided_source(fp4, orc, fmt, kind):
    """A column window of a wider matrix (leading dimension 1024 > 512 columns)
    in every quantize entry point."""
    xh = _mixed((96, 1024), 4)
    full = to_device(xh)
    view = full[:, 256:768]
    sub = np.ascontiguousarray(xh[:, 256:768])
    say("strided source", kind, "fmt", fmt)
    if kind in ("cols", "rows"):
        axis = 0 if kind == "cols" else 1
        want = orc.quantize(sub, axis=axis, fmt=fmt, rnd=1, seed=1)
        assert_same_quant(q_to_host(fp4.quantize(view, axis=axis, fmt=fmt, rnd=1, seed=1)), want, kind)
    elif kind == "dual":
        qc, qr = fp4.quantize_dual(view, fmt=fmt, rnd_cols=0, rnd_rows=1, seed_rows=3)
        assert_same_quant(q_to_host(qc), orc.quantize(sub, axis=0, fmt=fmt), "dual cols")
        assert_same_quant(q_to_host(qr), orc.quantize(sub, axis=1, fmt=fmt, rnd=1, seed=3), "dual rows")
    else:
        q, qt = fp4.quantize_2d(view, fmt=fmt, rnd=1, seed=5)
        w, wt = orc.quantize_2d(sub, fmt=fmt, rnd=1, seed=5)
        assert_same_quant(q_to_host(q), w, "2-D")
        assert_same_quant(q_to_host(qt), wt, "2-D transpose")


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("bf16out", [False, True])
def test_dequantize_matches_oracle(fp4, orc, fmt, bf16out):
    import torch
    xh = _mixed((96, 1056), 5)
    qo = orc.quantize(xh, fmt=fmt, had_on=fmt == 1, had_signs=123)
    q = q_from_oracle(qo, had_signs=123 if fmt == 1 else None)
    y = fp4.dequantize(q, dtype=torch.bfloat16 if bf16out else torch.float32)
    want = orc.dequantize_f32(qo)
    if bf16out:
        assert np.array_equal(to_host(y), orc.f32_to_bf16_bits(want))
    else:
        assert np.array_equal(to_host(y), want)



@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("bf16out", [False, True])
@pytest.mark.parametrize("axis", [0, 1])
def test_dequantize_unrotated_matches_oracle(fp4, orc, fmt, bf16out, axis):
    """fp4_dequantize_unrotated of a rotated quantization (MXFP4 32-wide,
    NVFP4 16-wide; either axis, the blocks lying along the quantized
    orientation's rows): bit-equal to the oracle's dequantization followed by
    its inverse rotation, bf16 rounded once at the end; without a rotation it
    equals fp4_dequantize."""
    import torch
    xh = _mixed((96, 1056), 6)
    signs = orc.hadamard_signs(21)
    say("dequantize unrotated fmt", fmt, "axis", axis, "bf16", bf16out)
    qo = orc.quantize(xh, axis=axis, fmt=fmt, had_on=True, had_signs=signs)
    q = q_from_oracle(qo, had_signs=signs)
    dt = torch.bfloat16 if bf16out else torch.float32
    y = to_host(fp4.dequantize(q, dtype=dt, unrotate=True))
    want = orc.dequantize_unrotated_f32(qo, signs)
    assert np.array_equal(y, orc.f32_to_bf16_bits(want) if bf16out else want)
    qo0 = orc.quantize(xh, axis=axis, fmt=fmt)
    q0 = q_from_oracle(qo0)
    iv = torch.int16 if bf16out else torch.int32
    assert torch.equal(fp4.dequantize(q0, dtype=dt, unrotate=True).view(iv), fp4.dequantize(q0, dtype=dt).view(iv))


def test_dequantize_unrotated_strided_output(fp4, orc):
    """Into rows of ld = cols + 8 (16-byte aligned): the padding stays untouched."""
    import torch
    xh = _mixed((40, 256), 7)
    signs = orc.hadamard_signs(22)
    qo = orc.quantize(xh, fmt=1, had_on=True, had_signs=signs)
    q = q_from_oracle(qo, had_signs=signs)
    full = torch.full((40, 264), 5.0, dtype=torch.float32, device="cuda")
    fp4.fp4_dequantize_unrotated(q, full[:, :256])
    yh = to_host(full)
    assert (yh[:, 256:] == 5.0).all()
    assert np.array_equal(yh[:, :256], orc.dequantize_unrotated_f32(qo, signs))

# ------------------------------------------------ both orientations in one read
DUAL = []
for fmt in (0, 1):
    for rc, rr in ((0, 1), (1, 1), (0, 0), (1, 0)):
        DUAL.append((fmt, rc, rr, (False, False)))
    for had in ((True, True), (False, True), (True, False)):
        for rc, rr in ((0, 1), (1, 1)):
            DUAL.append((fmt, rc, rr, had))


@pytest.mark.parametrize("fmt,rc,rr,had", DUAL)
@pytest.mark.parametrize("shape,bf16", [((96, 1056), True), ((256, 256), True), ((160, 96), False),
                                        ((32, 64), True), ((384, 4128), True)])
def test_quantize_dual_matches_two_oracle_passes(fp4, orc, fmt, rc, rr, had, shape, bf16):
    B = 16 if fmt == 0 else 32
    if shape[0] % B or shape[1] % B:
        pytest.skip("the dual pass needs both dimensions blocked")
    say("quantize_dual", shape, "fmt", fmt, "rnd", rc, rr, "had", had, "bf16", bf16)
    xh = _mixed(shape, 31 + shape[1], bf16)
    hc, hr = had
    sc = orc.hadamard_signs(5) if hc else 0
    sr = orc.hadamard_signs(6) if hr else 0
    want_c = orc.quantize(xh, axis=0, fmt=fmt, rnd=rc, seed=21, index_offset=8, had_on=hc, had_signs=sc)
    want_r = orc.quantize(xh, axis=1, fmt=fmt, rnd=rr, seed=22, index_offset=16, had_on=hr, had_signs=sr)
    qc, qr = fp4.quantize_dual(to_device(xh), fmt=fmt, rnd_cols=rc, seed_cols=21, index_offset_cols=8,
                               rnd_rows=rr, seed_rows=22, index_offset_rows=16,
                               had_signs_cols=sc if hc else None, had_signs_rows=sr if hr else None)
    assert_same_quant(q_to_host(qc), want_c, "dual, blocks along C")
    assert_same_quant(q_to_host(qr), want_r, "dual, blocks along R")


def test_quantize_dual_full_size_gradient(fp4, orc):
    """The Llama-7B layer's dY (32768 x 11008 bf16), SR in both orientations."""
    import torch
    from fp4_fully_quantized_amd import workloads
    say("quantize_dual full size dY")
    x = workloads.device_tensor("llama7b", "dY")
    qc, qr = fp4.quantize_dual(x, rnd_cols=1, seed_cols=(2 << 8) | 1, rnd_rows=1, seed_rows=(2 << 8) | 2)
    torch.cuda.synchronize()
    got_c, got_r = q_to_host(qc), q_to_host(qr)
    xh = to_host(x)
    del qc, qr, x
    assert_same_quant(got_c, orc.quantize(xh, axis=0, rnd=1, seed=(2 << 8) | 1), "dY, blocks along C")
    assert_same_quant(got_r, orc.quantize(xh, axis=1, rnd=1, seed=(2 << 8) | 2), "dY, blocks along R")


# ------------------------------------------------------- SR decision boundaries
def _sr_boundary_input(orc, R, C, axis, seed, offset):
    """fp32 [R, C] whose MXFP4 block exponents are all 0 (element 0 of every
    block along the blocked axis is 5.5), so the scaled values equal the
    inputs, and whose other values sit on or next to the stochastic-rounding
    boundary of their own draw h, where p's first 16 fraction bits reach
    2^16 - h: p * 2^22 = B - 1, B - 1/2, B, B + 1/2, B + 1 with
    B = 64 (2^16 - h), in each binade of the E2M1 grid (the integer ones
    where a binade's values give only integers), plus values far below the
    first grid step. The draw is the one of the element's index in the
    quantized orientation."""
    rng = np.random.default_rng(seed)
    x = np.zeros((R, C), dtype=np.float32)
    kinds = ["a1", "a2", "a4", "half", "tiny", "tinier"]
    for r in range(R):
        for c in range(C):
            pos = c % 32 if axis == 0 else r % 32
            if pos == 0:
                x[r, c] = 5.5
                continue
            idx = offset + (r * C + c if axis == 0 else c * R + r)
            h = orc.sr_draw16(seed, idx)
            kind = kinds[(r * 7 + c * 3) % len(kinds)]
            d = [-1.0, -0.5, 0.0, 0.5, 1.0][(r + c) % 5]
            g = min(64.0 * (65536 - h) + d, 4194303.0)   # target p * 2^22 (p < 1)
            if kind in ("a1", "a2", "a4"):     # [1,2), [2,4), [4,6): p * 2^22 = rem (22 bits)
                lo = {"a1": 1.0, "a2": 2.0, "a4": 4.0}[kind]
                q = {"a1": 0.5, "a2": 1.0, "a4": 2.0}[kind]
                g = np.floor(g)                # these binades hold integer p * 2^22 only
                a = lo + q * g / 4194304.0
            elif kind == "half":               # [0.5, 1): p * 2^22 = m / 2
                a = 0.5 + 0.5 * g / 4194304.0
            elif kind == "tiny":               # below 0.5: p * 2^22 = a * 2^23
                a = g / 8388608.0
            else:
                a = float(rng.choice([2.0 ** -30, 3.0 * 2 ** -40, 2.0 ** -24]))
            x[r, c] = np.float32(a) * (1.0 if rng.random() < 0.5 else -1.0)
    return x


@pytest.mark.parametrize("axis", [0, 1])
def test_sr_decision_boundaries(fp4, orc, axis):
    say("SR boundary cases, axis", axis)
    R, C = (8, 512) if axis == 0 else (512, 8)
    seed, offset = 29, 1024
    xh = _sr_boundary_input(orc, R, C, axis, seed, offset)
    want = orc.quantize(xh, axis=axis, fmt=1, rnd=1, seed=seed, index_offset=offset)
    assert (want["scales"] == 127).all()       # every block exponent is 0
    q = fp4.quantize(to_device(xh), axis=axis, fmt=1, rnd=1, seed=seed, index_offset=offset)
    assert_same_quant(q_to_host(q), want, "SR boundaries")


# ------------------------------------------------------------- full sizes
FULL = [
    # (workload, role, axis, fmt, rnd, had)  -- the passes of the layer steps
    ("llama7b", "X", 0, 0, 0, False),
    ("llama7b", "W", 0, 0, 0, False),
    ("llama7b", "dY", 0, 0, 1, False),
    ("llama7b", "dY", 1, 0, 1, False),
    ("llama7b", "X", 1, 0, 1, False),
    ("llama7b", "W", 1, 0, 1, False),
    ("llama7b", "X", 0, 1, 0, True),
    ("llama7b", "W", 0, 1, 0, True),
    # NVFP4 wgrad operands rotated 16-wide along the tokens
    ("llama7b", "dY", 1, 0, 1, True),
    ("llama7b", "X", 1, 0, 1, True),
    # the large-layer step (hidden 8192, MLP 28672, 16384 tokens)
    ("large", "X", 0, 0, 0, False),
    ("large", "W", 0, 0, 0, False),
    ("large", "dY", 0, 0, 1, False),
    ("large", "W", 1, 0, 1, False),
    ("large", "dY", 1, 0, 1, False),
    ("large", "X", 1, 0, 1, False),
]


@pytest.mark.parametrize("wl,role,axis,fmt,rnd,had", FULL)
def test_full_size_quantize_matches_oracle(fp4, orc, wl, role, axis, fmt, rnd, had):
    import torch
    from fp4_fully_quantized_amd import workloads
    say("full-size quantize", wl, role, "axis", axis, "fmt", fmt, "rnd", rnd, "had", had)
    x = workloads.device_tensor(wl, role)
    signs = fp4.fp4_hadamard_signs(3) if had else None
    q = fp4.quantize(x, axis=axis, fmt=fmt, rnd=rnd, seed=(1 << 8) | (axis + 1),
                     had_signs=signs)
    torch.cuda.synchronize()
    got = q_to_host(q)
    xh = to_host(x)
    del q, x
    want = orc.quantize(xh, axis=axis, fmt=fmt, rnd=rnd, seed=(1 << 8) | (axis + 1),
                        had_on=had, had_signs=signs or 0)
    assert_same_quant(got, want, f"{wl} {role}")


# ------------------------------------------------------- gradient-noise monitor
# Each partial sum is formed in FP32 over at most 32 elements (differences
# rounded once, squares accumulated by fma): relative error <= 33 * 2^-24
# (2e-6) of a sum of non-negative terms; the FP64 part is exact to 1e-15.
NOISE_RTOL = 1e-5


def _assert_noise(got, want, what):
    got = got.cpu().numpy()
    for k, name in ((0, "sum x^2"), (1, "sum (xhat - x)^2")):
        assert abs(got[k] - want[k]) <= NOISE_RTOL * want[k], (what, name, got[k], want[k])


def _assert_ratio(got, want, what):
    # sqrt of a quotient of two sums each within NOISE_RTOL: within NOISE_RTOL.
    got = float(got.cpu()[0])
    assert abs(got - want) <= NOISE_RTOL * want, (what, got, want)


def test_noise_ratio_special_values(fp4, orc):
    """The library's ratio on the device: ordinary sums, no noise (+inf), an
    all-zero tensor (0)."""
    import torch
    say("noise ratio special values")
    for sums in ([9.0, 0.25], [1e-30, 4e-34], [2.0, 0.0], [0.0, 0.0]):
        noise = torch.tensor(sums, dtype=torch.float64, device="cuda")
        got = float(fp4.noise_ratio(noise).cpu()[0])
        want = orc.noise_ratio(sums)
        assert got == want or abs(got - want) <= 1e-15 * want, (sums, got, want)


NOISE = [(fmt, rnd, axis, had) for fmt in (0, 1) for rnd in (0, 1) for axis in (0, 1) for had in (False, True)]


@pytest.mark.parametrize("fmt,rnd,axis,had", NOISE)
@pytest.mark.parametrize("shape,bf16", [((96, 1056), True), ((256, 256), False)])
def test_quantize_noise_matches_oracle(fp4, orc, fmt, rnd, axis, had, shape, bf16):
    import torch
    say("quantize noise", shape, "fmt", fmt, "rnd", rnd, "axis", axis, "had", had, "bf16", bf16)
    xh = _mixed(shape, 51 + shape[0], bf16)
    signs = orc.hadamard_signs(7) if had else 0
    want = orc.quantize(xh, axis=axis, fmt=fmt, rnd=rnd, seed=13, had_on=had, had_signs=signs, noise=True)
    noise = torch.zeros(2, dtype=torch.float64, device="cuda")
    x = to_device(xh)
    q = fp4.quantize(x, axis=axis, fmt=fmt, rnd=rnd, seed=13, had_signs=signs if had else None, noise=noise)
    assert_same_quant(q_to_host(q), want, "quantize with the noise monitor")
    _assert_noise(noise, want["noise"], "one call")
    _assert_ratio(fp4.noise_ratio(noise), orc.noise_ratio(want["noise"]), "one call")
    fp4.quantize(x, axis=axis, fmt=fmt, rnd=rnd, seed=13, had_signs=signs if had else None, noise=noise)
    _assert_noise(noise, 2 * want["noise"], "accumulated over two calls")


DUAL_NOISE = [(0, 1, 1, (False, False)), (0, 0, 1, (False, True)), (1, 1, 1, (True, True)),
              (1, 0, 1, (False, False))]


@pytest.mark.parametrize("fmt,rc,rr,had", DUAL_NOISE)
@pytest.mark.parametrize("which", ["both", "cols", "rows"])
def test_quantize_dual_noise_matches_oracle(fp4, orc, fmt, rc, rr, had, which):
    import torch
    say("quantize_dual noise", "fmt", fmt, "rnd", rc, rr, "had", had, which)
    xh = _mixed((160, 1056), 61)
    hc, hr = had
    sc = orc.hadamard_signs(8) if hc else 0
    sr = orc.hadamard_signs(9) if hr else 0
    want_c = orc.quantize(xh, axis=0, fmt=fmt, rnd=rc, seed=5, had_on=hc, had_signs=sc, noise=True)
    want_r = orc.quantize(xh, axis=1, fmt=fmt, rnd=rr, seed=6, had_on=hr, had_signs=sr, noise=True)
    nc = torch.zeros(2, dtype=torch.float64, device="cuda") if which != "rows" else None
    nr = torch.zeros(2, dtype=torch.float64, device="cuda") if which != "cols" else None
    qc, qr = fp4.quantize_dual(to_device(xh), fmt=fmt, rnd_cols=rc, seed_cols=5, rnd_rows=rr, seed_rows=6,
                               had_signs_cols=sc if hc else None, had_signs_rows=sr if hr else None,
                               noise_cols=nc, noise_rows=nr)
    assert_same_quant(q_to_host(qc), want_c, "dual cols")
    assert_same_quant(q_to_host(qr), want_r, "dual rows")
    if nc is not None:
        _assert_noise(nc, want_c["noise"], "dual cols")
    if nr is not None:
        _assert_noise(nr, want_r["noise"], "dual rows")


def test_noise_monitor_full_size_gradient(fp4, orc):
    """The Llama-7B layer's dY, SR in both orientations, with the monitor on both."""
    import torch
    from fp4_fully_quantized_amd import workloads
    say("noise monitor full size dY")
    x = workloads.device_tensor("llama7b", "dY")
    nc = torch.zeros(2, dtype=torch.float64, device="cuda")
    nr = torch.zeros(2, dtype=torch.float64, device="cuda")
    qc, qr = fp4.quantize_dual(x, rnd_cols=1, seed_cols=(2 << 8) | 1, rnd_rows=1, seed_rows=(2 << 8) | 2,
                               noise_cols=nc, noise_rows=nr)
    torch.cuda.synchronize()
    got_c = q_to_host(qc)
    xh = to_host(x)
    del qc, qr, x
    want_c = orc.quantize(xh, axis=0, rnd=1, seed=(2 << 8) | 1, noise=True)
    assert_same_quant(got_c, want_c, "dY cols")
    _assert_noise(nc, want_c["noise"], "dY cols")
    want_r = orc.quantize(xh, axis=1, rnd=1, seed=(2 << 8) | 2, noise=True)
    _assert_noise(nr, want_r["noise"], "dY rows")
    rc, rr = fp4.noise_ratio(nc), fp4.noise_ratio(nr)
    _assert_ratio(rc, orc.noise_ratio(want_c["noise"]), "dY cols ratio")
    _assert_ratio(rr, orc.noise_ratio(want_r["noise"]), "dY rows ratio")
    say("gradient / noise norm ratio", float(rc.cpu()[0]), float(rr.cpu()[0]))


# ------------------------------------------------------ 2-D block quantization
@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("rnd", [0, 1])
@pytest.mark.parametrize("shape,bf16", [((96, 1056), True), ((256, 256), True), ((160, 96), False),
                                        ((32, 64), True), ((384, 4128), True)])
def test_quantize_2d_matches_oracle(fp4, orc, fmt, rnd, shape, bf16):
    B = 16 if fmt == 0 else 32
    if shape[0] % B or shape[1] % B:
        pytest.skip("2-D blocks need both dimensions blocked")
    say("quantize_2d", shape, "fmt", fmt, "rnd", rnd, "bf16", bf16)
    xh = _mixed(shape, 71 + shape[1], bf16)
    want, want_t = orc.quantize_2d(xh, fmt=fmt, rnd=rnd, seed=31, index_offset=24)
    q, qt = fp4.quantize_2d(to_device(xh), fmt=fmt, rnd=rnd, seed=31, index_offset=24)
    assert_same_quant(q_to_host(q), want, "2-D, blocks along C")
    assert_same_quant(q_to_host(qt), want_t, "2-D, transpose")


def test_quantize_2d_full_size_weight(fp4, orc):
    """The Llama-7B layer's W (11008 x 4096 bf16), 16 x 16 NVFP4 blocks, RTN."""
    import torch
    from fp4_fully_quantized_amd import workloads
    say("quantize_2d full size W")
    x = workloads.device_tensor("llama7b", "W")
    q, qt = fp4.quantize_2d(x)
    torch.cuda.synchronize()
    got, got_t = q_to_host(q), q_to_host(qt)
    xh = to_host(x)
    del q, qt, x
    want, want_t = orc.quantize_2d(xh)
    assert_same_quant(got, want, "W 2-D")
    assert_same_quant(got_t, want_t, "W^T 2-D")


# --------------------------------------------------------- degenerate magnitudes
def _tiny(shape, seed, scale):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * scale).astype(np.float32)


TINY = [1e-32, 2.0 ** -99, 1e-38, 3e-39]   # below the NVFP4 floor, just above it, FP32 subnormal range


# Large and small tensor scales: amaxes that put s_g = amax / 2688 at exactly
# 2^-80 and 2^100 and at the bf16 neighbours either side (2688 = 21 * 2^7; the
# bf16 values next to it are 2672 and 2704), so that the tensor's values reach
# about 2^111 and its block scales span dozens of binades below s_g.
SG_EDGES = [2688.0 * 2.0 ** -80, 2672.0 * 2.0 ** -80, 2704.0 * 2.0 ** -80,
            2688.0 * 2.0 ** 100, 2704.0 * 2.0 ** 100, 2672.0 * 2.0 ** 100]


@pytest.mark.parametrize("amax", SG_EDGES)
@pytest.mark.parametrize("bf16", [False, True])
def test_large_and_small_tensor_scales(fp4, orc, amax, bf16):
    """NVFP4 tensors with s_g near 2^-80 and 2^100: codes, scale bytes and s_g
    equal the oracle's for both axes, RTN and SR, and the dual pass."""
    say("large and small tensor scales", amax, "bf16", bf16)
    rng = np.random.default_rng(17)
    x = (rng.uniform(-1.0, 1.0, (64, 256)) * rng.choice([1.0, 2.0 ** -6, 2.0 ** -14], (64, 256))
         * (0.999 * amax)).astype(np.float32)
    x[3, 5] = amax
    x[40, 200] = -amax
    xh = orc.f32_to_bf16_bits(x) if bf16 else x
    if bf16:   # the bf16 amax must still be the one chosen
        assert float(np.max(np.abs(orc.bf16_bits_to_f32(xh)))) == amax
    for axis in (0, 1):
        for rnd in (0, 1):
            want = orc.quantize(xh, axis=axis, fmt=0, rnd=rnd, seed=9)
            q = fp4.quantize(to_device(xh), axis=axis, fmt=0, rnd=rnd, seed=9)
            assert_same_quant(q_to_host(q), want, f"axis {axis} rnd {rnd}")
    want_c = orc.quantize(xh, axis=0, fmt=0, rnd=0)
    want_r = orc.quantize(xh, axis=1, fmt=0, rnd=1, seed=4)
    qc, qr = fp4.quantize_dual(to_device(xh), fmt=0, rnd_cols=0, rnd_rows=1, seed_rows=4)
    assert_same_quant(q_to_host(qc), want_c, "dual, blocks along C")
    assert_same_quant(q_to_host(qr), want_r, "dual, blocks along R")


@pytest.mark.parametrize("scale", TINY)
@pytest.mark.parametrize("fmt,axis", [(0, 0), (0, 1), (1, 0)])
@pytest.mark.parametrize("bf16", [False, True])
def test_tiny_and_subnormal_magnitudes(fp4, orc, scale, fmt, axis, bf16):
    """Tensors near and inside FP32's subnormal range (bf16 inputs round to
    bf16 subnormals): the tensor-scale floor and the block-scale rules agree
    with the oracle bit for bit, in RTN and SR."""
    say("tiny magnitudes", scale, "fmt", fmt, "axis", axis, "bf16", bf16)
    x = _tiny((64, 256), 81, scale)
    xh = orc.f32_to_bf16_bits(x) if bf16 else x
    for rnd in (0, 1):
        want = orc.quantize(xh, axis=axis, fmt=fmt, rnd=rnd, seed=5)
        q = fp4.quantize(to_device(xh), axis=axis, fmt=fmt, rnd=rnd, seed=5)
        assert_same_quant(q_to_host(q), want, f"tiny {scale} rnd {rnd}")
