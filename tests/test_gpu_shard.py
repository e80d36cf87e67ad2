"""GPU parity of the row-shard quantization entries: a tensor split by rows
(tokens) into ragged shards, each shard quantized on its own with the whole
tensor's amax (the per-shard amaxes reduced by max, as an all-reduce would)
and its global offsets, gives exactly the slices of the oracle's quantization
of the whole tensor: codes, scale bytes, amax and tensor scale, for both
formats, RTN and SR, with and without the rotation, on both axes and in the
one-read dual pass; with the noise monitor, the shards' sums add up to the
whole tensor's."""
import numpy as np
import pytest

from gpu_util import assert_same_quant, q_to_host, say, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp4_fully_quantized_amd as m
    m.lib()
    return m


def _data(shape, seed, bf16=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_t(3, size=shape).astype(np.float32)
    x[:, rng.permutation(shape[1])[:3]] *= 25
    x[7, :] = 0.0
    if bf16:
        from oracle.oracle import f32_to_bf16_bits
        return f32_to_bf16_bits(x)
    return x


def _bounds(sizes):
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(int)
    return list(zip(off[:-1].tolist(), sizes))


def _global_amax(fp4, shards, fmt, axis, signs):
    """Each shard's amax, reduced by max (the all-reduce of a data-parallel
    step, on one device)."""
    import torch
    if fmt != 0:
        return None
    part = torch.zeros(len(shards), dtype=torch.float32, device="cuda")
    for i, x in enumerate(shards):
        if signs:
            fp4.fp4_tensor_amax_hadamard16(x, axis, signs, part[i:i + 1])
        else:
            fp4.fp4_tensor_amax(x, part[i:i + 1])
    return part.max().reshape(1)


def _slice(want, off, n, axis, B):
    """Rows off .. off+n (COLS) or columns off .. off+n (ROWS) of a whole-tensor
    quantization."""
    d = dict(want)
    if axis == 0:
        d["codes"] = want["codes"][off:off + n]
        d["scales"] = want["scales"][off:off + n]
        d["rows"] = n
    else:
        d["codes"] = want["codes"][:, off // 2:(off + n) // 2]
        d["scales"] = want["scales"][:, off // B:(off + n) // B]
        d["cols"] = n
    return d


# Shard row counts: ragged for the COLS axis; whole 32-row blocks (both
# formats) where the blocks run along rows.
SIZES = {0: [37, 200, 3, 176], 1: [96, 224, 96]}
CASES = [(fmt, rnd, axis, had, bf16)
         for fmt in (0, 1) for rnd in (0, 1) for axis in (0, 1) for had in (False, True)
         for bf16 in (True, False) if not (bf16 is False and had)]


@pytest.mark.parametrize("fmt,rnd,axis,had,bf16", CASES)
def test_shards_equal_the_whole_tensor_quantization(fp4, orc, fmt, rnd, axis, had, bf16):
    import torch
    B = 16 if fmt == 0 else 32
    sizes = SIZES[axis]
    total, C = sum(sizes), 1056
    say("quantize_shard", (total, C), sizes, "fmt", fmt, "rnd", rnd, "axis", axis, "had", had, "bf16", bf16)
    xh = _data((total, C), 40 + fmt + 2 * axis, bf16)
    signs = orc.hadamard_signs(9) if had else 0
    want = orc.quantize(xh, axis=axis, fmt=fmt, rnd=rnd, seed=77, index_offset=24, had_on=had,
                        had_signs=signs)
    x = to_device(xh)
    shards = [x[o:o + n] for o, n in _bounds(sizes)]
    amax = _global_amax(fp4, shards, fmt, axis, signs)
    for (o, n), xs in zip(_bounds(sizes), shards):
        rows, cols = (C, n) if axis == 1 else (n, C)
        q = fp4.QTensor(rows, cols, fmt, had_signs=signs if had else None)
        if amax is not None:
            q.amax.copy_(amax)
        fp4.fp4_quantize_shard(xs, o, total, axis, rnd, 77, 24, True, q)
        torch.cuda.synchronize()
        assert_same_quant(q_to_host(q), _slice(want, o, n, axis, B), f"shard at row {o}")


@pytest.mark.parametrize("had", [False, True])
def test_nvfp4_row_shards_on_16_row_boundaries(fp4, orc, had):
    """NVFP4 blocks down the columns are 16 rows: shards may start on any
    multiple of 16 (here 48, 256), with and without the 16-wide rotation."""
    import torch
    sizes = [48, 208, 160]
    total, C = sum(sizes), 544
    say("quantize_shard NVFP4 rows on 16-row boundaries", sizes, "had", had)
    xh = _data((total, C), 95)
    signs = orc.hadamard_signs(12) if had else 0
    want = orc.quantize(xh, axis=1, fmt=0, rnd=1, seed=41, index_offset=0, had_on=had, had_signs=signs)
    x = to_device(xh)
    shards = [x[o:o + n] for o, n in _bounds(sizes)]
    amax = _global_amax(fp4, shards, 0, 1, signs)
    for (o, n), xs in zip(_bounds(sizes), shards):
        q = fp4.QTensor(C, n, 0, had_signs=signs if had else None)
        q.amax.copy_(amax)
        fp4.fp4_quantize_shard(xs, o, total, 1, 1, 41, 0, True, q)
        torch.cuda.synchronize()
        assert_same_quant(q_to_host(q), _slice(want, o, n, 1, 16), f"16-row shard at row {o}")


def test_single_shard_equals_fp4_quantize(fp4, orc):
    """row_offset 0, rows_total R: the plain quantization, amax computed in the call."""
    xh = _data((128, 512), 5)
    x = to_device(xh)
    for axis in (0, 1):
        say("quantize_shard whole tensor, axis", axis)
        q = fp4.QTensor(*((512, 128) if axis else (128, 512)), 0)
        fp4.fp4_quantize_shard(x, 0, 128, axis, 1, 3, 8, False, q)
        assert_same_quant(q_to_host(q), orc.quantize(xh, axis=axis, rnd=1, seed=3, index_offset=8),
                          f"one shard, axis {axis}")


DUAL = [(fmt, rc, rr, had) for fmt in (0, 1) for rc, rr in ((0, 1), (1, 1))
        for had in ((False, False), (True, True), (False, True))]


@pytest.mark.parametrize("fmt,rc,rr,had", DUAL)
def test_dual_shards_equal_the_whole_tensor_quantization(fp4, orc, fmt, rc, rr, had):
    import torch
    B = 16 if fmt == 0 else 32
    sizes = [96, 224, 32, 64]
    total, C = sum(sizes), 544
    hc, hr = had
    say("quantize_dual_shard", (total, C), sizes, "fmt", fmt, "rnd", rc, rr, "had", had)
    xh = _data((total, C), 60 + fmt)
    sc = orc.hadamard_signs(5) if hc else 0
    sr = orc.hadamard_signs(6) if hr else 0
    want_c = orc.quantize(xh, axis=0, fmt=fmt, rnd=rc, seed=21, index_offset=8, had_on=hc, had_signs=sc)
    want_r = orc.quantize(xh, axis=1, fmt=fmt, rnd=rr, seed=22, index_offset=16, had_on=hr, had_signs=sr)
    x = to_device(xh)
    shards = [x[o:o + n] for o, n in _bounds(sizes)]
    two = fmt == 0 and (hc or hr)
    amax_c = _global_amax(fp4, shards, fmt, 0, sc)
    amax_r = _global_amax(fp4, shards, fmt, 1, sr) if two else None
    for (o, n), xs in zip(_bounds(sizes), shards):
        qc = fp4.QTensor(n, C, fmt, had_signs=sc if hc else None)
        qr = fp4.QTensor(C, n, fmt, had_signs=sr if hr else None)
        if fmt == 0:
            qc.amax.copy_(amax_c)
            if two:
                qr.amax.copy_(amax_r)
            else:
                qr.amax = qc.amax
        fp4.fp4_quantize_dual_shard(xs, o, total, rc, 21, 8, rr, 22, 16, True, qc, qr)
        torch.cuda.synchronize()
        assert_same_quant(q_to_host(qc), _slice(want_c, o, n, 0, B), f"dual shard at row {o}, cols")
        assert_same_quant(q_to_host(qr), _slice(want_r, o, n, 1, B), f"dual shard at row {o}, rows")


def test_full_size_gradient_shard(fp4, orc):
    """One 8-way shard of the Llama-7B layer's dY (rows 12288 .. 16383 of
    32768 x 11008), SR in both orientations: equal to the same rows / columns
    of the whole tensor's quantization by the oracle."""
    import torch
    from fp4_fully_quantized_amd import workloads
    say("quantize_dual_shard full-size dY shard")
    x = workloads.device_tensor("llama7b", "dY")
    total, C = x.shape
    o, n = 12288, 4096
    amax = torch.zeros(8, dtype=torch.float32, device="cuda")
    for i in range(8):
        fp4.fp4_tensor_amax(x[i * n:(i + 1) * n], amax[i:i + 1])
    qc = fp4.QTensor(n, C, 0)
    qr = fp4.QTensor(C, n, 0)
    qc.amax.copy_(amax.max().reshape(1))
    qr.amax = qc.amax
    fp4.fp4_quantize_dual_shard(x[o:o + n], o, total, 1, 5, 0, 1, 6, 0, True, qc, qr)
    torch.cuda.synchronize()
    got_c, got_r = q_to_host(qc), q_to_host(qr)
    xh = to_host(x)
    del qc, qr, x
    assert_same_quant(got_c, _slice(orc.quantize(xh, axis=0, rnd=1, seed=5), o, n, 0, 16), "dY shard, cols")
    want_r = orc.quantize(xh, axis=1, rnd=1, seed=6)
    assert_same_quant(got_r, _slice(want_r, o, n, 1, 16), "dY shard, rows")


# Noise-monitor sums of shards, added into one buffer (as an all-reduce(sum)
# across ranks would): the whole tensor's sums. Each partial is formed in FP32
# over at most 32 elements (relative error <= 33 * 2^-24 of a sum of
# non-negative terms) and added in FP64, as in one call on the whole tensor.
NOISE_RTOL = 1e-5


def _assert_noise(got, want, what):
    got = got.cpu().numpy()
    for k in (0, 1):
        assert abs(got[k] - want[k]) <= NOISE_RTOL * want[k], (what, k, got[k], want[k])


@pytest.mark.parametrize("fmt,rnd,axis", [(0, 1, 0), (0, 1, 1), (1, 0, 0), (1, 1, 1)])
def test_monitored_shards_add_up_to_the_whole_tensor(fp4, orc, fmt, rnd, axis):
    import torch
    B = 16 if fmt == 0 else 32
    sizes = SIZES[axis]
    total, C = sum(sizes), 544
    say("quantize_shard with noise", (total, C), sizes, "fmt", fmt, "rnd", rnd, "axis", axis)
    xh = _data((total, C), 80 + fmt + 2 * axis)
    want = orc.quantize(xh, axis=axis, fmt=fmt, rnd=rnd, seed=9, index_offset=0, noise=True)
    x = to_device(xh)
    shards = [x[o:o + n] for o, n in _bounds(sizes)]
    amax = _global_amax(fp4, shards, fmt, axis, 0)
    noise = torch.zeros(2, dtype=torch.float64, device="cuda")
    for (o, n), xs in zip(_bounds(sizes), shards):
        q = fp4.QTensor(*((C, n) if axis == 1 else (n, C)), fmt)
        if amax is not None:
            q.amax.copy_(amax)
        fp4.fp4_quantize_shard(xs, o, total, axis, rnd, 9, 0, True, q, noise=noise)
        assert_same_quant(q_to_host(q), _slice(want, o, n, axis, B), f"monitored shard at row {o}")
    _assert_noise(noise, want["noise"], "shards")


@pytest.mark.parametrize("fmt", [0, 1])
def test_monitored_dual_shards_add_up_to_the_whole_tensor(fp4, orc, fmt):
    import torch
    B = 16 if fmt == 0 else 32
    sizes = [96, 224, 32, 64]
    total, C = sum(sizes), 544
    say("quantize_dual_shard with noise", (total, C), sizes, "fmt", fmt)
    xh = _data((total, C), 90 + fmt)
    want_c = orc.quantize(xh, axis=0, fmt=fmt, rnd=1, seed=3, noise=True)
    want_r = orc.quantize(xh, axis=1, fmt=fmt, rnd=1, seed=4, noise=True)
    x = to_device(xh)
    shards = [x[o:o + n] for o, n in _bounds(sizes)]
    amax = _global_amax(fp4, shards, fmt, 0, 0)
    nc = torch.zeros(2, dtype=torch.float64, device="cuda")
    nr = torch.zeros(2, dtype=torch.float64, device="cuda")
    for (o, n), xs in zip(_bounds(sizes), shards):
        qc, qr = fp4.QTensor(n, C, fmt), fp4.QTensor(C, n, fmt)
        if amax is not None:
            qc.amax.copy_(amax)
            qr.amax = qc.amax
        fp4.fp4_quantize_dual_shard(xs, o, total, 1, 3, 0, 1, 4, 0, True, qc, qr, noise_cols=nc, noise_rows=nr)
        assert_same_quant(q_to_host(qc), _slice(want_c, o, n, 0, B), f"monitored dual shard at row {o}, cols")
        assert_same_quant(q_to_host(qr), _slice(want_r, o, n, 1, B), f"monitored dual shard at row {o}, rows")
    _assert_noise(nc, want_c["noise"], "dual shards, cols")
    _assert_noise(nr, want_r["noise"], "dual shards, rows")
