"""GPU parity of the FP4 GEMMs against the oracle's FP64 product of the
dequantized operands: |y - ref| <= 1e-5 * sum_k |a_k b_k| per element (FP32
output; a bf16 output adds its own rounding 2^-8 |ref|). Operands are quantized
by the oracle and uploaded, so the GEMM is tested on its own; one case runs
the GPU quantizer end to end."""
import numpy as np
import pytest

from gpu_util import q_from_oracle, say, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp4_fully_quantized_amd as m
    m.lib()
    return m


def _data(shape, seed, std=1.0, outliers=False):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32) * np.float32(std)
    if outliers:
        x[:, rng.permutation(shape[1])[: max(1, shape[1] // 100)]] *= 20
    from oracle.oracle import f32_to_bf16_bits
    return f32_to_bf16_bits(x)


def _run(fp4, orc, qa, qb, out, signs=None):
    import torch
    A = q_from_oracle(qa, had_signs=signs)
    B = q_from_oracle(qb, had_signs=signs)
    y = fp4.gemm(A, B, dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    yh = to_host(y)
    if out == "bf16":
        yh = orc.bf16_bits_to_f32(yh)
    return yh


SHAPES = [(200, 136, 256), (77, 300, 384), (256, 256, 128), (1, 1, 128), (513, 129, 1024)]


@pytest.mark.parametrize("fmt,had", [(0, False), (0, True), (1, False), (1, True)])
@pytest.mark.parametrize("out", ["fp32", "bf16"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_gemm_matches_oracle(fp4, orc, fmt, had, out, M, N, K):
    say("gemm", M, N, K, "fmt", fmt, "had", had, "out", out)
    signs = orc.hadamard_signs(9) if had else 0
    qa = orc.quantize(_data((M, K), 1, outliers=True), fmt=fmt, had_on=had, had_signs=signs)
    qb = orc.quantize(_data((N, K), 2, std=0.02), fmt=fmt, had_on=had, had_signs=signs)
    y = _run(fp4, orc, qa, qb, out, signs if had else None)
    ref, S = orc.gemm_ref(qa, qb)
    ok, worst = orc.gemm_check(y, ref, S, out)
    assert ok, f"worst error {worst:.3g} of the bound"


def test_gemm_zero_operand_gives_exact_zero(fp4, orc):
    qa = orc.quantize(np.zeros((64, 256), dtype=np.float32))
    qb = orc.quantize(_data((64, 256), 3))
    y = _run(fp4, orc, qa, qb, "fp32")
    assert np.all(y == 0.0)


def test_gpu_quantizer_into_gemm_end_to_end(fp4, orc):
    import torch
    xh, wh = _data((320, 512), 4, outliers=True), _data((192, 512), 5, std=0.02)
    X, W = to_device(xh), to_device(wh)
    y = fp4.gemm(fp4.quantize(X), fp4.quantize(W), dtype=torch.float32)
    ref, S = orc.gemm_ref(orc.quantize(xh), orc.quantize(wh))
    ok, worst = orc.gemm_check(to_host(y), ref, S, "fp32")
    assert ok, worst


def test_nvfp4_rotated_wgrad_end_to_end(fp4, orc):
    """wgrad dW = dY^T X with both operands quantized by the GPU along the
    tokens with the same 16-wide rotation (SR, one dual pass each): equal to
    the oracle's GEMM of the oracle's quantizations, and the rotation cancels
    (close to the unrotated product)."""
    import torch
    T, N, K = 512, 192, 256
    dyh, xh = _data((T, N), 6), _data((T, K), 7, outliers=True)
    signs = orc.hadamard_signs(21)
    _, a = fp4.quantize_dual(to_device(dyh), rnd_cols=1, seed_cols=1, rnd_rows=1, seed_rows=2,
                             had_signs_rows=signs)
    _, b = fp4.quantize_dual(to_device(xh), rnd_cols=0, rnd_rows=1, seed_rows=3, had_signs_rows=signs)
    y = to_host(fp4.gemm(a, b, dtype=torch.float32))
    qa = orc.quantize(dyh, axis=1, rnd=1, seed=2, had_on=True, had_signs=signs)
    qb = orc.quantize(xh, axis=1, rnd=1, seed=3, had_on=True, had_signs=signs)
    ref, S = orc.gemm_ref(qa, qb)
    ok, worst = orc.gemm_check(y, ref, S, "fp32")
    assert ok, worst
    # The rotation cancels: the error against the exact product is that of an
    # unrotated FP4 quantization of the same operands (a mask mismatch would
    # leave an error of the order of the product itself).
    exact = orc.bf16_bits_to_f32(dyh).astype(np.float64).T @ orc.bf16_bits_to_f32(xh).astype(np.float64)
    plain, _ = orc.gemm_ref(orc.quantize(dyh, axis=1, rnd=1, seed=2), orc.quantize(xh, axis=1, rnd=1, seed=3))
    rel = np.linalg.norm(y - exact) / np.linalg.norm(exact)
    rel_plain = np.linalg.norm(plain - exact) / np.linalg.norm(exact)
    say("relative error rotated", rel, "unrotated", rel_plain)
    assert rel < 1.5 * rel_plain, (rel, rel_plain)


def test_2d_weight_serves_forward_and_dgrad(fp4, orc):
    """W quantized once with 16 x 16 blocks: the forward GEMM takes it blocked
    along K, dgrad takes its transpose blocked along N; both match the oracle's
    GEMMs of the oracle's 2-D quantization."""
    import torch
    T, N, K = 384, 256, 512
    xh, wh, dyh = _data((T, K), 8, outliers=True), _data((N, K), 9, std=0.02), _data((T, N), 10)
    qw, qwt = fp4.quantize_2d(to_device(wh))
    qx = fp4.quantize(to_device(xh))
    qdy = fp4.quantize(to_device(dyh), rnd=1, seed=4)
    y = to_host(fp4.gemm(qx, qw, dtype=torch.float32))
    dx = to_host(fp4.gemm(qdy, qwt, dtype=torch.float32))
    ow, owt = orc.quantize_2d(wh)
    for got, a, b, what in ((y, orc.quantize(xh), ow, "forward"),
                            (dx, orc.quantize(dyh, rnd=1, seed=4), owt, "dgrad")):
        ref, S = orc.gemm_ref(a, b)
        ok, worst = orc.gemm_check(got, ref, S, "fp32")
        assert ok, (what, worst)


def _rows_of(q, rows):
    d = dict(q)
    d["codes"], d["scales"], d["rows"] = q["codes"][rows], q["scales"][rows], len(rows)
    return d


def _sample_rows(M, seed, n=64, tile=256):
    """The first and last n rows and one random row of every `tile`-row band,
    so that every output tile of the kernel (256 x 256) has a checked row, in
    every column."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, M, tile)
    per_tile = starts + rng.integers(0, tile, len(starts))
    per_tile = np.minimum(per_tile, M - 1)
    return np.unique(np.concatenate([np.arange(n), np.arange(M - n, M), per_tile]))


def test_sampled_rows_reach_every_row_tile():
    for M in (32768, 16384, 11008, 28672, 300):
        rows = _sample_rows(M, 17)
        assert set(rows // 256) == set(range((M + 255) // 256)), M


# Full-size GEMMs. Llama-7B-shaped layer (32768 tokens, 4096 in, 11008 out):
# the forward on NVFP4 and MXFP4+Hadamard operands, dgrad and wgrad on SR
# operands. Large layer (16384 tokens, 8192 in, 28672 out): the NVFP4 step.
FULL = [
    ("llama7b", "fwd-nvfp4", "bf16"),
    ("llama7b", "fwd-mxfp4", "bf16"),
    ("llama7b", "dgrad", "fp32"),
    ("llama7b", "wgrad", "fp32"),
    ("large", "fwd-nvfp4", "bf16"),
    ("large", "dgrad", "fp32"),
    ("large", "wgrad", "fp32"),
]


@pytest.mark.parametrize("wl,which,out", FULL)
def test_full_size_gemm_sampled_rows(fp4, orc, wl, which, out):
    from fp4_fully_quantized_amd import workloads
    import torch
    say("full-size gemm", wl, which, out)
    dev = lambda role: to_host(workloads.device_tensor(wl, role))
    signs = 0
    if which.startswith("fwd"):
        fmt = 0 if which == "fwd-nvfp4" else 1
        had = fmt == 1
        signs = orc.hadamard_signs(3) if had else 0
        xh, wh = dev("X"), dev("W")
        qa = orc.quantize(xh, fmt=fmt, had_on=had, had_signs=signs)
        qb = orc.quantize(wh, fmt=fmt, had_on=had, had_signs=signs)
        del xh, wh
    elif which == "dgrad":
        had = False
        dyh, wh = dev("dY"), dev("W")
        qa = orc.quantize(dyh, axis=0, rnd=1, seed=(2 << 8) | 1)
        qb = orc.quantize(wh, axis=1, rnd=1, seed=(2 << 8) | 4)
        del dyh, wh
    else:
        had = False
        dyh, xh = dev("dY"), dev("X")
        qa = orc.quantize(dyh, axis=1, rnd=1, seed=(2 << 8) | 2)
        qb = orc.quantize(xh, axis=1, rnd=1, seed=(2 << 8) | 3)
        del dyh, xh
    A = q_from_oracle(qa, had_signs=signs if had else None)
    B = q_from_oracle(qb, had_signs=signs if had else None)
    y = fp4.gemm(A, B, dtype=torch.bfloat16 if out == "bf16" else torch.float32)
    rows = _sample_rows(qa["rows"], 17, 256)   # the whole first and last row tiles, a row of every other
    say("checked rows", len(rows), "of", qa["rows"], "covering", len(set(rows // 256)), "row tiles")
    yh = to_host(y[torch.from_numpy(rows).cuda()])
    if out == "bf16":
        yh = orc.bf16_bits_to_f32(yh)
    ref, S = orc.gemm_ref(_rows_of(qa, rows), qb)
    ok, worst = orc.gemm_check(yh, ref, S, out)
    say("worst error / bound", worst)
    assert ok, worst


def test_gemm_at_the_operand_size_limit(fp4, orc):
    """The largest A the ABI accepts (codes just below 2^31 bytes: M = 1048575
    rows at K = 4096) against a ragged N = 200, NVFP4, FP32 out; operands are
    random codes and E4M3 scale bytes (the GEMM's own inputs), checked on
    sampled rows including the last row tile."""
    import torch
    M, N, K = (2 ** 31 - 1) // 2048, 200, 4096
    say("gemm at the size limit", M, N, K)
    rng = np.random.default_rng(91)

    def operand(rows, seed):
        r = np.random.default_rng(seed)
        q = {"codes": r.integers(0, 256, (rows, K // 2), dtype=np.uint8),
             "scales": r.integers(0x30, 0x48, (rows, K // 16), dtype=np.uint8),
             "fmt": 0, "rows": rows, "cols": K, "amax": 1.0, "sg": 0.5 if seed % 2 else 0.25}
        return q

    qa, qb = operand(M, 3), operand(N, 4)
    A, B = q_from_oracle(qa), q_from_oracle(qb)
    y = fp4.gemm(A, B, dtype=torch.float32)
    rows = np.unique(np.concatenate([np.arange(32), np.arange(M - 300, M), rng.integers(0, M, 64)]))
    yh = to_host(y[torch.from_numpy(rows).cuda()])
    del y, A
    sub = dict(qa)
    sub["codes"], sub["scales"], sub["rows"] = qa["codes"][rows], qa["scales"][rows], len(rows)
    ref, S = orc.gemm_ref(sub, qb)
    ok, worst = orc.gemm_check(yh, ref, S, "fp32")
    say("worst error / bound", worst)
    assert ok, worst


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("out,pad", [("fp32", 4), ("fp32", 1), ("bf16", 8), ("bf16", 3)])
def test_gemm_into_a_strided_output(fp4, orc, fmt, out, pad):
    """Output with a leading dimension ldc = N + pad: 16-byte aligned rows
    (pad 4 fp32 / 8 bf16) take the staged row-store epilogue, the others the
    element-wise one; the padding columns stay untouched."""
    import torch
    M, N, K = 320, 256, 512
    say("gemm strided output", fmt, out, pad)
    qa = orc.quantize(_data((M, K), 11, outliers=True), fmt=fmt)
    qb = orc.quantize(_data((N, K), 12, std=0.02), fmt=fmt)
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    full = torch.full((M, N + pad), 7.0, dtype=dt, device="cuda")
    fp4.gemm(q_from_oracle(qa), q_from_oracle(qb), out=full[:, :N])
    yh = to_host(full)
    if out == "bf16":
        yh = orc.bf16_bits_to_f32(yh)
    assert (yh[:, N:] == 7.0).all()
    ref, S = orc.gemm_ref(qa, qb)
    ok, worst = orc.gemm_check(yh[:, :N], ref, S, out)
    assert ok, worst


def test_mxfp4_rotated_wgrad_end_to_end(fp4, orc):
    """MXFP4 wgrad with both operands rotated 32-wide along the tokens by the
    GPU quantizer (ROWS axis, SR): equal to the oracle's GEMM of the oracle's
    quantizations."""
    import torch
    T, N, K = 512, 192, 256
    dyh, xh = _data((T, N), 13), _data((T, K), 14, outliers=True)
    signs = orc.hadamard_signs(22)
    a = fp4.quantize(to_device(dyh), axis=1, fmt=1, rnd=1, seed=2, had_signs=signs)
    b = fp4.quantize(to_device(xh), axis=1, fmt=1, rnd=1, seed=3, had_signs=signs)
    y = to_host(fp4.gemm(a, b, dtype=torch.float32))
    qa = orc.quantize(dyh, axis=1, fmt=1, rnd=1, seed=2, had_on=True, had_signs=signs)
    qb = orc.quantize(xh, axis=1, fmt=1, rnd=1, seed=3, had_on=True, had_signs=signs)
    ref, S = orc.gemm_ref(qa, qb)
    ok, worst = orc.gemm_check(y, ref, S, "fp32")
    assert ok, worst


# ------------------------------------------------------------ raw operands
RAW = [(fmt, rnd, la, lb, had) for fmt in (0, 1) for rnd in (0, 1) for la in (0, 1) for lb in (0, 1)
       for had in (False, True) if not (had and la != lb)]


@pytest.mark.parametrize("fmt,rnd,la,lb,had", RAW)
def test_raw_operand_gemm(fp4, orc, fmt, rnd, la, lb, had):
    """fp4_gemm with raw operands (quantized by the library into the
    workspace, each stored K-major (layout N) or transposed (layout T)):
    bit-equal to fp4_quantize of each operand followed by the quantized GEMM,
    and within the tolerance of the oracle's GEMM of the oracle's
    quantizations."""
    import torch
    M, N, K = 200, 136, 256
    say("raw-operand gemm fmt", fmt, "rnd", rnd, "layouts", la, lb, "had", had)
    xh = _data((M, K), 31, outliers=True)
    wh = _data((N, K), 32, std=0.02)
    stored = lambda h, lay: np.ascontiguousarray(h.T) if lay == 1 else h
    xs, ws_ = stored(xh, la), stored(wh, lb)
    signs = orc.hadamard_signs(17) if had else None
    A = fp4.RawOperand(to_device(xs), layout=la, fmt=fmt, rnd=rnd, seed=41, index_offset=8 * rnd,
                       had_signs=signs)
    B = fp4.RawOperand(to_device(ws_), layout=lb, fmt=fmt, rnd=rnd, seed=42, had_signs=signs)
    assert (A.rows, A.k, B.rows, B.k) == (M, K, N, K)
    y = fp4.gemm(A, B, dtype=torch.float32)
    qa = fp4.quantize(A.data, axis=la, fmt=fmt, rnd=rnd, seed=41, index_offset=8 * rnd, had_signs=signs)
    qb = fp4.quantize(B.data, axis=lb, fmt=fmt, rnd=rnd, seed=42, had_signs=signs)
    y_ref = fp4.gemm(qa, qb, dtype=torch.float32)
    assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32))
    oa = orc.quantize(xs, axis=la, fmt=fmt, rnd=rnd, seed=41, index_offset=8 * rnd, had_on=had,
                      had_signs=signs or 0)
    ob = orc.quantize(ws_, axis=lb, fmt=fmt, rnd=rnd, seed=42, had_on=had, had_signs=signs or 0)
    ref, S = orc.gemm_ref(oa, ob)
    ok, worst = orc.gemm_check(to_host(y), ref, S, "fp32")
    assert ok, worst


def test_raw_and_quantized_operands_mixed(fp4, orc):
    """dgrad with dY already quantized and W raw (layout T, quantized along
    its rows by the call), bf16 output."""
    import torch
    T, N, K = 256, 128, 384
    dyh, wh = _data((T, N), 33), _data((N, K), 34, std=0.02)
    say("mixed raw / quantized operands")
    qdy = fp4.quantize(to_device(dyh), rnd=1, seed=5)
    Wt = fp4.RawOperand(to_device(wh), layout=fp4.FP4_LAYOUT_T, rnd=1, seed=6)
    ws = torch.empty(fp4.fp4_gemm_workspace_bytes(qdy, Wt), dtype=torch.uint8, device="cuda")
    dx = torch.empty((T, K), dtype=torch.bfloat16, device="cuda")
    fp4.fp4_gemm(qdy, Wt, dx, ws=ws)
    ref, S = orc.gemm_ref(orc.quantize(dyh, rnd=1, seed=5), orc.quantize(wh, axis=1, rnd=1, seed=6))
    ok, worst = orc.gemm_check(orc.bf16_bits_to_f32(to_host(dx)), ref, S, "bf16")
    assert ok, worst


# Split along K of the last, partial wave of output tiles (fp4_gemm_splitk_bytes).
@pytest.mark.parametrize("fmt,out", [(0, "fp32"), (0, "bf16"), (1, "fp32"), (1, "bf16")])
def test_split_k_gemm(fp4, orc, fmt, out):
    """520 x 300 x 8192 (6 output tiles, 32 K tiles): with the split-K area
    each tile is computed in 4 K ranges whose FP32 partial tiles a second
    kernel adds, ragged edges included. Within the oracle's tolerance, the
    same bits on a second call, and the unsplit product (no workspace) within
    the same tolerance: the two differ only in the order of FP32 additions."""
    import torch
    M, N, K = 520, 300, 8192
    say("split-k gemm fmt", fmt, "out", out)
    qa = orc.quantize(_data((M, K), 61, outliers=True), fmt=fmt)
    qb = orc.quantize(_data((N, K), 62, std=0.02), fmt=fmt)
    A, B = q_from_oracle(qa), q_from_oracle(qb)
    assert fp4.fp4_gemm_splitk_bytes(A, B) == 6 * 4 * 256 * 256 * 4
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    y1 = fp4.gemm(A, B, dtype=dt)
    y2 = fp4.gemm(A, B, dtype=dt)
    iv = torch.int16 if out == "bf16" else torch.int32
    assert torch.equal(y1.view(iv), y2.view(iv))
    y0 = torch.empty_like(y1)
    fp4.fp4_gemm(A, B, y0)
    ref, S = orc.gemm_ref(qa, qb)
    for what, y in (("split", y1), ("unsplit", y0)):
        yh = to_host(y)
        if out == "bf16":
            yh = orc.bf16_bits_to_f32(yh)
        ok, worst = orc.gemm_check(yh, ref, S, out)
        say(what, "worst error / bound", worst)
        assert ok, (what, worst)


def test_split_k_gemm_after_whole_tiles(fp4, orc):
    """4352 x 4096 x 8192: 272 tiles, the first 256 computed whole and the
    last 16 split in 4; sampled rows cover every tile row, all columns."""
    import torch
    M, N, K = 4352, 4096, 8192
    say("split-k gemm after a whole wave")
    qa = orc.quantize(_data((M, K), 63), rnd=1, seed=7)
    qb = orc.quantize(_data((N, K), 64, std=0.02), rnd=1, seed=8)
    A, B = q_from_oracle(qa), q_from_oracle(qb)
    assert fp4.fp4_gemm_splitk_bytes(A, B) == 16 * 4 * 256 * 256 * 4
    y = fp4.gemm(A, B, dtype=torch.float32)
    rows = _sample_rows(M, 23, 16)
    yh = to_host(y[torch.from_numpy(rows).cuda()])
    ref, S = orc.gemm_ref(_rows_of(qa, rows), qb)
    ok, worst = orc.gemm_check(yh, ref, S, "fp32")
    say("worst error / bound", worst)
    assert ok, worst


@pytest.mark.parametrize("fmt", [0, 1])
@pytest.mark.parametrize("out,pad", [("fp32", 0), ("fp32", 19), ("bf16", 0), ("bf16", 19)])
def test_split_k_gemm_into_a_strided_output(fp4, orc, fmt, out, pad):
    """Split-K into an output of 301 columns (not a multiple of 4) with
    ldc = 301 + pad: pad 19 gives 16-byte aligned fp32 rows (ldc 320), so the
    reduction stores whole 4-column pieces and the last columns element by
    element; pad 0 stores every element alone. The padding stays untouched."""
    import torch
    M, N, K = 300, 301, 8192
    say("split-k gemm strided output", fmt, out, pad)
    qa = orc.quantize(_data((M, K), 71, outliers=True), fmt=fmt)
    qb = orc.quantize(_data((N, K), 72, std=0.02), fmt=fmt)
    A, B = q_from_oracle(qa), q_from_oracle(qb)
    assert fp4.fp4_gemm_splitk_bytes(A, B) > 0
    dt = torch.bfloat16 if out == "bf16" else torch.float32
    full = torch.full((M, N + pad), 7.0, dtype=dt, device="cuda")
    fp4.gemm(A, B, out=full[:, :N])
    yh = to_host(full)
    if out == "bf16":
        yh = orc.bf16_bits_to_f32(yh)
    assert (yh[:, N:] == 7.0).all()
    ref, S = orc.gemm_ref(qa, qb)
    ok, worst = orc.gemm_check(yh[:, :N], ref, S, out)
    assert ok, worst
