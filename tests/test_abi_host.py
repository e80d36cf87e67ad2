"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/fp4.h declares, computes its host-only helpers, and
rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_entry_points():
    names = []
    for fn in sorted(os.listdir(os.path.join(ROOT, "include"))):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w \*]*?\b(fp4_\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def fp4():
    # The rejection cases pass fake device pointers: they must never reach a
    # launch, so this module only runs where no GPU is visible.
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("host-only ABI checks run without a GPU")
    import fp4_fully_quantized_amd as m
    if not os.path.exists(m.LIB_PATH):
        pytest.skip("libfp4.so not built")
    m.lib()
    return m


def test_every_declared_symbol_is_exported(fp4):
    names = declared_entry_points()
    assert len(names) >= 8
    L = ctypes.CDLL(fp4.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n
    assert sorted(fp4.EXPORTS) == names


def test_size_helpers(fp4):
    assert fp4.fp4_codes_bytes(32768, 4096) == 32768 * 2048
    assert fp4.fp4_scales_bytes(32768, 4096, fp4.FP4_NVFP4) == 32768 * 256
    assert fp4.fp4_scales_bytes(32768, 4096, fp4.FP4_MXFP4) == 32768 * 128
    assert fp4.fp4_scales_bytes(4, 40, fp4.FP4_MXFP4) == 0
    assert fp4.fp4_codes_bytes(0, 16) == 0


def test_hadamard_mask_matches_oracle(fp4, orc):
    for seed in (0, 1, 3, 77, 2 ** 33 + 9):
        assert fp4.fp4_hadamard_signs(seed) == orc.hadamard_signs(seed)


def test_status_strings(fp4):
    for s in range(8):
        assert fp4.fp4_status_str(s) != "unknown status"
    assert fp4.fp4_status_str(8) == "unknown status"


def _t(fp4, **kw):
    d = fp4.fp4_tensor()
    d.codes = kw.get("codes", 0x10000)
    d.scales = kw.get("scales", 0x20000)
    d.amax = kw.get("amax", 0x30000)
    d.tscale = kw.get("tscale", 0x40000)
    d.rows, d.cols = kw.get("rows", 64), kw.get("cols", 128)
    d.fmt = kw.get("fmt", 0)
    d.had_on = kw.get("had_on", 0)
    d.had_signs = kw.get("had_signs", 0)
    return d


# Every case below must fail validation (the pointers are fake).
QUANT_BAD = [
    # (src, dtype, R, C, ld, axis, rnd, offset, tensor overrides, expected status)
    (0, 1, 64, 128, 128, 0, 0, 0, {}, 1),
    (0x1000, 1, 0, 128, 128, 0, 0, 0, {}, 2),
    (0x1000, 1, 64, 100, 128, 0, 0, 0, {}, 2),          # C % 8
    (0x1000, 1, 64, 120, 128, 0, 0, 0, {}, 2),          # C not a multiple of 16 (NVFP4, COLS)
    (0x1000, 1, 64, 128, 120, 0, 0, 0, {}, 2),          # ld < C
    (0x1008, 1, 64, 128, 128, 0, 0, 0, {}, 3),          # src misaligned
    (0x1000, 1, 64, 128, 132, 0, 0, 0, {}, 3),          # ld % 8
    (0x1000, 1, 40, 128, 128, 1, 0, 0, {}, 2),          # R not a multiple of 16 (ROWS)
    (0x1000, 1, 64, 80, 128, 0, 0, 0, {"fmt": 1}, 2),   # C not a multiple of 32 (MXFP4)
    (0x1000, 1, 40, 128, 128, 1, 0, 0, {"had_on": 1}, 2),  # NVFP4 rotation, R not a multiple of 16
    (0x1000, 1, 64, 128, 128, 0, 1, 4, {}, 3),          # SR offset % 8
    (0x1000, 2, 64, 128, 128, 0, 0, 0, {}, 5),          # bad dtype
    (0x1000, 1, 64, 128, 128, 2, 0, 0, {}, 5),          # bad axis
    (0x1000, 1, 64, 128, 128, 0, 2, 0, {}, 5),          # bad rounding
    (0x1000, 1, 64, 128, 128, 0, 0, 0, {"fmt": 3}, 5),  # bad format
    (0x1000, 1, 64, 128, 128, 0, 0, 0, {"codes": 0}, 1),
    (0x1000, 1, 64, 128, 128, 0, 0, 0, {"amax": 0}, 1),
    (0x1000, 1, 64, 128, 128, 0, 0, 0, {"scales": 0x20004}, 3),
]


@pytest.mark.parametrize("case", QUANT_BAD)
def test_quantize_rejects_bad_arguments(fp4, case):
    src, dt, R, C, ld, axis, rnd, off, over, want = case
    d = _t(fp4, **over)
    st = fp4.lib().fp4_quantize(src, dt, R, C, ld, axis, rnd, 0, off, 1, ctypes.byref(d), None)
    assert st == want


def test_quantize_rejects_null_descriptor(fp4):
    assert fp4.lib().fp4_quantize(0x1000, 1, 64, 128, 128, 0, 0, 0, 0, 1, None, None) == 1


DUAL_BAD = [
    # (src, dtype, R, C, ld, rnd_c, off_c, rnd_r, off_r, cols overrides, rows overrides, expected)
    (0, 1, 64, 128, 128, 0, 0, 1, 0, {}, {}, 1),
    (0x1000, 1, 40, 128, 128, 0, 0, 1, 0, {}, {}, 2),          # R not a multiple of 16
    (0x1000, 1, 64, 120, 128, 0, 0, 1, 0, {}, {}, 2),          # C not a multiple of 16
    (0x1000, 1, 64, 128, 128, 0, 0, 1, 0, {"fmt": 1}, {}, 4),  # formats differ
    # NVFP4 with a rotation: the orientations need their own amax scalars
    (0x1000, 1, 64, 128, 128, 0, 0, 1, 0, {"had_on": 1}, {"had_on": 1}, 4),
    (0x1000, 1, 64, 128, 128, 0, 0, 1, 0, {}, {"had_on": 1}, 4),
    (0x1000, 1, 64, 128, 128, 0, 0, 1, 0, {"had_on": 1}, {"amax": 0}, 1),
    (0x1000, 1, 64, 128, 128, 0, 0, 1, 0, {}, {"had_on": 1, "amax": 0x30008}, 4),  # shared tscale
    (0x1000, 1, 64, 128, 128, 1, 4, 1, 0, {}, {}, 3),          # SR offset % 8 (cols)
    (0x1000, 1, 64, 128, 128, 0, 0, 1, 12, {}, {}, 3),         # SR offset % 8 (rows)
    (0x1000, 1, 64, 128, 128, 2, 0, 1, 0, {}, {}, 5),          # bad rounding
    (0x1000, 1, 64, 128, 128, 0, 0, 1, 0, {}, {"codes": 0}, 1),
    (0x1000, 1, 64, 128, 128, 0, 0, 1, 0, {}, {"tscale": 0}, 1),
    (0x1000, 1, 64, 128, 128, 0, 0, 1, 0, {"scales": 0x20004}, {}, 3),
]


@pytest.mark.parametrize("case", DUAL_BAD)
def test_quantize_dual_rejects_bad_arguments(fp4, case):
    src, dt, R, C, ld, rc, oc, rr, orr, over_c, over_r, want = case
    dc, dr = _t(fp4, **over_c), _t(fp4, **over_r)
    st = fp4.lib().fp4_quantize_dual(src, dt, R, C, ld, rc, 0, oc, rr, 0, orr, 1, ctypes.byref(dc),
                                     ctypes.byref(dr), None)
    assert st == want


def test_quantize_dual_rejects_null_descriptors(fp4):
    d = _t(fp4)
    assert fp4.lib().fp4_quantize_dual(0x1000, 1, 64, 128, 128, 0, 0, 0, 1, 0, 0, 1, None,
                                       ctypes.byref(d), None) == 1


SHARD_BAD = [
    # (R, C, row_offset, rows_total, axis, tensor overrides, expected status)
    (64, 128, -16, 128, 0, {}, 2),          # negative offset
    (64, 128, 80, 128, 0, {}, 2),           # shard runs past the whole tensor
    (64, 128, 0, 0, 0, {}, 2),              # no whole tensor
    (64, 128, 0, (1 << 62), 0, {}, 2),      # rows_total * C overflows the index
    (64, 128, 0, 132, 0, {}, 3),            # rows_total % 8
    (64, 128, 8, 128, 1, {}, 3),            # ROWS shard starts inside a block
    (64, 128, 16, 128, 1, {"fmt": 1}, 3),   # ... an MXFP4 block
    (64, 128, 0, 128, 2, {}, 5),            # bad axis
    (64, 128, 0, 128, 0, {"fmt": 3}, 5),    # bad format
    (40, 128, 0, 128, 1, {}, 2),            # ROWS shard rows not a multiple of 16 (as fp4_quantize)
    (64, 100, 0, 128, 0, {}, 2),            # C % 8 (as fp4_quantize)
]


@pytest.mark.parametrize("case", SHARD_BAD)
def test_quantize_shard_rejects_bad_arguments(fp4, case):
    R, C, off, total, axis, over, want = case
    d = _t(fp4, **over)
    st = fp4.lib().fp4_quantize_shard(0x1000, 1, R, C, C, off, total, axis, 1, 0, 0, 1, ctypes.byref(d), None,
                                      None)
    assert st == want
    assert fp4.lib().fp4_quantize_shard(0x1000, 1, R, C, C, off, total, axis, 1, 0, 0, 1, None, None, None) == 1


def test_quantize_shard_rejects_a_misaligned_noise_buffer(fp4):
    d = _t(fp4)
    assert fp4.lib().fp4_quantize_shard(0x1000, 1, 64, 128, 128, 0, 128, 0, 1, 0, 0, 1, ctypes.byref(d),
                                        0x50004, None) == 3
    dc, dr = _t(fp4), _t(fp4)
    for nc, nr in ((0x50004, None), (None, 0x50004)):
        assert fp4.lib().fp4_quantize_dual_shard(0x1000, 1, 64, 128, 128, 0, 128, 0, 0, 0, 1, 0, 0, 1,
                                                 ctypes.byref(dc), ctypes.byref(dr), nc, nr, None) == 3


DUAL_SHARD_BAD = [
    # (R, C, row_offset, rows_total, cols overrides, expected status)
    (64, 128, 8, 128, {}, 3),               # the row blocks straddle shards
    (64, 128, 96, 128, {}, 2),              # past the end
    (64, 128, 0, 36, {}, 2),                # shard larger than the whole tensor
    (64, 128, 0, 132, {}, 3),               # rows_total % 8
    (64, 128, 0, 128, {"fmt": 3}, 5),
    (40, 128, 0, 128, {}, 2),               # shard rows not a multiple of 16 (as fp4_quantize_dual)
]


@pytest.mark.parametrize("case", DUAL_SHARD_BAD)
def test_quantize_dual_shard_rejects_bad_arguments(fp4, case):
    R, C, off, total, over, want = case
    dc, dr = _t(fp4, **over), _t(fp4)
    st = fp4.lib().fp4_quantize_dual_shard(0x1000, 1, R, C, C, off, total, 0, 0, 0, 1, 0, 0, 1,
                                           ctypes.byref(dc), ctypes.byref(dr), None, None, None)
    assert st == want
    assert fp4.lib().fp4_quantize_dual_shard(0x1000, 1, R, C, C, off, total, 0, 0, 0, 1, 0, 0, 1,
                                             None, ctypes.byref(dr), None, None, None) == 1


def test_noise_entry_points_reject_bad_arguments(fp4):
    L = fp4.lib()
    d = _t(fp4)
    args = (0x1000, 1, 64, 128, 128, 0, 0, 0, 0, 1, ctypes.byref(d))
    assert L.fp4_quantize_noise(*args, None, None) == 1
    assert L.fp4_quantize_noise(*args, 0x60004, None) == 3          # noise not 8-byte aligned
    assert L.fp4_quantize_noise(0x1000, 1, 64, 120, 128, 0, 0, 0, 0, 1, ctypes.byref(d), 0x60000,
                                None) == 2                            # checks of fp4_quantize still apply
    dc, dr = _t(fp4), _t(fp4)
    dargs = (0x1000, 1, 64, 128, 128, 0, 0, 0, 1, 0, 0, 1, ctypes.byref(dc), ctypes.byref(dr))
    assert L.fp4_quantize_dual_noise(*dargs, None, None, None) == 1
    assert L.fp4_quantize_dual_noise(*dargs, None, 0x60002, None) == 3
    assert L.fp4_quantize_dual_noise(0x1000, 1, 40, 128, 128, 0, 0, 0, 1, 0, 0, 1, ctypes.byref(dc),
                                     ctypes.byref(dr), 0x60000, None, None) == 2


Q2D_BAD = [
    # (src, R, C, ld, rnd, offset, out overrides, out_t overrides, expected)
    (0, 64, 128, 128, 0, 0, {}, {}, 1),
    (0x1000, 40, 128, 128, 0, 0, {}, {}, 2),            # R not a multiple of 16
    (0x1000, 64, 136, 136, 0, 0, {}, {}, 2),            # C not a multiple of 16
    (0x1000, 64, 80, 128, 0, 0, {"fmt": 1}, {"fmt": 1}, 2),  # C not a multiple of 32 (MXFP4)
    (0x1000, 64, 128, 128, 0, 0, {"fmt": 1}, {}, 4),    # formats differ
    (0x1000, 64, 128, 128, 0, 0, {"had_on": 1}, {}, 4),  # no rotation with 2-D blocks
    (0x1000, 64, 128, 128, 1, 4, {}, {}, 3),            # SR offset % 8
    (0x1000, 64, 128, 128, 2, 0, {}, {}, 5),            # bad rounding
    (0x1000, 64, 128, 128, 0, 0, {}, {"codes": 0}, 1),
    (0x1000, 64, 128, 128, 0, 0, {}, {"tscale": 0}, 1),
    (0x1000, 64, 128, 128, 0, 0, {"scales": 0x20008}, {}, 3),
]


@pytest.mark.parametrize("case", Q2D_BAD)
def test_quantize_2d_rejects_bad_arguments(fp4, case):
    src, R, C, ld, rnd, off, over, over_t, want = case
    d, dt = _t(fp4, **over), _t(fp4, **over_t)
    st = fp4.lib().fp4_quantize_2d(src, 1, R, C, ld, rnd, 0, off, 1, ctypes.byref(d), ctypes.byref(dt), None)
    assert st == want
    assert fp4.lib().fp4_quantize_2d(0x1000, 1, 64, 128, 128, 0, 0, 0, 1, ctypes.byref(d), None, None) == 1


AMAX_H16_BAD = [
    # (src, dtype, R, C, ld, axis, amax, expected)
    (0, 1, 64, 128, 128, 0, 0x30000, 1),
    (0x1000, 1, 64, 128, 128, 0, 0, 1),
    (0x1000, 1, 64, 136, 136, 0, 0x30000, 2),   # C not a multiple of 16 (COLS)
    (0x1000, 1, 40, 128, 128, 1, 0x30000, 2),   # R not a multiple of 16 (ROWS)
    (0x1000, 1, 64, 128, 128, 2, 0x30000, 5),   # bad axis
    (0x1000, 3, 64, 128, 128, 0, 0x30000, 5),   # bad dtype
    (0x1004, 1, 64, 128, 128, 0, 0x30000, 3),   # misaligned
]


@pytest.mark.parametrize("case", AMAX_H16_BAD)
def test_amax_hadamard16_rejects_bad_arguments(fp4, case):
    src, dt, R, C, ld, axis, amax, want = case
    assert fp4.lib().fp4_tensor_amax_hadamard16(src, dt, R, C, ld, axis, 5, amax, None) == want


def _q_op(fp4, t):
    o = fp4.fp4_operand()
    o.kind = fp4.FP4_OPERAND_QUANTIZED
    o.q = ctypes.pointer(t)
    return o


def _raw_op(fp4, **kw):
    o = fp4.fp4_operand()
    o.kind = kw.get("kind", fp4.FP4_OPERAND_RAW)
    o.dtype = kw.get("dtype", 1)
    o.data = kw.get("data", 0x70000)
    o.rows, o.k = kw.get("rows", 64), kw.get("k", 128)
    o.ld = kw.get("ld", o.rows if kw.get("layout", 0) == 1 else o.k)
    o.layout = kw.get("layout", 0)
    o.fmt, o.rnd = kw.get("fmt", 0), kw.get("rnd", 0)
    o.seed, o.index_offset = kw.get("seed", 0), kw.get("index_offset", 0)
    o.had_on, o.had_signs = kw.get("had_on", 0), kw.get("had_signs", 0)
    return o


GEMM_BAD = [
    ({}, {"fmt": 1}, 1, 128, 4),                      # mixed formats
    ({"fmt": 1, "had_on": 1, "had_signs": 5}, {"fmt": 1, "had_on": 1, "had_signs": 6}, 1, 128, 4),
    ({"fmt": 1, "had_on": 1}, {"fmt": 1}, 1, 128, 4),
    ({"cols": 64}, {"cols": 64}, 1, 128, 2),          # K % 128
    ({"cols": 256}, {"cols": 128}, 1, 128, 2),        # K mismatch
    ({"rows": 0}, {}, 1, 128, 2),
    ({}, {"rows": 200}, 1, 128, 2),                   # ldc < N
    ({"tscale": 0}, {}, 1, 128, 1),
    ({"codes": 0x10008}, {}, 1, 128, 3),
    ({}, {}, 3, 128, 5),
    ({"fmt": 4}, {}, 1, 128, 5),
    ({"rows": 2 ** 20, "cols": 4096}, {"cols": 4096}, 1, 128, 2),   # A codes reach 2^31 bytes
    ({"cols": 4096}, {"rows": 2 ** 20, "cols": 4096}, 1, 2 ** 20, 2),  # B codes reach 2^31 bytes
]


@pytest.mark.parametrize("case", GEMM_BAD)
def test_gemm_rejects_bad_arguments(fp4, case):
    a_over, b_over, out_t, ldc, want = case
    A, B = _t(fp4, **a_over), _t(fp4, **b_over)
    st = fp4.lib().fp4_gemm(ctypes.byref(_q_op(fp4, A)), ctypes.byref(_q_op(fp4, B)), out_t, 0x50000, ldc,
                            None, 0, None)
    assert st == want
    A, B = _t(fp4), _t(fp4)
    oa, ob = _q_op(fp4, A), _q_op(fp4, B)
    assert fp4.lib().fp4_gemm(ctypes.byref(oa), ctypes.byref(ob), 0, 0x50002, 128, None, 0, None) == 3
    assert fp4.lib().fp4_gemm(None, ctypes.byref(ob), 1, 0x50000, 128, None, 0, None) == 1
    assert fp4.lib().fp4_gemm(ctypes.byref(oa), ctypes.byref(ob), 1, None, 128, None, 0, None) == 1
    nullq = fp4.fp4_operand()
    nullq.kind = fp4.FP4_OPERAND_QUANTIZED
    assert fp4.lib().fp4_gemm(ctypes.byref(nullq), ctypes.byref(ob), 1, 0x50000, 128, None, 0, None) == 1


def _ws_bytes(rows, k, fmt):
    up = lambda n: (n + 255) // 256 * 256
    return up(rows * k // 2) + up(rows * k // (16 if fmt == 0 else 32)) + (256 if fmt == 0 else 0)


def test_gemm_workspace_bytes(fp4):
    L = fp4.lib()
    A, B = _t(fp4), _t(fp4)
    qa, qb = _q_op(fp4, A), _q_op(fp4, B)
    assert L.fp4_gemm_workspace_bytes(ctypes.byref(qa), ctypes.byref(qb)) == 0
    ra = _raw_op(fp4, rows=100, k=256)
    rb = _raw_op(fp4, rows=48, k=256, layout=1, fmt=0)
    assert L.fp4_gemm_workspace_bytes(ctypes.byref(ra), ctypes.byref(qb)) == _ws_bytes(100, 256, 0)
    assert L.fp4_gemm_workspace_bytes(ctypes.byref(qa), ctypes.byref(rb)) == _ws_bytes(48, 256, 0)
    assert L.fp4_gemm_workspace_bytes(ctypes.byref(ra), ctypes.byref(rb)) == \
        _ws_bytes(100, 256, 0) + _ws_bytes(48, 256, 0)
    mx = _raw_op(fp4, rows=4096, k=4096, fmt=1)
    assert L.fp4_gemm_workspace_bytes(ctypes.byref(mx), ctypes.byref(mx)) == 2 * _ws_bytes(4096, 4096, 1)
    # the Llama-7B forward with both operands raw: X 32768 x 4096 and W 11008 x 4096 in NVFP4
    x = _raw_op(fp4, rows=32768, k=4096)
    w = _raw_op(fp4, rows=11008, k=4096)
    assert L.fp4_gemm_workspace_bytes(ctypes.byref(x), ctypes.byref(w)) == \
        32768 * 2048 + 32768 * 256 + 256 + 11008 * 2048 + 11008 * 256 + 256
    for bad in (_raw_op(fp4, rows=0), _raw_op(fp4, k=120), _raw_op(fp4, fmt=2), _raw_op(fp4, kind=7)):
        assert L.fp4_gemm_workspace_bytes(ctypes.byref(bad), ctypes.byref(qb)) == 0
    assert L.fp4_gemm_workspace_bytes(None, ctypes.byref(qb)) == 0



def _splitk(fp4, M, N, K, fmt=0):
    L = fp4.lib()
    a = _q_op(fp4, _t(fp4, rows=M, cols=K, fmt=fmt))
    b = _q_op(fp4, _t(fp4, rows=N, cols=K, fmt=fmt))
    return L.fp4_gemm_splitk_bytes(ctypes.byref(a), ctypes.byref(b))


def test_gemm_splitk_bytes(fp4):
    """The split-K area: the tiles of the last, partial wave (tiles mod 256)
    times the pieces the plan chooses times one FP32 256 x 256 tile. The plan
    prices a wave of n tiles at max(n / 256, 1.7 / 2.4) of a full one (the
    clock rises when fewer CUs run) against the partial tiles' traffic."""
    tile = 256 * 256 * 4
    # Llama-7B: wgrad's last wave of 176 of its 688 tiles already runs at the
    # higher clock; forward (5504 tiles, K = 4096) and dgrad (2048) neither
    assert _splitk(fp4, 11008, 4096, 32768) == 0
    assert _splitk(fp4, 11008, 4096, 32768, fmt=1) == 0
    assert _splitk(fp4, 32768, 11008, 4096) == 0
    assert _splitk(fp4, 32768, 4096, 11008) == 0
    # the large layer: 7168, 2048 and 3584 tiles, all whole waves
    assert _splitk(fp4, 16384, 28672, 8192) == 0
    assert _splitk(fp4, 16384, 8192, 28672) == 0
    assert _splitk(fp4, 28672, 8192, 16384) == 0
    # few tiles: 6 tiles with K = 8192 (32 K tiles) in 4 pieces of 8, with 4096 in 2
    assert _splitk(fp4, 520, 300, 8192) == 6 * 4 * tile
    assert _splitk(fp4, 520, 300, 4096) == 6 * 2 * tile
    assert _splitk(fp4, 520, 300, 7936) == 6 * 3 * tile
    # K % 256 != 0 counts 128-wide K tiles: 8064 = 63 of them, 7 pieces of 9
    assert _splitk(fp4, 520, 300, 8064) == 6 * 7 * tile
    # 272 tiles: the 16 of the second wave in 4 pieces
    assert _splitk(fp4, 4352, 4096, 8192) == 16 * 4 * tile
    # a 2048 x 2048 weight gradient over 32768 tokens: 64 tiles in 3 pieces
    assert _splitk(fp4, 2048, 2048, 32768) == 64 * 3 * tile
    # too short for a piece of 8 K tiles
    assert _splitk(fp4, 520, 300, 3840) == 0
    assert _splitk(fp4, 200, 136, 256) == 0
    # invalid pairs
    L = fp4.lib()
    qa = _q_op(fp4, _t(fp4, rows=64, cols=8192))
    qb = _q_op(fp4, _t(fp4, rows=64, cols=4096))
    assert L.fp4_gemm_splitk_bytes(ctypes.byref(qa), ctypes.byref(qb)) == 0
    assert L.fp4_gemm_splitk_bytes(None, ctypes.byref(qb)) == 0


RAW_BAD = [
    # (A overrides (raw), ws, ws_bytes, expected): B is a valid quantized NVFP4 64 x 128 operand
    ({}, None, 0, 7),                                   # no workspace
    ({}, 0x800000, _ws_bytes(64, 128, 0) - 1, 7),       # workspace too small
    ({}, 0x800010, 1 << 20, 7),                         # workspace not 256-byte aligned
    ({"data": 0}, 0x800000, 1 << 20, 1),
    ({"data": 0x70008}, 0x800000, 1 << 20, 3),          # source misaligned
    ({"ld": 132}, 0x800000, 1 << 20, 3),                # ld % 8
    ({"ld": 64}, 0x800000, 1 << 20, 2),                 # ld < K (layout N)
    ({"layout": 1, "ld": 32}, 0x800000, 1 << 20, 2),    # ld < rows (layout T)
    ({"layout": 2}, 0x800000, 1 << 20, 5),
    ({"rnd": 3}, 0x800000, 1 << 20, 5),
    ({"dtype": 4}, 0x800000, 1 << 20, 5),
    ({"rnd": 1, "index_offset": 12}, 0x800000, 1 << 20, 3),   # SR offset % 8
    ({"fmt": 1}, 0x800000, 1 << 20, 4),                 # formats differ
    ({"had_on": 1, "had_signs": 3}, 0x800000, 1 << 20, 4),  # rotation on one side only
    ({"k": 256}, 0x800000, 1 << 20, 2),                 # K differs from B's
    ({"rows": 60, "layout": 1, "ld": 64}, 0x800000, 1 << 20, 2),  # layout T: rows are the contiguous axis, % 8
]


@pytest.mark.parametrize("case", RAW_BAD)
def test_gemm_rejects_bad_raw_operands(fp4, case):
    over, ws, ws_bytes, want = case
    A = _raw_op(fp4, **over)
    B = _t(fp4)
    st = fp4.lib().fp4_gemm(ctypes.byref(A), ctypes.byref(_q_op(fp4, B)), 1, 0x50000, 128, ws, ws_bytes, None)
    assert st == want


def test_gemm_rejects_bad_raw_b(fp4):
    # The same checks apply to B; a too-small workspace counts both operands.
    A = _raw_op(fp4, rows=64, k=128)
    B = _raw_op(fp4, rows=48, k=128, layout=1, ld=48)
    need = _ws_bytes(64, 128, 0) + _ws_bytes(48, 128, 0)
    L = fp4.lib()
    assert L.fp4_gemm(ctypes.byref(A), ctypes.byref(B), 1, 0x50000, 48, 0x800000, need - 256, None) == 7
    Bbad = _raw_op(fp4, rows=48, k=128, layout=1, ld=40)
    assert L.fp4_gemm(ctypes.byref(A), ctypes.byref(Bbad), 1, 0x50000, 48, 0x800000, need, None) == 2
    Bsr = _raw_op(fp4, rows=48, k=128, layout=1, ld=48, rnd=1, index_offset=4)
    assert L.fp4_gemm(ctypes.byref(A), ctypes.byref(Bsr), 1, 0x50000, 48, 0x800000, need, None) == 3


def test_gemm_noalloc_rejects_operands_beyond_its_workspace(fp4):
    # Raw operands whose workspace exceeds the static array are refused before
    # anything touches a device; so are the checks fp4_gemm makes.
    L = fp4.lib()
    assert fp4.FP4_GEMM_NOALLOC_MAX_BYTES == 128 << 20
    x = _raw_op(fp4, rows=32768, k=4096)
    w = _raw_op(fp4, rows=11008, k=4096)
    assert L.fp4_gemm_workspace_bytes(ctypes.byref(x), ctypes.byref(w)) <= fp4.FP4_GEMM_NOALLOC_MAX_BYTES
    big = _raw_op(fp4, rows=65536, k=4096)
    need = L.fp4_gemm_workspace_bytes(ctypes.byref(big), ctypes.byref(w))
    assert need > fp4.FP4_GEMM_NOALLOC_MAX_BYTES
    assert L.fp4_gemm_noalloc(ctypes.byref(big), ctypes.byref(w), 1, 0x50000, 11008, None) == 7
    assert L.fp4_gemm_noalloc(ctypes.byref(x), ctypes.byref(w), 1, None, 11008, None) == 1
    assert L.fp4_gemm_noalloc(None, ctypes.byref(w), 1, 0x50000, 11008, None) == 1
    A, B = _t(fp4), _t(fp4, fmt=1)
    assert L.fp4_gemm_noalloc(ctypes.byref(_q_op(fp4, A)), ctypes.byref(_q_op(fp4, B)), 1, 0x50000, 128,
                              None) == 4


def test_noise_ratio_rejects_bad_arguments(fp4):
    L = fp4.lib()
    assert L.fp4_noise_ratio(None, 0x60000, None) == 1
    assert L.fp4_noise_ratio(0x60000, None, None) == 1
    assert L.fp4_noise_ratio(0x60004, 0x60010, None) == 3
    assert L.fp4_noise_ratio(0x60000, 0x60014, None) == 3


DEQ_BAD = [
    ({}, 1, 0, 128, 1),                # null dst
    ({"fmt": 5}, 1, 0x50000, 128, 5),
    ({"cols": 120}, 1, 0x50000, 128, 2),
    ({}, 1, 0x50000, 64, 2),           # ld < cols
    ({}, 1, 0x50004, 128, 3),
    ({"tscale": 0}, 1, 0x50000, 128, 1),
]


@pytest.mark.parametrize("case", DEQ_BAD)
@pytest.mark.parametrize("entry", ["fp4_dequantize", "fp4_dequantize_unrotated"])
def test_dequantize_rejects_bad_arguments(fp4, case, entry):
    over, dt, dst, ld, want = case
    q = _t(fp4, **over)
    assert getattr(fp4.lib(), entry)(ctypes.byref(q), dt, dst, ld, None) == want


def test_amax_rejects_bad_arguments(fp4):
    L = fp4.lib()
    assert L.fp4_tensor_amax(0x1000, 1, 64, 128, 128, None, None) == 1
    assert L.fp4_tensor_amax(0x1000, 1, 64, 12, 128, 0x2000, None) == 2
    assert L.fp4_tensor_amax(0x1004, 1, 64, 128, 128, 0x2000, None) == 3


def test_product_path_fails_loudly_without_the_library(monkeypatch, tmp_path):
    import fp4_fully_quantized_amd as m
    monkeypatch.setattr(m, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(m, "_lib", None)
    with pytest.raises(RuntimeError):
        m.lib()


# ---------------------------------------------------------------- the binding's own checks
# The Python binding refuses tensors the library cannot see through raw
# pointers (host memory, wrong dtype or shape, transposed views, buffers too
# small) before calling it. These run on CPU and meta tensors: nothing here
# reaches the library's compute calls.
def test_binding_rejects_host_and_meta_tensors(fp4):
    import torch
    x = torch.zeros((64, 128), dtype=torch.float32)
    q = fp4.QTensor(64, 128, fp4.FP4_NVFP4, device="cpu")
    with pytest.raises(ValueError, match="GPU"):
        fp4.fp4_quantize(x, 0, 0, 0, 0, False, q)
    with pytest.raises(ValueError, match="GPU"):
        fp4.fp4_tensor_amax(x, torch.zeros(1))
    m = torch.empty((64, 128), dtype=torch.float32, device="meta")
    with pytest.raises(ValueError, match="GPU"):
        fp4.fp4_quantize(m, 0, 0, 0, 0, False, q)
    with pytest.raises(ValueError, match="GPU"):
        fp4.RawOperand(x)


def test_binding_checks_shapes_and_buffers(fp4, monkeypatch):
    import torch
    # Pretend CPU tensors are device tensors to reach the shape and size checks
    # (the library is never called: every case raises first).
    monkeypatch.setattr(fp4, "_check_device", lambda t, name, device=None: None)
    calls = []
    real = fp4.lib()

    class OnlySizeHelpers:
        # the host-only size helpers answer; any other entry point is recorded
        def __getattr__(self, name):
            if name in ("fp4_codes_bytes", "fp4_scales_bytes", "fp4_status_str"):
                return getattr(real, name)
            calls.append(name)
            return lambda *a: 0

    monkeypatch.setattr(fp4, "_lib", OnlySizeHelpers())
    x = torch.zeros((64, 128), dtype=torch.float32)
    q = fp4.QTensor(64, 128, fp4.FP4_NVFP4, device="cpu")
    with pytest.raises(ValueError, match="needs 128 x 64"):
        fp4.fp4_quantize(x, fp4.FP4_AXIS_ROWS, 0, 0, 0, False, q)      # output not transposed
    with pytest.raises(ValueError, match="unit column stride"):
        fp4.fp4_quantize(torch.zeros((128, 64)).t(), 0, 0, 0, 0, False, q)
    with pytest.raises(TypeError):
        fp4.fp4_quantize(x.to(torch.float16), 0, 0, 0, 0, False, q)
    small = fp4.QTensor(64, 128, fp4.FP4_NVFP4, device="cpu")
    small.codes = small.codes[:10]
    with pytest.raises(ValueError, match="codes holds"):
        fp4.fp4_quantize(x, 0, 0, 0, 0, False, small)
    small = fp4.QTensor(64, 128, fp4.FP4_NVFP4, device="cpu")
    small.scales = small.scales.flatten()[:100]
    with pytest.raises(ValueError, match="scales holds"):
        fp4.fp4_quantize(x, 0, 0, 0, 0, False, small)
    noamax = fp4.QTensor(64, 128, fp4.FP4_NVFP4, device="cpu")
    noamax.amax = torch.zeros(1, dtype=torch.float64)
    with pytest.raises(ValueError, match="amax"):
        fp4.fp4_quantize(x, 0, 0, 0, 0, False, noamax)
    # GEMM: output shape, output layout, K of the operands
    qa = fp4.QTensor(64, 128, fp4.FP4_NVFP4, device="cpu")
    qb = fp4.QTensor(48, 128, fp4.FP4_NVFP4, device="cpu")
    with pytest.raises(ValueError, match="the product is 64 x 48"):
        fp4.fp4_gemm(qa, qb, torch.zeros((48, 64)))
    with pytest.raises(ValueError, match="unit column stride"):
        fp4.fp4_gemm(qa, qb, torch.zeros((48, 64)).t())
    # dequantize: destination shape
    with pytest.raises(ValueError, match="dst is"):
        fp4.fp4_dequantize(qa, torch.zeros((128, 64)))
    # dual: each output in its own orientation
    qr_bad = fp4.QTensor(64, 128, fp4.FP4_NVFP4, device="cpu")
    with pytest.raises(ValueError, match="out_rows"):
        fp4.fp4_quantize_dual(x, 0, 0, 0, 1, 0, 0, False, q, qr_bad)
    # noise buffers
    with pytest.raises(ValueError, match="noise"):
        fp4.fp4_quantize_noise(x, 0, 0, 0, 0, False, q, torch.zeros(2, dtype=torch.float32))
    with pytest.raises(ValueError, match="ratio"):
        fp4.fp4_noise_ratio(torch.zeros(2, dtype=torch.float64), torch.zeros(1, dtype=torch.float32))
    # raw operands: layout, and a workspace of the wrong type
    with pytest.raises(ValueError, match="layout"):
        fp4.RawOperand(x, layout=3)
    ra = fp4.RawOperand(x)
    assert (ra.rows, ra.k) == (64, 128)
    rt = fp4.RawOperand(x, layout=fp4.FP4_LAYOUT_T)
    assert (rt.rows, rt.k) == (128, 64)
    with pytest.raises(ValueError, match="ws"):
        fp4.fp4_gemm(ra, qb, torch.zeros((64, 48)), ws=torch.zeros(10, dtype=torch.float32))
    assert calls == []
