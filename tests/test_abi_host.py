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
    for s in range(7):
        assert fp4.fp4_status_str(s)


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
    ({"rows": 2 ** 20, "cols": 4096}, {"cols": 4096}, 1, 128, 2),   # A codes reach 2^31 bytes
    ({"cols": 4096}, {"rows": 2 ** 20, "cols": 4096}, 1, 2 ** 20, 2),  # B codes reach 2^31 bytes
]


@pytest.mark.parametrize("case", GEMM_BAD)
def test_gemm_rejects_bad_arguments(fp4, case):
    a_over, b_over, out_t, ldc, want = case
    A, B = _t(fp4, **a_over), _t(fp4, **b_over)
    st = fp4.lib().fp4_gemm(ctypes.byref(A), ctypes.byref(B), out_t, 0x50000, ldc, None)
    assert st == want
    A, B = _t(fp4), _t(fp4)
    assert fp4.lib().fp4_gemm(ctypes.byref(A), ctypes.byref(B), 0, 0x50002, 128, None) == 3
    assert fp4.lib().fp4_gemm(None, ctypes.byref(B), 1, 0x50000, 128, None) == 1


DEQ_BAD = [
    ({}, 1, 0, 128, 1),                # null dst
    ({"fmt": 5}, 1, 0x50000, 128, 5),
    ({"cols": 120}, 1, 0x50000, 128, 2),
    ({}, 1, 0x50000, 64, 2),           # ld < cols
    ({}, 1, 0x50004, 128, 3),
    ({"tscale": 0}, 1, 0x50000, 128, 1),
]


@pytest.mark.parametrize("case", DEQ_BAD)
def test_dequantize_rejects_bad_arguments(fp4, case):
    over, dt, dst, ld, want = case
    q = _t(fp4, **over)
    assert fp4.lib().fp4_dequantize(ctypes.byref(q), dt, dst, ld, None) == want


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
