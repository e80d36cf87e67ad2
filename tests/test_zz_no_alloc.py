"""The allocation-free GEMM (fp4_gemm_noalloc) through the C ABI: the same
products as fp4_gemm with a caller workspace, bit for bit, on consecutive
calls that reuse the library's static workspace, each smaller than the one
before (a stale tensor amax or code left there by an earlier call would
change the later results)."""
import pytest

from gpu_util import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fp4():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import fp4_fully_quantized_amd as m
    m.lib()
    return m


def _bits_equal(a, b):
    import torch
    view = torch.int16 if a.dtype == torch.bfloat16 else torch.int32
    return torch.equal(a.view(view), b.view(view))


def test_noalloc_gemm_matches_fp4_gemm_on_consecutive_calls(fp4):
    import numpy as np
    import torch
    from fp4_fully_quantized_amd import workloads

    # 1. The Llama-7B-shaped forward with both operands raw (NVFP4, round to
    #    nearest, bf16 out): 100.9 MB of the 128 MiB workspace.
    say("noalloc call 1: 32768 x 11008 x 4096, both operands raw NVFP4")
    X = workloads.device_tensor("llama7b", "X")
    W = workloads.device_tensor("llama7b", "W")
    A, B = fp4.RawOperand(X), fp4.RawOperand(W)
    need = fp4.fp4_gemm_workspace_bytes(A, B)
    assert 0 < need <= fp4.FP4_GEMM_NOALLOC_MAX_BYTES
    y = torch.empty((32768, 11008), dtype=torch.bfloat16, device="cuda")
    fp4.fp4_gemm_noalloc(A, B, y)
    ref = fp4.gemm(A, B, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert _bits_equal(y, ref)
    del X, W, A, B, y, ref

    # 2. Smaller: MXFP4 with the 32-wide rotation and stochastic rounding, A
    #    stored transposed (layout T, a wgrad-like operand), FP32 out.
    say("noalloc call 2: 384 x 256 x 1024, MXFP4 rotated SR, A layout T")
    rng = np.random.default_rng(5)
    at = to_device(rng.standard_normal((1024, 384)).astype(np.float32))
    bn = to_device((rng.standard_normal((256, 1024)) * 0.02).astype(np.float32))
    signs = fp4.fp4_hadamard_signs(11)
    A = fp4.RawOperand(at, layout=fp4.FP4_LAYOUT_T, fmt=fp4.FP4_MXFP4, rnd=fp4.FP4_SR, seed=3,
                       had_signs=signs)
    B = fp4.RawOperand(bn, fmt=fp4.FP4_MXFP4, rnd=fp4.FP4_SR, seed=4, had_signs=signs)
    y = torch.empty((384, 256), dtype=torch.float32, device="cuda")
    fp4.fp4_gemm_noalloc(A, B, y)
    ref = fp4.gemm(A, B, dtype=torch.float32)
    torch.cuda.synchronize()
    assert _bits_equal(y, ref)

    # 3. Smaller still, NVFP4 SR with values far below call 1's amax, one
    #    operand already quantized: the tensor amax in the workspace must be
    #    recomputed from zero, not kept from call 1.
    say("noalloc call 3: 128 x 64 x 256, NVFP4 SR, small values, B quantized")
    a = to_device((rng.standard_normal((128, 256)) * 1e-3).astype(np.float32))
    b = to_device((rng.standard_normal((64, 256)) * 1e-2).astype(np.float32))
    A = fp4.RawOperand(a, rnd=fp4.FP4_SR, seed=9, index_offset=16)
    Bq = fp4.quantize(b, rnd=fp4.FP4_SR, seed=10)
    y = torch.empty((128, 64), dtype=torch.float32, device="cuda")
    fp4.fp4_gemm_noalloc(A, Bq, y)
    ref = fp4.gemm(A, Bq, dtype=torch.float32)
    torch.cuda.synchronize()
    assert _bits_equal(y, ref)

    # 4. No raw operand: the static workspace is not needed at all.
    say("noalloc call 4: both operands quantized")
    Aq = fp4.quantize(a)
    y = torch.empty((128, 64), dtype=torch.float32, device="cuda")
    fp4.fp4_gemm_noalloc(Aq, Bq, y)
    torch.cuda.synchronize()
    assert _bits_equal(y, fp4.gemm(Aq, Bq, dtype=torch.float32))


def test_noalloc_gemm_refuses_more_than_its_workspace(fp4):
    import torch
    say("noalloc limit")
    X = torch.zeros((65536, 4096), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((11008, 4096), dtype=torch.bfloat16, device="cuda")
    A, B = fp4.RawOperand(X), fp4.RawOperand(W)
    assert fp4.fp4_gemm_workspace_bytes(A, B) > fp4.FP4_GEMM_NOALLOC_MAX_BYTES
    y = torch.full((65536, 8), 3.0, dtype=torch.float32, device="cuda")
    with pytest.raises(fp4.Fp4Error) as e:
        fp4.fp4_gemm_noalloc(A, fp4.RawOperand(W[:8]), y)
    assert e.value.status == fp4.FP4_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((y == 3.0).all())
