"""Benchmark of the FP4 quantize + FP4 GEMM hot path on one MI355X.

One step = one pass of the whole path over the Llama-7B-shaped linear layer
(32768 tokens = batch 64 x sequence 512, 4096 in, 11008 out; Quartet's kernel
measurements use this shape), inputs resident in HBM:

  NVFP4 forward   X, W quantized along K (round to nearest, two-level scaling),
                  Y = X W^T (bf16 out)
  NVFP4 backward  dY along out-features (SR), W^T (SR, amax reused),
                  dgrad dX = dY W (fp32 out); dY^T and X^T (SR, amax reused),
                  wgrad dW = dY^T X (fp32 out)
  MXFP4 forward   X, W with the 32-wide random-sign Hadamard (RTN),
                  Y = X W^T on the block-scaled FP4 MFMA (bf16 out)

Each NVFP4 tensor's two quantizations (X and W: RTN along K for the forward,
SR along the other axis for the backward; dY: SR along both) come from one
read of the tensor (fp4_quantize_dual); `--separate-passes` runs them as
separate fp4_quantize calls instead (same outputs).

Printed: one JSON line. `value` = GEMM FLOPs of the step / step time (TFLOP/s).
Quantize records give GB/s of algorithmic bytes, as a fraction of 8 TB/s
(`frac_hbm`) and of a 1 GiB device copy measured in the same run
(`frac_copy`, `hbm_copy_GBps`); `per_op_cold` times the step's quantize calls
with the caches evicted before each call.
`roofline` is for the dominant kernel (the NVFP4 GEMM), timed with HIP events
on the stream it runs on; `cpu_baseline` times the CPU oracle on a bounded
sample of the same step and scales it to the same unit.
`large_step` times the large-layer step the same way (hidden 8192, MLP 28672,
16384 tokens: NVFP4 fwd + bwd, RTN forward, SR on the backward operands).
`dp8_shard_step` times the NVFP4 step on one GPU's share of 8-way data
parallelism over the Llama-7B layer's tokens (4096 tokens: X [4096, 4096],
dY [4096, 11008], W whole), the shape each GPU would run, X and dY quantized
with the whole batch's SR indices (tokens 12288 .. 16383).
`measured_ceilings` puts what the chip reaches on this machine beside the
data-sheet peaks: loops of the two MFMA instructions the GEMMs issue, and
streaming passes (read only, copy, and a quantize-like 4:1 read:write pass)
at their best grid size.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

TOKENS, D_IN, D_OUT = 32768, 4096, 11008
GEMM_FLOP = 2.0 * TOKENS * D_IN * D_OUT          # each of fwd, dgrad, wgrad
L_TOKENS, L_IN, L_OUT = 16384, 8192, 28672       # the large layer
SHARD_TOKENS = TOKENS // 8                       # one GPU's share of 8-way data parallelism
SHARD_RANK = 3                                   # the share timed: tokens 12288 .. 16383
PEAK_F16_TFLOPS = 2500.0                         # dense MFMA, MI355X
PEAK_FP4_TFLOPS = 10100.0
PEAK_HBM_GBS = 8000.0


def algorithmic_bytes(n_elem: int, src_bytes: int, block: int, amax_pass: bool, outputs: int = 1) -> float:
    """Read the input once per pass, write 0.5 B of codes and 1/B B of scale
    per element for each output orientation; an NVFP4 pass without a ready
    amax reads the input once more."""
    b = n_elem * (src_bytes + outputs * (0.5 + 1.0 / block))
    if amax_pass:
        b += n_elem * src_bytes
    return b


def gemm_workspace(fp4, A, B):
    """The split-K area of this product (allocated once, before the timed
    steps), or None when the shape never splits."""
    import torch
    n = fp4.fp4_gemm_workspace_bytes(A, B) + fp4.fp4_gemm_splitk_bytes(A, B)
    return torch.empty(n, dtype=torch.uint8, device="cuda") if n else None


def make_step(fp4, X, W, dY, signs, separate=False):
    import torch

    outs = {
        "Y": torch.empty((TOKENS, D_OUT), dtype=torch.bfloat16, device="cuda"),
        "dX": torch.empty((TOKENS, D_IN), dtype=torch.float32, device="cuda"),
        "dW": torch.empty((D_OUT, D_IN), dtype=torch.float32, device="cuda"),
        "Ymx": torch.empty((TOKENS, D_OUT), dtype=torch.bfloat16, device="cuda"),
    }
    Q = fp4.QTensor
    NV, MX = fp4.FP4_NVFP4, fp4.FP4_MXFP4
    q = {
        "X": Q(TOKENS, D_IN, NV), "W": Q(D_OUT, D_IN, NV),
        "dY": Q(TOKENS, D_OUT, NV), "Wt": Q(D_IN, D_OUT, NV),
        "dYt": Q(D_OUT, TOKENS, NV), "Xt": Q(D_IN, TOKENS, NV),
        "mX": Q(TOKENS, D_IN, MX, had_signs=signs), "mW": Q(D_OUT, D_IN, MX, had_signs=signs),
    }
    # transposed quantizations reuse the tensor amax of the same tensor
    q["Wt"].amax = q["W"].amax
    q["dYt"].amax = q["dY"].amax
    q["Xt"].amax = q["X"].amax
    COLS, ROWS, RTN, SR = fp4.FP4_AXIS_COLS, fp4.FP4_AXIS_ROWS, fp4.FP4_RTN, fp4.FP4_SR
    seed = lambda role: (2 << 8) | role
    ws = {"fwd": gemm_workspace(fp4, q["X"], q["W"]), "dgrad": gemm_workspace(fp4, q["dY"], q["Wt"]),
          "wgrad": gemm_workspace(fp4, q["dYt"], q["Xt"]), "mx": gemm_workspace(fp4, q["mX"], q["mW"])}

    mx_ops = [
        ("quant X mx had", "q", lambda: fp4.fp4_quantize(X, COLS, RTN, 0, 0, False, q["mX"]),
         algorithmic_bytes(TOKENS * D_IN, 2, 32, False)),
        ("quant W mx had", "q", lambda: fp4.fp4_quantize(W, COLS, RTN, 0, 0, False, q["mW"]),
         algorithmic_bytes(D_OUT * D_IN, 2, 32, False)),
        ("gemm fwd mx", "g_mx", lambda: fp4.fp4_gemm(q["mX"], q["mW"], outs["Ymx"], ws["mx"]), GEMM_FLOP),
    ]
    if not separate:
        dual = lambda src, rc, sc, rr, sr, qc, qr: fp4.fp4_quantize_dual(src, rc, sc, 0, rr, sr, 0, False, qc, qr)
        ops = [
            ("quant X nv dual (rtn K, sr tokens)", "q",
             lambda: dual(X, RTN, 0, SR, seed(3), q["X"], q["Xt"]),
             algorithmic_bytes(TOKENS * D_IN, 2, 16, True, 2)),
            ("quant W nv dual (rtn K, sr out)", "q",
             lambda: dual(W, RTN, 0, SR, seed(4), q["W"], q["Wt"]),
             algorithmic_bytes(D_OUT * D_IN, 2, 16, True, 2)),
            ("gemm fwd nv", "g_nv", lambda: fp4.fp4_gemm(q["X"], q["W"], outs["Y"], ws["fwd"]), GEMM_FLOP),
            ("quant dY nv dual (sr both)", "q",
             lambda: dual(dY, SR, seed(1), SR, seed(2), q["dY"], q["dYt"]),
             algorithmic_bytes(TOKENS * D_OUT, 2, 16, True, 2)),
            ("gemm dgrad nv", "g_nv", lambda: fp4.fp4_gemm(q["dY"], q["Wt"], outs["dX"], ws["dgrad"]), GEMM_FLOP),
            ("gemm wgrad nv", "g_nv", lambda: fp4.fp4_gemm(q["dYt"], q["Xt"], outs["dW"], ws["wgrad"]), GEMM_FLOP),
        ] + mx_ops
        return ops, outs, q

    # (name, kind, callable, algorithmic units)
    ops = [
        ("quant X nv rtn", "q", lambda: fp4.fp4_quantize(X, COLS, RTN, 0, 0, False, q["X"]),
         algorithmic_bytes(TOKENS * D_IN, 2, 16, True)),
        ("quant W nv rtn", "q", lambda: fp4.fp4_quantize(W, COLS, RTN, 0, 0, False, q["W"]),
         algorithmic_bytes(D_OUT * D_IN, 2, 16, True)),
        ("gemm fwd nv", "g_nv", lambda: fp4.fp4_gemm(q["X"], q["W"], outs["Y"], ws["fwd"]), GEMM_FLOP),
        ("quant dY nv sr", "q", lambda: fp4.fp4_quantize(dY, COLS, SR, seed(1), 0, False, q["dY"]),
         algorithmic_bytes(TOKENS * D_OUT, 2, 16, True)),
        ("quant W^T nv sr", "q", lambda: fp4.fp4_quantize(W, ROWS, SR, seed(4), 0, True, q["Wt"]),
         algorithmic_bytes(D_OUT * D_IN, 2, 16, False)),
        ("gemm dgrad nv", "g_nv", lambda: fp4.fp4_gemm(q["dY"], q["Wt"], outs["dX"], ws["dgrad"]), GEMM_FLOP),
        ("quant dY^T nv sr", "q", lambda: fp4.fp4_quantize(dY, ROWS, SR, seed(2), 0, True, q["dYt"]),
         algorithmic_bytes(TOKENS * D_OUT, 2, 16, False)),
        ("quant X^T nv sr", "q", lambda: fp4.fp4_quantize(X, ROWS, SR, seed(3), 0, True, q["Xt"]),
         algorithmic_bytes(TOKENS * D_IN, 2, 16, False)),
        ("gemm wgrad nv", "g_nv", lambda: fp4.fp4_gemm(q["dYt"], q["Xt"], outs["dW"], ws["wgrad"]), GEMM_FLOP),
    ] + mx_ops
    return ops, outs, q


def make_extras(fp4, X, W, dY, signs16):
    """Adjacent passes timed beside the step (not part of it): the NVFP4
    quantizations of the wgrad operands with the 16-wide random-sign Hadamard
    along the tokens (with a rotation on one orientation the two orientations
    have their own tensor amax, the plain one and the rotated one, both taken
    in one read of the tensor before the dual pass); dY's dual SR pass with
    the gradient-noise monitor on both orientations; the two-dimensional
    (16 x 16) quantization of W that serves the forward GEMM and dgrad."""
    Q = fp4.QTensor
    NV = fp4.FP4_NVFP4
    COLS, ROWS, RTN, SR = fp4.FP4_AXIS_COLS, fp4.FP4_AXIS_ROWS, fp4.FP4_RTN, fp4.FP4_SR
    seed = lambda role: (2 << 8) | role
    import torch

    q = {
        "X": Q(TOKENS, D_IN, NV), "Xt": Q(D_IN, TOKENS, NV, had_signs=signs16),
        "dY": Q(TOKENS, D_OUT, NV), "dYt": Q(D_OUT, TOKENS, NV, had_signs=signs16),
        "dYm": Q(TOKENS, D_OUT, NV), "dYmt": Q(D_OUT, TOKENS, NV),
        "W2": Q(D_OUT, D_IN, NV), "W2t": Q(D_IN, D_OUT, NV),
    }
    q["W2t"].amax = q["W2"].amax
    q["dYmt"].amax = q["dYm"].amax
    noise = torch.zeros(4, dtype=torch.float64, device="cuda")
    dual = lambda src, rc, sc, rr, sr, qc, qr: fp4.fp4_quantize_dual(src, rc, sc, 0, rr, sr, 0, False, qc, qr)
    ops = [
        ("amax dY had16 tokens", "q", lambda: fp4.fp4_tensor_amax_hadamard16(dY, ROWS, signs16, q["dYt"].amax),
         TOKENS * D_OUT * 2.0),
        ("quant X nv dual (rtn K, sr+had16 tokens)", "q",
         lambda: dual(X, RTN, 0, SR, seed(3), q["X"], q["Xt"]),
         algorithmic_bytes(TOKENS * D_IN, 2, 16, True, 2)),
        ("quant dY nv dual (sr K, sr+had16 tokens)", "q",
         lambda: dual(dY, SR, seed(1), SR, seed(2), q["dY"], q["dYt"]),
         algorithmic_bytes(TOKENS * D_OUT, 2, 16, True, 2)),
        ("quant W nv 2-D 16x16 (rtn, W and W^T)", "q",
         lambda: fp4.fp4_quantize_2d(W, RTN, 0, 0, False, q["W2"], q["W2t"]),
         algorithmic_bytes(D_OUT * D_IN, 2, 16, True, 2)),
        ("quant dY nv dual (sr both) + noise monitor on both", "q",
         lambda: fp4.fp4_quantize_dual_noise(dY, SR, seed(1), 0, SR, seed(2), 0, False, q["dYm"], q["dYmt"],
                                             noise[0:2], noise[2:4]),
         algorithmic_bytes(TOKENS * D_OUT, 2, 16, True, 2)),
    ]
    return ops, q


def make_large_step(fp4, X, W, dY, cfg=4, shard=None):
    """The NVFP4 step of a layer (the large layer's, or a shard's): each
    tensor's amax pass and one fused pass for both of its orientations (X, W:
    RTN along K + SR along the other axis; dY: SR along both), then the three
    GEMMs (fwd bf16 out, dgrad and wgrad fp32 out). Shapes from the tensors;
    SR seeds (cfg << 8) | role. `shard` = (row_offset, rows_total): X and dY
    are rows row_offset .. of the whole token batch, quantized with the whole
    batch's SR indices (fp4_quantize_dual_shard)."""
    import torch

    (T, I), O = X.shape, W.shape[0]
    gf = 2.0 * T * I * O
    Q = fp4.QTensor
    NV = fp4.FP4_NVFP4
    RTN, SR = fp4.FP4_RTN, fp4.FP4_SR
    seed = lambda role: (cfg << 8) | role
    q = {"X": Q(T, I, NV), "Xt": Q(I, T, NV), "W": Q(O, I, NV), "Wt": Q(I, O, NV),
         "dY": Q(T, O, NV), "dYt": Q(O, T, NV)}
    for a, b in (("Xt", "X"), ("Wt", "W"), ("dYt", "dY")):
        q[a].amax = q[b].amax
    outs = {"Y": torch.empty((T, O), dtype=torch.bfloat16, device="cuda"),
            "dX": torch.empty((T, I), dtype=torch.float32, device="cuda"),
            "dW": torch.empty((O, I), dtype=torch.float32, device="cuda")}
    ws = {"fwd": gemm_workspace(fp4, q["X"], q["W"]), "dgrad": gemm_workspace(fp4, q["dY"], q["Wt"]),
          "wgrad": gemm_workspace(fp4, q["dYt"], q["Xt"])}
    dual = lambda src, rc, sc, rr, sr, qc, qr: fp4.fp4_quantize_dual(src, rc, sc, 0, rr, sr, 0, False, qc, qr)
    tok = dual
    if shard is not None:
        tok = lambda src, rc, sc, rr, sr, qc, qr: fp4.fp4_quantize_dual_shard(src, *shard, rc, sc, 0, rr, sr, 0,
                                                                              False, qc, qr)
    ops = [
        ("quant X nv dual (rtn K, sr tokens)", "q", lambda: tok(X, RTN, 0, SR, seed(3), q["X"], q["Xt"]),
         algorithmic_bytes(T * I, 2, 16, True, 2)),
        ("quant W nv dual (rtn K, sr out)", "q", lambda: dual(W, RTN, 0, SR, seed(4), q["W"], q["Wt"]),
         algorithmic_bytes(O * I, 2, 16, True, 2)),
        ("gemm fwd nv", "g_nv", lambda: fp4.fp4_gemm(q["X"], q["W"], outs["Y"], ws["fwd"]), gf),
        ("quant dY nv dual (sr both)", "q", lambda: tok(dY, SR, seed(1), SR, seed(2), q["dY"], q["dYt"]),
         algorithmic_bytes(T * O, 2, 16, True, 2)),
        ("gemm dgrad nv", "g_nv", lambda: fp4.fp4_gemm(q["dY"], q["Wt"], outs["dX"], ws["dgrad"]), gf),
        ("gemm wgrad nv", "g_nv", lambda: fp4.fp4_gemm(q["dYt"], q["Xt"], outs["dW"], ws["wgrad"]), gf),
    ]
    return ops, outs, q


def run_step(ops, steps, warmup):
    """Time `steps` passes of the op list after `warmup` untimed ones: the
    wall-clock step time between two synchronizations, and each op's HIP-event
    times on the current stream."""
    import torch

    for _ in range(warmup):
        for _, _, fn, _ in ops:
            fn()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in ops] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(steps):
        for i, (_, _, fn, _) in enumerate(ops):
            ev[s][i][0].record()
            fn()
            ev[s][i][1].record()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    per_op = [op_record(name, kind, units, [ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)])
              for i, (name, kind, _, units) in enumerate(ops)]
    return ms_per_step, per_op


def large_step_record(fp4, steps, warmup):
    """Time the large layer's step (hidden 8192, MLP 28672, 16384 tokens)."""
    import torch

    from fp4_fully_quantized_amd import workloads

    X = workloads.device_tensor("large", "X")
    W = workloads.device_tensor("large", "W")
    dY = workloads.device_tensor("large", "dY")
    rec = nv_step_record(fp4, X, W, dY, 4, steps, warmup)
    del X, W, dY
    torch.cuda.empty_cache()
    return {
        "workload": ("large-layer step: hidden 8192, MLP 28672, 16384 tokens; NVFP4 amax + one fused "
                     "quantize pass per tensor (RTN fwd, SR bwd), fwd (bf16 out), dgrad and wgrad (fp32 out)"),
        **rec,
        "targets": {
            "quantize_ms": 1.067,     # 5976.9 MB of separate passes at 70% of 8 TB/s
            "gemm_nv_ms_at_60pct_f16_peak": 5.097,
            "gemm_ms_at_60pct_fp4_peak": 1.274,
        },
    }


def shard_step_record(fp4, X, W, dY, row_offset, steps, warmup):
    """Time the NVFP4 step on one GPU's share of 8-way data parallelism over
    the Llama-7B layer's tokens (rows row_offset .. of X and dY, W whole; SR
    indices those of the whole batch)."""
    import torch

    rec = nv_step_record(fp4, X, W, dY, 5, steps, warmup, shard=(row_offset, TOKENS))
    torch.cuda.empty_cache()
    return {
        "workload": (f"one GPU's share of 8-way data parallelism over the Llama-7B layer: {X.shape[0]} "
                     f"tokens, X [{X.shape[0]}, {X.shape[1]}], W [{W.shape[0]}, {W.shape[1]}], dY "
                     f"[{dY.shape[0]}, {dY.shape[1]}] (tokens {row_offset} .. {row_offset + X.shape[0] - 1} of "
                     f"{TOKENS}); NVFP4 amax + one fused quantize pass per tensor (RTN fwd, SR bwd; X and dY "
                     "with the whole batch's SR indices), fwd (bf16 out), dgrad and wgrad (fp32 out); the "
                     "tensor amaxes would be "
                     "all-reduced (4 bytes each) and dW all-reduced across the 8 GPUs, not done here"),
        **rec,
    }


def nv_step_record(fp4, X, W, dY, cfg, steps, warmup, shard=None):
    import torch

    ops, outs, q = make_large_step(fp4, X, W, dY, cfg, shard)
    torch.cuda.synchronize()
    ms, per_op = run_step(ops, steps, warmup)
    gemms = [r for r, o in zip(per_op, ops) if o[1] == "g_nv"]
    quant = [(r, o) for r, o in zip(per_op, ops) if o[1] == "q"]
    q_ms = sum(r["avg_ms"] for r, _ in quant)
    q_bytes = sum(o[3] for _, o in quant)
    gf = 2.0 * X.shape[0] * X.shape[1] * W.shape[0]
    del ops, outs, q
    return {
        "ms_per_step": round(ms, 3),
        "TFLOPs": round(3 * gf / (ms * 1e-3) / 1e12, 1),
        "gemm_avg_ms": round(sum(r["avg_ms"] for r in gemms) / len(gemms), 4),
        "gemm_frac_f16_peak": round(sum(r["frac_f16_peak"] for r in gemms) / len(gemms), 4),
        "gemm_frac_fp4_peak": round(sum(r["frac_fp4_peak"] for r in gemms) / len(gemms), 4),
        "quantize_ms": round(q_ms, 4),
        "quantize_GBps": round(q_bytes / (q_ms * 1e-3) / 1e9, 1),
        "quantize_frac_hbm": round(q_bytes / (q_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 3),
        "per_op": per_op,
    }


def measure_ceilings(steps: int = 10):
    """What the chip reaches on this machine: the two MFMA instructions in tight
    loops (every SIMD busy, four changing operand sets, eight independent
    accumulators per wave) and streaming passes over 2 GiB buffers, each at
    the best of a few grid sizes."""
    import ctypes

    import torch

    from fp4_fully_quantized_amd import build as fp4_build

    if not os.path.exists(fp4_build.MEASURE_LIB):
        raise RuntimeError(f"{fp4_build.MEASURE_LIB} is not built; run python -m fp4_fully_quantized_amd.build")
    L = ctypes.CDLL(fp4_build.MEASURE_LIB)
    c = ctypes
    for fn in ("fp4m_mfma_f16", "fp4m_mfma_fp4"):
        getattr(L, fn).argtypes = [c.c_void_p, c.c_void_p, c.c_int, c.c_int, c.c_void_p]
    L.fp4m_stream_read.argtypes = [c.c_void_p, c.c_uint64, c.c_void_p, c.c_int, c.c_void_p]
    for fn in ("fp4m_stream_copy", "fp4m_stream_read4_write1"):
        getattr(L, fn).argtypes = [c.c_void_p, c.c_void_p, c.c_uint64, c.c_int, c.c_void_p]
    stream = c.c_void_p(torch.cuda.current_stream().cuda_stream)

    def timed(launch, reps):
        for _ in range(2):
            assert launch() == 0
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record()
            assert launch() == 0
            b.record()
        torch.cuda.synchronize()
        return sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]   # median, ms

    out = {}
    # MFMA loops. f16 operands: decoded NVFP4-like values (e2m1 x E4M3, exact
    # in f16); FP4 operands: random codes with unit E8M0 scales.
    g = torch.Generator(device="cuda").manual_seed(5)
    grid, iters = 1024, 4000
    sink = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
    grid_vals = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], device="cuda")
    codes = torch.randint(0, 8, (8 * 64 * 8,), generator=g, device="cuda")
    sign = torch.randint(0, 2, (8 * 64 * 8,), generator=g, device="cuda") * 2 - 1
    scl = torch.pow(2.0, torch.randint(-3, 4, (8 * 64 * 8,), generator=g, device="cuda").float()) * \
        (1 + torch.randint(0, 8, (8 * 64 * 8,), generator=g, device="cuda").float() / 8)
    ops_f16 = (grid_vals[codes] * sign * scl).to(torch.float16).contiguous()
    ops_fp4 = torch.randint(0, 256, (8 * 64 * 16,), generator=g, dtype=torch.int32, device="cuda").to(torch.uint8)
    for name, fn, ops, flop in (("mfma_f16", L.fp4m_mfma_f16, ops_f16, 32768),
                                ("mfma_fp4", L.fp4m_mfma_fp4, ops_fp4, 131072)):
        ms = timed(lambda: fn(ops.data_ptr(), sink.data_ptr(), grid, iters, stream), steps)
        out[name + "_TFLOPs"] = round(grid * 4 * iters * 8 * flop / (ms * 1e-3) / 1e12, 1)
    out["mfma_f16_frac_of_spec"] = round(out["mfma_f16_TFLOPs"] / PEAK_F16_TFLOPS, 3)
    out["mfma_fp4_frac_of_spec"] = round(out["mfma_fp4_TFLOPs"] / PEAK_FP4_TFLOPS, 3)
    del sink, ops_f16, ops_fp4
    # Streaming passes over 2 GiB (beyond the 256 MB memory-side cache).
    nbytes = 2 << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    word = torch.zeros(1, dtype=torch.int32, device="cuda")
    passes = {
        "hbm_stream_read": (lambda gr: L.fp4m_stream_read(src.data_ptr(), nbytes, word.data_ptr(), gr, stream),
                            nbytes),
        "hbm_stream_copy": (lambda gr: L.fp4m_stream_copy(src.data_ptr(), dst.data_ptr(), nbytes, gr, stream),
                            2 * nbytes),
        "hbm_stream_read4_write1": (lambda gr: L.fp4m_stream_read4_write1(src.data_ptr(), dst.data_ptr(),
                                                                          nbytes, gr, stream),
                                    nbytes + nbytes // 4),
    }
    for name, (launch, moved) in passes.items():
        best = None
        for gr in (1024, 2048, 4096, 8192, 16384):
            ms = timed(lambda: launch(gr), steps)
            gbps = moved / (ms * 1e-3) / 1e9
            if best is None or gbps > best[0]:
                best = (gbps, gr)
        out[name + "_GBps"] = round(best[0], 1)
        out[name + "_grid"] = best[1]
    out["hbm_best_frac_of_spec"] = round(max(out[k + "_GBps"] for k in passes) / PEAK_HBM_GBS, 3)
    del src, dst
    torch.cuda.empty_cache()
    return out


def time_ops(ops, steps, warmup, flush=None):
    """Per-op records (HIP events around each call on the current stream).
    With `flush` (a device buffer larger than the 256 MB last-level cache),
    each timed call is preceded by a read of that buffer, so the call finds
    none of its input in L2 or the memory-side cache."""
    import torch

    for _ in range(warmup):
        for _, _, fn, _ in ops:
            fn()
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in ops] for _ in range(steps)]
    torch.cuda.synchronize()
    for s in range(steps):
        for i, (_, _, fn, _) in enumerate(ops):
            if flush is not None:
                flush.sum()
            ev[s][i][0].record()
            fn()
            ev[s][i][1].record()
    torch.cuda.synchronize()
    return [op_record(name, kind, units, [ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(steps)])
            for i, (name, kind, _, units) in enumerate(ops)]


def measure_copy_GBps(steps: int = 10) -> float:
    """Device-to-device copy of 1 GiB with the runtime's own copy (one read
    and one write of every byte): what a plain streaming pass reaches on this
    GPU, the practical ceiling beside the 8 TB/s data-sheet figure."""
    import torch

    n = 1 << 29                                  # bf16 elements: 1 GiB
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    for a, b in ev:
        a.record()
        dst.copy_(src)
        b.record()
    torch.cuda.synchronize()
    avg_ms = sum(a.elapsed_time(b) for a, b in ev) / steps
    del src, dst
    return 2.0 * n * 2 / (avg_ms * 1e-3) / 1e9


def add_copy_frac(records, copy_gbps):
    for r in records:
        if "GBps" in r:
            r["frac_copy"] = round(r["GBps"] / copy_gbps, 3)


def op_record(name, kind, units, times_ms):
    ms = sorted(times_ms)
    avg = sum(ms) / len(ms)
    rec = {"op": name, "avg_ms": round(avg, 4), "median_ms": round(ms[len(ms) // 2], 4)}
    if kind == "q":
        rec["GBps"] = round(units / (avg * 1e-3) / 1e9, 1)
        rec["frac_hbm"] = round(rec["GBps"] / PEAK_HBM_GBS, 3)
    else:
        tf = units / (avg * 1e-3) / 1e12
        rec["TFLOPs"] = round(tf, 1)
        rec["frac_f16_peak" if kind == "g_nv" else "frac_fp4_peak"] = round(
            tf / (PEAK_F16_TFLOPS if kind == "g_nv" else PEAK_FP4_TFLOPS), 3)
        if kind == "g_nv":
            rec["frac_fp4_peak"] = round(tf / PEAK_FP4_TFLOPS, 3)
    return rec


def to_host_bits(t):
    """A bf16 device tensor as numpy uint16 bit patterns on the host."""
    import numpy as np
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(host):
    """The oracle on the host cores: every quantization pass of the step at
    full size on the step's own tensors (host copies), and every GEMM
    reference on a bounded sample of output rows scaled linearly to the full
    step, reported in the bench's unit."""
    import numpy as np

    from oracle import oracle as orc

    orc.lib()
    X, W, dY = host["X"], host["W"], host["dY"]
    t_quant = 0.0
    sg = orc.hadamard_signs(3)
    passes = [
        (X, dict(fmt=0)), (X, dict(axis=1, fmt=0, rnd=1, seed=(2 << 8) | 3)),
        (W, dict(fmt=0)), (W, dict(axis=1, fmt=0, rnd=1, seed=(2 << 8) | 4)),
        (dY, dict(fmt=0, rnd=1, seed=(2 << 8) | 1)), (dY, dict(axis=1, fmt=0, rnd=1, seed=(2 << 8) | 2)),
        (X, dict(fmt=1, had_on=True, had_signs=sg)), (W, dict(fmt=1, had_on=True, had_signs=sg)),
    ]
    for src, kw in passes:
        t0 = time.perf_counter()
        orc.quantize(src, **kw)
        t_quant += time.perf_counter() - t0
    # GEMM references (the oracle's gemm_ref: dequantize both operands exactly
    # to FP64, then the FP64 products A B^T and |A| |B|^T), on rows_g output
    # rows x up to 1024 columns, timed step by step so that B's dequantization
    # counts once per GEMM and the products scale with the full output size.
    rows_g = 512
    t_gemm = 0.0
    rng = np.random.default_rng(0)
    for M, N, K in [(TOKENS, D_OUT, D_IN), (TOKENS, D_IN, D_OUT), (D_OUT, D_IN, TOKENS),
                    (TOKENS, D_OUT, D_IN)]:
        nb = min(N, 1024)
        qa = orc.quantize(rng.standard_normal((rows_g, K)).astype(np.float32))
        qb = orc.quantize(rng.standard_normal((nb, K)).astype(np.float32))
        t0 = time.perf_counter()
        A = orc.dequantize_f64(qa)
        t1 = time.perf_counter()
        Bm = orc.dequantize_f64(qb)
        t2 = time.perf_counter()
        _ = A @ Bm.T
        _ = np.abs(A) @ np.abs(Bm).T
        t3 = time.perf_counter()
        t_gemm += (t1 - t0) * (M / rows_g) + (t2 - t1) * (N / nb) + (t3 - t2) * (M / rows_g) * (N / nb)
    t_step = t_quant + t_gemm
    flops = 4 * GEMM_FLOP
    return {
        "value": flops / t_step / 1e12,
        "unit": "TFLOP/s",
        "cores": orc.num_threads(),
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": (f"every quantization pass of the Llama-7B step at full size on the step's own tensors "
                   f"({t_quant:.1f} s measured), and every GEMM reference on {rows_g} output rows x up to 1024 "
                   f"columns scaled linearly to the full outputs ({t_gemm:.1f} s extrapolated); step "
                   f"{t_step:.1f} s"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-large-step", action="store_true",
                    help="skip the large layer's step (timed after the Llama-7B step)")
    ap.add_argument("--no-shard-step", action="store_true",
                    help="skip the 8-way data-parallel shard's step (timed after the large layer's)")
    ap.add_argument("--separate-passes", action="store_true",
                    help="quantize each orientation with its own pass instead of one read per tensor")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the FP4 quantize + GEMM path is built and timed on a "
              "single MI355X (multi-GPU sharding is a design note only); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import fp4_fully_quantized_amd as fp4
    from fp4_fully_quantized_amd import workloads

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    fp4.lib()
    torch.manual_seed(0)
    X = workloads.device_tensor("llama7b", "X")
    W = workloads.device_tensor("llama7b", "W")
    dY = workloads.device_tensor("llama7b", "dY")
    signs = fp4.fp4_hadamard_signs(3)
    ops, outs, q = make_step(fp4, X, W, dY, signs, separate=args.separate_passes)
    torch.cuda.synchronize()

    ms_per_step, per_op = run_step(ops, args.steps, args.warmup)

    # Adjacent passes, timed after the step's timed region.
    extra_ops, extra_q = make_extras(fp4, X, W, dY, fp4.fp4_hadamard_signs(4))
    extras = time_ops(extra_ops, args.steps, 2)
    del extra_ops, extra_q
    # The step's quantize calls again, each after a 1 GiB read that evicts the
    # caches (in the step, a tensor's second read -- the amax pass, then the
    # quantize pass -- can hit the 256 MB memory-side cache).
    flush = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    cold = time_ops([o for o in ops if o[1] == "q"], args.steps, 2, flush=flush)
    del flush
    copy_gbps = measure_copy_GBps()
    for recs in (per_op, extras, cold):
        add_copy_frac(recs, copy_gbps)

    nv = [r for r, o in zip(per_op, ops) if o[1] == "g_nv"]
    nv_avg_ms = sum(r["avg_ms"] for r in nv) / len(nv)
    achieved = GEMM_FLOP / (nv_avg_ms * 1e-3) / 1e12
    step_flop = 4 * GEMM_FLOP
    quant_bytes = sum(o[3] for o in ops if o[1] == "q")
    quant_ms = sum(r["avg_ms"] for r, o in zip(per_op, ops) if o[1] == "q")

    # HBM bytes per NVFP4 GEMM launch from the committed rocprofv3 counter runs,
    # valid only while the GEMM sources are the ones the counters were taken on.
    from fp4_fully_quantized_amd import profiling

    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            rec = json.load(f)
        if rec.get("source_digest") == profiling.source_digest():
            traffic = rec.get("nv_gemm_bytes_per_launch")

    out = {
        "metric": "FP4 quantize GB/s + FP4 GEMM TFLOPS (fwd/dgrad/wgrad), % of MI355X roofline",
        "value": round(step_flop / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4",
        "data": "synthetic",
        "config": {
            "workload": ("Llama-7B-shaped linear layer step: NVFP4 fwd + bwd (RTN fwd, SR bwd, "
                         "transposed quantization) and MXFP4+Hadamard fwd"),
            "tokens": TOKENS, "in_features": D_IN, "out_features": D_OUT,
            "gemms_per_step": 4, "quantizations_per_step": 8,
            "quantize_launches": ("separate passes: an amax pass and one quantize pass per orientation"
                                  if args.separate_passes else
                                  "per NVFP4 tensor: an amax pass, then one pass that quantizes both "
                                  "orientations (two reads of the tensor)"),
        },
        "quantize_GBps_aggregate": round(quant_bytes / (quant_ms * 1e-3) / 1e9, 1),
        "hbm_copy_GBps": round(copy_gbps, 1),
        "per_op": per_op,
        "per_op_cold": cold,
        "extras": extras,
        "roofline": {
            "kernel": "NVFP4 GEMM (e2m1*E4M3 decoded exactly to f16, f16 MFMA)",
            "bound": "mfma",
            "achieved": round(achieved, 1),
            "peak": PEAK_F16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_F16_TFLOPS, 4),
            "traffic": traffic,
        },
    }
    # The chip's measured ceilings, then the large layer's step.
    ceilings = measure_ceilings()
    ceilings["rocclr_copy_GBps"] = round(copy_gbps, 1)
    out["measured_ceilings"] = ceilings
    out["roofline"]["measured_peak"] = ceilings["mfma_f16_TFLOPs"]
    out["roofline"]["frac_of_measured_peak"] = round(achieved / ceilings["mfma_f16_TFLOPs"], 4)
    stream_q = ceilings["hbm_stream_read4_write1_GBps"]
    for recs in (per_op, extras, cold):
        for r in recs:
            if "GBps" in r:
                r["frac_stream"] = round(r["GBps"] / stream_q, 3)
    host = None
    if not args.no_cpu_baseline:
        host = {k: to_host_bits(v) for k, v in (("X", X), ("W", W), ("dY", dY))}
    shard = None
    if not args.no_shard_step:
        r0 = SHARD_RANK * SHARD_TOKENS
        shard = (X[r0:r0 + SHARD_TOKENS].clone(), W, dY[r0:r0 + SHARD_TOKENS].clone(), r0)
    del X, W, dY, ops, outs, q
    torch.cuda.empty_cache()
    if not args.no_large_step:
        out["large_step"] = large_step_record(fp4, args.steps, args.warmup)
    if shard is not None:
        out["dp8_shard_step"] = shard_step_record(fp4, *shard, args.steps, args.warmup)
        del shard
        torch.cuda.empty_cache()
    if host is not None:
        out["cpu_baseline"] = cpu_baseline(host)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
