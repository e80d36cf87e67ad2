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

    mx_ops = [
        ("quant X mx had", "q", lambda: fp4.fp4_quantize(X, COLS, RTN, 0, 0, False, q["mX"]),
         algorithmic_bytes(TOKENS * D_IN, 2, 32, False)),
        ("quant W mx had", "q", lambda: fp4.fp4_quantize(W, COLS, RTN, 0, 0, False, q["mW"]),
         algorithmic_bytes(D_OUT * D_IN, 2, 32, False)),
        ("gemm fwd mx", "g_mx", lambda: fp4.fp4_gemm(q["mX"], q["mW"], outs["Ymx"]), GEMM_FLOP),
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
            ("gemm fwd nv", "g_nv", lambda: fp4.fp4_gemm(q["X"], q["W"], outs["Y"]), GEMM_FLOP),
            ("quant dY nv dual (sr both)", "q",
             lambda: dual(dY, SR, seed(1), SR, seed(2), q["dY"], q["dYt"]),
             algorithmic_bytes(TOKENS * D_OUT, 2, 16, True, 2)),
            ("gemm dgrad nv", "g_nv", lambda: fp4.fp4_gemm(q["dY"], q["Wt"], outs["dX"]), GEMM_FLOP),
            ("gemm wgrad nv", "g_nv", lambda: fp4.fp4_gemm(q["dYt"], q["Xt"], outs["dW"]), GEMM_FLOP),
        ] + mx_ops
        return ops, outs, q

    # (name, kind, callable, algorithmic units)
    ops = [
        ("quant X nv rtn", "q", lambda: fp4.fp4_quantize(X, COLS, RTN, 0, 0, False, q["X"]),
         algorithmic_bytes(TOKENS * D_IN, 2, 16, True)),
        ("quant W nv rtn", "q", lambda: fp4.fp4_quantize(W, COLS, RTN, 0, 0, False, q["W"]),
         algorithmic_bytes(D_OUT * D_IN, 2, 16, True)),
        ("gemm fwd nv", "g_nv", lambda: fp4.fp4_gemm(q["X"], q["W"], outs["Y"]), GEMM_FLOP),
        ("quant dY nv sr", "q", lambda: fp4.fp4_quantize(dY, COLS, SR, seed(1), 0, False, q["dY"]),
         algorithmic_bytes(TOKENS * D_OUT, 2, 16, True)),
        ("quant W^T nv sr", "q", lambda: fp4.fp4_quantize(W, ROWS, SR, seed(4), 0, True, q["Wt"]),
         algorithmic_bytes(D_OUT * D_IN, 2, 16, False)),
        ("gemm dgrad nv", "g_nv", lambda: fp4.fp4_gemm(q["dY"], q["Wt"], outs["dX"]), GEMM_FLOP),
        ("quant dY^T nv sr", "q", lambda: fp4.fp4_quantize(dY, ROWS, SR, seed(2), 0, True, q["dYt"]),
         algorithmic_bytes(TOKENS * D_OUT, 2, 16, False)),
        ("quant X^T nv sr", "q", lambda: fp4.fp4_quantize(X, ROWS, SR, seed(3), 0, True, q["Xt"]),
         algorithmic_bytes(TOKENS * D_IN, 2, 16, False)),
        ("gemm wgrad nv", "g_nv", lambda: fp4.fp4_gemm(q["dYt"], q["Xt"], outs["dW"]), GEMM_FLOP),
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


def cpu_baseline():
    """The oracle on a bounded sample of the step: every quantization pass on a
    row slab of its tensor and every GEMM reference on a few output rows, each
    scaled linearly to the full step, reported in the bench's unit."""
    import numpy as np

    from fp4_fully_quantized_amd import workloads
    from oracle import oracle as orc

    orc.lib()
    rows_q = 1024         # rows of each quantized tensor in the sample
    rows_g = 512          # output rows of each GEMM in the sample
    t_quant = 0.0
    t_gemm = 0.0
    X = workloads.host_tensor("llama7b", "X", shape=(rows_q, D_IN))
    W = workloads.host_tensor("llama7b", "W", shape=(rows_q, D_IN))
    dY = workloads.host_tensor("llama7b", "dY", shape=(rows_q, D_OUT))
    # (tensor slab, full element count of the pass, kwargs)
    passes = [
        (X, TOKENS * D_IN, dict(fmt=0)), (W, D_OUT * D_IN, dict(fmt=0)),
        (dY, TOKENS * D_OUT, dict(fmt=0, rnd=1, seed=1)),
        (W, D_OUT * D_IN, dict(axis=1, fmt=0, rnd=1, seed=4)),
        (dY, TOKENS * D_OUT, dict(axis=1, fmt=0, rnd=1, seed=2)),
        (X, TOKENS * D_IN, dict(axis=1, fmt=0, rnd=1, seed=3)),
        (X, TOKENS * D_IN, dict(fmt=1, had_on=True, had_signs=orc.hadamard_signs(3))),
        (W, D_OUT * D_IN, dict(fmt=1, had_on=True, had_signs=orc.hadamard_signs(3))),
    ]
    for slab, full, kw in passes:
        t0 = time.perf_counter()
        orc.quantize(slab, **kw)
        dt = time.perf_counter() - t0
        t_quant += dt * full / slab.size
    # GEMM references (the oracle's gemm_ref: dequantize both operands exactly
    # to FP64, then the FP64 products A B^T and |A| |B|^T), timed step by step
    # so that B's dequantization counts once per GEMM and the products scale
    # with the full output size.
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
        "sample": (f"every quantization pass of the step on a {rows_q}-row slab of its tensor "
                   f"and every GEMM reference on {rows_g} output rows x up to 1024 columns, "
                   f"each scaled linearly to the full Llama-7B step; extrapolated step "
                   f"{t_step:.1f} s (quantize {t_quant:.1f} s, FP64 GEMM {t_gemm:.1f} s)"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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

    def step(events=None):
        for i, (_, _, fn, _) in enumerate(ops):
            if events is not None:
                events[i][0].record()
            fn()
            if events is not None:
                events[i][1].record()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in ops] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(ev[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    per_op = [op_record(name, kind, units, [ev[s][i][0].elapsed_time(ev[s][i][1]) for s in range(args.steps)])
              for i, (name, kind, _, units) in enumerate(ops)]

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
            "quantize_launches": "separate" if args.separate_passes else "one read per NVFP4 tensor",
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
    if not args.no_cpu_baseline:
        del X, W, dY, ops, outs, q
        torch.cuda.empty_cache()
        out["cpu_baseline"] = cpu_baseline()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
