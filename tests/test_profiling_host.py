"""Host-side checks of the profiling summaries: the labelling of a benchmark
run's dispatches, which every per-kernel counter table rests on."""
import json

import pytest

from fp4_fully_quantized_amd import profiling as p


def _names(steps, warmup):
    # Kernel short names as a benchmark run launches them (GEMMs included),
    # written out independently of the tables under test.
    step = ["k_amax<true, false>", "k_quant_dual<0, 0, 1, true, false, false, false>",
            "k_amax<true, false>", "k_quant_dual<0, 0, 1, true, false, false, false>",
            "k_gemm<0, 256, true, false>",
            "k_amax<true, false>", "k_quant_dual<0, 1, 1, true, false, false, false>",
            "k_gemm<0, 256, false, false>", "k_gemm<0, 256, false, false>",
            "k_quant_cols<1, 0, true, true, false>", "k_quant_cols<1, 0, true, true, false>",
            "k_gemm_mx8<true>"]
    extras = ["k_amax_rot_rows<true>", "k_amax_pair<true, false, true>",
              "k_quant_dual<0, 0, 1, true, false, true, false>", "k_amax_pair<true, false, true>",
              "k_quant_dual<0, 1, 1, true, false, true, false>", "k_amax<true, false>",
              "k_quant_2d<0, 0, true>", "k_amax<true, false>",
              "k_quant_dual_w4<0, 1, 1, true, false, false, true>"]
    cold = [n for n in step if not n.startswith("k_gemm")]
    return step * (warmup + steps) + extras * (2 + steps) + cold * (2 + steps)


def test_label_dispatches_accepts_a_benchmark_run():
    labels = p.label_dispatches(_names(1, 1), 1, 1)
    assert len(labels) == 2 * 12 + 3 * 9 + 3 * 8
    assert labels[0][0] == "amax X" and labels[4][0].startswith("NVFP4 GEMM fwd")
    assert labels[-1][0] == "MXFP4+Hadamard W (cold)"
    # algorithmic bytes: dual pass over X reads bf16 once, writes two orientations
    x_dual = [u for l, u, _ in labels if l.startswith("dual X (RTN")][0]
    assert x_dual == 32768 * 4096 * (2 + 2 * (0.5 + 1 / 16))
    # element-orientation counts: 2 for dual passes, 1 for amax and MXFP4 passes, 0 for GEMMs
    d = {l: e for l, _, e in labels}
    assert d["dual dY (SR both)"] == 2 * 32768 * 11008
    assert d["amax W"] == 11008 * 4096 and d["MXFP4+Hadamard X"] == 32768 * 4096
    assert d["NVFP4 GEMM wgrad (fp32 out)"] == 0


def test_label_dispatches_rejects_a_changed_run():
    names = _names(1, 1)
    with pytest.raises(ValueError):
        p.label_dispatches(names[:-1], 1, 1)
    swapped = list(names)
    swapped[0], swapped[1] = swapped[1], swapped[0]
    with pytest.raises(ValueError):
        p.label_dispatches(swapped, 1, 1)


def _write_csv(path, header, rows):
    import csv
    import os
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def _raw(name):
    # as rocprofv3 prints it
    return f"void (anonymous namespace)::{name}(void const*, long)"


def test_summarize_on_synthetic_counters(tmp_path):
    """summarize() on made-up counter files whose figures are known: every
    quantize dispatch moves exactly its algorithmic bytes (ratio 1.000 after
    the copy calibration), every dispatch runs at 2 GHz with the MFMA pipe half
    busy and VALU issuing a quarter of the time."""
    out, prof = tmp_path / "out", tmp_path / "profiles"
    prof.mkdir()
    names = _names(p.PMC_STEPS, p.PMC_WARMUP)
    labels = p.label_dispatches(names, p.PMC_STEPS, p.PMC_WARMUP)
    ph = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value", "Start_Timestamp",
          "End_Timestamp"]
    fetch, write, util = [], [], []
    cyc, dur = 2_000_000, 1_000_000          # cycles per XCD over 1 ms: 2 GHz
    for i, (n, (_, units, elems)) in enumerate(zip(names, labels)):
        t0 = 10_000_000 * (i + 1)
        row = lambda c, v: [i + 1, _raw(n), 1024, c, v, t0, t0 + dur]
        fetch.append(row("FETCH_SIZE", units * 0.6 / 2048))      # read bytes / 1024 / factor 2
        write.append(row("WRITE_SIZE", units * 0.4 / 1024))      # written bytes / 1024 / factor 1
        util += [row("GRBM_GUI_ACTIVE", 8 * cyc), row("SQ_VALU_MFMA_BUSY_CYCLES", 0.5 * 1024 * cyc),
                 row("SQ_ACTIVE_INST_VALU", 0.25 * 1024 * cyc / 4), row("SQ_INSTS_VALU", 1000.0),
                 row("SQ_INSTS_MFMA", 100.0)]
    _write_csv(str(out / "pmc_fetch" / "bench_counter_collection.csv"), ph, fetch)
    _write_csv(str(out / "pmc_write" / "bench_counter_collection.csv"), ph, write)
    _write_csv(str(out / "pmc_util" / "bench_counter_collection.csv"), ph, util)
    copy = lambda c, v: [[k + 2, "__amd_rocclr_copyBuffer", 1, c, v, 0, 1] for k in range(3)]
    _write_csv(str(out / "pmc_copy_fetch" / "copy_counter_collection.csv"), ph,
               [[1, "fill", 1, "FETCH_SIZE", 7.0, 0, 1]] + copy("FETCH_SIZE", (1 << 30) / 1024 / 2))
    _write_csv(str(out / "pmc_copy_write" / "copy_counter_collection.csv"), ph, copy("WRITE_SIZE", (1 << 30) / 1024))
    trace = [[_raw(n), 0, 1000 * (k + 1)] for k, n in enumerate(_names(p.STEPS, p.WARMUP))]
    _write_csv(str(out / "prof_bench" / "bench_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp",
                                                                    "End_Timestamp"], trace)
    _write_csv(str(out / "prof_bench" / "bench_kernel_stats.csv"),
               ["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"],
               [[_raw("k_gemm<0, 256, true, false>"), 13, 2e6, 1.9e6, 2.1e6, 30.0]])
    p.summarize(str(out), str(prof))

    q = (prof / "quantize_llama7b_hbm_traffic.md").read_text()
    rows = [l for l in q.splitlines() if l.startswith("| ") and not l.startswith("| dispatch")]
    assert len(rows) == 8 + 9 + 8 and all(l.rstrip(" |").endswith("1.000") for l in rows)
    u = 32768 * 11008 * (2 + 2 * (0.5 + 1 / 16))   # bf16 read + two orientations written
    assert f"| dual dY (SR both) | 2 | {0.6 * u / 1e6:.1f} | {0.4 * u / 1e6:.1f} | {u / 1e6:.1f} | {u / 1e6:.1f} | 1.000 |" in q
    u = (prof / "llama7b_step_mfma_valu_utilisation.md").read_text()
    assert "| NVFP4 GEMM fwd (bf16 out) | 2 | 1000.0 | 2.00 | 0.500 | 0.250 | 10.00 |" in u
    t = json.loads((prof / "traffic.json").read_text())
    assert t["fetch_factor"] == 2.0 and t["write_factor"] == 1.0
    assert t["nv_gemm_bytes_per_launch"] == round(p._GF * 1.0)


def _large_names(steps, warmup):
    step = ["k_amax<true, false>", "k_quant_dual<0, 0, 1, true, false, false, false>",
            "k_amax<true, false>", "k_quant_dual<0, 0, 1, true, false, false, false>",
            "k_gemm<0, 256, true, false>",
            "k_amax<true, false>", "k_quant_dual<0, 1, 1, true, false, false, false>",
            "k_gemm<0, 256, false, false>", "k_gemm<0, 256, false, false>"]
    return step * (warmup + steps)


def test_trace_split_into_llama_ceilings_and_large_step(tmp_path):
    """The kernel trace of a full benchmark run: the Llama-7B part, the ceiling
    measurements, then the large layer's step, each summarized on its own
    (durations chosen so each group's timed average is known)."""
    ceil = ["k_mfma_f16", "k_mfma_fp4"] + ["k_stream_read", "k_stream_copy", "k_stream_read4_write1"]
    names = _names(p.STEPS, p.WARMUP) + ["__amd_rocclr_copyBuffer"] + ceil + ["fill"] + \
        _large_names(p.STEPS, p.WARMUP)
    dur = {"k_gemm<0, 256, true, false>": 5_000_000, "k_gemm<0, 256, false, false>": 6_000_000}
    trace, t = [], 0
    n_large = len(_large_names(p.STEPS, p.WARMUP))
    first_large = len(names) - n_large
    for k, n in enumerate(names):
        d = dur.get(n, 100_000) if k >= first_large else 1000
        if k >= first_large and n == "k_gemm<0, 256, false, false>":
            d = 6_000_000 if (k - first_large) % 9 == 7 else 7_000_000   # dgrad, then wgrad
        trace.append([_raw(n), t, t + d])
        t += d + 10
    out = tmp_path / "out" / "prof_bench"
    _write_csv(str(out / "bench_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    llama, ce, large = p._trace_parts(str(out / "bench_kernel_trace.csv"))
    assert [n for n, _ in ce] == ceil
    # the large part also holds the generation of its inputs ("fill")
    assert len(large) == n_large + 1 and len(llama) == len(_names(p.STEPS, p.WARMUP)) + 1
    prof = tmp_path / "profiles"
    prof.mkdir()
    p._write_large_step(large, "CMD", str(prof))
    text = (prof / "large_layer_step_kernel_stats.md").read_text()
    assert "| NVFP4 GEMM fwd 16384x28672x8192 (bf16 out) | 13 | 5000.0 | 5000.0 |" in text
    assert "| NVFP4 GEMM dgrad 16384x8192x28672 (fp32 out) | 13 | 6000.0 | 6000.0 |" in text
    assert "| NVFP4 GEMM wgrad 28672x8192x16384 (fp32 out) | 13 | 7000.0 | 7000.0 |" in text
    assert "| tensor amax (X, W, dY) | 39 | 100.0 |" in text
    p._write_ceilings(ce, "CMD", str(prof))
    assert "| f16 MFMA loop" in (prof / "chip_ceilings_kernel_stats.md").read_text()


def test_trace_tail_split_into_large_and_shard_steps(tmp_path):
    """After the ceilings: the large layer's step (9 library dispatches a
    step), then the data-parallel shard's step; each gets its own table."""
    large = _large_names(p.STEPS, p.WARMUP)
    tail = ["fill"] + large + ["copy", "copy"] + large
    trace = []
    for k, n in enumerate(tail):
        shard = k > len(large) + 2
        d = 1000 if not n.startswith("k_gemm") else (500_000 if shard else 5_000_000)
        trace.append((n, d))
    big, shard = p._split_after_steps(trace, 9)
    assert len(big) == len(large) + 1 and len(shard) == len(large) + 2
    prof = tmp_path / "profiles"
    prof.mkdir()
    p._write_shard_step(shard, "CMD", str(prof))
    text = (prof / "dp8_shard_step_kernel_stats.md").read_text()
    assert "| NVFP4 GEMM fwd 4096x11008x4096 (bf16 out) | 13 | 500.0 | 500.0 |" in text
    assert "| NVFP4 GEMM dgrad 4096x4096x11008 (fp32 out) | 13 | 500.0 |" in text
    assert "| NVFP4 GEMM wgrad 11008x4096x4096 (fp32 out) | 13 | 500.0 |" in text
    # a run without the shard step leaves nothing after the large step
    assert p._split_after_steps(trace[:len(large) + 1], 9)[1] == []


def test_code_digest_ignores_comments_only():
    from fp4_fully_quantized_amd.profiling import code_digest
    a = "int f(int x) {\n  return x + 1;  // one more\n}\n"
    b = "/* f: the successor */\nint f(int x) {\n    return x + 1;\n}\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert code_digest([a]) == code_digest([b])
    assert code_digest([a]) != code_digest([c])
    # the files are hashed as separate texts
    assert code_digest([a, c]) != code_digest([c, a])


def test_summarize_lds_on_synthetic_counters(tmp_path):
    """summarize_lds() on made-up counters whose per-K-tile figures are known:
    every GEMM dispatch reports 1000 LDS and 64 MFMA instructions per K tile,
    2 GHz over 1 ms, and waits of a tenth (LDS) and a fifth (any) of its wave
    cycles."""
    out, prof = tmp_path / "out", tmp_path / "profiles"
    prof.mkdir()
    names = _names(p.PMC_STEPS, p.PMC_WARMUP)
    labels = p.label_dispatches(names, p.PMC_STEPS, p.PMC_WARMUP)
    units = {l: t * (k // 256) for l, k, t, _ in p._STEP_GEMMS}
    ph = ["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name", "Counter_Value", "Start_Timestamp",
          "End_Timestamp"]
    rows = []
    cyc, dur = 2_000_000, 1_000_000
    for i, (n, (l, _, _)) in enumerate(zip(names, labels)):
        u = units.get(l, 1)
        t0 = 10_000_000 * (i + 1)
        row = lambda c, v: [i + 1, _raw(n), 1024, c, v, t0, t0 + dur]
        rows += [row("GRBM_GUI_ACTIVE", 8 * cyc), row("SQ_INSTS_LDS", 1000.0 * u), row("SQ_INSTS_MFMA", 64.0 * u),
                 row("SQ_ACTIVE_INST_LDS", 400.0 * u), row("SQ_LDS_BANK_CONFLICT", 40.0 * u),
                 row("SQ_WAIT_INST_LDS", 10.0), row("SQ_WAIT_ANY", 20.0), row("SQ_WAVE_CYCLES", 100.0)]
    _write_csv(str(out / "pmc_lds" / "bench_counter_collection.csv"), ph, rows)
    p.summarize_lds(str(out), str(prof))
    t = (prof / "gemm_llama7b_lds_per_k_tile.md").read_text()
    body = [l for l in t.splitlines() if l.startswith("| ") and not l.startswith("| GEMM")]
    assert len(body) == 4
    fwd_units = 128 * 43 * 16
    assert (f"| NVFP4 GEMM fwd (bf16 out) | 2 | 1000.0 | {cyc * 256 / fwd_units:.0f} | 1000 | 64 | 400 | 40 | "
            "0.100 | 0.100 | 0.200 |") in t
    assert "| MXFP4 GEMM fwd (bf16 out) | 2 |" in t
