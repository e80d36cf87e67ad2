"""Helpers for profiling runs.

    python -m fp4_fully_quantized_amd.profiling copy

runs a plain device copy of a known size (1 GiB, bf16) a few times, so that
the HBM byte counters read for it (FETCH_SIZE, WRITE_SIZE) can calibrate the
same counters read for the library's kernels.

    python -m fp4_fully_quantized_amd.profiling summarize OUT

reads the rocprofv3 CSV output of the profiling commands listed in
PROFILE_COMMANDS (under the folder OUT) and writes the text summaries and
profiles/traffic.json that the benchmark's roofline figure reads.

    python -m fp4_fully_quantized_amd.profiling summarize-trace OUT

writes only the kernel-time summaries, from the kernel-trace run ("stats").

    python -m fp4_fully_quantized_amd.profiling summarize-lds OUT

writes only the GEMMs' LDS summary per K tile, from the "lds" counter run
(summarize includes it when that run's folder is there).
"""
import sys

COPY_BYTES = 1 << 30


def copy(reps: int = 3) -> None:
    import torch

    src = torch.empty(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {COPY_BYTES} bytes x {reps}", flush=True)


# ---------------------------------------------------------------- summaries
def short_name(name: str) -> str:
    base = name.replace("(anonymous namespace)::", "")
    if base.startswith("void "):
        base = base[5:]
    return base.split("(")[0].strip()


def kernel_stats_table(csv_path: str, top: int = 20) -> str:
    """Markdown table of a rocprofv3 --stats kernel_stats.csv."""
    import csv

    rows = list(csv.DictReader(open(csv_path)))
    out = ["| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows[:top]:
        out.append(f"| `{short_name(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.2f} |")
    return "\n".join(out)


def counter_per_dispatch(csv_path: str, counter: str, name_regex: str):
    """[(kernel short name, grid size, value)] for every dispatch of kernels whose
    name matches, from a rocprofv3 --pmc counter_collection.csv."""
    import csv
    import re

    pat = re.compile(name_regex)
    out = []
    for r in csv.DictReader(open(csv_path)):
        if r["Counter_Name"] == counter and pat.search(r["Kernel_Name"]):
            out.append((short_name(r["Kernel_Name"]), int(r["Grid_Size"]), float(r["Counter_Value"])))
    return out


def code_digest(texts) -> str:
    """Digest of C++/HIP sources with comments and whitespace removed, so that
    only a change of the code itself (not of its comments) changes it."""
    import hashlib
    import re

    h = hashlib.sha256()
    for t in texts:
        t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        h.update(" ".join(t.split()).encode())
        h.update(b"\0")
    return h.hexdigest()[:16]


def source_digest() -> str:
    """Digest of the GEMM sources' code: a traffic figure is valid for this digest only."""
    import os

    here = os.path.dirname(os.path.abspath(__file__))
    texts = []
    for fn in ("gemm.hip", "fp4_device.hpp"):
        with open(os.path.join(here, "csrc", fn)) as f:
            texts.append(f.read())
    return code_digest(texts)


# ---------------------------------------------------------------- the profile set
# The commands whose output `summarize` reads, run from the repository root on one
# MI355X after `cd /tmp && export TMPDIR=/tmp` (OUT = their output folder).
PROFILE_COMMANDS = {
    "stats": "rocprofv3 --kernel-trace --stats --output-format csv -d OUT/prof_bench -o bench -- "
             "python3 bench.py --steps 10 --warmup 3 --no-cpu-baseline",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --kernel-include-regex \"k_gemm|k_quant|k_amax\" --output-format csv "
             "-d OUT/pmc_fetch -o bench -- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline "
             "--no-large-step --no-shard-step",
    "write": "rocprofv3 --pmc WRITE_SIZE --kernel-include-regex \"k_gemm|k_quant|k_amax\" --output-format csv "
             "-d OUT/pmc_write -o bench -- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline "
             "--no-large-step --no-shard-step",
    "util": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_ACTIVE_INST_VALU SQ_INSTS_VALU SQ_INSTS_MFMA "
            "GRBM_GUI_ACTIVE --kernel-include-regex \"k_gemm|k_quant|k_amax\" --output-format csv "
            "-d OUT/pmc_util -o bench -- python3 bench.py --steps 1 --warmup 1 --no-cpu-baseline "
            "--no-large-step --no-shard-step",
    "lds": "rocprofv3 --pmc SQ_INSTS_LDS SQ_ACTIVE_INST_LDS SQ_LDS_BANK_CONFLICT SQ_WAIT_INST_LDS SQ_WAIT_ANY "
           "SQ_WAVE_CYCLES SQ_INSTS_MFMA GRBM_GUI_ACTIVE --kernel-include-regex \"k_gemm|k_quant|k_amax\" "
           "--output-format csv -d OUT/pmc_lds -o bench -- python3 bench.py --steps 1 --warmup 1 "
           "--no-cpu-baseline --no-large-step --no-shard-step",
    "copy_fetch": "rocprofv3 --pmc FETCH_SIZE --output-format csv -d OUT/pmc_copy_fetch -o copy -- "
                  "python3 -m fp4_fully_quantized_amd.profiling copy",
    "copy_write": "rocprofv3 --pmc WRITE_SIZE --output-format csv -d OUT/pmc_copy_write -o copy -- "
                  "python3 -m fp4_fully_quantized_amd.profiling copy",
}

# Kernel groups of one benchmark step, in step order: (label, name regex, bytes or
# flops per launch is computed by the benchmark itself).
GROUPS = [
    ("NVFP4 GEMM (fwd bf16 out; dgrad, wgrad fp32 out)", r"^k_gemm<0,"),
    ("MXFP4 GEMM (fwd, bf16 out)", r"^k_gemm(<1,|_mx8<)"),
    ("quantize, both orientations from one read", r"^k_quant_dual(_w4)?<"),
    ("quantize, blocks along the contiguous axis", r"^k_quant_cols<"),
    ("quantize, blocks along rows (transposed output)", r"^k_quant_rows<"),
    ("tensor amax", r"^k_amax(_flat)?<"),
    ("tensor amax of the values rotated down the columns", r"^k_amax_rot_rows<"),
    ("both orientations' amaxes, one rotated (one read)", r"^k_amax_pair<"),
    ("2-D block quantize (both orientations)", r"^k_quant_2d<"),
]
# The benchmark's on-box ceiling measurements (libfp4_measure.so), launched
# between the Llama-7B part of the run and the large layer's step.
CEILING_KERNELS = [
    ("f16 MFMA loop (v_mfma_f32_32x32x16_f16)", r"^k_mfma_f16$"),
    ("scaled FP4 MFMA loop (v_mfma_scale_f32_32x32x64_f8f6f4)", r"^k_mfma_fp4$"),
    ("streaming read", r"^k_stream_read$"),
    ("streaming copy", r"^k_stream_copy$"),
    ("streaming read 16 B / write 4 B per lane", r"^k_stream_read4_write1$"),
]
STEPS, WARMUP = 10, 3   # of the stats command
PMC_STEPS, PMC_WARMUP = 1, 1   # of the counter commands
CUS, SIMDS_PER_CU, XCDS = 256, 4, 8


# The library's dispatches in one `bench.py --steps K --warmup W` run, in launch
# order: (label, kernel-name regex, algorithmic bytes or FLOPs per dispatch,
# elements x orientations a quantize or amax dispatch processes). The
# benchmark runs the step W + K times, then the adjacent passes 2 + K times, then
# the step's quantize calls 2 + K times with the caches evicted before each.
TOKENS, D_IN, D_OUT = 32768, 4096, 11008
_NX, _NW, _NY = TOKENS * D_IN, D_OUT * D_IN, TOKENS * D_OUT
# Algorithmic bytes of each NVFP4 GEMM: both operands' codes (0.5 B) and E4M3
# scales (1/16 B) per element read once, the output written once.
_OPND = 0.5 + 1 / 16
GEMM_ALGO_BYTES = {
    "fwd": (_NX + _NW) * _OPND + TOKENS * D_OUT * 2,      # Y bf16
    "dgrad": (_NY + _NW) * _OPND + TOKENS * D_IN * 4,     # dX fp32
    "wgrad": (_NY + _NX) * _OPND + D_OUT * D_IN * 4,      # dW fp32
}
_DUAL = 2 + 2 * (0.5 + 1 / 16)      # bf16 read + two orientations of codes and E4M3 scales
_MX = 2 + 0.5 + 1 / 32
_GF = 2.0 * TOKENS * D_IN * D_OUT
STEP_DISPATCHES = [
    ("amax X", r"^k_amax(_flat)?<", 2 * _NX, _NX),
    ("dual X (RTN along K, SR along tokens)", r"^k_quant_dual<0, 0, 1,", _DUAL * _NX, 2 * _NX),
    ("amax W", r"^k_amax(_flat)?<", 2 * _NW, _NW),
    ("dual W (RTN along K, SR along out)", r"^k_quant_dual<0, 0, 1,", _DUAL * _NW, 2 * _NW),
    ("NVFP4 GEMM fwd (bf16 out)", r"^k_gemm<0, 256, true, false>", _GF, 0),
    ("amax dY", r"^k_amax(_flat)?<", 2 * _NY, _NY),
    ("dual dY (SR both)", r"^k_quant_dual<0, 1, 1,", _DUAL * _NY, 2 * _NY),
    ("NVFP4 GEMM dgrad (fp32 out)", r"^k_gemm<0, 256, false, false>", _GF, 0),
    ("NVFP4 GEMM wgrad (fp32 out)", r"^k_gemm<0, 256, false, false>", _GF, 0),
    ("MXFP4+Hadamard X", r"^k_quant_cols<1,", _MX * _NX, _NX),
    ("MXFP4+Hadamard W", r"^k_quant_cols<1,", _MX * _NW, _NW),
    ("MXFP4 GEMM fwd (bf16 out)", r"^k_gemm_mx8<true>", _GF, 0),
]
EXTRA_DISPATCHES = [
    ("amax dY rotated 16-wide along tokens", r"^k_amax_rot_rows<", 2 * _NY, _NY),
    ("amax pair X (plain, rotated along tokens)", r"^k_amax_pair<", 2 * _NX, _NX),
    ("dual X, 16-wide rotation along tokens", r"^k_quant_dual<0, 0, 1, true, false, true,", _DUAL * _NX, 2 * _NX),
    ("amax pair dY (plain, rotated along tokens)", r"^k_amax_pair<", 2 * _NY, _NY),
    ("dual dY, 16-wide rotation along tokens", r"^k_quant_dual<0, 1, 1, true, false, true,", _DUAL * _NY, 2 * _NY),
    ("amax W (2-D)", r"^k_amax(_flat)?<", 2 * _NW, _NW),
    ("2-D 16x16 W", r"^k_quant_2d<", _DUAL * _NW, 2 * _NW),
    ("amax dY (monitored)", r"^k_amax(_flat)?<", 2 * _NY, _NY),
    ("dual dY + noise monitor", r"^k_quant_dual_w4<0, 1, 1, true, false, false, true>", _DUAL * _NY, 2 * _NY),
]


def label_dispatches(names, steps: int, warmup: int):
    """Labels of a benchmark run's dispatches (kernel short names in launch
    order, as filtered by the profiling commands), checked against the kernel
    each position must run."""
    import re

    cold = [(l + " (cold)", rx, u, e) for l, rx, u, e in STEP_DISPATCHES if not rx.startswith("^k_gemm")]
    expect = STEP_DISPATCHES * (warmup + steps) + EXTRA_DISPATCHES * (2 + steps) + cold * (2 + steps)
    if len(names) != len(expect):
        raise ValueError(f"{len(names)} dispatches, expected {len(expect)}")
    for n, (l, rx, _, _) in zip(names, expect):
        if not re.search(rx, n):
            raise ValueError(f"dispatch {n!r} where {l} ({rx}) was expected")
    return [(l, u, e) for l, _, u, e in expect]


def _per_dispatch(csv_path: str):
    """[(kernel name, {counter: value}, duration ns)] in dispatch order."""
    import csv

    d = {}
    for r in csv.DictReader(open(csv_path)):
        k = int(r["Dispatch_Id"])
        e = d.setdefault(k, [short_name(r["Kernel_Name"]), {},
                             int(r["End_Timestamp"]) - int(r["Start_Timestamp"])])
        e[1][r["Counter_Name"]] = float(r["Counter_Value"])
    return [tuple(d[k]) for k in sorted(d)]


def _trace_parts(trace_csv: str):
    """The kernel trace's dispatches [(short name, duration ns)] in launch
    order, split into the Llama-7B part of the run, the ceiling measurements
    and the large layer's part (after the last measurement kernel)."""
    import csv
    import re

    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    d = [(short_name(r["Kernel_Name"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) for r in rows]
    meas = [i for i, (n, _) in enumerate(d) if any(re.search(rx, n) for _, rx in CEILING_KERNELS)]
    if not meas:
        return d, [], []
    return d[:meas[0]], d[meas[0]:meas[-1] + 1], d[meas[-1] + 1:]


def _group(dispatches, groups):
    """{group label: [durations in ns]} of the dispatches whose names match."""
    import re

    out = {label: [] for label, _ in groups}
    for name, dur in dispatches:
        for label, rx in groups:
            if re.search(rx, name):
                out[label].append(dur)
    return out


def _gemm_shape(grid: int, index: int):
    names = ["fwd 32768x11008x4096 (bf16 out)", "dgrad 32768x4096x11008 (fp32 out)",
             "wgrad 11008x4096x32768 (fp32 out)"]
    return names[index % 3]


def _stats_lines(groups):
    """Group rows of a part of the run that launches each group the same
    number of times per step: all launches, and the timed steps' alone."""
    out = ["| group | launches | avg us | avg us (timed) | min us | max us |", "|---|---|---|---|---|---|"]
    for label, d in groups.items():
        if d:
            per_step = len(d) // (WARMUP + STEPS)
            timed = d[per_step * WARMUP:]
            out.append(f"| {label} | {len(d)} | {sum(d) / len(d) / 1e3:.1f} | {sum(timed) / len(timed) / 1e3:.1f} | "
                       f"{min(d) / 1e3:.1f} | {max(d) / 1e3:.1f} |")
    return out


# The large layer's step in launch order (bench.py make_large_step).
L_TOKENS, L_IN, L_OUT = 16384, 8192, 28672
LARGE_GROUPS = [
    ("tensor amax (X, W, dY)", r"^k_amax(_flat)?<"),
    ("quantize X, both orientations (RTN along K, SR along tokens)", r"^k_quant_dual<0, 0, 1,"),
    ("quantize dY, both orientations (SR)", r"^k_quant_dual<0, 1, 1,"),
    ("NVFP4 GEMM fwd 16384x28672x8192 (bf16 out)", r"^k_gemm<0, 256, true, false>"),
    ("NVFP4 GEMM dgrad 16384x8192x28672 / wgrad 28672x8192x16384 (fp32 out)", r"^k_gemm<0, 256, false, false>"),
]


def _split_after_steps(dispatches, per_step: int):
    """(the dispatches up to the last library dispatch of WARMUP + STEPS steps
    of `per_step` library dispatches each, the rest)."""
    import re

    lib = re.compile(r"^k_(amax|quant|gemm|split)")
    need, seen = per_step * (WARMUP + STEPS), 0
    for i, (name, _) in enumerate(dispatches):
        if lib.search(name):
            seen += 1
            if seen == need:
                return dispatches[:i + 1], dispatches[i + 1:]
    return dispatches, []


def _write_nv_step(dispatches, groups, pair_label, dgrad_label, wgrad_label, title, intro, path):
    """Kernel-time table of an NVFP4 step (amax + dual passes + three GEMMs);
    dgrad and wgrad run the same kernel and are told apart by launch order."""
    g = _group(dispatches, groups)
    d = g.pop(pair_label)
    g[dgrad_label] = d[0::2]
    g[wgrad_label] = d[1::2]
    with open(path, "w") as f:
        f.write("\n".join([f"# {title}", ""] + intro + [""] + _stats_lines(g) + [""]))


def _command_lines(command):
    return ["Command (run from the repository root on one MI355X, `cd /tmp && export TMPDIR=/tmp` first; "
            "`OUT` = the folder the run writes its CSV files to):", "", "```", command, "```", ""]


def _write_large_step(dispatches, command, profiles_dir):
    import os

    intro = _command_lines(command) + [
        f"The large layer: hidden {L_IN}, MLP {L_OUT}, {L_TOKENS} tokens. One step = for each of X, W and dY "
        "an amax pass and one pass that quantizes both orientations (NVFP4; X and W: RTN along K, SR along "
        "the other axis; dY: SR along both), the fwd GEMM (bf16 out), dgrad and wgrad (fp32 out); "
        f"{WARMUP} warm-up + {STEPS} timed steps, after the rest of the run. `avg us (timed)` leaves out the "
        "warm-up steps. X's and W's dual passes run the same kernel (the group holds both).",
    ]
    _write_nv_step(dispatches, LARGE_GROUPS,
                   "NVFP4 GEMM dgrad 16384x8192x28672 / wgrad 28672x8192x16384 (fp32 out)",
                   "NVFP4 GEMM dgrad 16384x8192x28672 (fp32 out)", "NVFP4 GEMM wgrad 28672x8192x16384 (fp32 out)",
                   "Kernel time of the large layer's step (bench.py `large_step`)", intro,
                   os.path.join(profiles_dir, "large_layer_step_kernel_stats.md"))


# One GPU's share of 8-way data parallelism over the Llama-7B layer's tokens.
S_TOKENS = TOKENS // 8
SHARD_GROUPS = [
    ("tensor amax (X, W, dY)", r"^k_amax(_flat)?<"),
    ("quantize X and W, both orientations (RTN along K, SR along the other axis)", r"^k_quant_dual<0, 0, 1,"),
    ("quantize dY, both orientations (SR)", r"^k_quant_dual<0, 1, 1,"),
    (f"NVFP4 GEMM fwd {S_TOKENS}x{D_OUT}x{D_IN} (bf16 out)", r"^k_gemm<0, 256, true, false>"),
    (f"NVFP4 GEMM dgrad {S_TOKENS}x{D_IN}x{D_OUT} / wgrad {D_OUT}x{D_IN}x{S_TOKENS} (fp32 out)",
     r"^k_gemm<0, 256, false, false>"),
]


def _write_shard_step(dispatches, command, profiles_dir):
    import os

    intro = _command_lines(command) + [
        f"One GPU's share of 8-way data parallelism over the Llama-7B layer's tokens: X [{S_TOKENS}, {D_IN}], "
        f"dY [{S_TOKENS}, {D_OUT}], W [{D_OUT}, {D_IN}] whole (bench.py `dp8_shard_step`, timed after the "
        "large layer's step). One step = amax + one dual pass for each of X, W and dY (RTN along K, SR on the "
        f"backward orientations), the fwd GEMM (bf16 out), dgrad and wgrad (fp32 out); {WARMUP} warm-up + "
        f"{STEPS} timed steps. `avg us (timed)` leaves out the warm-up steps.",
    ]
    _write_nv_step(dispatches, SHARD_GROUPS, SHARD_GROUPS[-1][0],
                   f"NVFP4 GEMM dgrad {S_TOKENS}x{D_IN}x{D_OUT} (fp32 out)",
                   f"NVFP4 GEMM wgrad {D_OUT}x{D_IN}x{S_TOKENS} (fp32 out)",
                   "Kernel time of one 8-way data-parallel shard's step (bench.py `dp8_shard_step`)", intro,
                   os.path.join(profiles_dir, "dp8_shard_step_kernel_stats.md"))


def _write_ceilings(dispatches, command, profiles_dir):
    import os

    groups = _group(dispatches, CEILING_KERNELS)
    lines = [
        "# Kernel time of the chip-ceiling measurements (bench.py `measured_ceilings`)",
        "",
        "Command (run from the repository root on one MI355X, `cd /tmp && export TMPDIR=/tmp` first; "
        "`OUT` = the folder the run writes its CSV files to):",
        "",
        "```", command, "```",
        "",
        "The MFMA loops run 1024 workgroups of 4 waves, each wave 4000 iterations of 8 MFMAs "
        "(32768 FLOP per f16 instruction, 131072 per FP4 instruction); the streaming passes cover 2 GiB "
        "at five grid sizes each (2 warm-up + 10 timed launches per size, so the averages mix grid sizes; "
        "the benchmark reports the best size's median).",
        "",
        "| kernel | launches | avg us | min us | max us |",
        "|---|---|---|---|---|",
    ]
    for label, d in groups.items():
        if d:
            lines.append(f"| {label} | {len(d)} | {sum(d) / len(d) / 1e3:.1f} | {min(d) / 1e3:.1f} | "
                         f"{max(d) / 1e3:.1f} |")
    lines.append("")
    with open(os.path.join(profiles_dir, "chip_ceilings_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines))


def summarize(out_dir: str, profiles_dir: str) -> None:
    summarize_trace(out_dir, profiles_dir)
    summarize_counters(out_dir, profiles_dir)


def summarize_trace(out_dir: str, profiles_dir: str) -> None:
    """Kernel-time summaries of the kernel-trace run: the Llama-7B part of the
    benchmark, the large layer's step and the chip-ceiling measurements."""
    import os

    stats_csv = os.path.join(out_dir, "prof_bench", "bench_kernel_stats.csv")
    trace_csv = os.path.join(out_dir, "prof_bench", "bench_kernel_trace.csv")
    cmd = lambda k: PROFILE_COMMANDS[k]   # OUT: the folder the runs write their CSV files to

    # ---- kernel time of the step
    llama, ceil, large = _trace_parts(trace_csv)
    groups = _group(llama, GROUPS)
    lines = [
        "# Kernel time of the Llama-7B layer step (bench.py)",
        "",
        "Command (run from the repository root on one MI355X, `cd /tmp && export TMPDIR=/tmp` first; "
        "`OUT` = the folder the run writes its CSV files to):",
        "",
        "```", cmd("stats"), "```",
        "",
        "One step = NVFP4 quantization of X, W and dY, each tensor read once for both of its orientations "
        "(X, W: RTN along K + SR along the other axis; dY: SR along both), the fwd GEMM (bf16 out), dgrad and "
        f"wgrad GEMMs (fp32 out), MXFP4+Hadamard fwd (quantize X, W; GEMM bf16 out). {WARMUP + STEPS} steps "
        f"traced ({WARMUP} warm-up + {STEPS} timed), then the adjacent passes the benchmark times after the "
        "step (`extras`: NVFP4 16-wide rotation of the wgrad operands with their amax pass, the noise-monitored "
        "dY pass, the 2-D quantization of W), 2 warm-up + 10 timed calls each, then the step's quantize "
        "calls again with the caches evicted before each call (torch's reduction over a 1 GiB buffer), "
        "2 + 10 calls each, and a 1 GiB device copy (`__amd_rocclr_copyBuffer`, 13 launches) that measures "
        "the copy bandwidth; the other torch kernels are the one-time input generation. The same run then "
        "measures the chip's ceilings (`chip_ceilings_kernel_stats.md`) and times the large layer's step "
        "(`large_layer_step_kernel_stats.md`) and an 8-way data-parallel shard's step "
        "(`dp8_shard_step_kernel_stats.md`); this table covers the dispatches before those.",
        "",
        "`avg us (timed)` (GEMMs, which only the step launches) leaves out the warm-up steps' launches (the "
        "first launches of a run are slower while the clock settles); that is the figure to set against the "
        "benchmark's HIP-event times.",
        "",
        "`k_gemm<0, 256, *, *>` = NVFP4 GEMM (f16 MFMA), `k_gemm_mx8<*>` (whole tiles) and `k_gemm<1, *, *, *>` "
        "= MXFP4 GEMM (scaled FP4 MFMA); the bf16 flag = bf16 output, the last `k_gemm` flag = a split-K piece "
        "(none in this step).",
        "",
        "## Kernel groups (from the kernel trace)",
        "",
        "| group | launches | avg us | avg us (timed) | min us | max us |",
        "|---|---|---|---|---|---|",
    ]
    for label, _ in GROUPS:
        d = groups[label]
        if d:
            # Kernels launched only by the step (the GEMMs): drop the warm-up launches.
            timed = "-"
            if label.endswith("GEMM") or "GEMM (" in label:
                per_step = len(d) // (WARMUP + STEPS)
                t = d[per_step * WARMUP:]
                timed = f"{sum(t) / len(t) / 1e3:.1f}"
            lines.append(f"| {label} | {len(d)} | {sum(d) / len(d) / 1e3:.1f} | {timed} | "
                         f"{min(d) / 1e3:.1f} | {max(d) / 1e3:.1f} |")
    lines += ["", "## Per kernel over the whole run (`--stats` summary)", "", kernel_stats_table(stats_csv), ""]
    with open(os.path.join(profiles_dir, "llama7b_step_kernel_stats.md"), "w") as f:
        f.write("\n".join(lines))
    large, shard = _split_after_steps(large, 9)
    if large:
        _write_large_step(large, cmd("stats"), profiles_dir)
    if shard:
        _write_shard_step(shard, cmd("stats"), profiles_dir)
    if ceil:
        _write_ceilings(ceil, cmd("stats"), profiles_dir)


def summarize_counters(out_dir: str, profiles_dir: str) -> None:
    """HBM traffic and MFMA / VALU utilisation from the counter runs."""
    import json
    import os

    cmd = lambda k: PROFILE_COMMANDS[k]   # OUT: the folder the runs write their CSV files to

    # ---- HBM traffic of the NVFP4 GEMM
    # Only the copy dispatches (the fill that creates the source is left out).
    def copy_avg(path, counter):
        v = [x for _, _, x in counter_per_dispatch(path, counter, "copyBuffer")]
        return sum(v) / len(v)

    cf = copy_avg(os.path.join(out_dir, "pmc_copy_fetch", "copy_counter_collection.csv"), "FETCH_SIZE")
    cw = copy_avg(os.path.join(out_dir, "pmc_copy_write", "copy_counter_collection.csv"), "WRITE_SIZE")
    reps_kib = COPY_BYTES / 1024
    f_fac = reps_kib / cf
    w_fac = reps_kib / cw
    fe = counter_per_dispatch(os.path.join(out_dir, "pmc_fetch", "bench_counter_collection.csv"),
                              "FETCH_SIZE", r"k_gemm<0,")
    wr = counter_per_dispatch(os.path.join(out_dir, "pmc_write", "bench_counter_collection.csv"),
                              "WRITE_SIZE", r"k_gemm<0,")
    assert len(fe) == len(wr) and len(fe) % 3 == 0, (len(fe), len(wr))
    rows = []
    for i, ((_, grid, fk), (_, _, wk)) in enumerate(zip(fe, wr)):
        rows.append((_gemm_shape(grid, i), grid // 256, fk, wk, (fk * f_fac + wk * w_fac) * 1024,
                     list(GEMM_ALGO_BYTES.values())[i % 3]))
    avg = sum(r[4] for r in rows) / len(rows)
    lines = [
        "# HBM traffic of the NVFP4 GEMM (Llama-7B layer: fwd, dgrad, wgrad)",
        "",
        "Commands (from the repository root on one MI355X, after `cd /tmp && export TMPDIR=/tmp`; "
        "`OUT` = the folder the runs write their CSV files to):",
        "",
        "```", cmd("fetch"), cmd("write"), cmd("copy_fetch"), cmd("copy_write"), "```",
        "",
        "## Calibration with a plain copy of 1 GiB (`__amd_rocclr_copyBuffer`, average of 3 dispatches)",
        "",
        f"FETCH_SIZE reads {cf:.0f} KiB for {reps_kib:.0f} KiB read -> factor {f_fac:.3f}; "
        f"WRITE_SIZE reads {cw:.0f} KiB for {reps_kib:.0f} KiB written -> factor {w_fac:.3f}.",
        "",
        "## Per dispatch (KiB as read, then bytes after calibration)",
        "",
        "| GEMM | grid | FETCH_SIZE KiB | WRITE_SIZE KiB | HBM bytes (calibrated) | algorithmic | ratio |",
        "|---|---|---|---|---|---|---|",
    ]
    for name, wgs, fk, wk, b, algo in rows:
        lines.append(f"| {name} | {wgs} WGs | {fk:.0f} | {wk:.0f} | {b / 1e6:.1f} MB | {algo / 1e6:.1f} MB | "
                     f"{b / algo:.2f} |")
    algo_avg = sum(GEMM_ALGO_BYTES.values()) / 3
    lines += [
        "",
        f"Average over the NVFP4 GEMM launches: {avg / 1e6:.1f} MB per launch (this is `roofline.traffic`), "
        f"against {algo_avg / 1e6:.1f} MB of algorithmic bytes on average ({avg / algo_avg:.2f}x).",
        "Algorithmic bytes per launch: both operands' codes (0.5 B) and E4M3 scales (1/16 B) per element, read "
        "once, plus the output written once: fwd X + W (75.5 + 25.4 MB) + Y bf16 (721.4 MB) = "
        f"{GEMM_ALGO_BYTES['fwd'] / 1e6:.1f} MB; dgrad dY + W^T (202.9 + 25.4 MB) + dX fp32 (536.9 MB) = "
        f"{GEMM_ALGO_BYTES['dgrad'] / 1e6:.1f} MB; wgrad dY^T + X^T (202.9 + 75.5 MB) + dW fp32 (180.4 MB) = "
        f"{GEMM_ALGO_BYTES['wgrad'] / 1e6:.1f} MB.",
        "",
        f"GEMM source digest: `{source_digest()}`.",
        "",
    ]
    with open(os.path.join(profiles_dir, "nvfp4_gemm_llama7b_hbm_traffic.md"), "w") as f:
        f.write("\n".join(lines))
    # ---- HBM bytes of the quantize-side dispatches
    fd = _per_dispatch(os.path.join(out_dir, "pmc_fetch", "bench_counter_collection.csv"))
    wd = _per_dispatch(os.path.join(out_dir, "pmc_write", "bench_counter_collection.csv"))
    labels = label_dispatches([n for n, _, _ in fd], PMC_STEPS, PMC_WARMUP)
    assert [n for n, _, _ in fd] == [n for n, _, _ in wd]
    agg = {}
    for (l, units, _), (_, fc, _), (_, wc, _) in zip(labels, fd, wd):
        if l.startswith(("NVFP4 GEMM", "MXFP4 GEMM")):
            continue
        a = agg.setdefault(l, [0, 0.0, 0.0, units])
        a[0] += 1
        a[1] += fc["FETCH_SIZE"] * f_fac * 1024
        a[2] += wc["WRITE_SIZE"] * w_fac * 1024
    lines = [
        "# HBM traffic of the quantize-side kernels (Llama-7B layer step and adjacent passes)",
        "",
        "Same counter runs and copy calibration as the NVFP4 GEMM traffic "
        "(`nvfp4_gemm_llama7b_hbm_traffic.md`):",
        "",
        "```", cmd("fetch"), cmd("write"), cmd("copy_fetch"), cmd("copy_write"), "```",
        "",
        "Read and write bytes are FETCH_SIZE and WRITE_SIZE per dispatch (averaged over the run's launches of "
        f"that dispatch), times the copy factors {f_fac:.3f} and {w_fac:.3f}. The counters see the traffic "
        "between L2 and the memory fabric, so a read served by the 256 MB memory-side cache counts as a read "
        "here. Algorithmic bytes: the bf16 input once, 0.5 B of codes and 1/16 B (NVFP4) or 1/32 B (MXFP4) "
        "of scale per element and orientation written; an amax pass reads the input once. `(cold)` = the "
        "benchmark's repeat of the step's quantize calls with the caches evicted before each call.",
        "",
        "| dispatch | launches | read MB | written MB | total MB | algorithmic MB | total / algorithmic |",
        "|---|---|---|---|---|---|---|",
    ]
    for l, (n, fb, wb, units) in agg.items():
        lines.append(f"| {l} | {n} | {fb / n / 1e6:.1f} | {wb / n / 1e6:.1f} | {(fb + wb) / n / 1e6:.1f} | "
                     f"{units / 1e6:.1f} | {(fb + wb) / n / units:.3f} |")
    lines.append("")
    with open(os.path.join(profiles_dir, "quantize_llama7b_hbm_traffic.md"), "w") as f:
        f.write("\n".join(lines))

    # ---- MFMA and VALU utilisation
    ud = _per_dispatch(os.path.join(out_dir, "pmc_util", "bench_counter_collection.csv"))
    labels = label_dispatches([n for n, _, _ in ud], PMC_STEPS, PMC_WARMUP)
    simds = CUS * SIMDS_PER_CU
    agg = {}
    for (l, units, elems), (_, c, dur) in zip(labels, ud):
        cyc = c["GRBM_GUI_ACTIVE"] / XCDS
        a = agg.setdefault(l, [0, 0.0, 0.0, 0.0, 0.0, 0.0, units])
        a[0] += 1
        a[1] += dur
        a[2] += cyc / dur                                        # GHz
        a[3] += c["SQ_VALU_MFMA_BUSY_CYCLES"] / (simds * cyc)
        a[4] += 4 * c["SQ_ACTIVE_INST_VALU"] / (simds * cyc)
        a[5] += c["SQ_INSTS_VALU"] / c["SQ_INSTS_MFMA"] if elems == 0 else c["SQ_INSTS_VALU"] * 64 / elems
    lines = [
        "# MFMA and VALU utilisation of the Llama-7B layer step's kernels",
        "",
        "Command (from the repository root on one MI355X, after `cd /tmp && export TMPDIR=/tmp`; "
        "`OUT` = the folder the run writes its CSV files to):",
        "",
        "```", cmd("util"), "```",
        "",
        f"Per dispatch, averaged over the run's launches of that dispatch. GRBM_GUI_ACTIVE sums the "
        f"{XCDS} XCDs' cycles, so the kernel's cycles are GRBM_GUI_ACTIVE / {XCDS} (the `clock` column, "
        f"those cycles over the dispatch's duration, checks it). MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / "
        f"({simds} SIMDs x cycles). VALU issue = 4 x SQ_ACTIVE_INST_VALU / ({simds} SIMDs x cycles): "
        "SQ_ACTIVE_INST_VALU counts one per VALU instruction of a wave (it equals SQ_INSTS_VALU to 0.01% "
        "here), and a wave64 instruction holds a 16-lane SIMD for 4 cycles, so 1.0 = every SIMD issuing "
        "VALU work every cycle. `VALU / unit` = VALU instructions (MFMA included) per MFMA for GEMMs; "
        "VALU instructions x 64 lanes per element and orientation for quantize passes (per element for "
        "amax passes). Durations are longer than in unprofiled runs (counters serialise the dispatches). "
        "A clock above the 2.4 GHz maximum means the counters' window outlasted the dispatch (short "
        "kernels); the busy fractions of those rows are then low by that ratio.",
        "",
        "| dispatch | launches | avg us | clock GHz | MFMA busy | VALU issue | VALU / unit |",
        "|---|---|---|---|---|---|---|",
    ]
    for l, (n, dur, ghz, mf, va, per, _) in agg.items():
        lines.append(f"| {l} | {n} | {dur / n / 1e3:.1f} | {ghz / n:.2f} | {mf / n:.3f} | {va / n:.3f} | "
                     f"{per / n:.2f} |")
    lines.append("")
    with open(os.path.join(profiles_dir, "llama7b_step_mfma_valu_utilisation.md"), "w") as f:
        f.write("\n".join(lines))

    if os.path.isdir(os.path.join(out_dir, "pmc_lds")):
        summarize_lds(out_dir, profiles_dir)

    with open(os.path.join(profiles_dir, "traffic.json"), "w") as f:
        json.dump({"nv_gemm_bytes_per_launch": round(avg), "source_digest": source_digest(),
                   "fetch_factor": round(f_fac, 4), "write_factor": round(w_fac, 4)}, f, indent=1)
        f.write("\n")


# The step's GEMMs: (label in STEP_DISPATCHES, K, output tiles of 256 x 256, threads per workgroup).
_STEP_GEMMS = [
    ("NVFP4 GEMM fwd (bf16 out)", D_IN, (TOKENS // 256) * -(-D_OUT // 256), 256),
    ("NVFP4 GEMM dgrad (fp32 out)", D_OUT, (TOKENS // 256) * (D_IN // 256), 256),
    ("NVFP4 GEMM wgrad (fp32 out)", TOKENS, -(-D_OUT // 256) * (D_IN // 256), 256),
    ("MXFP4 GEMM fwd (bf16 out)", D_IN, (TOKENS // 256) * -(-D_OUT // 256), 512),
]


def summarize_lds(out_dir: str, profiles_dir: str) -> None:
    """LDS work and waits of the step's GEMMs per K tile of 256 (one workgroup's
    256 x 256 output tile over 256 K values), from the "lds" counter run."""
    import os

    cmd = PROFILE_COMMANDS["lds"]
    dd = _per_dispatch(os.path.join(out_dir, "pmc_lds", "bench_counter_collection.csv"))
    labels = label_dispatches([n for n, _, _ in dd], PMC_STEPS, PMC_WARMUP)
    shapes = {l: (k, t, th) for l, k, t, th in _STEP_GEMMS}
    agg = {}
    for (l, _, _), (_, c, dur) in zip(labels, dd):
        if l not in shapes:
            continue
        k, tiles, _ = shapes[l]
        units = tiles * (k // 256)                   # workgroup K tiles of the dispatch
        cyc = c["GRBM_GUI_ACTIVE"] / XCDS
        a = agg.setdefault(l, [0] + [0.0] * 9)
        a[0] += 1
        a[1] += dur
        a[2] += cyc * CUS / units                    # CU cycles per K tile
        a[3] += c["SQ_INSTS_LDS"] / units
        a[4] += c["SQ_INSTS_MFMA"] / units
        a[5] += c["SQ_LDS_BANK_CONFLICT"] / units
        a[6] += c["SQ_LDS_BANK_CONFLICT"] / c["SQ_ACTIVE_INST_LDS"]
        a[7] += c["SQ_WAIT_INST_LDS"] / c["SQ_WAVE_CYCLES"]
        a[8] += c["SQ_WAIT_ANY"] / c["SQ_WAVE_CYCLES"]
        a[9] += c["SQ_ACTIVE_INST_LDS"] / units
    lines = [
        "# LDS work and waits per K tile of the Llama-7B step's GEMMs",
        "",
        "Command (from the repository root on one MI355X, after `cd /tmp && export TMPDIR=/tmp`; "
        "`OUT` = the folder the run writes its CSV files to):",
        "",
        "```", cmd, "```",
        "",
        "A K tile here is one workgroup's 256 x 256 output tile over 256 values of K: the unit of the GEMMs' "
        "K loop (staging writes of the next tile's operands, fragment reads, one barrier). Per dispatch, "
        "averaged over the run's launches: `CU cycles / K tile` = the kernel's cycles (GRBM_GUI_ACTIVE / "
        f"{XCDS}) x {CUS} CUs / (output tiles x K / 256), so it includes each tile's prologue and epilogue; "
        "`LDS instr`, `MFMA instr`, `active LDS` (SQ_ACTIVE_INST_LDS) and `conflict` (SQ_LDS_BANK_CONFLICT) "
        "are the counters' sums over the dispatch divided by its K tiles; `conflict / active LDS` and the "
        "two wait fractions (SQ_WAIT_INST_LDS and SQ_WAIT_ANY over SQ_WAVE_CYCLES, summed over waves) are "
        "ratios of the counters as the hardware reports them. The NVFP4 kernel runs 4 waves per workgroup "
        "(one per SIMD, 128 x 128 outputs each), the MXFP4 kernel 8 (two per SIMD, 128 x 64 each).",
        "",
        "| GEMM | launches | avg us | CU cycles / K tile | LDS instr / K tile | MFMA instr / K tile | "
        "active LDS / K tile | conflict / K tile | conflict / active LDS | LDS wait / wave cycles | "
        "any wait / wave cycles |",
        "|---|---|---|---|---|---|---|---|---|---|---|",
    ]
    for l, (n, dur, cpk, lds, mfma, conf, cfr, wl, wa, act) in agg.items():
        lines.append(f"| {l} | {n} | {dur / n / 1e3:.1f} | {cpk / n:.0f} | {lds / n:.0f} | {mfma / n:.0f} | "
                     f"{act / n:.0f} | {conf / n:.0f} | {cfr / n:.3f} | {wl / n:.3f} | {wa / n:.3f} |")
    lines.append("")
    with open(os.path.join(profiles_dir, "gemm_llama7b_lds_per_k_tile.md"), "w") as f:
        f.write("\n".join(lines))


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "copy":
        copy()
    elif len(sys.argv) > 2 and sys.argv[1] in ("summarize", "summarize-trace", "summarize-lds"):
        import os

        prof = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "profiles")
        {"summarize": summarize, "summarize-trace": summarize_trace,
         "summarize-lds": summarize_lds}[sys.argv[1]](sys.argv[2], prof)
    else:
        print(__doc__)
