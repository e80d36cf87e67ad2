"""Helpers for profiling runs.

    python -m fp4_fully_quantized_amd.profiling copy

runs a plain device copy of a known size (1 GiB, bf16) a few times, so that
the HBM byte counters read for it (FETCH_SIZE, WRITE_SIZE) can calibrate the
same counters read for the library's kernels.
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


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "copy":
        copy()
    else:
        print(__doc__)


# ---------------------------------------------------------------- summaries
def short_name(name: str) -> str:
    base = name.split("(")[0].replace("void ", "").replace("(anonymous namespace)::", "")
    return base.strip()


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


def source_digest() -> str:
    """Digest of the GEMM sources: a traffic figure is valid for this digest only."""
    import hashlib
    import os

    h = hashlib.sha256()
    here = os.path.dirname(os.path.abspath(__file__))
    for fn in ("gemm.hip", "fp4_device.hpp"):
        with open(os.path.join(here, "csrc", fn), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]
