"""Builds libfp4.so (gfx950) in-tree from csrc/ with hipcc, and beside it
libfp4_measure.so (the benchmark's on-box ceiling measurements).

    python -m fp4_fully_quantized_amd.build

Every HIP source is compiled with -ffp-contract=off (the quantizer's FP32
arithmetic must not be contracted into FMAs) and with packed-FP32 VALU
instructions disabled.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfp4.so")
SOURCES = ["quant.hip", "quant_dual.hip", "quant_2d.hip", "gemm.hip", "abi.cpp"]
# The chip's measured ceilings (MFMA loops, streaming passes) for the benchmark.
MEASURE_SOURCES = ["measure.hip"]
MEASURE_LIB = os.path.join(PKG, "libfp4_measure.so")
ARCH = os.environ.get("FP4_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    return os.path.join(rocm, "bin", "hipcc")


def flags() -> list[str]:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-Wall", "-Wno-unused-function"]


def build(verbose: bool = False) -> str:
    _build_lib(SOURCES, LIB, verbose)
    _build_lib(MEASURE_SOURCES, MEASURE_LIB, verbose)
    return LIB


def _build_lib(sources: list[str], lib: str, verbose: bool) -> None:
    os.makedirs(BUILD, exist_ok=True)
    procs = []
    objs = []
    for src in sources:
        obj = os.path.join(BUILD, src + ".o")
        cmd = [hipcc()] + flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".cpp"):
            cmd = [hipcc()] + flags() + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
    failed = False
    for src, p in procs:
        out = p.communicate()[0].decode(errors="replace")
        out = "\n".join(l for l in out.splitlines() if "packed-fp32-ops" not in l)
        if p.returncode != 0:
            failed = True
            sys.stderr.write(f"[fp4 build] {src} failed:\n{out}\n")
        elif verbose and out.strip():
            sys.stderr.write(f"[fp4 build] {src}:\n{out}\n")
    if failed:
        raise RuntimeError("hipcc failed")
    tmp = lib + ".tmp"
    subprocess.run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, check=True)
    os.replace(tmp, lib)


if __name__ == "__main__":
    print(build(verbose=True))
