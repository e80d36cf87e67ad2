"""Seeded synthetic inputs for the FP4 quantize + GEMM path.

This module only draws numbers: it holds none of the quantizer's or the GEMM's
arithmetic, so both the GPU library's tests and the CPU oracle can take their
inputs from it. Shapes and distributions follow the workloads the pages
measure on (Quartet, Measured effects table: Llama-7B-shaped linear layers,
batch 64 x sequence 512 = 32768 tokens), with the distributions described in
the design notes:

  tiny           X, W fp32 [256, 256] ~ N(0, 1)
  llama7b        X bf16 [32768, 4096] ~ N(0, 1) with 1% of the columns x20,
                 W bf16 [11008, 4096] ~ N(0, 0.02),
                 dY bf16 [32768, 11008] = 1e-3 * t3 / sqrt(3) (Student-t, nu = 3)
  large          X bf16 [16384, 8192] ~ N(0, 1) with 1% of the columns x20,
                 W bf16 [28672, 8192] ~ N(0, 0.01), dY bf16 [16384, 28672] ~ N(0, 1e-3)

Values are drawn in fp32 and rounded to nearest-even into bf16. Two backends
draw the same distributions: numpy on the host (small cases, bit-identical on
every machine) and torch on the GPU (full sizes, where host drawing is slow);
either way the same bytes then feed the GPU library and the oracle.
"""
from __future__ import annotations

import math

import numpy as np

SHAPES = {
    "tiny": {"X": (256, 256), "W": (256, 256)},
    "llama7b": {"X": (32768, 4096), "W": (11008, 4096), "dY": (32768, 11008)},
    "large": {"X": (16384, 8192), "W": (28672, 8192), "dY": (16384, 28672)},
}
W_STD = {"tiny": 1.0, "llama7b": 0.02, "large": 0.01}
OUTLIER_FRACTION = 0.01
OUTLIER_GAIN = 20.0
GRAD_STD = 1e-3


def _seed(workload: str, role: str, extra: int = 0) -> int:
    base = {"tiny": 0, "llama7b": 1000, "large": 4000}[workload]
    return base + {"X": 1, "W": 2, "dY": 3, "perm": 4}[role] + 10 * extra


def outlier_columns(n_cols: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    k = max(1, int(round(OUTLIER_FRACTION * n_cols)))
    return np.sort(rng.permutation(n_cols)[:k])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even fp32 -> bf16 bit patterns (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------- host (numpy)
def host_normal(shape, std, seed, outliers=False, bf16=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32) * np.float32(std)
    if outliers:
        cols = outlier_columns(shape[1], seed + 3)
        x[:, cols] *= np.float32(OUTLIER_GAIN)
    return f32_to_bf16_bits(x) if bf16 else x


def host_student_t(shape, scale, seed, nu=3, bf16=True):
    rng = np.random.default_rng(seed)
    t = rng.standard_t(nu, size=shape).astype(np.float32)
    x = t * np.float32(scale / math.sqrt(nu / (nu - 2)))
    return f32_to_bf16_bits(x) if bf16 else x


def host_tensor(workload: str, role: str, shape=None, extra: int = 0):
    """Host copy of one input: uint16 bf16 bits (fp32 for the tiny workload).
    `shape` overrides the workload's shape (same distribution)."""
    shape = tuple(shape or SHAPES[workload][role])
    bf16 = workload != "tiny"
    s = _seed(workload, role, extra)
    if role == "X":
        return host_normal(shape, 1.0, s, outliers=workload != "tiny", bf16=bf16)
    if role == "W":
        return host_normal(shape, W_STD[workload], s, bf16=bf16)
    if role == "dY":
        if workload == "llama7b":
            return host_student_t(shape, GRAD_STD, s, bf16=bf16)
        return host_normal(shape, GRAD_STD, s, bf16=bf16)
    raise KeyError(role)


# ---------------------------------------------------------------- device (torch)
def device_tensor(workload: str, role: str, device="cuda", shape=None, extra: int = 0):
    """Same distributions drawn by torch on `device`, returned as a bf16 tensor
    (fp32 for the tiny workload)."""
    import torch

    shape = tuple(shape or SHAPES[workload][role])
    s = _seed(workload, role, extra)
    g = torch.Generator(device=device)
    g.manual_seed(s)
    out_dtype = torch.float32 if workload == "tiny" else torch.bfloat16
    if role == "dY" and workload == "llama7b":
        z = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        chi = torch.zeros(shape, device=device, dtype=torch.float32)
        for _ in range(3):
            chi += torch.randn(shape, generator=g, device=device, dtype=torch.float32) ** 2
        x = z / torch.sqrt(chi / 3.0) * (GRAD_STD / math.sqrt(3.0))
        del chi, z
    else:
        std = {"X": 1.0, "W": W_STD[workload], "dY": GRAD_STD}[role]
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32) * std
        if role == "X" and workload != "tiny":
            cols = torch.from_numpy(outlier_columns(shape[1], s + 3)).to(device)
            x[:, cols] *= OUTLIER_GAIN
    return x.to(out_dtype)
