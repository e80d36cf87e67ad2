"""Helpers for the GPU parity tests: move host inputs and oracle results to
the device and GPU results back, print what names each case before it runs."""
import sys

import numpy as np


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def to_device(x_host, device="cuda"):
    """numpy fp32 or bf16 bits (uint16) -> torch device tensor (float32 / bfloat16)."""
    import torch
    if x_host.dtype == np.uint16:
        return torch.from_numpy(x_host.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(x_host).to(device)


def to_host(x):
    """torch device tensor -> numpy (bf16 as uint16 bits)."""
    import torch
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).cpu().numpy().view(np.uint16)
    return x.cpu().numpy()


def q_to_host(q):
    import fp4_fully_quantized_amd as fp4
    d = {"codes": q.codes.cpu().numpy(), "scales": q.scales.cpu().numpy(), "fmt": q.fmt,
         "rows": q.rows, "cols": q.cols}
    if q.fmt == fp4.FP4_NVFP4:
        d["amax"] = float(q.amax.cpu()[0])
        d["sg"] = float(q.tscale.cpu()[0])
    else:
        d["amax"], d["sg"] = None, 1.0
    return d


def q_from_oracle(qo, had_signs=None, device="cuda"):
    """Upload an oracle quantization into a device QTensor (oracle -> GPU only)."""
    import torch
    import fp4_fully_quantized_amd as fp4
    q = fp4.QTensor(qo["rows"], qo["cols"], qo["fmt"], device=device, had_signs=had_signs)
    q.codes.copy_(torch.from_numpy(np.ascontiguousarray(qo["codes"])))
    q.scales.copy_(torch.from_numpy(np.ascontiguousarray(qo["scales"])))
    if qo["fmt"] == fp4.FP4_NVFP4:
        q.amax.fill_(qo["amax"])
        q.tscale.fill_(qo["sg"])
    return q


def assert_same_quant(got, want, what=""):
    assert got["codes"].shape == want["codes"].shape, what
    bad = np.argwhere(got["codes"] != want["codes"])
    assert bad.size == 0, f"{what}: {len(bad)} code bytes differ, first at {bad[:5].tolist()}"
    bad = np.argwhere(got["scales"] != want["scales"])
    assert bad.size == 0, f"{what}: {len(bad)} scale bytes differ, first at {bad[:5].tolist()}"
    if want["fmt"] == 0:
        assert got["amax"] == want["amax"], what
        assert got["sg"] == want["sg"], what
