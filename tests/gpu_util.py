"""Helpers for the GPU parity tests: device upload and the error metric.

Tolerance metric: max |x - ref| / sqrt(mean(ref^2)) per tensor over all its
elements, separately for the outputs and the final state, against the float64
oracle.  Bars: 1e-4 for fp32 q/k/v, 2e-2 for bf16 q/k/v with fp32 gates,
state and accumulation.
"""
import numpy as np

TOL = {"f32": 1e-4, "bf16": 2e-2}


def rel_err(x, ref):
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(x - ref)) / max(rms, 1e-300))


def to_device(x, qkv_dtype, device="cuda"):
    import torch
    dt = torch.bfloat16 if qkv_dtype == "bf16" else torch.float32
    d = {n: torch.from_numpy(np.ascontiguousarray(x[n])).to(device=device, dtype=dt)
         for n in ("q", "k", "v")}
    for n in ("log_gate", "beta", "h0"):
        d[n] = torch.from_numpy(np.ascontiguousarray(x[n])).to(device)
    return d


def to_numpy(t):
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def oracle_args(x, heads=None):
    """Oracle inputs, optionally restricted to a subset of heads."""
    a = [x[n] for n in ("q", "k", "v", "log_gate", "beta")]
    h0 = x["h0"]
    if heads is not None:
        a = [t[:, :, heads] for t in a]
        h0 = h0[:, heads]
    return a, h0
