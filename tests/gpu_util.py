"""Helpers for the GPU parity tests: device copies and the fp tolerance gate."""
from __future__ import annotations

import numpy as np

# fp32-accumulation gate (reading of "max relative error <= 2e-3 vs fp64"):
# relative error with the denominator floored at 1% of the rms of the
# reference, so outputs that are almost exactly zero do not make the ratio
# unbounded.  Integer paths are compared bit-exactly instead.
FP_TOL = 2e-3


def fp_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    den = np.maximum(np.abs(ref), 1e-2 * rms if rms > 0 else 1e-30)
    return float(np.max(np.abs(got - ref) / den))


def fp_errors(got: np.ndarray, ref: np.ndarray):
    """(gated error, unfloored element-wise max |x-r|/|r| over r != 0,
    normwise max|x-r| / max|r|)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0, 0.0, 0.0
    diff = np.abs(got - ref)
    nz = ref != 0
    unfloored = float(np.max(diff[nz] / np.abs(ref[nz]))) if np.any(nz) else 0.0
    if np.any(~nz & (diff > 0)):
        unfloored = float("inf")
    mx = float(np.max(np.abs(ref)))
    normwise = float(np.max(diff)) / mx if mx > 0 else float(np.max(diff))
    return fp_rel_err(got, ref), unfloored, normwise


def torch_dev():
    import torch

    return torch, torch.device("cuda:0")


def to_dev(a: np.ndarray):
    torch, dev = torch_dev()
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def empty_dev(shape, dtype):
    torch, dev = torch_dev()
    return torch.empty(shape, dtype=dtype, device=dev)


def workspace_for(nbytes: int):
    """A zero-filled device workspace of nbytes (None when no workspace is needed)."""
    if nbytes == 0:
        return None
    torch, dev = torch_dev()
    return torch.zeros(nbytes, dtype=torch.uint8, device=dev)


def sync():
    import torch

    torch.cuda.synchronize()


def to_host(t) -> np.ndarray:
    sync()
    return t.cpu().numpy()


def strided(a: np.ndarray, ld: int, fill=0) -> np.ndarray:
    """Embed a 2-D array in rows of length ld (>= a.shape[1])."""
    out = np.full((a.shape[0], ld), fill, a.dtype)
    out[:, : a.shape[1]] = a
    return out
