"""Helpers for the GPU parity tests (imported by tests only).

Inputs are the seeded synthetic workloads of ``synth``; the oracle runs in
float64 on exactly the float32 arrays that the GPU receives.
"""
from __future__ import annotations

import math
import sys

import numpy as np


def rel(a, b):
    """Relative Frobenius error ||a - b|| / ||b||."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def row_err(a, b, floor=0.1):
    """Worst row-relative error, max over rows i of
    ||a_i - b_i|| / max(||b_i||, floor * RMS_j ||b_j||).

    A 2-D array's rows are its last-axis vectors; a 1-D array's elements are
    rows of one entry.  Rows whose reference norm is below ``floor`` times
    the RMS row norm are measured against that floor instead (an absolute
    tolerance there), so an error confined to one element or one tile edge
    fails the bar instead of vanishing into a whole-array norm."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if b.ndim <= 1:
        a, b = a.reshape(-1, 1), b.reshape(-1, 1)
    else:
        a, b = a.reshape(-1, b.shape[-1]), b.reshape(-1, b.shape[-1])
    nb = np.linalg.norm(b, axis=1)
    rms = float(np.sqrt(np.mean(nb * nb))) if nb.size else 0.0
    den = np.maximum(nb, floor * rms)
    den[den == 0] = 1.0
    return float(np.max(np.linalg.norm(a - b, axis=1) / den)) if nb.size else 0.0


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def torch_dev():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("GPU test run without a visible GPU")
    return torch, torch.device("cuda:0")


def to_gpu(x, dtype=None):
    torch, dev = torch_dev()
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(dev).contiguous()


def empty(shape, dtype="f32"):
    torch, dev = torch_dev()
    dt = {"f32": torch.float32, "i32": torch.int32}[dtype]
    return torch.full(shape, float("nan") if dtype == "f32" else -7, dtype=dt, device=dev)


def workspace(nbytes):
    torch, dev = torch_dev()
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=dev)


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().cpu().numpy()


def pack(rows_per_problem, arrays):
    """Concatenate per-problem [k_p, d] arrays into packed [sum k, d]."""
    return np.ascontiguousarray(np.concatenate([a[:k] for a, k in zip(arrays, rows_per_problem)]))


def unpack(packed, ks):
    out, o = [], 0
    for k in ks:
        out.append(packed[o:o + k])
        o += k
    return out
