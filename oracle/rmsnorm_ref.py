"""RMS normalisation, the plain fp64 definition (test infrastructure only).

Only tests/, the package's smoke entry and bench.py's CPU-baseline leg use this
module; the library never calls it.

Page "CuTile Autotuning" ("Quick Reference -- Occupancy-Only Autotune") names
normalisation kernels among those whose only tuned parameter is occupancy.
The operation itself is the standard one (the pages give no formula):

    y[r, j] = x[r, j] / sqrt(mean_j(x[r, j]^2) + eps) * w[j]

Inputs are bf16 bit patterns (uint16) or floats; the result is fp64.
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def rmsnorm(x, w, eps: float):
    """Row-wise RMS normalisation times the weight vector, in fp64."""
    xf = bf16_to_f64(x)
    wf = bf16_to_f64(w)
    if xf.ndim != 2 or wf.shape != (xf.shape[1],):
        raise ValueError("x must be [rows, n] and w [n]")
    ms = np.mean(xf * xf, axis=1, keepdims=True)
    return xf / np.sqrt(ms + float(eps)) * wf[None, :]
