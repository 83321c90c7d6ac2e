"""Helpers for the GPU parity tests: uploads, downloads and the tolerance check.

The oracle values always come from oracle/ on the CPU; nothing here computes
a reference.
"""
import sys

import numpy as np

from tile_shape_autotuning_amd import workloads as wl

# tolerance on max |C_gpu - C_ref| relative to max |C_ref| (fp32 inputs / bf16 inputs)
TOL = {wl.F32: 1e-4, wl.BF16: 1e-2, wl.BF16_F32OUT: 1e-2}


def mark(msg):
    """Name the case about to run on the GPU (flushed, so a lost box still shows it)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def to_dev(x):
    import torch
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def out_f64(C):
    import torch
    return C.to(torch.float64).cpu().numpy() if C.dtype == torch.bfloat16 else C.double().cpu().numpy()


def out_bits(C):
    import torch
    assert C.dtype == torch.bfloat16
    return C.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def rel_err(got, ref):
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    return err, scale


def assert_close(got, ref, dtype, what=""):
    err, scale = rel_err(got, ref)
    tol = TOL[dtype] * scale
    assert err <= tol, f"{what}: max|err| {err:.3e} > {TOL[dtype]:g} * max|C| = {tol:.3e}"
    return err, scale
