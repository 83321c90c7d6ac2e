"""Python driver for the fp64 GEMM oracle in ``gemm_ref.c`` -- TEST INFRASTRUCTURE ONLY.

``gemm`` returns the full float64 product; ``gemm_entries`` returns chosen
entries only, for sampled parity checks at sizes where the full product would
take too long.  Both compute C = act(A @ B + bias) with every product and sum
in double precision (page "Tile Selection: Cost Models Against Measurement",
"The structure of the search space"; fused epilogue from page "Tiling the
hierarchy", fusion section).

Inputs are float32 arrays, or uint16 arrays holding bf16 bit patterns.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

from . import build as _build

_lib = None

ACT = {"none": 0, "relu": 1, "gelu": 2}


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        i64, vp, ip = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.oracle_gemm.argtypes = [i64, i64, i64, vp, vp, ip, vp, ip, vp]
        lib.oracle_gemm.restype = ip
        lib.oracle_gemm_entries.argtypes = [i64, i64, i64, vp, vp, ip, vp, ip, i64, vp, vp, vp]
        lib.oracle_gemm_entries.restype = ip
        lib.oracle_num_threads.restype = ip
        lib.oracle_set_threads.argtypes = [ip]
        _lib = lib
    return _lib


def num_threads() -> int:
    return _load().oracle_num_threads()


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def _prep(A, B, bias, act):
    A = np.ascontiguousarray(A)
    B = np.ascontiguousarray(B)
    if A.dtype == np.float32 and B.dtype == np.float32:
        in_bf16 = 0
    elif A.dtype == np.uint16 and B.dtype == np.uint16:
        in_bf16 = 1
    else:
        raise TypeError("A and B must both be float32 or both uint16 (bf16 bits)")
    if A.ndim != 2 or B.ndim != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch {A.shape} x {B.shape}")
    M, K = A.shape
    N = B.shape[1]
    if bias is not None:
        bias = np.ascontiguousarray(bias, dtype=np.float32)
        if bias.shape != (N,):
            raise ValueError("bias must have shape (N,)")
    a = ACT[act] if isinstance(act, str) else int(act)
    return A, B, bias, a, in_bf16, M, N, K


def _ptr(x):
    return None if x is None else x.ctypes.data


def gemm(A, B, bias=None, act="none") -> np.ndarray:
    A, B, bias, a, in_bf16, M, N, K = _prep(A, B, bias, act)
    C = np.empty((M, N), dtype=np.float64)
    rc = _load().oracle_gemm(M, N, K, _ptr(A), _ptr(B), in_bf16, _ptr(bias), a, _ptr(C))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm failed ({rc})")
    return C


def gemm_entries(A, B, rows, cols, bias=None, act="none") -> np.ndarray:
    A, B, bias, a, in_bf16, M, N, K = _prep(A, B, bias, act)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be equal-length 1-D arrays")
    out = np.empty(rows.shape[0], dtype=np.float64)
    rc = _load().oracle_gemm_entries(M, N, K, _ptr(A), _ptr(B), in_bf16, _ptr(bias), a,
                                     rows.shape[0], _ptr(rows), _ptr(cols), _ptr(out))
    if rc != 0:
        raise RuntimeError(f"oracle_gemm_entries failed ({rc})")
    return out
