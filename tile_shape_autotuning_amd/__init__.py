"""tilegemm: fused C = act(A @ B + bias) with per-shape tile selection on
AMD MI355X (gfx950).

The work happens in hand-written HIP kernels behind the C ABI of
include/tilegemm.h (libtilegemm.so); this package marshals PyTorch tensors
(device memory and the current stream) into that ABI.  Nothing computes on
the host: without the built library, importing the binding's entry points
raises.
"""
from __future__ import annotations

from . import _native
from ._native import (ACT, BF16, BF16_F32OUT, F32, Cfg, DeviceDesc, TileGemmError, autotune_table,
                      builtin_device_desc, cache_clear, cache_load, cache_lookup, cache_save, cache_size,
                      check_cfg, default_cfg, enumerate_feasible, gemm_autotune, get_device_desc, grid,
                      has_kernel, kernel_count, kernel_resources, streams_b, model_choice, model_time_us, resources,
                      set_device_override, set_shape_buckets, dispatch_m, space, stats, rmsnorm_autotune,
                      set_tile_order, tile_order,
                      rmsnorm_cache_lookup, rmsnorm_tunes)

__all__ = [
    "gemm_bias_act", "gemm_autotune", "Cfg", "DeviceDesc", "TileGemmError", "F32", "BF16", "BF16_F32OUT",
    "ACT", "enumerate_feasible", "space", "check_cfg", "model_time_us", "model_choice", "grid", "default_cfg",
    "resources", "builtin_device_desc", "set_device_override", "get_device_desc", "kernel_count",
    "has_kernel", "kernel_resources", "streams_b", "autotune_table", "cache_lookup", "cache_save", "cache_load",
    "cache_clear", "cache_size", "stats", "dtype_code", "set_shape_buckets", "dispatch_m", "set_tile_order",
    "tile_order",
    "rmsnorm", "rmsnorm_autotune", "rmsnorm_cache_lookup", "rmsnorm_tunes",
]


def dtype_code(in_dtype, out_dtype=None) -> int:
    """tg_dtype for torch input/output dtypes."""
    import torch
    if in_dtype == torch.float32:
        if out_dtype not in (None, torch.float32):
            raise TypeError("fp32 inputs produce fp32 output")
        return F32
    if in_dtype == torch.bfloat16:
        if out_dtype in (None, torch.bfloat16):
            return BF16
        if out_dtype == torch.float32:
            return BF16_F32OUT
        raise TypeError("bf16 inputs produce bf16 or fp32 output")
    raise TypeError(f"unsupported input dtype {in_dtype}")


class BoundGemm:
    """A gemm_bias_act call with its arguments marshalled once.

    Calling it issues exactly the C-ABI call ``gemm_bias_act`` (key lookup,
    launch) on the stream that was current when it was bound; for loops where
    per-call Python checks would dominate a microsecond-scale kernel.
    """

    def __init__(self, A, B, bias=None, act="none", out=None, out_dtype=None, cfg=None):
        import ctypes
        import torch
        self.out = gemm_bias_act(A, B, bias, act, out, out_dtype, cfg)   # validates, tunes if needed
        self._keep = (A, B, bias, self.out)
        M, K = A.shape
        N = B.shape[1]
        code = dtype_code(A.dtype, self.out.dtype)
        c = None if cfg is None else ctypes.byref(Cfg.of(cfg))
        self._stream = torch.cuda.current_stream(A.device).cuda_stream
        self._args = (M, N, K, A.data_ptr(), B.data_ptr(), bias.data_ptr() if bias is not None else None,
                      self.out.data_ptr(), code, ACT[act] if isinstance(act, str) else int(act), c)
        self._fn = _native.lib().gemm_bias_act

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            _native.check(st)
        return self.out

    def rebind_stream(self):
        _native.set_stream(self._stream)


def gemm_bias_act(A, B, bias=None, act="none", out=None, out_dtype=None, cfg=None):
    """C = act(A @ B + bias) on the GPU through libtilegemm.

    A: [M, K], B: [K, N] (both bfloat16 or both float32, contiguous, same
    CUDA/HIP device); bias: [N] float32 or None; act: "none" | "relu" |
    "gelu"; out_dtype: for bf16 inputs, torch.bfloat16 (default) or
    torch.float32; cfg: a Cfg (or 8-tuple) to force a configuration, else the
    tuned/cached choice.  Runs on the current stream and returns C.
    """
    import torch
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError(f"shape mismatch {tuple(A.shape)} x {tuple(B.shape)}")
    if A.dtype != B.dtype:
        raise TypeError("A and B must have the same dtype")
    if not (A.is_cuda and B.is_cuda) or A.device != B.device:
        raise ValueError("A and B must be on the same GPU")
    if not (A.is_contiguous() and B.is_contiguous()):
        raise ValueError("A and B must be contiguous (row-major)")
    M, K = A.shape
    N = B.shape[1]
    if out is not None and out_dtype is None:
        out_dtype = out.dtype
    code = dtype_code(A.dtype, out_dtype)
    odt = torch.bfloat16 if code == BF16 else torch.float32
    if out is None:
        out = torch.empty((M, N), dtype=odt, device=A.device)
    elif out.shape != (M, N) or out.dtype != odt or not out.is_contiguous() or out.device != A.device:
        raise ValueError("out must be a contiguous [M, N] tensor of the output dtype on A's device")
    if bias is not None:
        if bias.dtype != torch.float32 or bias.shape != (N,) or not bias.is_contiguous() or bias.device != A.device:
            raise ValueError("bias must be a contiguous float32 [N] tensor on A's device")
    with torch.cuda.device(A.device):
        _native.set_stream(torch.cuda.current_stream(A.device).cuda_stream)
        st = _native.gemm_bias_act_ptr(M, N, K, A.data_ptr(), B.data_ptr(),
                                       bias.data_ptr() if bias is not None else 0, out.data_ptr(),
                                       code, act, cfg)
    _native.check(st)
    return out


def rmsnorm(x, w, eps=1e-6, occupancy=0, out=None):
    """y = x / sqrt(mean(x^2, row) + eps) * w on the GPU through libtilegemm.

    x: [rows, n] bfloat16, w: [n] bfloat16 (contiguous, same device, n a
    multiple of 8 up to 32768); occupancy: 1, 2, 4 or 8 workgroups per CU,
    or 0 for the tuned choice (cached per shape).  Runs on the current stream
    and returns y (bfloat16, like x).
    """
    import torch
    if x.dim() != 2 or w.dim() != 1 or w.shape[0] != x.shape[1]:
        raise ValueError(f"shape mismatch {tuple(x.shape)} / {tuple(w.shape)}")
    if x.dtype != torch.bfloat16 or w.dtype != torch.bfloat16:
        raise TypeError("x and w must be bfloat16")
    if not (x.is_cuda and w.is_cuda) or x.device != w.device or not (x.is_contiguous() and w.is_contiguous()):
        raise ValueError("x and w must be contiguous tensors on the same GPU")
    rows, n = x.shape
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like x")
    with torch.cuda.device(x.device):
        _native.set_stream(torch.cuda.current_stream(x.device).cuda_stream)
        st = _native.rmsnorm_ptr(rows, n, x.data_ptr(), w.data_ptr(), out.data_ptr(), eps, occupancy)
    _native.check(st)
    return out
