"""ctypes binding of libtilegemm.so: argument marshalling only.

Every function here forwards to the C ABI declared in include/tilegemm.h.  The
library must have been built (``python -m tile_shape_autotuning_amd.build_lib``
or ``__graft_entry__.build()``); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libtilegemm.so")

F32, BF16, BF16_F32OUT = 0, 1, 2
ACT = {"none": 0, "relu": 1, "gelu": 2}

TG_OK, TG_E_INVAL, TG_E_INFEASIBLE, TG_E_UNSUPPORTED, TG_E_HIP, TG_E_NOMEM, TG_E_CACHE = 0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "TG_OK", -1: "TG_E_INVAL", -2: "TG_E_INFEASIBLE", -3: "TG_E_UNSUPPORTED",
                -4: "TG_E_HIP", -5: "TG_E_NOMEM", -6: "TG_E_CACHE"}

# every symbol include/tilegemm.h declares
EXPORTS = [
    "tg_last_error", "tg_version", "tg_set_stream", "gemm_bias_act", "gemm_autotune", "gemm_autotune_ep",
    "gemm_bias_act_noalloc", "tg_noalloc_scratch_bytes",
    "tg_enumerate", "tg_space", "tg_check_cfg", "tg_model_time", "tg_model_times", "tg_model_choice", "tg_grid",
    "tg_default_cfg", "tg_resources", "tg_set_device_override", "tg_get_device_desc",
    "tg_builtin_device_desc", "tg_kernel_count", "tg_has_kernel", "tg_kernel_resources", "tg_streams_b",
    "tg_autotune_table", "tg_cache_lookup", "tg_cache_save", "tg_cache_load", "tg_cache_clear",
    "tg_cache_size", "tg_stats", "tg_set_shape_buckets", "tg_dispatch_m", "tg_set_tile_order", "tg_tile_order",
    "tg_rmsnorm", "tg_rmsnorm_autotune", "tg_rmsnorm_cache_lookup", "tg_rmsnorm_tunes",
]


class Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("kind", "bm", "bn", "bk", "wgm", "wgn", "stages", "split_k")]

    def astuple(self):
        return tuple(getattr(self, n) for n, _ in self._fields_)

    @classmethod
    def of(cls, t):
        if isinstance(t, Cfg):
            return t
        if hasattr(t, "astuple"):
            t = t.astuple()
        return cls(*[int(x) for x in t])

    def __repr__(self):
        return "Cfg(kind=%d, bm=%d, bn=%d, bk=%d, wgm=%d, wgn=%d, stages=%d, split_k=%d)" % self.astuple()

    def __eq__(self, other):
        try:
            return self.astuple() == Cfg.of(other).astuple()
        except Exception:
            return NotImplemented

    def __hash__(self):
        return hash(self.astuple())


class DeviceDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("mode", "n_cu", "simds", "lds_cu", "lds_block", "max_threads",
                                              "waves_max", "blocks_max", "vgpr_max", "acc_max", "r0", "reserved")] + \
               [(n, ctypes.c_double) for n in ("peak_bf16", "peak_f32", "bw", "a_ref", "c_fill", "t0",
                                               "unaligned_eff", "lat_mem", "cu_bw", "lds_bw_cu", "lat_step", "lat_l2",
                                               "l2_bytes", "w1_eff", "skinny_eff", "hbm_eff", "sliced_eff")]


class TuneRow(ctypes.Structure):
    _fields_ = [("cfg", Cfg), ("predicted_us", ctypes.c_double), ("measured_us", ctypes.c_double),
                ("confirmed_us", ctypes.c_double)]


class TileGemmError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


_lib = None


def lib():
    """Load the native library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} not found: build it with `python -m tile_shape_autotuning_amd.build_lib`")
        L = ctypes.CDLL(LIB_PATH)
        i64, i32, vp, dp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.POINTER(ctypes.c_double)
        pc = ctypes.POINTER(Cfg)
        pi = ctypes.POINTER(ctypes.c_int)
        pi64 = ctypes.POINTER(ctypes.c_int64)
        sig = {
            "tg_last_error": ([], ctypes.c_char_p),
            "tg_version": ([], i32),
            "tg_set_stream": ([vp], i32),
            "gemm_bias_act": ([i64, i64, i64, vp, vp, vp, vp, i32, i32, pc], i32),
            "gemm_autotune": ([i64, i64, i64, i32, pc], i32),
            "gemm_bias_act_noalloc": ([i64, i64, i64, vp, vp, vp, vp, i32, i32, pc], i32),
            "tg_noalloc_scratch_bytes": ([], ctypes.c_size_t),
            "gemm_autotune_ep": ([i64, i64, i64, i32, i32, i32, pc], i32),
            "tg_enumerate": ([i64, i64, i64, i32, pc, i32, pi], i32),
            "tg_space": ([i32, pc, i32, pi], i32),
            "tg_check_cfg": ([i64, i64, i64, i32, pc, pi], i32),
            "tg_model_time": ([i64, i64, i64, i32, pc, dp], i32),
            "tg_model_choice": ([i64, i64, i64, i32, pc, dp], i32),
            "tg_model_times": ([i64, i64, i64, i32, pc, i32, dp], i32),
            "tg_grid": ([i64, i64, i64, pc, pi64, pi64], i32),
            "tg_default_cfg": ([i64, i64, i64, i32, pc], i32),
            "tg_resources": ([i32, pc, pi, pi, pi], i32),
            "tg_set_device_override": ([ctypes.POINTER(DeviceDesc)], i32),
            "tg_get_device_desc": ([ctypes.POINTER(DeviceDesc)], i32),
            "tg_builtin_device_desc": ([i32, ctypes.POINTER(DeviceDesc)], i32),
            "tg_kernel_count": ([], i32),
            "tg_has_kernel": ([i32, pc], i32),
            "tg_kernel_resources": ([i32, pc, pi], i32),
            "tg_streams_b": ([i64, i32, pc, pi], i32),
            "tg_autotune_table": ([i64, i64, i64, i32, i32, i32, ctypes.POINTER(TuneRow), i32, pi], i32),
            "tg_cache_lookup": ([i64, i64, i64, i32, i32, i32, pc, dp, pi], i32),
            "tg_cache_save": ([ctypes.c_char_p], i32),
            "tg_cache_load": ([ctypes.c_char_p, pi, pi], i32),
            "tg_cache_clear": ([], None),
            "tg_cache_size": ([], i32),
            "tg_stats": ([pi64, pi64, pi64], i32),
            "tg_set_shape_buckets": ([i32], i32),
            "tg_set_tile_order": ([i32], i32),
            "tg_tile_order": ([], i32),
            "tg_dispatch_m": ([i64, pi64], i32),
            "tg_rmsnorm": ([i64, i64, vp, vp, vp, ctypes.c_float, i32], i32),
            "tg_rmsnorm_autotune": ([i64, i64, pi, dp], i32),
            "tg_rmsnorm_cache_lookup": ([i64, i64, pi, dp, pi], i32),
            "tg_rmsnorm_tunes": ([pi64], i32),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def last_error() -> str:
    return lib().tg_last_error().decode()


def check(status: int):
    if status != TG_OK:
        raise TileGemmError(status, last_error())


# ---------------------------------------------------------------- compute
def set_stream(stream_handle: int | None):
    check(lib().tg_set_stream(stream_handle or None))


def gemm_bias_act_ptr(M, N, K, A, B, bias, C, dtype, act, cfg=None) -> int:
    """Raw C-ABI call with device addresses (ints); returns the status."""
    c = None if cfg is None else ctypes.byref(Cfg.of(cfg))
    a = ACT[act] if isinstance(act, str) else int(act)
    return lib().gemm_bias_act(M, N, K, A or None, B or None, bias or None, C or None, int(dtype), a, c)


def gemm_bias_act_noalloc_ptr(M, N, K, A, B, bias, C, dtype, act, cfg=None) -> int:
    """Raw C-ABI call of the entry point that allocates nothing (device
    addresses as ints); returns the status."""
    c = None if cfg is None else ctypes.byref(Cfg.of(cfg))
    a = ACT[act] if isinstance(act, str) else int(act)
    return lib().gemm_bias_act_noalloc(M, N, K, A or None, B or None, bias or None, C or None, int(dtype), a, c)


def noalloc_scratch_bytes() -> int:
    return int(lib().tg_noalloc_scratch_bytes())


def _act(act) -> int:
    return ACT[act] if isinstance(act, str) else int(act)


def gemm_autotune(M, N, K, dtype, act="none", bias=False) -> Cfg:
    """Tune (or look up) the call of this shape with activation `act` and,
    if `bias`, a bias vector: gemm_autotune for the plain call, else
    gemm_autotune_ep."""
    out = Cfg()
    if _act(act) == 0 and not bias:
        check(lib().gemm_autotune(M, N, K, int(dtype), ctypes.byref(out)))
    else:
        check(lib().gemm_autotune_ep(M, N, K, int(dtype), _act(act), 1 if bias else 0, ctypes.byref(out)))
    return out


# ---------------------------------------------------------------- selection queries
def enumerate_feasible(M, N, K, dtype):
    n = ctypes.c_int()
    check(lib().tg_enumerate(M, N, K, int(dtype), None, 0, ctypes.byref(n)))
    buf = (Cfg * max(1, n.value))()
    check(lib().tg_enumerate(M, N, K, int(dtype), buf, n.value, ctypes.byref(n)))
    return [buf[i] for i in range(n.value)]


def space(dtype):
    n = ctypes.c_int()
    check(lib().tg_space(int(dtype), None, 0, ctypes.byref(n)))
    buf = (Cfg * max(1, n.value))()
    check(lib().tg_space(int(dtype), buf, n.value, ctypes.byref(n)))
    return [buf[i] for i in range(n.value)]


def check_cfg(M, N, K, dtype, cfg) -> int:
    r = ctypes.c_int()
    check(lib().tg_check_cfg(M, N, K, int(dtype), ctypes.byref(Cfg.of(cfg)), ctypes.byref(r)))
    return r.value


def model_time_us(M, N, K, dtype, cfg) -> float:
    us = ctypes.c_double()
    check(lib().tg_model_time(M, N, K, int(dtype), ctypes.byref(Cfg.of(cfg)), ctypes.byref(us)))
    return us.value


def model_times_us(M, N, K, dtype, cfgs):
    """Model times (us) of many configurations in one call; -1 where infeasible."""
    n = len(cfgs)
    buf = (Cfg * max(1, n))(*[Cfg.of(c) for c in cfgs])
    out = (ctypes.c_double * max(1, n))()
    check(lib().tg_model_times(M, N, K, int(dtype), buf, n, out))
    return [out[i] for i in range(n)]


def model_choice(M, N, K, dtype):
    out, us = Cfg(), ctypes.c_double()
    check(lib().tg_model_choice(M, N, K, int(dtype), ctypes.byref(out), ctypes.byref(us)))
    return out, us.value


def grid(M, N, K, cfg):
    t, b = ctypes.c_int64(), ctypes.c_int64()
    check(lib().tg_grid(M, N, K, ctypes.byref(Cfg.of(cfg)), ctypes.byref(t), ctypes.byref(b)))
    return t.value, b.value


def default_cfg(M, N, K, dtype) -> Cfg:
    out = Cfg()
    check(lib().tg_default_cfg(M, N, K, int(dtype), ctypes.byref(out)))
    return out


def resources(dtype, cfg):
    lds, v, b = ctypes.c_int(), ctypes.c_int(), ctypes.c_int()
    check(lib().tg_resources(int(dtype), ctypes.byref(Cfg.of(cfg)), ctypes.byref(lds), ctypes.byref(v),
                             ctypes.byref(b)))
    return lds.value, v.value, b.value


def builtin_device_desc(which: int) -> DeviceDesc:
    d = DeviceDesc()
    check(lib().tg_builtin_device_desc(which, ctypes.byref(d)))
    return d


def set_device_override(desc: DeviceDesc | None):
    check(lib().tg_set_device_override(ctypes.byref(desc) if desc is not None else None))


def get_device_desc() -> DeviceDesc:
    d = DeviceDesc()
    check(lib().tg_get_device_desc(ctypes.byref(d)))
    return d


def kernel_count() -> int:
    return lib().tg_kernel_count()


def has_kernel(dtype, cfg) -> bool:
    return bool(lib().tg_has_kernel(int(dtype), ctypes.byref(Cfg.of(cfg))))


def kernel_resources(dtype, cfg):
    """(vgpr, agpr, scratch bytes per lane, lds bytes, occupancy) of the compiled kernel."""
    r = (ctypes.c_int * 5)()
    check(lib().tg_kernel_resources(int(dtype), ctypes.byref(Cfg.of(cfg)), r))
    return tuple(r)


def streams_b(M, dtype, cfg) -> bool:
    """Whether a call of M rows with cfg reads B with the non-temporal policy."""
    r = ctypes.c_int()
    check(lib().tg_streams_b(int(M), int(dtype), ctypes.byref(Cfg.of(cfg)), ctypes.byref(r)))
    return bool(r.value)


# ---------------------------------------------------------------- cache
def autotune_table(M, N, K, dtype, act="none", bias=False):
    """Rows of the last tuning run for the key: (cfg, model us, median of the
    short samples, median of the long confirmation samples); -1 where not
    measured or not confirmed."""
    n = ctypes.c_int()
    a, b = _act(act), 1 if bias else 0
    check(lib().tg_autotune_table(M, N, K, int(dtype), a, b, None, 0, ctypes.byref(n)))
    buf = (TuneRow * max(1, n.value))()
    check(lib().tg_autotune_table(M, N, K, int(dtype), a, b, buf, n.value, ctypes.byref(n)))
    return [(buf[i].cfg, buf[i].predicted_us, buf[i].measured_us, buf[i].confirmed_us) for i in range(n.value)]


def cache_lookup(M, N, K, dtype, act="none", bias=False):
    out, us, hit = Cfg(), ctypes.c_double(), ctypes.c_int()
    check(lib().tg_cache_lookup(M, N, K, int(dtype), _act(act), 1 if bias else 0, ctypes.byref(out),
                                ctypes.byref(us), ctypes.byref(hit)))
    return (out, us.value) if hit.value else None


def cache_save(path: str):
    check(lib().tg_cache_save(path.encode()))


def cache_load(path: str):
    a, b = ctypes.c_int(), ctypes.c_int()
    check(lib().tg_cache_load(path.encode(), ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def cache_clear():
    lib().tg_cache_clear()


def cache_size() -> int:
    return lib().tg_cache_size()


def set_tile_order(group_m: int):
    """Tile rows per scheduling group (0: the default)."""
    check(lib().tg_set_tile_order(int(group_m)))


def tile_order() -> int:
    return lib().tg_tile_order()


def set_shape_buckets(on: bool):
    """Key calls without a cfg on M's shape bucket (on) or on M itself (off)."""
    check(lib().tg_set_shape_buckets(1 if on else 0))


def dispatch_m(M: int) -> int:
    """The M a call without a cfg is keyed and tuned on."""
    k = ctypes.c_int64()
    check(lib().tg_dispatch_m(int(M), ctypes.byref(k)))
    return k.value


def rmsnorm_ptr(rows: int, n: int, x: int, w: int, y: int, eps: float, occupancy: int) -> int:
    """Raw C-ABI call on device pointers; returns the status."""
    return lib().tg_rmsnorm(int(rows), int(n), x or None, w or None, y or None, float(eps), int(occupancy))


def rmsnorm_autotune(rows: int, n: int):
    """(occupancy, measured us) chosen for the shape; tunes on a cache miss."""
    occ, us = ctypes.c_int(), ctypes.c_double()
    check(lib().tg_rmsnorm_autotune(int(rows), int(n), ctypes.byref(occ), ctypes.byref(us)))
    return occ.value, us.value


def rmsnorm_cache_lookup(rows: int, n: int):
    """(occupancy, measured us) if the shape is cached on the current device, else None."""
    occ, us, hit = ctypes.c_int(), ctypes.c_double(), ctypes.c_int()
    check(lib().tg_rmsnorm_cache_lookup(int(rows), int(n), ctypes.byref(occ), ctypes.byref(us), ctypes.byref(hit)))
    return (occ.value, us.value) if hit.value else None


def rmsnorm_tunes() -> int:
    k = ctypes.c_int64()
    check(lib().tg_rmsnorm_tunes(ctypes.byref(k)))
    return k.value


def stats():
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    check(lib().tg_stats(ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return {"tunes": a.value, "timed_launches": b.value, "cache_hits": c.value}
