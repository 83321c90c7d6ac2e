"""The library's native selection rules against the selection oracle (CPU only).

The shared library loads without a GPU; its host-only functions (space,
feasibility, cost model, grid, registry, cache) are called through the C ABI
with a device-description override, and must agree with oracle/select_ref.py
bit for bit: identical candidate spaces and feasible sets, identical
rejection reasons, bitwise-equal float64 model times, identical choices and
block counts.  The H100 replica reproduces the printed numbers of page
"Compilers and Kernel Languages" ("A different tile for every shape")
through the C ABI as well.
"""
import json
import os
import random
import re

import pytest

from oracle import select_ref as S

tg = pytest.importorskip("tile_shape_autotuning_amd")
from tile_shape_autotuning_amd import _native as N  # noqa: E402

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
GOLDEN = os.path.join(ROOT, "tests", "golden", "h100_model_page_results.json")


@pytest.fixture(scope="module", autouse=True)
def mi355x_rules():
    if not os.path.exists(N.LIB_PATH):
        pytest.skip("libtilegemm.so not built")
    N.set_device_override(N.builtin_device_desc(0))
    yield
    N.set_device_override(None)


def _t(c):
    return tuple(c.astuple())


SHAPES = [(256, 256, 256, S.F32), (1000, 1000, 8192, S.BF16_F32OUT), (8192, 8192, 8192, S.BF16),
          (16, 28672, 8192, S.BF16), (4100, 3000, 1000, S.BF16),
          (1, 1, 1, S.F32), (1, 1, 1, S.BF16), (17, 65, 15, S.BF16), (63, 17, 1, S.F32),
          (64, 64, 64, S.BF16_F32OUT), (65, 1000, 4100, S.BF16), (33, 4096, 4096, S.BF16), (5, 8, 0, S.BF16),
          (4096, 4096, 0, S.F32), (48, 512, 96, S.BF16), (2048, 24, 8, S.F32)]


def _random_shapes(n, seed=7):
    rng = random.Random(seed)
    out = []
    for _ in range(n):
        M = rng.choice([rng.randint(1, 80), rng.randint(1, 5000), rng.randint(1, 20000)])
        Nn = rng.choice([rng.randint(1, 80), rng.randint(1, 5000), rng.randint(1, 30000)])
        K = rng.choice([rng.randint(0, 100), rng.randint(1, 9000), 8 * rng.randint(1, 1000)])
        out.append((M, Nn, K, rng.choice([S.F32, S.BF16, S.BF16_F32OUT])))
    return out


def test_library_exports_every_declared_symbol():
    import ctypes
    with open(os.path.join(ROOT, "include", "tilegemm.h")) as f:
        text = f.read()
    declared = set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\);", text, re.M))
    assert {"gemm_bias_act", "gemm_autotune", "tg_enumerate", "tg_cache_save"} <= declared
    lib = ctypes.CDLL(N.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(N.EXPORTS)


def test_version():
    assert N.lib().tg_version() == 3


@pytest.mark.parametrize("dtype", [S.F32, S.BF16, S.BF16_F32OUT])
def test_space_identical(dtype):
    assert [_t(c) for c in N.space(dtype)] == [c.astuple() for c in S.space(dtype)]


@pytest.mark.parametrize("M,Nn,K,dtype", SHAPES + _random_shapes(60))
def test_feasible_set_identical(M, Nn, K, dtype):
    got = [_t(c) for c in N.enumerate_feasible(M, Nn, K, dtype)]
    want = [c.astuple() for c in S.enumerate_feasible(M, Nn, K, dtype)]
    assert got == want


@pytest.mark.parametrize("M,Nn,K,dtype", SHAPES[:8])
def test_rejection_reasons_identical(M, Nn, K, dtype):
    for c in S.space(dtype):
        assert N.check_cfg(M, Nn, K, dtype, c.astuple()) == S.check(M, Nn, K, dtype, c), c


@pytest.mark.parametrize("M,Nn,K,dtype", SHAPES + _random_shapes(40, seed=11))
def test_model_times_bitwise_and_choice(M, Nn, K, dtype):
    feas = S.enumerate_feasible(M, Nn, K, dtype)
    for c in feas:
        assert N.model_time_us(M, Nn, K, dtype, c.astuple()) == S.model_time(M, Nn, K, dtype, c) * 1e6, c
    got, got_us = N.model_choice(M, Nn, K, dtype)
    want, want_t = S.model_choice(M, Nn, K, dtype)
    assert _t(got) == want.astuple()
    assert got_us == want_t * 1e6


@pytest.mark.parametrize("M,Nn,K,dtype", SHAPES)
def test_grid_default_and_resources_identical(M, Nn, K, dtype):
    for c in S.enumerate_feasible(M, Nn, K, dtype)[::7]:
        assert N.grid(M, Nn, K, c.astuple()) == S.grid(M, Nn, c, K=K)
        lds, v, b = N.resources(dtype, c.astuple())
        assert lds == S.lds_bytes(c, dtype)
        assert v == S.vgpr_estimate(c, dtype, S.MI355X)
        assert b == S.blocks_per_cu(c, dtype, S.MI355X)
    assert _t(N.default_cfg(M, Nn, K, dtype)) == S.default_cfg(Nn, K, dtype).astuple()


def test_builtin_descriptions_match_oracle_constants():
    for which, ref in ((0, S.MI355X), (1, S.H100_REPLICA)):
        d = N.builtin_device_desc(which)
        for f in ("mode", "n_cu", "simds", "lds_cu", "lds_block", "max_threads", "waves_max", "blocks_max",
                  "vgpr_max", "acc_max", "r0", "peak_bf16", "peak_f32", "bw", "a_ref", "c_fill", "t0",
                  "unaligned_eff", "lat_mem", "cu_bw", "lds_bw_cu", "lat_step", "lat_l2", "l2_bytes", "w1_eff",
                  "skinny_eff", "hbm_eff", "sliced_eff"):
            assert getattr(d, f) == getattr(ref, f), f


def test_h100_replica_through_the_abi_reproduces_page_numbers():
    with open(GOLDEN) as f:
        g = json.load(f)
    N.set_device_override(N.builtin_device_desc(1))
    try:
        big, small, dec = g["cases"]
        c, us = N.model_choice(big["M"], big["N"], big["K"], S.BF16)
        assert [c.bm, c.bn] == big["best_tile"] and round(us) == big["best_us_rounded"]
        times = {(x.bm, x.bn): N.model_time_us(big["M"], big["N"], big["K"], S.BF16, x)
                 for x in N.enumerate_feasible(big["M"], big["N"], big["K"], S.BF16)}
        assert len(times) == 16
        assert round(max(times.values()) / us, 2) == big["worst_over_best_2dp"]
        assert round(times[(128, 128)] / us, 2) == big["fixed_128x128_over_best_2dp"]
        c, us = N.model_choice(small["M"], small["N"], small["K"], S.BF16)
        assert [c.bm, c.bn] == small["best_tile"]
        fixed = N.model_time_us(small["M"], small["N"], small["K"], S.BF16, (0, 128, 128, 64, 1, 1, 1, 1))
        assert round(fixed / us, 2) == small["fixed_128x128_over_best_2dp"]
        assert N.grid(small["M"], small["N"], small["K"], (0, 128, 128, 64, 1, 1, 1, 1))[0] == small["tiles_at_128x128"]
        ts = {N.model_time_us(dec["M"], dec["N"], dec["K"], S.BF16, x)
              for x in N.enumerate_feasible(dec["M"], dec["N"], dec["K"], S.BF16)}
        assert len(ts) == 1 and round(ts.pop(), 1) == dec["floor_us_1dp"]
    finally:
        N.set_device_override(N.builtin_device_desc(0))


def test_every_instantiable_configuration_has_a_kernel():
    n = 0
    for dtype in (S.F32, S.BF16):
        for c in S.space(dtype):
            # split_k is a run-time value except for the sliced-K kind
            compiled = c.split_k == 1 or c.kind == S.KIND_SLICEDK
            if compiled and S.check_static(dtype, c) == S.OK:
                assert N.has_kernel(dtype, c.astuple()), c
                n += 1
            elif compiled:
                assert not N.has_kernel(dtype, c.astuple()), c
    assert N.kernel_count() == n
    # bf16->fp32 output uses the bf16 kernels
    assert N.has_kernel(S.BF16_F32OUT, (0, 128, 128, 64, 2, 2, 2, 1))


def test_default_configurations_do_not_spill():
    for dtype in (S.F32, S.BF16):
        for K, Nn in ((4096, 4096), (15, 17)):
            c = S.default_cfg(Nn, K, dtype)
            vgpr, agpr, scratch, lds, occ = N.kernel_resources(dtype, c.astuple())
            assert scratch == 0 and vgpr > 0 and occ >= 1, (c, vgpr, agpr, scratch)


def test_error_codes_without_a_device():
    lib = N.lib()
    assert N.gemm_bias_act_ptr(-1, 4, 4, 16, 16, 0, 16, S.BF16, 0) == N.TG_E_INVAL
    assert N.gemm_bias_act_ptr(4, 4, 1 << 22, 16, 16, 0, 16, S.BF16, 0) == N.TG_E_UNSUPPORTED
    assert N.gemm_bias_act_ptr(4, 4, 4, 16, 16, 0, 16, 7, 0) == N.TG_E_INVAL
    assert N.gemm_bias_act_ptr(4, 4, 4, 16, 16, 0, 16, S.BF16, 9) == N.TG_E_INVAL
    assert N.gemm_bias_act_ptr(4, 4, 4, 0, 16, 0, 16, S.BF16, 0) == N.TG_E_INVAL
    assert "NULL" in N.last_error()
    assert N.gemm_bias_act_ptr(0, 4, 4, 0, 0, 0, 0, S.BF16, 0) == N.TG_OK      # empty: nothing to do
    with pytest.raises(N.TileGemmError) as e:
        N.model_time_us(256, 256, 256, S.BF16, (0, 256, 256, 32, 1, 1, 1, 1))   # accumulators exceed 256
    assert e.value.status == N.TG_E_INFEASIBLE
    with pytest.raises(N.TileGemmError):
        N.model_choice(4, 4, -1, S.F32)
    assert lib.tg_set_device_override(N.DeviceDesc()) == N.TG_E_INVAL          # all-zero description
    with pytest.raises(N.TileGemmError):
        N.grid(4, 4, 4, (0, 0, 32, 32, 1, 1, 1, 1))


def test_model_mode_tuning_and_cache_roundtrip(tmp_path, monkeypatch):
    monkeypatch.setenv("TILEGEMM_TUNE_MODE", "model")
    N.cache_clear()
    s0 = N.stats()
    shapes = [(4100, 3000, 1000, S.BF16), (256, 256, 256, S.F32), (16, 28672, 8192, S.BF16)]
    chosen = {}
    for M, Nn, K, dt in shapes:
        c = N.gemm_autotune(M, Nn, K, dt)
        assert _t(c) == S.model_choice(M, Nn, K, dt)[0].astuple()
        chosen[(M, Nn, K, dt)] = _t(c)
        assert _t(N.cache_lookup(M, Nn, K, dt)[0]) == _t(c)
        rows = N.autotune_table(M, Nn, K, dt)
        assert len(rows) == 1 and rows[0][2] == -1.0 and rows[0][3] == -1.0
    assert N.stats()["tunes"] == s0["tunes"] + 3
    # a second call is a cache hit: no new tuning run
    N.gemm_autotune(4100, 3000, 1000, S.BF16)
    assert N.stats()["tunes"] == s0["tunes"] + 3
    with pytest.raises(N.TileGemmError):
        N.gemm_autotune(64, 64, 64, S.BF16, act=7)
    # a different dtype is a different key, and so is a different epilogue
    assert N.cache_lookup(4100, 3000, 1000, S.BF16_F32OUT) is None
    assert N.cache_lookup(4100, 3000, 1000, S.BF16, act="relu", bias=True) is None
    c_ep = N.gemm_autotune(4100, 3000, 1000, S.BF16, act="gelu", bias=True)
    assert N.stats()["tunes"] == s0["tunes"] + 4
    assert _t(N.cache_lookup(4100, 3000, 1000, S.BF16, act="gelu", bias=True)[0]) == _t(c_ep)
    assert N.cache_lookup(4100, 3000, 1000, S.BF16, act="gelu", bias=False) is None
    chosen_ep = {(4100, 3000, 1000, S.BF16, "gelu", True): _t(c_ep)}
    path = str(tmp_path / "cache.txt")
    N.cache_save(path)
    N.cache_clear()
    assert N.cache_size() == 0
    assert N.cache_load(path) == (4, 0)
    for (M, Nn, K, dt), c in chosen.items():
        assert _t(N.cache_lookup(M, Nn, K, dt)[0]) == c
    for (M, Nn, K, dt, act, b), c in chosen_ep.items():
        assert _t(N.cache_lookup(M, Nn, K, dt, act=act, bias=b)[0]) == c
    # lines of another library version are skipped; stale configurations too
    lines = open(path).read().splitlines()
    other = lines[1].split()
    other[2] = "999"
    stale = lines[1].split()
    stale[9:17] = ["0", "256", "256", "32", "1", "1", "1", "1"]
    with open(path, "w") as f:
        f.write("\n".join([lines[0], " ".join(other), " ".join(stale)] + lines[2:]) + "\n")
    N.cache_clear()
    assert N.cache_load(path) == (3, 2)
    # a malformed file is rejected and leaves the cache as it was
    before = N.cache_size()
    bad = tmp_path / "bad.txt"
    bad.write_text(lines[0] + "\nnot a cache line\n")
    with pytest.raises(N.TileGemmError) as e:
        N.cache_load(str(bad))
    assert e.value.status == N.TG_E_CACHE and N.cache_size() == before
    bad.write_text("# something else\n")
    with pytest.raises(N.TileGemmError):
        N.cache_load(str(bad))
    with pytest.raises(N.TileGemmError):
        N.cache_load(str(tmp_path / "missing.txt"))
    N.cache_clear()


def test_tile_order_setting():
    try:
        assert N.tile_order() == 8
        N.set_tile_order(3)
        assert N.tile_order() == 3
        with pytest.raises(N.TileGemmError):
            N.set_tile_order(-1)
        with pytest.raises(N.TileGemmError):
            N.set_tile_order(5000)
        assert N.tile_order() == 3
    finally:
        N.set_tile_order(0)
    assert N.tile_order() == 8


def test_dispatch_keys_follow_the_oracle_buckets():
    try:
        N.set_shape_buckets(True)
        for M in range(0, 600):
            assert N.dispatch_m(M) == S.bucket_m(M), M
        N.set_shape_buckets(False)
        for M in (1, 3, 17, 100, 257):
            assert N.dispatch_m(M) == M
    finally:
        N.set_shape_buckets(True)
    with pytest.raises(N.TileGemmError) as e:
        N.dispatch_m(-1)
    assert e.value.status == N.TG_E_INVAL


def test_rmsnorm_argument_checks_without_a_device():
    assert N.rmsnorm_ptr(4, 12, 0, 0, 0, 1e-6, 1) == N.TG_E_UNSUPPORTED      # n not a multiple of 8
    assert N.rmsnorm_ptr(4, 32776, 0, 0, 0, 1e-6, 1) == N.TG_E_UNSUPPORTED   # n above 32768
    assert N.rmsnorm_ptr(-1, 16, 0, 0, 0, 1e-6, 1) == N.TG_E_INVAL
    assert N.rmsnorm_ptr(4, 16, 0, 0, 0, 1e-6, 5) == N.TG_E_INVAL            # occupancy not 0/1/2/4/8
    assert N.rmsnorm_ptr(4, 16, 0, 0, 0, float("nan"), 1) == N.TG_E_INVAL
    assert N.rmsnorm_ptr(0, 16, 0, 0, 0, 1e-6, 0) == N.TG_OK                  # nothing to do
    assert N.rmsnorm_ptr(4, 16, 0, 0, 0, 1e-6, 1) == N.TG_E_INVAL            # NULL operands


def test_measured_tuning_needs_a_device(monkeypatch):
    monkeypatch.setenv("TILEGEMM_TUNE_MODE", "hybrid")
    N.cache_clear()
    if N.lib().tg_kernel_count() and not _has_gpu():
        with pytest.raises(N.TileGemmError) as e:
            N.gemm_autotune(512, 512, 512, S.BF16)
        assert e.value.status == N.TG_E_UNSUPPORTED


def _has_gpu():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def test_b_streaming_rule():
    """B is read with the non-temporal policy exactly when every element of it
    is read by one workgroup: always for the skinny kind, and for bf16 tiled
    tiles of at most 64 rows when M fits in one tile row."""
    seen = {True: 0, False: 0}
    for dtype in (S.BF16, S.BF16_F32OUT, S.F32):
        for c in tg.space(dtype):
            if not tg.has_kernel(dtype, c):
                continue
            for M in (1, 16, 17, 40, 64, 65, 200):
                got = tg.streams_b(M, dtype, c)
                if c.kind == S.KIND_SKINNY:
                    want = True
                else:
                    want = dtype != S.F32 and c.kind == S.KIND_TILED and c.bm <= 64 and M <= c.bm
                assert got == want, (M, dtype, c.astuple())
                seen[got] += 1
    assert seen[True] > 100 and seen[False] > 100
    with pytest.raises(tg.TileGemmError):
        tg.streams_b(-1, S.BF16, tg.space(S.BF16)[0])


def _cfg_of(key):
    """The configuration an allocation-table key names (split_k = 1, or the
    compiled K groups of a sliced-K kernel)."""
    return key[1:8] + (key[8] if key[1] == S.KIND_SLICEDK else 1,)


def test_allocation_table_matches_the_built_kernels():
    # the oracle's fixed input (oracle/kernel_allocation.json) must describe the
    # kernels this library was built with; refresh it with
    # `python -m oracle.refresh_allocation` after a kernel change
    table = S.allocation_table()
    assert N.kernel_count() == len(table)
    for key, (vgpr, agpr, lds, scratch, occ) in table.items():
        in_bf16, cfg = key[0], _cfg_of(key)
        dt = S.BF16 if in_bf16 else S.F32
        assert N.kernel_resources(dt, cfg) == (vgpr, agpr, scratch, lds, occ), key


def test_spill_rule_through_the_abi():
    for key, v in S.allocation_table().items():
        if v[3] > 0:
            c = _cfg_of(key)
            dt = S.BF16 if key[0] else S.F32
            M = c[1] if c[0] == S.KIND_SKINNY else 1024
            assert N.check_cfg(M, 1024, 1024, dt, c) == S.R_SPILL
