"""GPU tests of the measuring autotuner and the shape-keyed cache.

Page "Tile Selection: Cost Models Against Measurement" ("Measurement, and
what it must control"; cache keyed by shape, dtype, device and version) and
page "CuTile Autotuning" (the fixed configuration is always measured, so
tuning never loses to it; correctness with tuning on and off).
"""
import numpy as np
import pytest

from oracle import gemm_ref
from oracle import select_ref as S
from tile_shape_autotuning_amd import workloads as wl

from gpu_util import assert_close, mark, out_f64, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tg = pytest.importorskip("tile_shape_autotuning_amd")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg.set_device_override(None)


def test_autotune_measures_default_and_picks_argmin(monkeypatch):
    monkeypatch.setenv("TILEGEMM_TUNE_MODE", "hybrid")
    M, N, K, dtype = 4100, 3000, 1000, wl.BF16
    tg.cache_clear()
    s0 = tg.stats()
    ep = dict(act="relu", bias=True)       # the epilogue of the call served below
    mark("autotune 4100x3000x1000 bf16")
    c = tg.gemm_autotune(M, N, K, dtype, **ep)
    s1 = tg.stats()
    assert s1["tunes"] == s0["tunes"] + 1 and s1["timed_launches"] > s0["timed_launches"]
    table = tg.autotune_table(M, N, K, dtype, **ep)
    measured = [(row[0].astuple(), row[2]) for row in table if row[2] > 0]
    confirmed = {row[0].astuple(): row[3] for row in table if row[3] > 0}
    assert len(measured) >= 2
    default = S.default_cfg(N, K, dtype).astuple()
    assert default in [m[0] for m in measured], "the fixed default must be measured"
    # the best eight by the short samples and the default are re-timed with long
    # samples, and the choice is the fastest of those
    top8 = [m[0] for m in sorted(measured, key=lambda m: m[1])[:8]]
    assert set(confirmed) == set(top8) | {default}
    best = min(confirmed.items(), key=lambda kv: kv[1])
    assert c.astuple() == best[0]
    assert best[1] <= confirmed[default]
    assert tg.cache_lookup(M, N, K, dtype, **ep)[1] == best[1]
    # every measured candidate is feasible and has a kernel that does not spill
    for cfg, _ in measured:
        assert tg.check_cfg(M, N, K, dtype, cfg) == 0
        assert tg.kernel_resources(dtype, cfg)[2] == 0
    # second request: cache hit, no new tuning
    assert tg.gemm_autotune(M, N, K, dtype, **ep).astuple() == c.astuple()
    assert tg.stats()["tunes"] == s1["tunes"]
    # gemm_bias_act without a cfg serves the cached choice and counts a hit
    A, B, bias = wl.workload_inputs(5)
    mark("cached launch 4100x3000x1000")
    C = tg.gemm_bias_act(to_dev(A), to_dev(B), to_dev(bias), act="relu")
    torch.cuda.synchronize()
    assert tg.stats()["cache_hits"] == s1["cache_hits"] + 1
    rng = np.random.default_rng(1)
    rows, cols = rng.integers(0, M, 2000), rng.integers(0, N, 2000)
    ref = gemm_ref.gemm_entries(A, B, rows, cols, bias, "relu")
    got = out_f64(C)[rows, cols]
    assert_close(got, ref, dtype, "cached choice")


def test_confirmation_stage_off_picks_short_sample_argmin(monkeypatch):
    monkeypatch.setenv("TILEGEMM_TUNE_MODE", "hybrid")
    monkeypatch.setenv("TILEGEMM_TUNE_TOPK", "6")
    monkeypatch.setenv("TILEGEMM_TUNE_CONFIRM", "0")
    M, N, K, dtype = 16, 4096, 2048, wl.BF16
    tg.cache_clear()
    mark("autotune 16x4096x2048 bf16, no confirmation stage")
    c = tg.gemm_autotune(M, N, K, dtype)
    table = tg.autotune_table(M, N, K, dtype)
    assert all(row[3] == -1.0 for row in table)
    measured = [(row[0].astuple(), row[2]) for row in table if row[2] > 0]
    assert c.astuple() == min(measured, key=lambda m: m[1])[0]
    tg.cache_clear()


def test_disable_autotune_uses_model_choice(monkeypatch):
    monkeypatch.setenv("TILEGEMM_DISABLE_AUTOTUNE", "1")
    tg.cache_clear()
    s0 = tg.stats()
    M, N, K, dtype = 1000, 1000, 8192, wl.BF16_F32OUT
    A, B, _ = wl.workload_inputs(2)
    mark("disable-autotune 1000x1000x8192")
    C = tg.gemm_bias_act(to_dev(A), to_dev(B), None, act="none", out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert tg.stats()["tunes"] == s0["tunes"]
    rng = np.random.default_rng(2)
    rows, cols = rng.integers(0, M, 2000), rng.integers(0, N, 2000)
    ref = gemm_ref.gemm_entries(A, B, rows, cols, None, "none")
    assert_close(out_f64(C)[rows, cols], ref, dtype, "model choice")


def test_cache_roundtrip_on_device(tmp_path, monkeypatch):
    monkeypatch.setenv("TILEGEMM_TUNE_MODE", "hybrid")
    monkeypatch.setenv("TILEGEMM_TUNE_TOPK", "4")
    tg.cache_clear()
    mark("autotune 256^3 f32 topk 4")
    c = tg.gemm_autotune(256, 256, 256, wl.F32)
    p = str(tmp_path / "tune.txt")
    tg.cache_save(p)
    tg.cache_clear()
    assert tg.cache_lookup(256, 256, 256, wl.F32) is None
    assert tg.cache_load(p) == (1, 0)
    hit = tg.cache_lookup(256, 256, 256, wl.F32)
    assert hit is not None and hit[0].astuple() == c.astuple() and hit[1] > 0


def test_shape_buckets_one_tuning_per_bucket(monkeypatch):
    # page "Tile Selection: Cost Models Against Measurement", "Hybrid strategies": a varying
    # batch is served by a few tuned variants picked from the real extents, not re-tuned per M
    monkeypatch.setenv("TILEGEMM_TUNE_MODE", "hybrid")
    monkeypatch.setenv("TILEGEMM_TUNE_TOPK", "4")
    N, K, dtype = 2048, 1024, wl.BF16
    rng_seed = 11

    def run(M):
        A, B, bias = wl.make_inputs(M, N, K, dtype, wl.Dist("normal"), wl.Dist("normal"), wl.Dist("normal"),
                                    rng_seed + M)
        mark(f"bucketed dispatch M={M}")
        C = tg.gemm_bias_act(to_dev(A), to_dev(B), to_dev(bias), act="relu")
        torch.cuda.synchronize()
        assert_close(out_f64(C), gemm_ref.gemm(A, B, bias, "relu"), dtype, f"bucketed M={M}")

    try:
        tg.set_shape_buckets(True)
        tg.cache_clear()
        s0 = tg.stats()
        for M in (17, 20, 25, 32):
            assert tg.dispatch_m(M) == 32
            run(M)
        s1 = tg.stats()
        assert s1["tunes"] == s0["tunes"] + 1, "one tuning for the whole bucket"
        assert s1["cache_hits"] == s0["cache_hits"] + 3
        ep = dict(act="relu", bias=True)
        assert tg.cache_lookup(32, N, K, dtype, **ep) is not None and tg.cache_lookup(20, N, K, dtype, **ep) is None
        # the key holds the epilogue the calls ran: the plain call has no entry yet
        assert tg.cache_lookup(32, N, K, dtype) is None
        # buckets off: every M is its own key
        tg.set_shape_buckets(False)
        tg.cache_clear()
        s2 = tg.stats()
        for M in (20, 25):
            assert tg.dispatch_m(M) == M
            run(M)
        assert tg.stats()["tunes"] == s2["tunes"] + 2
    finally:
        tg.set_shape_buckets(True)
        tg.cache_clear()


def test_first_use_tuning_times_the_callers_operands(monkeypatch, capfd):
    """A call without a configuration that misses the cache tunes on copies of
    its own operands (the values set the matrix cores' power draw and so the
    clock); explicit tuning, without operands, on synthetic uniform values."""
    monkeypatch.setenv("TILEGEMM_TUNE_MODE", "hybrid")
    monkeypatch.setenv("TILEGEMM_TUNE_TOPK", "4")
    monkeypatch.setenv("TILEGEMM_LOG", "1")
    tg.cache_clear()
    M, N, K, dtype = 40, 1024, 512, wl.BF16          # M's shape bucket is 48: 8 rows are synthetic
    A, B, bias = wl.make_inputs(M, N, K, dtype, wl.Dist("int", 2), wl.Dist("int", 2), wl.Dist("int", 4), 21)
    mark("first-use tuning 40x1024x512")
    C = tg.gemm_bias_act(to_dev(A), to_dev(B), to_dev(bias), act="relu")
    torch.cuda.synchronize()
    ref = gemm_ref.gemm(A, B, bias, "relu")
    want = wl.f32_to_bf16_bits(ref.astype(np.float32))
    from gpu_util import out_bits
    assert np.array_equal(out_bits(C), want)
    err = capfd.readouterr().err
    assert "tuning 48x1024x512 dt1 on the caller's operands" in err
    mark("explicit tuning 48x2048x512")
    tg.gemm_autotune(48, 2048, 512, dtype)
    assert "on uniform synthetic operands" in capfd.readouterr().err
    tg.cache_clear()
