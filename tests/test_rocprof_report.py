"""The rocprofv3 harness on synthetic result databases (CPU only).

rocprofv3 writes SQLite files with a `kernels` view (one row per dispatch,
duration in ns) and a `counters_collection` view (one row per dispatch and
counter, possibly several rows per counter that add up).  These tests build
such files by hand, with numbers whose derived figures are known exactly.
"""
import os
import sqlite3

import pytest

from tile_shape_autotuning_amd import rocprof_report as R

GEMM = "void tg::gemm_tiled_dma_kernel<64, 128, 64, 2, 4, 2>(tg::GemmParams)"
COPY = "void at::native::elementwise_kernel<copy>(int)"


def _trace_db(d, rows):
    os.makedirs(d, exist_ok=True)
    c = sqlite3.connect(os.path.join(d, "run_results.db"))
    c.execute("create table kernels (name text, duration integer, grid_x integer)")
    c.executemany("insert into kernels values (?, ?, ?)", [r if len(r) == 3 else (r[0], r[1], 1024) for r in rows])
    c.commit()
    c.close()


def _pmc_db(d, rows):
    os.makedirs(d, exist_ok=True)
    c = sqlite3.connect(os.path.join(d, "run_results.db"))
    c.execute("create table counters_collection (kernel_name text, dispatch_id integer, counter_name text, "
              "value real)")
    c.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    c.commit()
    c.close()


def test_kernel_times_average_per_name(tmp_path):
    d = str(tmp_path / "trace")
    _trace_db(d, [(GEMM, 30000), (GEMM, 40000), (COPY, 1000)])
    t = R.kernel_times(d)
    assert t[GEMM] == (2, 35000.0)
    assert t[COPY] == (1, 1000.0)
    assert "gemm_tiled_dma_kernel" in R.kernel_table(d)
    # the name filter keeps only the matching kernels, with their own averages
    only = R.kernel_table(d, match=("gemm_tiled_dma_kernel",)).splitlines()
    assert len(only) == 2 and "35.000" in only[1] and COPY not in "\n".join(only)


def test_kernel_times_split_one_template_by_grid(tmp_path):
    d = str(tmp_path / "trace")
    # the same kernel serving a big and a small problem in one run
    _trace_db(d, [(GEMM, 900000, 524288), (GEMM, 910000, 524288), (GEMM, 40000, 104448)])
    assert R.kernel_times(d, grid=524288)[GEMM] == (2, 905000.0)
    assert R.kernel_times(d, grid=104448)[GEMM] == (1, 40000.0)
    assert R.kernel_times(d)[GEMM][0] == 3


def test_counters_sum_rows_of_one_dispatch_then_average(tmp_path):
    d = str(tmp_path / "pmc")
    # dispatch 1 reports the counter in two rows (e.g. per XCD); dispatch 2 in one
    _pmc_db(d, [(GEMM, 1, "SQ_WAVES", 3.0), (GEMM, 1, "SQ_WAVES", 5.0), (GEMM, 2, "SQ_WAVES", 4.0)])
    assert R.counters(d)[GEMM]["SQ_WAVES"] == pytest.approx(6.0)


def test_summary_mfma_utilisation_and_rates(tmp_path):
    tr, pmc = str(tmp_path / "t"), str(tmp_path / "p")
    _trace_db(tr, [(GEMM, 50000)] * 4)            # 50 us per launch
    busy_cu = 1.0e6
    _pmc_db(pmc, [(GEMM, 1, "SQ_VALU_MFMA_BUSY_CYCLES", 2.0e6), (GEMM, 1, "SQ_BUSY_CU_CYCLES", busy_cu),
                  (GEMM, 1, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000.0), (GEMM, 1, "SQ_INSTS_LDS", 400.0),
                  (GEMM, 1, "SQ_LDS_BANK_CONFLICT", 100.0), (GEMM, 1, "SQ_WAVE_CYCLES", 1000.0),
                  (GEMM, 1, "SQ_WAIT_ANY", 250.0)])
    s = R.summary(tr, [pmc], kernel="gemm_tiled_dma_kernel<64, 128, 64, 2, 4, 2>", flops=1.0e12, nbytes=4.0e8)
    assert s["avg_us"] == pytest.approx(50.0)
    assert s["TFLOP/s"] == pytest.approx(1.0e12 / 50e-6 / 1e12)
    assert s["GB/s"] == pytest.approx(4.0e8 / 50e-6 / 1e9)
    assert s["mfma_util"] == pytest.approx(2.0e6 / (4 * busy_cu))       # four SIMDs per CU
    assert s["mfma_flops_per_dispatch"] == pytest.approx(1000.0 * 512)
    assert s["lds_conflict_cycles_per_lds_inst"] == pytest.approx(0.25)
    assert s["wait_any_frac"] == pytest.approx(0.25)


def test_hbm_traffic_scaled_by_the_copy_calibration(tmp_path):
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    copy_bytes = 1 << 30
    # the copy reads and writes copy_bytes; its counters read half and exactly that
    _pmc_db(fetch, [(COPY, 1, "FETCH_SIZE", copy_bytes / 1024 / 2), (GEMM, 2, "FETCH_SIZE", 1000.0)])
    _pmc_db(write, [(COPY, 1, "WRITE_SIZE", copy_bytes / 1024), (GEMM, 2, "WRITE_SIZE", 300.0)])
    t = R.hbm_traffic(fetch, write, copy_bytes, kernel="gemm")
    assert t["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert t["FETCH_SIZE"]["bytes"] == pytest.approx(1000.0 * 1024 * 2.0)
    assert t["WRITE_SIZE"]["bytes"] == pytest.approx(300.0 * 1024)
    assert t["bytes"] == pytest.approx(1000.0 * 1024 * 2.0 + 300.0 * 1024)


def test_copy_calibration_ignores_smaller_copies_of_the_same_kernel(tmp_path):
    # three calibration copies of 1 GiB plus the program's own 470 MB copy under
    # the same kernel name: the scale comes from the calibration copies alone
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    copy_bytes = 1 << 30
    half = copy_bytes / 1024 / 2
    fetch_rows = [(COPY, 1, "FETCH_SIZE", half + 8), (COPY, 2, "FETCH_SIZE", half),
                  (COPY, 3, "FETCH_SIZE", half), (COPY, 4, "FETCH_SIZE", 229406.0),
                  (GEMM, 5, "FETCH_SIZE", 1000.0), (GEMM, 6, "FETCH_SIZE", 1002.0)]
    # per-instance rows of one dispatch add up
    write_rows = [(COPY, 1, "WRITE_SIZE", copy_bytes / 2048), (COPY, 1, "WRITE_SIZE", copy_bytes / 2048),
                  (COPY, 4, "WRITE_SIZE", 450000.0), (GEMM, 5, "WRITE_SIZE", 300.0)]
    _pmc_db(fetch, fetch_rows)
    _pmc_db(write, write_rows)
    t = R.hbm_traffic(fetch, write, copy_bytes, kernel="gemm")
    assert t["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert t["FETCH_SIZE"]["kib_raw"] == pytest.approx(1001.0)
    assert t["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    # a mean over every copy dispatch would have given a scale of about 2.3
    per = R.dispatch_counters(fetch)
    assert sorted(per[COPY]["FETCH_SIZE"])[0] == 229406.0
    assert R.copy_calibration(per, "FETCH_SIZE") == pytest.approx(half)


def test_missing_results_raise(tmp_path):
    with pytest.raises(FileNotFoundError):
        R.kernel_times(str(tmp_path / "nothing"))


def test_kernel_names_match_the_template_instances():
    assert R.kernel_name((0, 64, 128, 64, 2, 4, 2, 4)) == "gemm_tiled_dma_kernel<64, 128, 64, 2, 4, 2, false, false, 1>"
    assert R.kernel_name((0, 32, 256, 32, 1, 2, 4, 2), stream_b=True) == \
        "gemm_tiled_dma_kernel<32, 256, 32, 1, 2, 4, true, false, 1>"
    assert R.kernel_name((0, 32, 32, 32, 2, 2, 4, 1), in_bf16=False) == \
        "gemm_tiled_dma_kernel<32, 32, 32, 2, 2, 4, false, true, 1>"
    assert R.kernel_name((4, 16, 32, 64, 1, 1, 2, 4), in_bf16=False) == \
        "gemm_tiled_dma_kernel<16, 32, 64, 1, 1, 2, false, true, 4>"
    assert R.kernel_name((1, 32, 128, 32, 4, 1, 2, 8)) == "gemm_skinny_kernel<2, 4, 2>"


def test_commands_give_one_counter_block_per_pass():
    cmds = R.commands(["--workload", "3", "--only"])
    pmc = [c for c in cmds if "--pmc" in c]
    assert len(pmc) == 3
    for c in pmc:
        ctrs = c.split("--pmc", 1)[1].split("-d", 1)[0].split()
        assert sum(1 for x in ctrs if x.startswith("SQ_")) <= 8
        assert sum(1 for x in ctrs if x.startswith("GRBM_")) <= 2
    assert any("FETCH_SIZE" in c and "WRITE_SIZE" not in c for c in pmc)
    assert any("WRITE_SIZE" in c and "FETCH_SIZE" not in c for c in pmc)


RED = "tg::splitk_reduce_kernel(float const*, int, long, long, int, float const*, void*, int, int, int)"


def test_split_k_calls_count_both_launches(tmp_path):
    tr, fetch, write = str(tmp_path / "t"), str(tmp_path / "f"), str(tmp_path / "w")
    # every call: the GEMM (30 us) then the second pass (5 us, its own grid)
    _trace_db(tr, [(GEMM, 30000, 131072), (RED, 5000, 250112)] * 3 + [(RED, 9000, 4096)])
    copy_bytes = 1 << 30
    _pmc_db(fetch, [(COPY, 1, "FETCH_SIZE", copy_bytes / 1024), (GEMM, 2, "FETCH_SIZE", 1000.0),
                    (RED, 3, "FETCH_SIZE", 400.0)])
    _pmc_db(write, [(COPY, 1, "WRITE_SIZE", copy_bytes / 1024), (GEMM, 2, "WRITE_SIZE", 400.0),
                    (RED, 3, "WRITE_SIZE", 100.0)])
    s = R.summary(tr, [], fetch, write, copy_bytes, kernel="gemm_tiled_dma_kernel", flops=1.0e12, grid=131072,
                  second=("splitk_reduce", 250112))
    assert s["avg_us"] == pytest.approx(30.0)
    assert s["second"]["avg_us"] == pytest.approx(5.0) and s["second"]["calls"] == 3
    assert s["call_us"] == pytest.approx(35.0)
    assert s["TFLOP/s"] == pytest.approx(1.0e12 / 35e-6 / 1e12)
    assert s["traffic"]["bytes"] == pytest.approx((1000.0 + 400.0 + 400.0 + 100.0) * 1024)
    text, _ = R.counters_text("w", (0, 128, 64, 64, 2, 2, 3, 4), "gemm_tiled_dma_kernel", tr, [], fetch, write,
                              copy_bytes, 1.0e12, 0, ["cmd"], 131072, ("splitk_reduce", 250112))
    assert "per call (both launches):   35.000 us" in text


def test_observed_clock_from_busy_cycles():
    # 8 XCDs busy 2.0e6 cycles each over a 1 ms kernel: 2.0 GHz
    assert R.observed_clock_ghz({"GRBM_GUI_ACTIVE": 8 * 2.0e6}, 1000.0) == pytest.approx(2.0)


def test_short_kernels_print_no_busy_cu_or_clock_figure(tmp_path):
    """GRBM_GUI_ACTIVE spans microseconds around each dispatch: the busy-CU
    count and the clock that divide by it are left out below 200 us."""
    from tile_shape_autotuning_amd import rocprof_report as R

    def fake_summary(*a, **k):
        return {"calls": 10, "avg_us": us, "call_us": us, "counters": {"GRBM_GUI_ACTIVE": 8.0e5,
                                                                     "SQ_BUSY_CU_CYCLES": 1.0e7}}
    import pytest as _pt
    mp = _pt.MonkeyPatch()
    mp.setattr(R, "summary", fake_summary)
    try:
        us = 27.0
        text, _ = R.counters_text("w", (0, 1, 1, 1, 1, 1, 1, 1), "k", "t", [], None, None, 0, None, None, [])
        assert "busy CUs" not in text and "clock" not in text
        us = 800.0
        text, _ = R.counters_text("w", (0, 1, 1, 1, 1, 1, 1, 1), "k", "t", [], None, None, 0, None, None, [])
        assert "busy CUs" in text and "clock" in text
    finally:
        mp.undo()


def test_workload_launch_picks_the_dispatches_of_a_workload():
    from tile_shape_autotuning_amd import rocprof_report as R
    # 8192^3 at 256 x 256 with 8 waves: 1024 workgroups of 512 lanes, no second pass
    assert R.workload_launch(3, (0, 256, 256, 64, 2, 4, 2, 1)) == (
        "gemm_tiled_dma_kernel<256, 256, 64, 2, 4, 2, false, false, 1>", 1024 * 512, None)
    # the decode with split 2 streams B (one tile row) and adds a second pass over 16 x 28672 outputs
    name, grid, second = R.workload_launch(4, (0, 64, 256, 32, 2, 4, 4, 2))
    assert name.endswith("true, false, 1>") and grid == 112 * 2 * 512
    assert second == ("splitk_reduce_kernel<2>", 448 * 256)
