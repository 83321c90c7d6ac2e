"""Host-side logic of bench.py (CPU only): the multi-GPU refusal, the
warm-up loop and the lookup of recorded HBM traffic."""
import os
import subprocess
import sys
import time

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


class _FakeCuda:
    def synchronize(self):
        pass


class _FakeTorch:
    cuda = _FakeCuda()


def test_warm_up_runs_at_least_min_steps_and_min_time():
    calls = []

    def step():
        calls.append(1)
        time.sleep(0.0005)

    t0 = time.perf_counter()
    n = bench.warm_up(step, 7, _FakeTorch(), min_seconds=0.03)
    assert n == len(calls) and n >= 7
    assert time.perf_counter() - t0 >= 0.03
    # a slow first batch needs no more steps
    calls.clear()
    n = bench.warm_up(lambda: (calls.append(1), time.sleep(0.02)), 3, _FakeTorch(), min_seconds=0.01)
    assert n == 3 == len(calls)


def _traffic_lines():
    with open(bench.TRAFFIC_FILE) as f:
        return [dict(t.split("=", 1) for t in line.split()[1:]) for line in f if line.startswith("traffic ")]


def test_recorded_traffic_is_used_only_for_matching_sources(monkeypatch):
    rows = _traffic_lines()
    assert rows, "profiles/hbm_traffic.txt holds records"
    kv = rows[0]
    cfg = [int(x) for x in kv["cfg"].split(",")]
    from tile_shape_autotuning_amd import build_lib
    if kv["kernel_src_sha256"] != build_lib.kernel_source_digest():
        pytest.skip("records were taken with other kernel sources")
    got = bench.measured_traffic(kv["workload"], cfg)
    assert got == int(float(kv["fetch_bytes"]) + float(kv["write_bytes"]))
    assert bench.measured_traffic(kv["workload"], cfg[:-1] + [cfg[-1] + 1]) is None
    monkeypatch.setattr(build_lib, "kernel_source_digest", lambda: "0" * 64)
    assert bench.measured_traffic(kv["workload"], cfg) is None


def test_persisted_report_matches_persisted_cache():
    """The tuning report shipped beside the persisted cache describes the runs
    that chose the cache's entries."""
    import json
    from tile_shape_autotuning_amd import workloads as wl
    with open(bench.DEFAULT_REPORT) as f:
        rep = json.load(f)
    with open(bench.DEFAULT_CACHE) as f:
        entries = [line.split() for line in f if line.startswith("gfx950")]
    # arch, CUs, version, M, N, K, dtype, act, bias, cfg (8 fields), measured us, predicted us
    cfg_of = {tuple(int(x) for x in e[3:9]): [int(x) for x in e[9:17]] for e in entries}
    for w in wl.WORKLOADS.values():
        r = rep["report"][w.name]
        key = (w.M, w.N, w.K, w.dtype, w.act, int(w.bias_dist is not None))
        assert r["chosen"]["cfg"] == cfg_of[key], w.name
        assert r["worst_over_best"] >= 1.0 and r["fixed_over_best"] >= 1.0
    out = bench.persisted_report({})
    assert set(out["workloads"]) == {w.name for w in wl.WORKLOADS.values()}
