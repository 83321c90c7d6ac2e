#!/usr/bin/env python3
"""Benchmark of the autotuned fused GEMM on one MI355X.

A step is one call of gemm_bias_act (cached autotuned configuration: key
lookup, launch geometry, the GEMM kernel, plus the second pass when the
configuration splits K) on inputs already resident in HBM.  The headline line
times the largest workload, the 8192^3 bf16 multiply with bias and GELU
(compute-bound); the other four workloads are reported under "shapes" with
their own throughput and roofline fraction.

Every workload is also timed, in the same run, with the fixed 128 x 128
default configuration and with the cost model's first choice: the ratios
fixed/tuned and model/tuned and the model's hit rate in the line are measured
here (page "Tile Selection: Cost Models Against Measurement", "Measurement,
and what it must control").  Worst/best needs every configuration measured;
that figure comes from the exhaustive tuning behind the persisted cache and
is labelled so ("tuning_report"), or from --report, which re-measures it.

All inputs are generated and copied to the GPU before anything is timed, and
the headline workload is timed last, right after the others, on a GPU whose
clocks are those of sustained use: exactly --warmup untimed steps of it, then
exactly --steps timed ones.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I]
                  [--report]   # also measure every feasible configuration
                               # (best/worst/fixed ratios, model hit rate)
                  [--copy-calib BYTES]   # plain copy for the HBM counter scale
                  [--only]     # time only the chosen workload (for profiling)
                  [--fresh | --cache FILE]   # tune now, or load a tuning cache
                                             # (default: the persisted MI355X one)
                  [--cache-out FILE]         # with --report: save the exhaustive tuning
                  [--buckets]  # also: shape-bucket dispatch against per-M tuning
                               # on the decode weights (M = 1 .. 256)
                  [--no-rmsnorm]  # skip the second workload: the occupancy-tuned
                                  # RMS normalisation (16384 x 8192 bf16) against
                                  # the HBM roofline, reported under "rmsnorm"
                  [--rmsnorm]     # report it also with --only
                  [--order]       # also: the headline at six tile scheduling orders

The per-shape configurations come from the persisted tuning cache when it is
present (the exhaustive measured autotune of every workload on MI355X, in the
library's own cache format); --fresh runs the library's hybrid tuner instead.
The JSON "config.tuning" says which.  Prints one JSON line.  Needs the built
library; the oracle is used only for the CPU-baseline leg.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from tile_shape_autotuning_amd import workloads as wl  # noqa: E402

PEAK = {"bf16": 2516.6, "f32": 157.3}   # dense MFMA TFLOP/s, MI355X spec
HBM_PEAK = 8000.0                       # GB/s


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _dev(x, torch):
    if x is None:
        return None
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def bound_of(w):
    """HBM-bound when the roofline time of the bytes exceeds that of the flops."""
    prec = "f32" if w.dtype == wl.F32 else "bf16"
    t_flop = w.flops / (PEAK[prec] * 1e12)
    t_mem = w.compulsory_bytes / (HBM_PEAK * 1e9)
    return ("hbm" if t_mem > t_flop else "mfma"), prec


class Prepared:
    """One workload's inputs on the GPU and its output buffer."""

    def __init__(self, index, torch, rotate=1):
        import tile_shape_autotuning_amd as tg
        self.w = w = wl.WORKLOADS[index]
        self.index = index
        A, B, bias = wl.workload_inputs(index)
        self.host = (A, B, bias)
        self.A, self.B, self.bias = _dev(A, torch), _dev(B, torch), _dev(bias, torch)
        self.Bs = [self.B] + [self.B.clone() for _ in range(rotate - 1)]
        self.act = ["none", "relu", "gelu"][w.act]
        self.out_dtype = torch.bfloat16 if w.dtype == wl.BF16 else torch.float32
        self.C = torch.empty((w.M, w.N), dtype=self.out_dtype, device="cuda")
        self.tg = tg

    def bind(self, cfg=None):
        """A step: one C-ABI call, rotating through the weight copies; cfg None
        takes the cached (tuned) configuration, tuning on a miss."""
        calls = [self.tg.BoundGemm(self.A, B, self.bias, act=self.act, out=self.C, cfg=cfg) for B in self.Bs]
        state = [0]

        def step():
            calls[state[0] % len(calls)]()
            state[0] += 1
        return step

    def tuned(self):
        """(cfg, tuner's measured us) of the cache entry a call without cfg uses."""
        w = self.w
        return self.tg.cache_lookup(self.tg.dispatch_m(w.M), w.N, w.K, w.dtype, act=self.act,
                                    bias=self.bias is not None)


def warm_up(step, min_steps, torch, min_seconds=0.1):
    """Untimed steps until the GPU has run for at least min_seconds (and at
    least min_steps steps); returns how many were run.  After the host-side
    input generation the GPU has idled for seconds and its clocks ramp up
    over tens of milliseconds: timed right away, a 200-step run of the
    16-row decode read 80 us per step that reads 74 us after 30 ms of warm-up
    (the 1000 x 1000 x 8192 case: 34.2 vs 32.3 us)."""
    t0 = time.perf_counter()
    n = max(1, min_steps)
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    while elapsed < min_seconds:
        more = max(1, int(n * (min_seconds - elapsed) / max(elapsed, 1e-6)) + 1)
        for _ in range(more):
            step()
        torch.cuda.synchronize()
        n += more
        elapsed = time.perf_counter() - t0
    return n


def time_steps(step, steps, torch):
    """Average seconds per step over `steps`, timed with HIP events on the
    launch stream (torch's current stream, which the binding hands to the
    library), and the host wall time of the region."""
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) * 1e-3 / steps, wall


def secondary_steps(p, sec_hint, steps):
    """Steps for a measurement off the headline: about 0.2 s of GPU time
    (between 10 and 5000 steps), whatever the headline's step count."""
    return max(10, min(5000, int(0.2 / max(1e-6, sec_hint))))


def compare_configs(p, torch, steps, tuned_sec):
    """The fixed 128 x 128 default and the cost model's first choice, each
    timed here after its own warm-up, against the tuned configuration."""
    w, tg = p.w, p.tg
    tuned_cfg = tuple(p.tuned()[0].astuple())
    out = {}
    for name, cfg in (("fixed_128x128", tg.default_cfg(w.M, w.N, w.K, w.dtype)),
                      ("model_choice", tg.model_choice(w.M, w.N, w.K, w.dtype)[0])):
        cfg = tuple(cfg.astuple())
        if cfg == tuned_cfg:
            sec = tuned_sec
        else:
            step = p.bind(cfg)
            warm_up(step, 3, torch)
            sec, _ = time_steps(step, secondary_steps(p, tuned_sec, steps), torch)
        out[name] = {"cfg": list(cfg), "us": round(sec * 1e6, 3), "over_tuned": round(sec / tuned_sec, 4),
                     "is_tuned": cfg == tuned_cfg}
    return out


def shape_summary(p, sec, forced_cfg=None):
    w = p.w
    bound, prec = bound_of(w)
    tflops = w.flops / sec / 1e12
    gbs = w.compulsory_bytes / sec / 1e9
    frac = gbs / HBM_PEAK if bound == "hbm" else tflops / PEAK[prec]
    if forced_cfg is not None:
        cfg, meas = p.tg.Cfg.of(forced_cfg), float("nan")
    else:
        cfg, meas = p.tuned()   # the entry the call used
    return {"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "dtype": wl.DTYPE_NAMES[w.dtype],
            "act": p.act, "us": round(sec * 1e6, 3), "TFLOP/s": round(tflops, 2), "GB/s": round(gbs, 1),
            "bound": bound, "roofline_frac": round(frac, 4), "cfg": list(cfg.astuple()),
            "tuned_us": round(meas, 3)}


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.txt")
# the report of the exhaustive measured tuning behind the persisted cache
DEFAULT_REPORT = os.path.join(ROOT, "tile_shape_autotuning_amd", "tuned", "mi355x_report.json")


def persisted_report(shapes):
    """Best/worst, best/fixed-128x128 and model-versus-measured figures of the
    exhaustive tuning that produced the persisted cache, per workload, each
    marked with whether the configuration timed here is the one that tuning
    chose."""
    with open(DEFAULT_REPORT) as f:
        rep = json.load(f)
    out = {"source": rep["source"], "measured_in_this_run": False, "model_hit_rate": rep["model_hit_rate"],
           "workloads": {}}
    for name, r in rep["report"].items():
        timed = shapes.get(name, {}).get("cfg")
        out["workloads"][name] = {
            "candidates_measured": r["measured"], "best_us": r["best"]["us"], "worst_us": r["worst"]["us"],
            "worst_over_best": r["worst_over_best"], "fixed_128x128_over_best": r["fixed_over_best"],
            "chosen": r["chosen"]["cfg"], "chosen_confirmed_us": r["chosen"]["us"],
            "model_choice": r["model_choice"], "model_choice_over_best": r["model_choice_over_best"],
            "model_hit": r["model_hit"], "rank_corr": r["rank_corr"],
            "timed_here_is_chosen": timed == r["chosen"]["cfg"] if timed is not None else None}
    return out
CALIBRATION_REPORT = os.path.join(ROOT, "tile_shape_autotuning_amd", "tuned", "calibration_report.json")


def calibration_summary():
    """The cost model's calibration, scored on shapes the fit did not see
    (offline: tile_shape_autotuning_amd.calibrate on the committed tables)."""
    with open(CALIBRATION_REPORT) as f:
        r = json.load(f)
    keep = ("tables", "model_hits", "best_in_topk", "near_best_in_topk", "geomean_choice_over_best",
            "mean_rank_corr", "msle")
    return {"measured_in_this_run": False, "source": r.get("source", ""),
            "train": r["split"]["train"], "held_out": r["split"]["held_out"],
            "constants_fitted": r["constants_fitted"],
            **{k: {x: r[k][x] for x in keep} for k in ("held_out_before", "held_out_after",
                                                       "train_before", "train_after")}}


# per-shape tuning results measured on MI355X (the library's cache file format)
DEFAULT_CACHE = os.path.join(ROOT, "tile_shape_autotuning_amd", "tuned", "mi355x.cache")


def measured_traffic(workload, cfg):
    """HBM bytes per call recorded by the rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs for this workload and configuration -- only if they were taken with
    the kernel sources, launch path and compile flags of this tree (else the
    kernel may have changed: None)."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    from tile_shape_autotuning_amd.build_lib import kernel_source_digest
    digest = kernel_source_digest()
    want = ",".join(str(x) for x in cfg)
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if not line.startswith("traffic "):
                continue
            kv = dict(t.split("=", 1) for t in line.split()[1:])
            if kv.get("workload") == workload and kv.get("cfg") == want and kv.get("kernel_src_sha256") == digest:
                return int(float(kv["fetch_bytes"]) + float(kv["write_bytes"]))
    return None


def cpu_baseline(index, host=None, target_s=12.0):
    """The oracle, as it stands, on a bounded row sample of the workload on
    the host's cores: the sample grows until one pass takes about a second
    (so fixed per-call costs do not set the rate), then is scaled to about
    target_s seconds; a workload that is done within that is repeated."""
    from oracle import gemm_ref
    w = wl.WORKLOADS[index]
    A, B, bias = host if host is not None else wl.workload_inputs(index)
    act = ["none", "relu", "gelu"][w.act]
    rows, dt = 8, 0.0
    while True:
        rows = min(rows, w.M)
        t0 = time.perf_counter()
        gemm_ref.gemm(A[:rows], B, bias, act)
        dt = time.perf_counter() - t0
        if dt >= 1.0 or rows == w.M:
            break
        rows *= 4
    rows2 = int(max(rows, min(w.M, rows * target_s / max(dt, 1e-3))))
    reps = 1
    if rows2 != rows:
        t0 = time.perf_counter()
        gemm_ref.gemm(A[:rows2], B, bias, act)
        dt = time.perf_counter() - t0
    if rows2 == w.M and dt < target_s:          # the whole workload is quick: repeat it
        reps = max(1, int(target_s / max(dt, 1e-3)))
        t0 = time.perf_counter()
        for _ in range(reps):
            gemm_ref.gemm(A, B, bias, act)
        dt = (time.perf_counter() - t0) / reps
    return {"value": round(2.0 * rows2 * w.N * w.K / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": gemm_ref.num_threads(), "kind": "oracle",
            "sample": f"first {rows2} of {w.M} rows of {w.name} (full K and N), fp64 oracle, "
                      f"{dt:.2f} s per pass x {reps} pass(es)"}


def report(indices, torch, dump_dir=None, cache_out=None):
    """Measure every feasible configuration per workload with the library's
    exhaustive tuner: best/worst/fixed ratios and the cost model's hit rate.
    With cache_out, the exhaustively tuned entries are saved there."""
    import tile_shape_autotuning_amd as tg
    from tile_shape_autotuning_amd import _native as N
    out = {}
    hits = 0
    tg.cache_clear()
    for i in indices:
        w = wl.WORKLOADS[i]
        os.environ["TILEGEMM_TUNE_MODE"] = "exhaustive"
        os.environ["TILEGEMM_TUNE_SAMPLES"] = "5"
        os.environ["TILEGEMM_PROGRESS"] = "1"
        # split-K cannot help a problem with thousands of tiles; keep its sweep short
        os.environ["TILEGEMM_TUNE_MAX_SPLIT"] = "1" if w.flops > 1e12 else "64"
        t0 = time.perf_counter()
        act, has_bias = ["none", "relu", "gelu"][w.act], w.bias_dist is not None
        tg.gemm_autotune(w.M, w.N, w.K, w.dtype, act=act, bias=has_bias)
        tune_s = time.perf_counter() - t0
        table = tg.autotune_table(w.M, w.N, w.K, w.dtype, act=act, bias=has_bias)
        rows = [(c.astuple(), pred, meas) for c, pred, meas, _ in table if meas > 0]
        confirmed = {c.astuple(): conf for c, _, _, conf in table if conf > 0}
        if dump_dir:
            os.makedirs(dump_dir, exist_ok=True)
            with open(os.path.join(dump_dir, f"table_{w.name}.json"), "w") as f:
                json.dump({"workload": w.name, "M": w.M, "N": w.N, "K": w.K, "dtype": w.dtype,
                           "rows": [[list(c), pred, meas, confirmed.get(c, -1.0)] for c, pred, meas in rows]}, f)
        best = min(rows, key=lambda r: r[2])
        worst = max(rows, key=lambda r: r[2])
        fixed = [r for r in rows if r[0] == tuple(tg.default_cfg(w.M, w.N, w.K, w.dtype).astuple())]
        model_cfg, _ = tg.model_choice(w.M, w.N, w.K, w.dtype)
        model_rows = [r for r in rows if r[0] == tuple(model_cfg.astuple())]
        hit = bool(model_rows) and model_rows[0][0] == best[0]
        hits += hit
        # rank correlation between predicted and measured times
        pr = np.argsort(np.argsort([r[1] for r in rows]))
        mr = np.argsort(np.argsort([r[2] for r in rows]))
        rho = float(np.corrcoef(pr, mr)[0, 1]) if len(rows) > 2 else float("nan")
        chosen = tg.cache_lookup(w.M, w.N, w.K, w.dtype, act=act, bias=has_bias)[0].astuple()
        out[w.name] = {
            "measured": len(rows), "tune_s": round(tune_s, 2),
            "best": {"cfg": list(best[0]), "us": round(best[2], 3)},
            # the tuner's choice: the fastest of the best few (and the default)
            # re-timed with long samples
            "chosen": {"cfg": list(chosen), "us": round(confirmed.get(chosen, -1.0), 3),
                       "confirmed": {",".join(str(x) for x in c): round(v, 3) for c, v in confirmed.items()}},
            "worst": {"cfg": list(worst[0]), "us": round(worst[2], 3)},
            "worst_over_best": round(worst[2] / best[2], 3),
            "fixed_over_best": round(fixed[0][2] / best[2], 3) if fixed else None,
            "model_choice": list(model_cfg.astuple()),
            "model_choice_over_best": round(model_rows[0][2] / best[2], 3) if model_rows else None,
            "model_hit": hit, "rank_corr": round(rho, 3),
        }
        log(f"report {w.name}: {out[w.name]}")
    if cache_out:
        tg.cache_save(cache_out)
        log(f"tuning cache written to {cache_out}")
    os.environ["TILEGEMM_TUNE_MODE"] = "hybrid"
    tg.cache_clear()
    return out, hits


BUCKET_MS = (1, 2, 3, 5, 8, 13, 16, 17, 24, 32, 40, 48, 56, 64, 80, 100, 128, 160, 200, 256)


def bucket_report(torch, steps):
    """Run-time dispatch over shape buckets on the decode weights (N = 28672,
    K = 8192, bf16): for each M, the time per call with the configuration of
    M's bucket (tuned once per bucket, at its largest M) and with a
    configuration tuned for M itself, and how many tuning runs each needed.
    Weights rotate through two copies, as in the decode workload."""
    import tile_shape_autotuning_amd as tg
    N, K = 28672, 8192
    A, B, bias = wl.make_inputs(max(BUCKET_MS), N, K, wl.BF16, wl.Dist("normal"), wl.Dist("normal"),
                                wl.Dist("normal"), 5)
    A_d, bias_d = _dev(A, torch), _dev(bias, torch)
    Bs = [_dev(B, torch)]
    Bs.append(Bs[0].clone())
    rows = {M: {"M": M, "key": None} for M in BUCKET_MS}
    tunes = {}
    try:
        for mode in ("bucketed", "exact"):
            tg.set_shape_buckets(mode == "bucketed")
            tg.cache_clear()
            t0 = tg.stats()["tunes"]
            for M in BUCKET_MS:
                a = A_d[:M]
                C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
                calls = [tg.BoundGemm(a, b, bias_d, act="none", out=C) for b in Bs]   # the first tunes
                for c in calls:
                    c()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for i in range(steps):
                    calls[i % 2]()
                e1.record()
                torch.cuda.synchronize()
                key = tg.dispatch_m(M)
                cfg = tg.cache_lookup(key, N, K, wl.BF16, act="none", bias=True)[0].astuple()
                rows[M][mode + "_us"] = round(e0.elapsed_time(e1) * 1e3 / steps, 3)
                rows[M][mode + "_cfg"] = list(cfg)
                if mode == "bucketed":
                    rows[M]["key"] = key
                log(f"buckets {mode} M={M}: {rows[M][mode + '_us']} us cfg {cfg}")
            tunes[mode] = tg.stats()["tunes"] - t0
    finally:
        tg.set_shape_buckets(True)
        tg.cache_clear()
    out = list(rows.values())
    for r in out:
        r["bucketed_over_exact"] = round(r["bucketed_us"] / r["exact_us"], 3)
    ratios = [r["bucketed_over_exact"] for r in out]
    return {"shape": f"M x {N} x {K} bf16", "tunings": tunes, "rows": out,
            "geomean_bucketed_over_exact": round(float(np.exp(np.mean(np.log(ratios)))), 4),
            "max_bucketed_over_exact": max(ratios)}


def tile_order_study(p, torch, groups=(1, 2, 4, 8, 16, 32)):
    """The headline workload's tuned call with each scheduling order (tile
    rows per group; the order changes which tiles share an XCD's L2 at a
    time, not what they compute)."""
    tg = p.tg
    out = {}
    try:
        for g in groups:
            tg.set_tile_order(g)
            step = p.bind(None)
            warm_up(step, 3, torch)
            sec, _ = time_steps(step, secondary_steps(p, 1e-3, 0), torch)
            out[str(g)] = round(sec * 1e6, 2)
    finally:
        tg.set_tile_order(0)
    best = min(out, key=out.get)
    res = {"workload": p.w.name, "us_per_group_rows": out, "default": tg.tile_order(), "best": int(best),
           "default_over_best": round(out[str(tg.tile_order())] / out[best], 4) if str(tg.tile_order()) in out
           else None}
    log(f"tile order study: {res}")
    return res


STREAMK_SHAPE = (4352, 4352, 8192)


def streamk_study(torch):
    """The stream-K kind where it pays: a bf16 problem of 17 x 17 tiles of
    256 x 256 (one full round of 256 and a tail of 33) with a long K.  Times
    the same tile data-parallel (two rounds) and with the stream-K tail, and
    the hybrid tuner's own choice for the shape (which sees both kinds)."""
    import tile_shape_autotuning_amd as tg
    M, N, K = STREAMK_SHAPE
    sk_ = 1.0 / np.sqrt(K)
    A, B, _ = wl.make_inputs(M, N, K, wl.BF16, wl.Dist("normal", sk_), wl.Dist("normal", sk_), None, 6)
    A_d, B_d = _dev(A, torch), _dev(B, torch)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    out = {"shape": f"{M} x {N} x {K} bf16", "tiles_256x256": 17 * 17}

    def timed(cfg):
        call = tg.BoundGemm(A_d, B_d, None, act="none", out=C, cfg=cfg)
        warm_up(call, 3, torch)
        sec, _ = time_steps(call, max(10, int(0.2 / max(1e-6, _one(call)))), torch)
        return sec

    def _one(call):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3

    dp_cfg, sk_cfg = (0, 256, 256, 64, 2, 4, 2, 1), (3, 256, 256, 64, 2, 4, 2, 1)
    t_dp, t_sk = timed(dp_cfg), timed(sk_cfg)
    out.update({"data_parallel": {"cfg": list(dp_cfg), "us": round(t_dp * 1e6, 2)},
                "stream_k": {"cfg": list(sk_cfg), "us": round(t_sk * 1e6, 2)},
                "data_parallel_over_stream_k": round(t_dp / t_sk, 3)})
    tuned = tuple(tg.gemm_autotune(M, N, K, wl.BF16).astuple())
    out["tuner_choice"] = {"cfg": list(tuned), "us": round(timed(tuned) * 1e6, 2), "kind_is_stream_k": tuned[0] == 3}
    model = tuple(tg.model_choice(M, N, K, wl.BF16)[0].astuple())
    out["model_choice"] = list(model)
    out["TFLOP/s_best"] = round(2.0 * M * N * K / min(t_dp, t_sk) / 1e12, 1)
    log(f"stream-K study: {out}")
    return out


PADDED_SHAPE = (513, 1001, 777)


def padded_study(torch):
    """The padded path where the shape is ragged: 513 x 1001 x 777 bf16 with
    bias and ReLU (K and N not whole 16-byte vectors).  Times the best
    element-load configuration and the best padded-path configuration of the
    committed exhaustive table of that shape, interleaved, and the hybrid
    tuner's own choice (which sees both)."""
    import gzip
    import tile_shape_autotuning_amd as tg
    M, N, K = PADDED_SHAPE
    path = os.path.join(ROOT, "tile_shape_autotuning_amd", "tuned", "tables", "table_c23_bf16_513x1001x777.json.gz")
    if not os.path.exists(path):
        return None
    with gzip.open(path, "rt") as f:
        rows = [r for r in json.load(f)["rows"] if r[2] is not None and r[2] > 0]
    elem = tuple(min((r for r in rows if r[0][0] == 2), key=lambda r: r[2])[0])
    padded = tuple(min((r for r in rows if r[0][0] == 0), key=lambda r: r[2])[0])
    A, B, bias = wl.make_inputs(M, N, K, wl.BF16, wl.Dist("normal", 1.0 / np.sqrt(K)), wl.Dist("normal", 1.0),
                                wl.Dist("uniform", 1.0), 9)
    A_d, B_d, b_d = _dev(A, torch), _dev(B, torch), _dev(bias, torch)
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    res = {}
    for rnd in range(3):
        for name, cfg in (("element_loads", elem), ("padded", padded)):
            call = tg.BoundGemm(A_d, B_d, b_d, act="relu", out=C, cfg=cfg)
            warm_up(call, 10, torch, 0.05)
            sec, _ = time_steps(call, 2000, torch)
            res[name] = min(res.get(name, 1e9), sec)
    tuned = tuple(tg.gemm_autotune(M, N, K, wl.BF16, act="relu", bias=True).astuple())
    call = tg.BoundGemm(A_d, B_d, b_d, act="relu", out=C, cfg=tuned)
    warm_up(call, 10, torch, 0.05)
    t_tuned, _ = time_steps(call, 2000, torch)
    out = {"shape": f"{M} x {N} x {K} bf16, bias + ReLU",
           "element_loads": {"cfg": list(elem), "us": round(res["element_loads"] * 1e6, 3)},
           "padded": {"cfg": list(padded), "us": round(res["padded"] * 1e6, 3)},
           "element_loads_over_padded": round(res["element_loads"] / res["padded"], 3),
           "tuner_choice": {"cfg": list(tuned), "us": round(t_tuned * 1e6, 3)},
           "picked_from": os.path.relpath(path, ROOT)}
    log(f"padded study: {out}")
    return out


def sliced_k_study(p, tuned_cfg, torch):
    """The sliced-K kind where it pays: the fp32 workload's tuned call (K
    split among the wave groups of each workgroup; `tuned_cfg`, the
    configuration its timed call used) against the best configuration
    without K groups in the committed exhaustive table of the same shape,
    both timed here, interleaved, with the same warm-up."""
    import gzip
    path = os.path.join(ROOT, "tile_shape_autotuning_amd", "tuned", "tables", f"table_{p.w.name}.json.gz")
    if not os.path.exists(path):
        return None
    with gzip.open(path, "rt") as f:
        rows = [r for r in json.load(f)["rows"] if r[2] is not None and r[2] > 0 and r[0][0] != 4]
    plain = tuple(min(rows, key=lambda r: r[2])[0])
    tuned = tuple(tuned_cfg)
    res = {}
    for rnd in range(3):
        for name, cfg in (("tuned", tuned), ("without_k_groups", plain)):
            step = p.bind(cfg)
            warm_up(step, 10, torch, 0.05)
            sec, _ = time_steps(step, 2000, torch)
            res[name] = min(res.get(name, 1e9), sec)
    out = {"workload": p.w.name, "tuned": {"cfg": list(tuned), "us": round(res["tuned"] * 1e6, 3)},
           "without_k_groups": {"cfg": list(plain), "us": round(res["without_k_groups"] * 1e6, 3),
                                "picked_from": os.path.relpath(path, ROOT)},
           "without_over_tuned": round(res["without_k_groups"] / res["tuned"], 3)}
    log(f"sliced-K study: {out}")
    return out


def rmsnorm_report(torch, steps, rows=16384, n=8192):
    """The second workload: RMS normalisation of rows x n bf16 with
    occupancy-only tuning.  Time per call at each occupancy and with the
    tuned one (HIP events, back-to-back calls), against the HBM roofline of
    reading x and writing y once."""
    import tile_shape_autotuning_amd as tg
    g = torch.Generator(device="cuda").manual_seed(7)
    x = torch.randn((rows, n), device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
    w = torch.randn(n, device="cuda", dtype=torch.float32, generator=g).to(torch.bfloat16)
    y = torch.empty_like(x)
    nbytes = 2 * rows * n * 2 + n * 2

    def timed(occ):
        warm_up(lambda: tg.rmsnorm(x, w, 1e-6, occupancy=occ, out=y), 3, torch)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            tg.rmsnorm(x, w, 1e-6, occupancy=occ, out=y)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    per = {occ: round(timed(occ), 3) for occ in (1, 2, 4, 8)}
    t0 = tg.rmsnorm_tunes()
    tuned_us = timed(0)
    occ, tuner_us = tg.rmsnorm_cache_lookup(rows, n)
    gbs = nbytes / (tuned_us * 1e-6) / 1e9
    log(f"rmsnorm {rows}x{n}: per occupancy {per}, tuned occupancy {occ}: {tuned_us:.2f} us, {gbs:.0f} GB/s")
    return {"shape": f"{rows} x {n} bf16", "us_per_occupancy": per, "tuned_occupancy": occ,
            "tuning_runs": tg.rmsnorm_tunes() - t0, "tuned_us": round(tuned_us, 3),
            "tuner_measured_us": round(tuner_us, 3),
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK, "unit": "GB/s",
                         "frac": round(gbs / HBM_PEAK, 4), "bytes_per_call": nbytes}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10,
                    help="untimed steps of the headline workload right before its timed ones")
    ap.add_argument("--workload", type=int, default=3)
    ap.add_argument("--only", action="store_true")
    ap.add_argument("--no-compare", action="store_true",
                    help="skip timing the fixed default and the model's choice (profiling runs)")
    ap.add_argument("--report", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-calib", type=int, default=0)
    ap.add_argument("--dump", type=str, default="", help="with --report: write every measured row here")
    ap.add_argument("--fresh", action="store_true",
                    help="tune from scratch instead of loading the persisted tuning cache")
    ap.add_argument("--cache", type=str, default=DEFAULT_CACHE, help="tuning cache file to load")
    ap.add_argument("--cache-out", type=str, default="", help="with --report: save the exhaustive tuning here")
    ap.add_argument("--report-out", type=str, default="",
                    help="with --report: save the report (ratios, confirmed choices, model hits) here as JSON")
    ap.add_argument("--buckets", action="store_true",
                    help="also report shape-bucket dispatch against per-M tuning on the decode weights")
    ap.add_argument("--rmsnorm", action="store_true",
                    help="report the occupancy-tuned RMS normalisation also with --only")
    ap.add_argument("--no-rmsnorm", action="store_true", help="skip the RMS normalisation report")
    ap.add_argument("--streamk", action="store_true", help="report the stream-K study also with --only")
    ap.add_argument("--order", action="store_true",
                    help="also time the headline call at six tile scheduling orders (tile_order_study); off by "
                         "default, so that a kernel trace of the default run holds the headline's own launches only")
    ap.add_argument("--padded", action="store_true", help="report the padded-path study also with --only")
    ap.add_argument("--no-padded", action="store_true",
                    help="skip the padded-path study (513 x 1001 x 777: element loads against padded operands)")
    ap.add_argument("--no-streamk", action="store_true",
                    help="skip the stream-K study (4352 x 4352 x 8192: data-parallel against stream-K tail)")
    ap.add_argument("--cfg", type=str, default="",
                    help="force a configuration for the main workload: kind,bm,bn,bk,wgm,wgn,stages,split_k")
    a = ap.parse_args()
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    import tile_shape_autotuning_amd as tg
    tg._native.lib()   # fails loudly if the library is missing

    if a.copy_calib:
        n = a.copy_calib // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 3 copies of {a.copy_calib} bytes")

    tuning = "fresh"
    if not a.fresh and a.cache and os.path.exists(a.cache):
        loaded, skipped = tg.cache_load(a.cache)
        tuning = f"cache {os.path.relpath(a.cache, ROOT)} ({loaded} entries, {skipped} skipped)"
        log(f"tuning: {tuning}")

    main_idx = a.workload
    # the headline goes last: it is timed on a GPU that the others kept busy
    indices = [main_idx] if a.only else [i for i in sorted(wl.WORKLOADS) if i != main_idx] + [main_idx]
    forced = tuple(int(x) for x in a.cfg.split(",")) if a.cfg else None
    # every input is generated and resident before anything is timed
    prepared = {}
    for i in indices:
        # decode: stream distinct weights every call (copies together exceed the 256 MiB
        # last-level cache twice over, as the library's tuner times it)
        wi = wl.WORKLOADS[i]
        b_bytes = wi.K * wi.N * (4 if wi.dtype == wl.F32 else 2)
        rotate = min(8, max(2, -(-(512 << 20) // b_bytes))) if wi.M <= 64 else 1
        log(f"workload {i}: preparing")
        prepared[i] = Prepared(i, torch, rotate=rotate)
    torch.cuda.synchronize()

    shapes = {}
    main_res = None
    hits, compared = 0, 0
    for i in indices:
        p = prepared[i]
        is_main = i == main_idx
        cfg = forced if (is_main and forced) else None
        step = p.bind(cfg)     # the first call tunes (without a persisted entry) and caches
        tuned_us = p.tuned()[1] if cfg is None else float("nan")
        if not is_main:
            warm_up(step, 10, torch)
            steps = secondary_steps(p, (tuned_us if tuned_us > 0 else 100.0) * 1e-6, a.steps)
            sec, wall = time_steps(step, steps, torch)
            s = shape_summary(p, sec, cfg)
            s["steps"] = steps
        if not a.no_compare and cfg is None:
            hint = sec if not is_main else max(tuned_us, 1.0) * 1e-6
            cmp_ = compare_configs(p, torch, a.steps, hint)
        if is_main:
            # exactly --warmup untimed steps, then exactly --steps timed ones
            for _ in range(a.warmup):
                step()
            sec, wall = time_steps(step, a.steps, torch)
            s = shape_summary(p, sec, cfg)
            s["steps"] = a.steps
            main_res = (p, sec, wall, a.steps)
        if not a.no_compare and cfg is None:
            # re-express the ratios against this run's tuned time
            for v in cmp_.values():
                if v["is_tuned"]:
                    v["us"] = round(sec * 1e6, 3)
                v["over_tuned"] = round(v["us"] * 1e-6 / sec, 4)
            s["fixed_128x128"] = cmp_["fixed_128x128"]
            s["model_choice"] = cmp_["model_choice"]
            hits += cmp_["model_choice"]["is_tuned"]
            compared += 1
        shapes[p.w.name] = s
        log(f"workload {i}: {s}")

    p, sec, wall, steps = main_res
    w = p.w
    bound, prec = bound_of(w)
    achieved = w.flops / sec / 1e12 if bound == "mfma" else w.compulsory_bytes / sec / 1e9
    peak = PEAK[prec] if bound == "mfma" else HBM_PEAK
    line = {
        "metric": "autotuned GEMM TFLOP/s (or GB/s) per shape and % of MI355X roofline",
        "value": round(achieved, 3) if bound == "mfma" else round(achieved, 1),
        "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": a.warmup,
        "ms_per_step": round(sec * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": prec, "data": "synthetic",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "dtype": wl.DTYPE_NAMES[w.dtype], "act": p.act, "bias": p.bias is not None,
                   "cfg": shapes[w.name]["cfg"], "tuning": tuning, "parallelism": "single-gpu",
                   "order": "headline timed last, after " + (", ".join(wl.WORKLOADS[i].name for i in indices[:-1])
                                                            or "nothing")},
        "roofline": {"bound": bound, "achieved": round(achieved, 2), "peak": peak,
                     "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                     "frac": round(achieved / peak, 4),
                     "traffic": measured_traffic(w.name, shapes[w.name]["cfg"])},
        "shapes": shapes,
    }
    if compared:
        line["measured_here"] = {
            "model_hit_rate": f"{hits}/{compared}",
            "fixed_128x128_over_tuned": {k: v["fixed_128x128"]["over_tuned"] for k, v in shapes.items()
                                         if "fixed_128x128" in v},
            "model_choice_over_tuned": {k: v["model_choice"]["over_tuned"] for k, v in shapes.items()
                                        if "model_choice" in v},
            "note": "hit = the cost model's first choice is the configuration the measured tuning chose"}
    if a.report:
        rep, hits = report([i for i in indices], torch, a.dump, a.cache_out or None)
        line["report"] = rep
        line["model_hit_rate"] = f"{hits}/{len(indices)}"
        if a.report_out:
            with open(a.report_out, "w") as f:
                json.dump({"source": "bench.py --report on MI355X (exhaustive measured autotune of each workload)",
                           "model_hit_rate": line["model_hit_rate"], "report": rep}, f, indent=1)
    elif tuning.startswith("cache") and os.path.exists(DEFAULT_REPORT):
        line["tuning_report"] = persisted_report(shapes)
    if os.path.exists(CALIBRATION_REPORT):
        line["calibration"] = calibration_summary()
    if a.buckets:
        line["buckets"] = bucket_report(torch, 100)
    if (a.rmsnorm or not a.only) and not a.no_rmsnorm:
        line["rmsnorm"] = rmsnorm_report(torch, 50)
    if (a.streamk or not a.only) and not a.no_streamk:
        line["streamk_study"] = streamk_study(torch)
    if 1 in prepared and not a.only and forced is None:
        line["sliced_k_study"] = sliced_k_study(prepared[1], shapes[prepared[1].w.name]["cfg"], torch)
    if (a.padded or not a.only) and forced is None and not a.no_padded:
        line["padded_study"] = padded_study(torch)
    if a.order and forced is None:
        line["tile_order_study"] = tile_order_study(p, torch)
    if not a.no_cpu:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(main_idx, p.host)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
