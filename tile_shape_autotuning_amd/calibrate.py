"""Fit the cost model's device constants on some measured tables and score
the fit on others.

Page "Tile Selection: Cost Models Against Measurement", "Hybrid strategies":
measure some configurations, fit the model to them, and let the fitted model
rank what was not measured -- with no guarantee outside what the fit saw
("Analytical models and where they break": correction terms leave residual
error away from the calibration shapes).  So the shapes are split: the fit
sees the training tables only, and the report gives the model's quality on
the held-out tables before and after the fit.

The model's form stays the analytical one; only calibration constants of the
MI355X description are fitted (effective LDS and L2-to-CU bandwidth per CU,
the memory latency a K step waits for from HBM and from L2, the issue
efficiency of a lone wave on a SIMD and of the sliced-K kind, the achievable
HBM fraction, the L2-to-CU efficiency of element loads), by grid
search: fewest training tables whose measured best is outside the model's
top k (the hybrid tuner measures the top k), then the smallest geometric
mean of the measured time of the model's first choice over the best, then
the smallest mean squared log error of predicted against measured times.  The
report also counts the tables with a configuration within 2 % of the
measured best in the model's top k, which box-to-box noise of that size
does not move.  The model is
evaluated by the library (tg_model_times under a device-description
override), so a fitted set can be written into the built-in description as
it is.

Tables: `python -m tile_shape_autotuning_amd.tables --out DIR` (gzipped JSON,
one per shape: configuration, model time, measured median).  The split is
fixed: the five benchmark workloads and the even-numbered calibration shapes
train, the odd-numbered ones are held out.

    python -m tile_shape_autotuning_amd.calibrate DIR [--topk 16] [--out FILE] [--jobs N]
"""
from __future__ import annotations

import argparse
import glob
import gzip
import itertools
import json
import math
import os
import re
import sys

from . import _native as N

GRID = {
    "lds_bw_cu": [128.0e9, 160.0e9, 192.0e9, 230.0e9],
    "cu_bw": [40.0e9, 50.0e9, 60.0e9, 75.0e9],
    "lat_step": [0.8e-6, 1.0e-6, 1.25e-6, 1.5e-6],
    "lat_l2": [0.25e-6, 0.3e-6, 0.4e-6, 0.5e-6],
    "w1_eff": [0.35, 0.4, 0.5, 0.55],
    "hbm_eff": [0.9125],
    "sliced_eff": [0.4, 0.55, 0.7, 1.0],
    "unaligned_eff": [0.0625, 0.125, 0.25],
}


def load_tables(d):
    tabs = []
    for f in sorted(glob.glob(os.path.join(d, "table_*.json*"))):
        opener = gzip.open if f.endswith(".gz") else open
        with opener(f, "rt") as fh:
            tabs.append(json.load(fh))
    if not tabs:
        raise FileNotFoundError(f"no table_*.json[.gz] in {d}")
    return tabs


def held_out(name: str) -> bool:
    """The fixed split: calibration shapes cNN with odd NN are held out."""
    m = re.match(r"c(\d+)_", name)
    return bool(m) and int(m.group(1)) % 2 == 1


def split(tabs):
    return [t for t in tabs if not held_out(t["workload"])], [t for t in tabs if held_out(t["workload"])]


def _spearman(x, y):
    n = len(x)
    if n < 3:
        return float("nan")
    rx = {i: r for r, i in enumerate(sorted(range(n), key=lambda i: x[i]))}
    ry = {i: r for r, i in enumerate(sorted(range(n), key=lambda i: y[i]))}
    return 1 - 6 * sum((rx[i] - ry[i]) ** 2 for i in range(n)) / (n * (n * n - 1))


# a configuration measured within this fraction of the best counts as
# near-best: boxes differ by about that much between runs, so which of two
# such configurations is "the" best is not a property of the shape
NEAR = 0.02


def table_stats(tab, desc, topk):
    """Model quality on one table: (msle, best in top k, measured time of the
    model's first choice over the best measured, Spearman rank correlation,
    first choice is the measured best, a near-best configuration in top k)."""
    N.set_device_override(desc)
    rows = tab["rows"]
    pred_all = N.model_times_us(tab["M"], tab["N"], tab["K"], tab["dtype"], [r[0] for r in rows])
    keep = [i for i, p in enumerate(pred_all) if p > 0 and rows[i][2] > 0]
    pred = [pred_all[i] for i in keep]
    meas = [rows[i][2] for i in keep]
    err = sum((math.log(p) - math.log(m)) ** 2 for p, m in zip(pred, meas)) / max(1, len(meas))
    # ties in model time keep the first configuration in canonical order
    order = sorted(range(len(pred)), key=lambda i: (pred[i], rows[keep[i]][0]))
    best = min(range(len(meas)), key=lambda i: meas[i])
    near = any(meas[i] <= (1.0 + NEAR) * meas[best] for i in order[:topk])
    return (err, best in set(order[:topk]), meas[order[0]] / meas[best], _spearman(pred, meas), order[0] == best,
            near)


def evaluate(tabs, desc, topk):
    if not tabs:
        return {}
    stats = [table_stats(t, desc, topk) for t in tabs]
    n = len(stats)
    return {"tables": n,
            "msle": round(sum(s[0] for s in stats) / n, 5),
            "model_hits": sum(s[4] for s in stats),
            "best_in_topk": sum(s[1] for s in stats),
            "near_best_in_topk": sum(s[5] for s in stats),
            "geomean_choice_over_best": round(math.exp(sum(math.log(s[2]) for s in stats) / n), 4),
            "mean_rank_corr": round(sum(s[3] for s in stats if s[3] == s[3]) / max(1, sum(s[3] == s[3] for s in stats)),
                                    4),
            "per_table": {t["workload"]: {"hit": s[4], "in_topk": s[1], "near_in_topk": s[5],
                                          "choice_over_best": round(s[2], 4),
                                          "rank_corr": round(s[3], 4), "msle": round(s[0], 5)}
                          for t, s in zip(tabs, stats)}}


def _desc(base, vals):
    d = N.DeviceDesc.from_buffer_copy(base)
    for k, v in vals.items():
        setattr(d, k, v)
    return d


_FIT = {}


def _score(cand):
    """Score of one candidate set on the training tables (smaller is better):
    fewest tables whose measured best is outside the model's top k (the
    hybrid tuner measures the top k, so that is what the model has to get
    right), then the geometric mean of the measured time of the model's first
    choice over the best, then the mean squared log error."""
    train, topk, base = _FIT["train"], _FIT["topk"], _FIT["base"]
    try:
        stats = [table_stats(t, _desc(base, cand), topk) for t in train]
    finally:
        N.set_device_override(None)
    return (-sum(s[1] for s in stats), round(sum(math.log(s[2]) for s in stats) / len(stats), 9),
            sum(s[0] for s in stats) / len(stats))


def fit(train, topk=16, grid=None, base=None, jobs=None):
    """Grid search on the training tables; returns the best constants (ties:
    the first in grid order).  jobs > 1 scores the grid in that many forked
    processes, with the same result."""
    grid = grid or GRID
    base = base if base is not None else N.builtin_device_desc(0)
    cands = [dict(zip(grid, vals)) for vals in itertools.product(*grid.values())]
    _FIT.update(train=train, topk=topk, base=N.DeviceDesc.from_buffer_copy(base))
    try:
        if jobs and jobs > 1 and len(cands) > 1:
            import multiprocessing as mp
            with mp.get_context("fork").Pool(jobs) as pool:
                keys = pool.map(_score, cands, chunksize=max(1, len(cands) // (4 * jobs)))
        else:
            keys = [_score(c) for c in cands]
    finally:
        _FIT.clear()
        N.set_device_override(None)
    i = min(range(len(cands)), key=lambda i: (keys[i], i))
    return cands[i]


def calibrate(tabs, topk=16, grid=None, jobs=None):
    base = N.builtin_device_desc(0)
    train, test = split(tabs)
    fitted = fit(train, topk, grid, base, jobs)
    after = _desc(base, fitted)
    try:
        rep = {"split": {"train": [t["workload"] for t in train], "held_out": [t["workload"] for t in test]},
               "topk": topk,
               "constants_before": {k: getattr(base, k) for k in (grid or GRID)},
               "constants_fitted": fitted,
               "train_before": evaluate(train, base, topk), "train_after": evaluate(train, after, topk),
               "held_out_before": evaluate(test, base, topk), "held_out_after": evaluate(test, after, topk)}
    finally:
        N.set_device_override(None)
    return rep


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("dir")
    ap.add_argument("--topk", type=int, default=16)
    ap.add_argument("--out", default="")
    ap.add_argument("--jobs", type=int, default=min(8, os.cpu_count() or 1))
    a = ap.parse_args(argv)
    rep = calibrate(load_tables(a.dir), a.topk, jobs=a.jobs)
    text = json.dumps(rep, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
