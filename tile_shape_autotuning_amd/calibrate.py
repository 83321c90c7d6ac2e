"""Fit the cost model's device constants to measured autotuning tables.

Page "Tile Selection: Cost Models Against Measurement", "Hybrid strategies":
measure a set of configurations, fit the model to those measurements, and use
the fitted model to rank configurations that were not measured.  Here the
model's form stays the analytical one; only its calibration constants (the
pipeline latency per K step, LDS bandwidth per CU, the tile-efficiency area
and the launch/fill terms) are fitted, by grid search on the mean squared
log error over every measured row of every table.

Input tables are the JSON files `bench.py --report --dump DIR` writes (one
per workload: the measured median per configuration).  The model is
evaluated by the library itself (tg_model_time under a device-description
override), so a fitted set can be pasted into the built-in MI355X
description as it is.

    python -m tile_shape_autotuning_amd.calibrate DIR [--topk 16]
"""
from __future__ import annotations

import argparse
import glob
import itertools
import json
import math
import os
import sys

from . import _native as N

GRID = {
    "lds_bw_cu": [192.0e9, 230.0e9, 307.2e9],
    "cu_bw": [60.0e9, 75.0e9, 90.0e9, 120.0e9],
    "lat_step": [0.6e-6, 0.8e-6, 1.0e-6],
    "lat_l2": [0.4e-6, 0.5e-6, 0.75e-6],
    "w1_eff": [0.5, 0.55, 0.6, 0.75],
    "t0": [4.0e-6],
}


def load_tables(d):
    tabs = []
    for f in sorted(glob.glob(os.path.join(d, "table_*.json"))):
        with open(f) as fh:
            tabs.append(json.load(fh))
    if not tabs:
        raise FileNotFoundError(f"no table_*.json in {d}")
    return tabs


def _rank_stats(tab, desc, topk):
    M, Nn, K, dt = tab["M"], tab["N"], tab["K"], tab["dtype"]
    N.set_device_override(desc)
    pred, meas = [], []
    for row in tab["rows"]:
        cfg, m = row[0], row[2]
        try:
            pred.append(N.model_time_us(M, Nn, K, dt, cfg))
            meas.append(m)
        except N.TileGemmError:
            continue
    err = sum((math.log(p) - math.log(m)) ** 2 for p, m in zip(pred, meas)) / max(1, len(meas))
    order = sorted(range(len(pred)), key=lambda i: pred[i])
    best = min(range(len(meas)), key=lambda i: meas[i])
    top = set(order[:topk])
    # measured time of the model's first choice relative to the best measured
    choice_ratio = meas[order[0]] / meas[best]
    # Spearman rank correlation
    rp = {i: r for r, i in enumerate(order)}
    rm = {i: r for r, i in enumerate(sorted(range(len(meas)), key=lambda i: meas[i]))}
    n = len(meas)
    rho = 1 - 6 * sum((rp[i] - rm[i]) ** 2 for i in range(n)) / (n * (n * n - 1)) if n > 2 else float("nan")
    return err, best in top, choice_ratio, rho, order[0] == best


def evaluate(tabs, desc, topk):
    stats = [_rank_stats(t, desc, topk) for t in tabs]
    return {"msle": sum(s[0] for s in stats) / len(stats),
            "model_hits": sum(s[4] for s in stats),
            "best_in_topk": sum(s[1] for s in stats),
            "choice_over_best": [round(s[2], 3) for s in stats],
            "rank_corr": [round(s[3], 3) for s in stats]}


def fit(tabs, topk=16, grid=GRID):
    base = N.builtin_device_desc(0)
    best = None
    for vals in itertools.product(*grid.values()):
        d = N.builtin_device_desc(0)
        for k, v in zip(grid, vals):
            setattr(d, k, v)
        e = evaluate(tabs, d, topk)
        key = (-e["model_hits"], -e["best_in_topk"], e["msle"])
        if best is None or key < best[0]:
            best = (key, dict(zip(grid, vals)), e)
    N.set_device_override(None)
    return {"before": evaluate(tabs, base, topk), "fitted": best[1], "after": best[2]}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("dir")
    ap.add_argument("--topk", type=int, default=16)
    a = ap.parse_args(argv)
    tabs = load_tables(a.dir)
    res = fit(tabs, a.topk)
    N.set_device_override(None)
    print(json.dumps({"tables": [t["workload"] for t in tabs], **res}, indent=1))


if __name__ == "__main__":
    sys.exit(main())
