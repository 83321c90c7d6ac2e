"""Exhaustive measured tuning tables for a set of shapes (GPU).

For each shape the library's tuner runs in exhaustive mode on its own
synthetic operands (uniform values in [-1, 1)): every feasible configuration
that has a compiled kernel is timed, interleaved over several rounds, and
the table of (configuration, model time, measured median) is written as
gzipped JSON -- the input of the cost model's calibration
(tile_shape_autotuning_amd.calibrate), which fits on some shapes and scores
the fit on shapes it has not seen (page "Tile Selection: Cost Models Against
Measurement", "Hybrid strategies": fit the model to measured configurations,
predict the unmeasured ones).

    python -m tile_shape_autotuning_amd.tables --out DIR [--only NAME ...]
"""
from __future__ import annotations

import argparse
import gzip
import json
import os
import sys
import time

F32, BF16, BF16_F32OUT = 0, 1, 2

# Shapes beyond the five workloads, chosen to span M (decode rows, shape-bucket
# edges, tall), N and K, ragged sizes and all three dtype pairs.
CALIBRATION_SHAPES = [
    ("c01_bf16_1x4096x4096", 1, 4096, 4096, BF16),
    ("c02_bf16_8x14336x4096", 8, 14336, 4096, BF16),
    ("c03_bf16_32x8192x8192", 32, 8192, 8192, BF16),
    ("c04_bf16_48x4096x11008", 48, 4096, 11008, BF16),
    ("c05_bf16_64x28672x4096", 64, 28672, 4096, BF16),
    ("c06_bf16_100x8192x2048", 100, 8192, 2048, BF16),
    ("c07_bf16_200x4096x4096", 200, 4096, 4096, BF16),
    ("c08_bf16_512x512x512", 512, 512, 512, BF16),
    ("c09_bf16_1024x1024x1024", 1024, 1024, 1024, BF16),
    ("c10_bf16_2048x2048x2048", 2048, 2048, 2048, BF16),
    ("c11_bf16_777x1240x2056", 777, 1240, 2056, BF16),
    ("c12_bf16_1536x4096x1024", 1536, 4096, 1024, BF16),
    ("c13_bf16_3000x1000x4096", 3000, 1000, 4096, BF16),
    ("c14_bf16_4096x4096x4096", 4096, 4096, 4096, BF16),
    ("c15_bf16_8192x4096x1024", 8192, 4096, 1024, BF16),
    ("c16_bf16_6000x7000x512", 6000, 7000, 512, BF16),
    ("c17_bf16_2048x8192x8192", 2048, 8192, 8192, BF16),
    ("c18_bf16f32_512x2048x8192", 512, 2048, 8192, BF16_F32OUT),
    ("c19_bf16f32_1000x3000x504", 1000, 3000, 504, BF16_F32OUT),
    ("c20_f32_128x128x128", 128, 128, 128, F32),
    ("c21_f32_512x512x512", 512, 512, 512, F32),
    ("c22_f32_384x640x256", 384, 640, 256, F32),
    ("c23_bf16_513x1001x777", 513, 1001, 777, BF16),     # N, K not multiples of 8: element loads or padded
    ("c24_bf16_4096x256x147", 4096, 256, 147, BF16),     # K ragged only: A padded, B read in place
    ("c25_bf16_1024x1001x1024", 1024, 1001, 1024, BF16),  # N ragged only: B padded, output pass
]


def workload_shapes():
    """The five benchmark workloads, measured the same way."""
    from . import workloads as wl
    return [(w.name, w.M, w.N, w.K, w.dtype) for _, w in sorted(wl.WORKLOADS.items())]


def dump_table(tg, name, M, N, K, dtype, out_dir, max_split=None):
    os.environ["TILEGEMM_TUNE_MODE"] = "exhaustive"
    os.environ.setdefault("TILEGEMM_TUNE_SAMPLES", "3")
    os.environ.setdefault("TILEGEMM_TUNE_SAMPLE_US", "500")
    os.environ["TILEGEMM_TUNE_CONFIRM"] = "0"
    # split-K cannot help a problem that fills the chip many times over
    flops = 2.0 * M * N * K
    os.environ["TILEGEMM_TUNE_MAX_SPLIT"] = str(max_split or (1 if flops > 2e11 else 64))
    t0 = time.perf_counter()
    tg.gemm_autotune(M, N, K, dtype)
    rows = [[list(c.astuple()), pred, meas] for c, pred, meas, _ in tg.autotune_table(M, N, K, dtype) if meas > 0]
    doc = {"workload": name, "M": M, "N": N, "K": K, "dtype": dtype, "operands": "uniform [-1, 1)",
           "tune_s": round(time.perf_counter() - t0, 2), "rows": rows}
    with gzip.open(os.path.join(out_dir, f"table_{name}.json.gz"), "wt") as f:
        json.dump(doc, f, separators=(",", ":"))
    tg.cache_clear()
    return doc


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True)
    ap.add_argument("--only", nargs="*", default=None)
    a = ap.parse_args(argv)
    import tile_shape_autotuning_amd as tg
    tg._native.lib()
    os.makedirs(a.out, exist_ok=True)
    for name, M, N, K, dt in workload_shapes() + CALIBRATION_SHAPES:
        if a.only and name not in a.only:
            continue
        doc = dump_table(tg, name, M, N, K, dt, a.out)
        best = min(doc["rows"], key=lambda r: r[2])
        print(f"[tables] {name}: {len(doc['rows'])} configurations in {doc['tune_s']} s, best {best[0]} "
              f"{best[2]:.2f} us", flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
