"""rocprofv3 harness: commands and summaries for the GEMM kernels.

The measurement side of the method (page "Tile Selection: Cost Models Against
Measurement", "Measurement, and what it must control") reports what the
hardware did: per-kernel average duration from a kernel trace, matrix-core
utilisation and LDS bank conflicts from SQ counters, and HBM traffic from the
L2 fetch/write counters, scaled by what the same counters read for a plain
copy of known size.

    python -m tile_shape_autotuning_amd.rocprof_report commands [bench args...]
    python -m tile_shape_autotuning_amd.rocprof_report summary --trace DIR [--pmc DIR ...]
        [--fetch DIR --write DIR --copy-bytes N] [--kernel SUBSTR] [--flops F] [--bytes B]

rocprofv3 writes SQLite databases (`*_results.db`); this module reads them
with the standard library only.
"""
from __future__ import annotations

import argparse
import collections
import glob
import json
import os
import sqlite3
import sys

MFMA_PASS = ["SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES",
             "SQ_LDS_BANK_CONFLICT", "SQ_INSTS_LDS", "SQ_WAIT_INST_LDS", "SQ_WAVE_CYCLES", "SQ_WAIT_ANY",
             "GRBM_GUI_ACTIVE"]
SIMDS_PER_CU = 4
MFMA_FLOPS_PER_MOP = 512        # SQ_INSTS_VALU_MFMA_MOPS_* counts 512-flop units


def commands(bench_args, outdir="rocprof_out"):
    """The rocprofv3 invocations that produce the summaries (one pass each)."""
    b = " ".join(["python3", "bench.py"] + list(bench_args))
    return [
        f"rocprofv3 --kernel-trace --stats -d {outdir}/trace -o run -- {b}",
        f"rocprofv3 --pmc {' '.join(MFMA_PASS)} -d {outdir}/pmc -o run -- {b}",
        f"rocprofv3 --pmc FETCH_SIZE -d {outdir}/fetch -o run -- {b} --copy-calib 1073741824",
        f"rocprofv3 --pmc WRITE_SIZE -d {outdir}/write -o run -- {b} --copy-calib 1073741824",
    ]


def _dbs(d):
    out = sorted(glob.glob(os.path.join(d, "**", "*_results.db"), recursive=True))
    if not out:
        raise FileNotFoundError(f"no *_results.db under {d}")
    return out


def kernel_times(trace_dir, grid=None):
    """{kernel name: (calls, average ns)} from a kernel trace; with grid, only
    the dispatches of that many work-items (one template can serve several
    problems in one run)."""
    acc = collections.defaultdict(lambda: [0, 0.0])
    for db in _dbs(trace_dir):
        c = sqlite3.connect(db)
        for name, dur, gx in c.execute("select name, duration, grid_x from kernels"):
            if grid is not None and int(gx) != int(grid):
                continue
            acc[name][0] += 1
            acc[name][1] += float(dur)
    return {k: (n, s / n) for k, (n, s) in acc.items()}


def dispatch_counters(pmc_dir):
    """{kernel name: {counter: [value of each dispatch]}} (a counter's
    per-instance values summed within a dispatch)."""
    acc = collections.defaultdict(lambda: collections.defaultdict(dict))
    for db in _dbs(pmc_dir):
        c = sqlite3.connect(db)
        q = "select kernel_name, dispatch_id, counter_name, value from counters_collection"
        for name, disp, ctr, val in c.execute(q):
            acc[name][ctr][(db, disp)] = acc[name][ctr].get((db, disp), 0.0) + float(val)
    return {k: {ctr: list(v.values()) for ctr, v in d.items()} for k, d in acc.items()}


def counters(pmc_dir):
    """{kernel name: {counter: mean value per dispatch}}."""
    return {k: {ctr: sum(v) / len(v) for ctr, v in d.items()}
            for k, d in dispatch_counters(pmc_dir).items()}


def copy_calibration(per_dispatch, counter):
    """The counter's reading for the calibration copy: the median over the
    largest copy dispatches (those within 10 % of the largest).  The program
    may run smaller copies of its own under the same kernel name (a weight
    replica, say); a mean over every dispatch of that name would mix them in."""
    vals = [v for n, d in per_dispatch.items() if "copy" in n.lower() or "elementwise" in n.lower()
            for v in d.get(counter, [])]
    if not vals or max(vals) <= 0:
        return 0.0
    top = sorted(v for v in vals if v >= 0.9 * max(vals))
    return top[len(top) // 2]


def _pick(d, sub):
    keys = [k for k in d if sub in k]
    if not keys:
        raise KeyError(f"no kernel matching {sub!r}; have {list(d)[:5]}")
    return max(keys, key=lambda k: d[k][0] if isinstance(d[k], tuple) else 0)


def summary(trace_dir, pmc_dirs=(), fetch_dir=None, write_dir=None, copy_bytes=0, kernel="gemm",
            flops=None, nbytes=None, grid=None, second=None):
    """Figures of one kernel.  `second` = (name substring, grid) of a kernel
    that every call launches after it (the split-K second pass): its average
    duration and HBM bytes are reported too, and the per-call figures cover
    both launches."""
    times = kernel_times(trace_dir, grid)
    kname = _pick(times, kernel)
    calls, avg_ns = times[kname]
    out = {"kernel": kname, "calls": calls, "avg_us": avg_ns / 1e3, "call_us": avg_ns / 1e3}
    if second:
        t2 = kernel_times(trace_dir, second[1])
        k2 = _pick(t2, second[0])
        out["second"] = {"kernel": k2, "calls": t2[k2][0], "avg_us": t2[k2][1] / 1e3}
        out["call_us"] = out["avg_us"] + out["second"]["avg_us"]
        avg_ns = out["call_us"] * 1e3
    if flops:
        out["TFLOP/s"] = flops / (avg_ns * 1e-9) / 1e12
    if nbytes:
        out["GB/s"] = nbytes / (avg_ns * 1e-9) / 1e9
    for d in pmc_dirs:
        cs = counters(d)
        k = next((n for n in cs if kernel in n), None)
        if k is None:
            continue
        s = cs[k]
        if "SQ_VALU_MFMA_BUSY_CYCLES" in s and s.get("SQ_BUSY_CU_CYCLES"):
            out["mfma_util"] = s["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMDS_PER_CU * s["SQ_BUSY_CU_CYCLES"])
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in s:
            out["mfma_flops_per_dispatch"] = s["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * MFMA_FLOPS_PER_MOP
        if s.get("SQ_INSTS_LDS"):
            out["lds_conflict_cycles_per_lds_inst"] = s.get("SQ_LDS_BANK_CONFLICT", 0.0) / s["SQ_INSTS_LDS"]
        if s.get("SQ_WAVE_CYCLES"):
            out["wait_any_frac"] = s.get("SQ_WAIT_ANY", 0.0) / s["SQ_WAVE_CYCLES"]
            out["wait_lds_frac"] = s.get("SQ_WAIT_INST_LDS", 0.0) / s["SQ_WAVE_CYCLES"]
        out.setdefault("counters", {}).update({c: s[c] for c in s})
    if fetch_dir and write_dir and copy_bytes:
        out["traffic"] = hbm_traffic(fetch_dir, write_dir, copy_bytes, kernel)
        if second:
            t2 = hbm_traffic(fetch_dir, write_dir, copy_bytes, second[0])
            out["second"]["traffic"] = t2
            tr = out["traffic"]
            out["traffic"] = {n: {"kib_raw": tr[n]["kib_raw"] + t2[n]["kib_raw"], "scale": tr[n]["scale"],
                                  "bytes": tr[n]["bytes"] + t2[n]["bytes"]} for n in ("FETCH_SIZE", "WRITE_SIZE")}
            out["traffic"]["bytes"] = tr["bytes"] + t2["bytes"]
    return out


def observed_clock_ghz(ctrs, avg_us, xcds=8):
    """Shader clock while the kernel ran: GRBM_GUI_ACTIVE (summed over the
    XCDs) per XCD, over the kernel's average duration."""
    return ctrs["GRBM_GUI_ACTIVE"] / xcds / (avg_us * 1e-6) / 1e9


def hbm_traffic(fetch_dir, write_dir, copy_bytes, kernel="gemm"):
    """HBM bytes per dispatch of the kernel, from FETCH_SIZE and WRITE_SIZE (KiB),
    each scaled so that a plain copy of copy_bytes reads and writes exactly
    copy_bytes."""
    res = {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = dispatch_counters(d)
        cs = {n: {c: sum(v) / len(v) for c, v in dd.items()} for n, dd in per.items()}
        k = next((n for n in cs if kernel in n), None)
        copy_kib = copy_calibration(per, name)
        if k is None or copy_kib <= 0:
            raise KeyError(f"{name}: kernel or copy calibration missing")
        scale = (copy_bytes / 1024.0) / copy_kib if copy_kib > 0 else float("nan")
        res[name] = {"kib_raw": cs[k].get(name, 0.0), "copy_kib_raw": copy_kib, "scale": scale,
                     "bytes": cs[k].get(name, 0.0) * 1024.0 * scale}
    res["bytes"] = res["FETCH_SIZE"]["bytes"] + res["WRITE_SIZE"]["bytes"]
    return res


def kernel_table(trace_dir, top=12, match=()):
    """Text table of the kernels in a trace (one row per kernel and grid
    size), by total time; with `match`, only kernels whose name contains one
    of those strings."""
    acc = collections.defaultdict(lambda: [0, 0.0])
    for db in _dbs(trace_dir):
        c = sqlite3.connect(db)
        for name, dur, gx in c.execute("select name, duration, grid_x from kernels"):
            if match and not any(m in name for m in match):
                continue
            acc[(name, int(gx))][0] += 1
            acc[(name, int(gx))][1] += float(dur)
    rows = sorted(acc.items(), key=lambda kv: -kv[1][1])[:top]
    out = [f"{'calls':>7} {'avg us':>10} {'total ms':>9} {'work-items':>10}  kernel"]
    for (name, gx), (n, tot) in rows:
        out.append(f"{n:>7} {tot / n / 1e3:>10.3f} {tot / 1e6:>9.3f} {gx:>10}  {name}")
    return "\n".join(out)


def kernel_name(cfg, in_bf16=True, stream_b=False):
    """The template name rocprofv3 prints for a configuration's kernel
    (stream_b: the instantiation that reads B with the non-temporal policy,
    which launches with a single row of tiles use)."""
    kind, bm, bn, bk, wgm, wgn, st, split = cfg
    if kind in (0, 4):
        # the sliced-K kind is the same kernel with its K groups compiled in
        return (f"gemm_tiled_dma_kernel<{bm}, {bn}, {bk}, {wgm}, {wgn}, {st}, {'true' if stream_b else 'false'}, "
                f"{'false' if in_bf16 else 'true'}, {split if kind == 4 else 1}>")
    if kind == 1:
        return f"gemm_skinny_kernel<{bm // 16}, {wgm}, {st}>"
    return f"gemm_tiled_kernel<{'true' if in_bf16 else 'false'}, {bm}, {bn}, {bk}, {wgm}, {wgn}, {st}"


def counters_text(workload, cfg, kname, trace_dir, pmc_dirs, fetch_dir, write_dir, copy_bytes, flops,
                  algo_bytes, commands_used, grid=None, second=None):
    """Summary of one kernel on one workload: duration, MFMA utilisation, LDS
    bank conflicts, L2 hit rate and HBM bytes (FETCH_SIZE / WRITE_SIZE scaled
    by the same counters for a plain copy of copy_bytes).  With `second` (the
    split-K second pass) the rates and bytes are per call, both launches."""
    sm = summary(trace_dir, pmc_dirs, fetch_dir, write_dir, copy_bytes, kname, flops, algo_bytes, grid, second)
    c = sm.get("counters", {})
    lines = [f"# {kname} on {workload}", "", "cfg (kind,bm,bn,bk,wgm,wgn,stages,split_k): " +
             ",".join(str(x) for x in cfg), "", "commands (run from the repository root on MI355X):"]
    lines += [f"  {cmd}" for cmd in commands_used]
    lines += ["", f"launches traced:            {sm['calls']}" + (f" (dispatches of {grid} work-items)" if grid else ""),
              f"average duration:           {sm['avg_us']:.3f} us"]
    if second:
        s2 = sm["second"]
        lines += [f"second pass {s2['kernel']}: {s2['calls']} launches, average {s2['avg_us']:.3f} us",
                  f"per call (both launches):   {sm['call_us']:.3f} us"]
    per = "call" if second else "launch"
    if flops:
        lines.append(f"algorithmic TFLOP/s:        {sm['TFLOP/s']:.1f}   (2MNK = {flops:.4g} flop per {per})")
    if algo_bytes:
        lines.append(f"algorithmic GB/s:           {sm['GB/s']:.1f}   (compulsory {algo_bytes:.4g} B per {per})")
    if "mfma_util" in sm:
        lines.append(f"MFMA busy / (4 x CU busy):  {sm['mfma_util']:.3f}")
    if c.get("GRBM_GUI_ACTIVE") and sm["avg_us"] >= 200.0:
        # the GPU-busy counter also spans several microseconds around each
        # dispatch (a 27 us kernel read as 80,000 cycles per XCD, 3 GHz): both
        # figures that divide by it are printed for long kernels only
        if c.get("SQ_BUSY_CU_CYCLES"):
            lines.append(f"busy CUs (CU-busy / GPU-busy cycles, 8 XCDs): "
                         f"{c['SQ_BUSY_CU_CYCLES'] / (c['GRBM_GUI_ACTIVE'] / 8):.0f}")
        lines.append(f"clock (GPU-busy cycles per XCD / duration): {observed_clock_ghz(c, sm['avg_us']):.2f} GHz")
    if "lds_conflict_cycles_per_lds_inst" in sm:
        lines.append(f"LDS bank-conflict cycles per LDS instruction: {sm['lds_conflict_cycles_per_lds_inst']:.2f}")
    if "wait_any_frac" in sm:
        lines.append(f"wave cycles waiting (any): {sm['wait_any_frac']:.3f}")
    if c.get("TCC_HIT_sum") is not None and c.get("TCC_MISS_sum") is not None:
        h, m = c["TCC_HIT_sum"], c["TCC_MISS_sum"]
        lines.append(f"L2 hit rate:                {h / max(1.0, h + m):.3f}  ({h:.4g} hits, {m:.4g} misses per launch)")
    tr = sm.get("traffic")
    if tr:
        f, w = tr["FETCH_SIZE"], tr["WRITE_SIZE"]
        lines += ["", f"HBM traffic per {per} (counter KiB x scale; scale = copy bytes / copy counter):",
                  f"  FETCH_SIZE {f['kib_raw']:.1f} KiB x {f['scale']:.4f} = {f['bytes']:.4g} B",
                  f"  WRITE_SIZE {w['kib_raw']:.1f} KiB x {w['scale']:.4f} = {w['bytes']:.4g} B",
                  f"  total {tr['bytes']:.4g} B" + (f" = {tr['bytes'] / algo_bytes:.2f} x the compulsory bytes"
                                                     if algo_bytes else ""),
                  f"  achieved HBM rate {tr['bytes'] / (sm['call_us'] * 1e-6) / 1e9:.1f} GB/s"]
    lines += ["", "raw counters (mean per dispatch):"]
    lines += [f"  {k} = {v:.6g}" for k, v in sorted(c.items())]
    return "\n".join(lines) + "\n", sm


def workload_launch(index, cfg):
    """Kernel name, work-items of its dispatch, and the second pass (name,
    work-items) or None, for a workload run with cfg -- the figures that pick
    its dispatches out of a trace of several workloads."""
    from . import workloads as wl
    w = wl.WORKLOADS[index]
    kind, bm, bn, bk, wgm, wgn, st, split = cfg
    in_bf16 = w.dtype != wl.F32
    tiles = -(-w.M // bm) * -(-w.N // bn)
    stream_b = kind == 0 and in_bf16 and bm <= 64 and w.M <= bm
    if kind == 1:
        threads = 64 * wgm
        tiles = -(-w.N // 128)
    else:
        threads = 64 * wgm * wgn
    name = kernel_name(cfg, in_bf16, stream_b)
    if kind == 4:
        # sliced-K: split groups of waves inside each tile's one workgroup
        return name, tiles * threads * split, None
    second = None
    if split > 1:
        blocks = min(-(-w.M * w.N // 1024), 65536)
        second = (f"splitk_reduce_kernel<{split}>", blocks * 256)
    return name, tiles * split * threads, second


def render(index, cfg, trace, pmc_dirs, fetch, write, commands_used, out_path=None):
    """Text summary of one workload's kernel: average duration of its
    dispatches in `trace` (picked by kernel name and work-items, so a trace of
    several workloads serves), counters from the pmc passes, HBM traffic from
    the FETCH_SIZE / WRITE_SIZE passes (each run with a 1 GiB copy for the
    scale); `commands_used` are the commands printed at the top."""
    from . import workloads as wl
    w = wl.WORKLOADS[index]
    name, grid, second = workload_launch(index, cfg)
    text, sm = counters_text(w.name, cfg, name, trace, pmc_dirs, fetch, write, 1 << 30, w.flops,
                             w.compulsory_bytes, commands_used, grid=grid, second=second)
    if out_path:
        with open(out_path, "w") as f:
            f.write(text)
    return text, sm


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("render")
    r.add_argument("--workload", type=int, required=True)
    r.add_argument("--cfg", required=True, help="kind,bm,bn,bk,wgm,wgn,stages,split_k")
    r.add_argument("--trace", required=True)
    r.add_argument("--pmc", action="append", default=[])
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--command", action="append", default=[], help="a command that made the data (repeatable)")
    r.add_argument("--out", default="")
    c = sub.add_parser("commands")
    c.add_argument("bench_args", nargs=argparse.REMAINDER)
    k = sub.add_parser("kernels", help="the kernel table of a trace, by total time")
    k.add_argument("--trace", required=True)
    k.add_argument("--top", type=int, default=12)
    k.add_argument("--match", action="append", default=[], help="keep kernels whose name contains this (repeatable)")
    s = sub.add_parser("summary")
    s.add_argument("--trace", required=True)
    s.add_argument("--pmc", action="append", default=[])
    s.add_argument("--fetch")
    s.add_argument("--write")
    s.add_argument("--copy-bytes", type=int, default=0)
    s.add_argument("--kernel", default="gemm")
    s.add_argument("--flops", type=float)
    s.add_argument("--bytes", type=float)
    a = ap.parse_args(argv)
    if a.cmd == "render":
        cfg = tuple(int(x) for x in a.cfg.split(","))
        text, _ = render(a.workload, cfg, a.trace, a.pmc, a.fetch, a.write, a.command, a.out or None)
        print(text)
        return 0
    if a.cmd == "kernels":
        print(kernel_table(a.trace, a.top, tuple(a.match)))
        return 0
    if a.cmd == "commands":
        print("\n".join(commands(a.bench_args)))
    else:
        print(json.dumps(summary(a.trace, a.pmc, a.fetch, a.write, a.copy_bytes, a.kernel, a.flops, a.bytes),
                         indent=1))


if __name__ == "__main__":
    sys.exit(main())
