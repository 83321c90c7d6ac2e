"""Launch geometry on the device: the workgroups and threads per workgroup
that the runtime dispatched, as its tracer records them, are the ones the
selection plans (tg_grid: ceil(M/BM) ceil(N/BN) tiles times the workgroups
per tile, page "Tile Selection: Cost Models Against Measurement", "The
structure of the search space"), for every kernel kind, and the second pass
runs exactly where the plan has one (split-K across workgroups, a stream-K
tail cut into pieces), as do the padded path's copies and output pass."""
import json

import pytest

from oracle import select_ref as S
from tile_shape_autotuning_amd import workloads as wl

from gpu_util import mark

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tg = pytest.importorskip("tile_shape_autotuning_amd")

# (M, N, K, dtype, cfg): every kind, split-K, a single row of tiles (B
# streamed), an unaligned shape, fp32; K is exact in bf16 (the outputs of
# all-ones operands are K)
CASES = [
    (300, 264, 520, wl.BF16, (0, 64, 64, 64, 2, 2, 2, 2)),
    (200, 168, 392, wl.BF16, (0, 16, 32, 64, 1, 2, 3, 1)),
    (16, 2048, 1024, wl.BF16, (0, 32, 256, 32, 1, 2, 4, 2)),
    (16, 1024, 512, wl.BF16, (1, 16, 128, 32, 4, 1, 2, 2)),
    (300, 262, 516, wl.BF16, (2, 64, 64, 32, 2, 2, 2, 1)),
    (1024, 1040, 2048, wl.BF16_F32OUT, (3, 256, 256, 64, 2, 4, 2, 1)),
    (300, 264, 520, wl.BF16, (4, 32, 64, 128, 1, 2, 2, 4)),
    (256, 256, 256, wl.F32, (4, 16, 32, 64, 1, 1, 2, 4)),
    # the tiled kind's padded path: copies, the kernel on the padded extents, output pass
    (300, 262, 516, wl.BF16, (0, 64, 64, 64, 2, 2, 2, 1)),
    (300, 262, 1020, wl.BF16, (0, 64, 64, 64, 2, 2, 2, 2)),
    (130, 130, 258, wl.F32, (0, 32, 64, 32, 2, 2, 3, 1)),
]


def _threads(c):
    kind, bm, bn, bk, wgm, wgn, st, s = c
    if kind == S.KIND_SKINNY:
        return 64 * wgm
    return 64 * wgm * wgn * (s if kind == S.KIND_SLICEDK else 1)


def _other_kernels(M, N, K, dt, c):
    """Kernels the call runs besides the GEMM: the split-K or stream-K second
    pass, or the padded path's copies and output pass."""
    kind, s = c[0], c[7]
    if S.padded_path(N, K, dt, S.Cfg(*c), S.MI355X):
        return 2
    if kind == S.KIND_STREAMK:
        return int(S.streamk_plan(M, N, K, S.Cfg(*c))["smax"] >= 2)
    return int(kind != S.KIND_SLICEDK and s > 1)


def test_dispatched_grid_is_the_planned_one(tmp_path):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from torch.profiler import ProfilerActivity, profile
    calls = []
    for M, N, K, dt, c in CASES:
        assert tg.check_cfg(M, N, K, dt, c) == 0 and tg.has_kernel(dt, c), c
        t = torch.float32 if dt == wl.F32 else torch.bfloat16
        A = torch.ones((M, K), device="cuda", dtype=t)
        B = torch.ones((K, N), device="cuda", dtype=t)
        calls.append((A, B, torch.float32 if dt != wl.BF16 else torch.bfloat16, c))
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CPU, ProfilerActivity.CUDA]) as prof:
        for (M, N, K, dt, c), (A, B, odt, cfg) in zip(CASES, calls):
            mark(f"launch grid {M}x{N}x{K} dt{dt} {cfg}")
            C = tg.gemm_bias_act(A, B, out_dtype=odt, cfg=cfg)
            torch.cuda.synchronize()
            # all-ones operands: every output is K
            assert torch.all(C.float() == float(K)), cfg
    path = tmp_path / "trace.json"
    prof.export_chrome_trace(str(path))
    with open(path) as f:
        events = json.load(f)["traceEvents"]
    kernels = sorted((e for e in events if e.get("cat") == "kernel" and "tg::" in e.get("name", "")),
                     key=lambda e: e["ts"])
    gemms = [e for e in kernels if "gemm_" in e["name"]]
    assert len(gemms) == len(CASES), [e["name"] for e in kernels]
    for e, (M, N, K, dt, c) in zip(gemms, CASES):
        tiles, blocks = tg.grid(M, N, K, c)
        assert e["args"]["grid"] == [blocks, 1, 1], (c, e["name"], e["args"])
        assert e["args"]["block"] == [_threads(c), 1, 1], (c, e["name"], e["args"])
        if c[0] == S.KIND_SLICEDK:
            assert e["name"].rstrip(")").split("(")[0].endswith(f", {c[7]}>"), e["name"]
        if c[0] != S.KIND_SLICEDK and c[0] != S.KIND_STREAMK and c[7] > 1:
            assert blocks == tiles * c[7]
    others = [e for e in kernels if "gemm_" not in e["name"]]
    assert len(others) == sum(_other_kernels(M, N, K, dt, c) for M, N, K, dt, c in CASES), [e["name"] for e in others]
    assert sum("pad_operands" in e["name"] for e in others) == sum(
        S.padded_path(N, K, dt, S.Cfg(*c), S.MI355X) for M, N, K, dt, c in CASES)
