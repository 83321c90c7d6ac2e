"""GPU parity of the occupancy-tuned RMS normalisation against the fp64 oracle.

Page "CuTile Autotuning" ("Quick Reference -- Occupancy-Only Autotune"):
occupancy is the only tuned parameter of such kernels; tune once per shape,
cache, launch directly.  The bound: bf16 output is the round-to-nearest of
an fp32 computation, so |y - ref| <= (2^-8 + 1e-5) |ref| (half a bf16 unit in
the last place plus the fp32 arithmetic).  Every occupancy must give the
same bits: a row is reduced in a fixed order whichever workgroup takes it.
"""
import numpy as np
import pytest

from oracle import rmsnorm_ref as R
from tile_shape_autotuning_amd import workloads as wl

from gpu_util import mark, out_bits

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tg = pytest.importorskip("tile_shape_autotuning_amd")


@pytest.fixture(autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs(rows, n, seed):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, n)) * rng.uniform(0.01, 100.0, (rows, 1))   # rows of different scales
    w = rng.uniform(-2.0, 2.0, n)
    return wl.f32_to_bf16_bits(x.astype(np.float32)), wl.f32_to_bf16_bits(w.astype(np.float32))


def _dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _check(y, ref, what):
    got = wl.bf16_bits_to_f32(out_bits(y)).astype(np.float64)
    err = np.abs(got - ref)
    bound = (2.0 ** -8 + 1e-5) * np.abs(ref) + 1e-30
    bad = np.count_nonzero(err > bound)
    assert bad == 0, f"{what}: {bad} outputs beyond the bound, worst {np.max(err / bound):.3g}x"


@pytest.mark.parametrize("rows,n", [(1, 8), (3, 1000), (64, 4096), (257, 8192), (1000, 12288), (17, 32768)])
def test_every_occupancy_matches_the_oracle_and_each_other(rows, n):
    x, w = _inputs(rows, n, rows + n)
    eps = 1e-5
    ref = R.rmsnorm(x, w, eps)
    x_d, w_d = _dev(x), _dev(w)
    first = None
    for occ in (1, 2, 4, 8):
        mark(f"rmsnorm {rows}x{n} occupancy {occ}")
        y = tg.rmsnorm(x_d, w_d, eps, occupancy=occ)
        torch.cuda.synchronize()
        _check(y, ref, f"{rows}x{n} occupancy {occ}")
        if first is None:
            first = y.clone()
        else:
            assert torch.equal(y.view(torch.int16), first.view(torch.int16)), f"occupancy {occ} differs"


def test_tuned_once_per_shape_then_cached():
    rows, n = 2048, 4096
    x, w = _inputs(rows, n, 5)
    ref = R.rmsnorm(x, w, 1e-6)
    x_d, w_d = _dev(x), _dev(w)
    t0 = tg.rmsnorm_tunes()
    mark("rmsnorm tuned 2048x4096")
    y = tg.rmsnorm(x_d, w_d, 1e-6)
    torch.cuda.synchronize()
    _check(y, ref, "tuned")
    assert tg.rmsnorm_tunes() == t0 + 1
    hit = tg.rmsnorm_cache_lookup(rows, n)
    assert hit is not None and hit[0] in (1, 2, 4, 8) and hit[1] > 0
    y2 = tg.rmsnorm(x_d, w_d, 1e-6)
    torch.cuda.synchronize()
    assert tg.rmsnorm_tunes() == t0 + 1, "a cached shape is not tuned again"
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))
    assert tg.rmsnorm_autotune(rows, n) == hit


def test_argument_errors():
    x = torch.zeros((4, 16), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    y = torch.empty_like(x)
    N = tg._native
    assert N.rmsnorm_ptr(4, 16, x.data_ptr(), w.data_ptr(), y.data_ptr(), 1e-6, 3) == N.TG_E_INVAL
    assert N.rmsnorm_ptr(4, 16, x.data_ptr() + 2, w.data_ptr(), y.data_ptr(), 1e-6, 1) == N.TG_E_INVAL
    assert N.rmsnorm_ptr(4, 12, x.data_ptr(), w.data_ptr(), y.data_ptr(), 1e-6, 1) == N.TG_E_UNSUPPORTED
    assert N.rmsnorm_ptr(4, 16, x.data_ptr(), w.data_ptr(), y.data_ptr(), -1.0, 1) == N.TG_E_INVAL
    assert N.rmsnorm_ptr(0, 16, 0, 0, 0, 1e-6, 0) == N.TG_OK
