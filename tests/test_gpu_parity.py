"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

* Integer-exact inputs (entries in {-2..2}, integer bias, K small enough that
  every partial sum is an integer below 2^24): fp32 accumulation is exact in
  any order, so every feasible configuration -- every tile, wave grid,
  pipeline depth, split-K and edge tile -- must match the oracle bitwise
  (fp32 output) or be exactly the round-to-nearest-even bf16 of it.
* The five workloads with the autotuned and the fixed default
  configuration, within max|err| <= tol * max|C_ref| (tol 1e-4 for fp32
  inputs, 1e-2 for bf16 inputs), on the full output of every workload
  (8192^3 included: the oracle's product takes about 10 s on the host).
* Edge shapes, empty and K = 0 problems, determinism, maximum sizes.
* 48 seeded random problems (ragged or aligned, every dtype, with and
  without bias) with the cost model's choice and random feasible
  configurations of every kind the shape admits, integer-exact.
"""
import numpy as np
import pytest

from oracle import gemm_ref
from oracle import select_ref as S
from tile_shape_autotuning_amd import workloads as wl

from gpu_util import assert_close, mark, out_bits, out_f64, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tg = pytest.importorskip("tile_shape_autotuning_amd")

ACT_NAMES = ["none", "relu", "gelu"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg._native.lib()
    tg.set_device_override(None)
    yield
    torch.cuda.synchronize()


def _int_inputs(M, N, K, dtype, seed):
    return wl.make_inputs(M, N, K, dtype, wl.Dist("int", 2), wl.Dist("int", 2), wl.Dist("int", 4), seed)


def _run(A_d, B_d, bias_d, act, dtype, cfg=None):
    out_dtype = torch.float32 if dtype in (wl.F32, wl.BF16_F32OUT) else torch.bfloat16
    return tg.gemm_bias_act(A_d, B_d, bias_d, act=act, out_dtype=out_dtype, cfg=cfg)


def _exact_check(C, ref, dtype, what):
    if dtype == wl.BF16:
        want = wl.f32_to_bf16_bits(ref.astype(np.float32))
        got = out_bits(C)
        bad = np.count_nonzero(got != want)
        assert bad == 0, f"{what}: {bad} of {want.size} bf16 outputs differ from RNE(exact)"
    else:
        got = out_f64(C)
        bad = np.count_nonzero(got != ref)
        assert bad == 0, f"{what}: {bad} of {ref.size} outputs differ from the exact result"


def test_first_kernel_default_cfg_integer_exact():
    for dtype in (wl.BF16, wl.F32, wl.BF16_F32OUT):
        M = N = K = 256
        A, B, bias = _int_inputs(M, N, K, dtype, 1)
        ref = gemm_ref.gemm(A, B, bias, "relu")
        cfg = S.default_cfg(N, K, dtype).astuple()
        mark(f"default cfg {cfg} dtype {dtype} 256^3")
        C = _run(to_dev(A), to_dev(B), to_dev(bias), "relu", dtype, cfg)
        torch.cuda.synchronize()
        _exact_check(C, ref, dtype, f"dtype {dtype} cfg {cfg}")


@pytest.mark.parametrize("M,N,K,dtype", [
    (200, 136, 328, wl.BF16),         # ragged in M and N, K not a multiple of 64
    (96, 264, 520, wl.BF16_F32OUT),
    (130, 100, 260, wl.F32),          # fp32: ragged everywhere, K mod 16 = 4
    (40, 200, 300, wl.F32),
])
def test_every_feasible_cfg_integer_exact(M, N, K, dtype):
    A, B, bias = _int_inputs(M, N, K, dtype, 2)
    ref = gemm_ref.gemm(A, B, bias, "relu")
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    feas = [c for c in tg.enumerate_feasible(M, N, K, dtype) if tg.has_kernel(dtype, c)]
    assert len(feas) > 50
    for c in feas:
        mark(f"sweep {M}x{N}x{K} dt{dtype} {c.astuple()}")
        C = _run(A_d, B_d, b_d, "relu", dtype, c)
        torch.cuda.synchronize()
        _exact_check(C, ref, dtype, f"{M}x{N}x{K} dt{dtype} {c.astuple()}")


@pytest.mark.parametrize("M,N,K,dtype", [
    (17, 65, 15, wl.BF16), (63, 17, 1, wl.F32), (1, 1, 1, wl.BF16), (65, 33, 63, wl.BF16_F32OUT),
    (300, 47, 129, wl.F32), (5, 1000, 77, wl.BF16),                 # ... and K ragged only
    (40, 1001, 512, wl.BF16), (100, 130, 128, wl.F32),               # N ragged only
    (100, 128, 130, wl.F32), (70, 264, 515, wl.BF16_F32OUT),          # K ragged only
])
def test_unaligned_shapes_integer_exact(M, N, K, dtype):
    # every configuration of the element-load kind and of the tiled kind's
    # padded path (zero-padded copies of A and B, slabs, output pass)
    A, B, bias = _int_inputs(M, N, K, dtype, 3)
    ref = gemm_ref.gemm(A, B, bias, "relu")
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    feas = [c for c in tg.enumerate_feasible(M, N, K, dtype) if tg.has_kernel(dtype, c)]
    assert {c.kind for c in feas} == {S.KIND_UNALIGNED, S.KIND_TILED}
    assert all(S.padded_path(N, K, dtype, S.Cfg(*c.astuple()), S.MI355X) for c in feas if c.kind == S.KIND_TILED)
    for c in feas:
        mark(f"unaligned {M}x{N}x{K} dt{dtype} {c.astuple()}")
        C = _run(A_d, B_d, b_d, "relu", dtype, c)
        torch.cuda.synchronize()
        _exact_check(C, ref, dtype, f"{M}x{N}x{K} {c.astuple()}")
    mark(f"unaligned {M}x{N}x{K} dt{dtype} autotuned")
    C = _run(A_d, B_d, b_d, "relu", dtype)
    torch.cuda.synchronize()
    _exact_check(C, ref, dtype, f"{M}x{N}x{K} autotuned")


def _random_problem(rng):
    """A seeded random problem: M from 1 to 1500, N and K mostly on the
    16-byte alignment the tiled kinds need (else only the element-load kind
    is feasible), any dtype, ReLU or none, bias or none."""
    dtype = int(rng.choice([wl.BF16, wl.F32, wl.BF16_F32OUT]))
    unit = 4 if dtype == wl.F32 else 8
    M = int(rng.integers(1, 1501))
    if rng.random() < 0.8:
        N, K = unit * int(rng.integers(1, 1501 // unit + 1)), unit * int(rng.integers(1, 2049 // unit + 1))
    else:
        N, K = int(rng.integers(1, 1501)), int(rng.integers(1, 2049))
    act = str(rng.choice(["none", "relu"]))
    return M, N, K, dtype, act, bool(rng.random() < 0.7)


@pytest.mark.parametrize("seed", range(48))
def test_random_problems_random_cfgs_integer_exact(seed):
    """Random shapes (ragged or aligned, every dtype) with the cost model's
    choice and up to six random feasible configurations, at least one of each
    kind the shape admits (data-parallel, split-K, sliced-K, stream-K, skinny,
    element-load), all integer-exact against the oracle."""
    rng = np.random.default_rng(1000 + seed)
    M, N, K, dtype, act, with_bias = _random_problem(rng)
    A, B, bias = _int_inputs(M, N, K, dtype, 10 + seed)
    if not with_bias:
        bias = None
    ref = gemm_ref.gemm(A, B, bias, act)
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    feas = [c for c in tg.enumerate_feasible(M, N, K, dtype) if tg.has_kernel(dtype, c)]
    assert feas
    picks = {}
    for c in feas:                                   # one of each kind, then random others
        key = (c.kind, c.split_k > 1)
        picks.setdefault(key, c)
    chosen = list(picks.values())
    rest = [c for c in feas if c not in chosen]
    for i in rng.permutation(len(rest))[:max(0, 6 - len(chosen))]:
        chosen.append(rest[int(i)])
    chosen.append(tg.model_choice(M, N, K, dtype)[0])
    for c in chosen:
        mark(f"random {seed}: {M}x{N}x{K} dt{dtype} {act} bias={with_bias} {c.astuple()}")
        C = _run(A_d, B_d, b_d, act, dtype, c)
        torch.cuda.synchronize()
        _exact_check(C, ref, dtype, f"{M}x{N}x{K} dt{dtype} {act} {c.astuple()}")


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
@pytest.mark.parametrize("K", [515, 512])
def test_padded_path_misaligned_pointers(dtype, K):
    # a shape with only K ragged reads B in place and stores C directly, and
    # an aligned shape reads both in place -- unless B or C (or A) sits off
    # 16-byte alignment, which the tiled kind's padded path then copies (A, B)
    # or sends through the output pass (C)
    M, N = 96, 264
    A, B, bias = _int_inputs(M, N, K, dtype, 12)
    ref = gemm_ref.gemm(A, B, bias, "relu")
    tdt = torch.float32 if dtype == wl.F32 else torch.bfloat16
    odt = tdt
    b_d = to_dev(bias)

    def shifted(x, shift):
        t = to_dev(x)
        buf = torch.zeros(t.numel() + 1, dtype=tdt, device="cuda")
        v = buf[shift:shift + t.numel()].view(t.shape)
        v.copy_(t)
        return v

    cfgs = [(0, 64, 64, 64, 2, 2, 2, 1), (0, 64, 64, 64, 2, 2, 2, 2)] if dtype != wl.F32 else \
        [(0, 64, 64, 32, 2, 2, 2, 1), (0, 64, 64, 32, 2, 2, 2, 2)]
    for sa, sb, sc in ((0, 0, 0), (1, 0, 0), (0, 1, 0), (0, 0, 1), (1, 1, 1)):
        A_d, B_d = shifted(A, sa), shifted(B, sb)
        cbuf = torch.zeros(M * N + 1, dtype=odt, device="cuda")
        out = cbuf[sc:sc + M * N].view(M, N)
        for cfg in cfgs:
            assert tg.check_cfg(M, N, K, dtype, cfg) == 0
            mark(f"padded misaligned dt{dtype} K {K} shifts {sa}{sb}{sc} {cfg}")
            out.fill_(0)
            tg.gemm_bias_act(A_d, B_d, b_d, act="relu", out=out, cfg=cfg)
            torch.cuda.synchronize()
            _exact_check(out, ref, dtype, f"shifts {sa}{sb}{sc} {cfg}")
            if sc:
                assert float(cbuf[0]) == 0.0, "wrote before C"
        if (sa, sb, sc) == (1, 1, 1):
            # without a configuration: the tuned choice, whatever its kind
            mark(f"padded misaligned dt{dtype} K {K} tuned")
            out.fill_(0)
            tg.gemm_bias_act(A_d, B_d, b_d, act="relu", out=out)
            torch.cuda.synchronize()
            _exact_check(out, ref, dtype, "misaligned, tuned")
            assert float(cbuf[0]) == 0.0, "wrote before C"


def test_misaligned_operands_of_a_selected_sliced_k_call(monkeypatch):
    # a call without a configuration whose selection (here the cost model's
    # choice: the sliced-K kind) cannot take operands off 16-byte alignment
    # runs the same tile on the tiled kind, padded
    monkeypatch.setenv("TILEGEMM_DISABLE_AUTOTUNE", "1")
    tg.cache_clear()
    M = N = K = 256
    dtype = wl.F32
    assert tg.model_choice(M, N, K, dtype)[0].kind == S.KIND_SLICEDK
    A, B, bias = _int_inputs(M, N, K, dtype, 13)
    ref = gemm_ref.gemm(A, B, bias, "relu")
    bufs = []
    for x in (A, B):
        t = to_dev(x)
        buf = torch.zeros(t.numel() + 1, dtype=torch.float32, device="cuda")
        v = buf[1:1 + t.numel()].view(t.shape)
        v.copy_(t)
        bufs.append(v)
    cbuf = torch.zeros(M * N + 1, dtype=torch.float32, device="cuda")
    out = cbuf[1:].view(M, N)
    mark("misaligned operands, selected sliced-K")
    tg.gemm_bias_act(bufs[0], bufs[1], to_dev(bias), act="relu", out=out)
    torch.cuda.synchronize()
    _exact_check(out, ref, dtype, "misaligned, selected sliced-K")
    assert float(cbuf[0]) == 0.0
    tg.cache_clear()


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32, wl.BF16_F32OUT])
def test_padded_path_gelu_random_inputs(dtype):
    # the padded path with bias and GELU on random operands, against the fp64
    # oracle within the dtype's tolerance, and twice in a row bit for bit
    M, N, K = 257, 1001, 515
    A, B, bias = wl.make_inputs(M, N, K, dtype, wl.Dist("normal", 1.0), wl.Dist("normal", 1.0 / 23.0),
                                wl.Dist("normal", 0.1), 77)
    ref = gemm_ref.gemm(A, B, bias, "gelu")
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    for cfg in ((0, 64, 64, 64, 2, 2, 2, 1), (0, 128, 128, 64, 2, 4, 2, 2)):
        c = S.Cfg(*cfg)
        if dtype == wl.F32:
            c = S.Cfg(0, 64, 64, 32, 2, 2, 2, cfg[7])
        assert S.padded_path(N, K, dtype, c, S.MI355X) and tg.check_cfg(M, N, K, dtype, c.astuple()) == 0
        mark(f"padded gelu dt{dtype} {c.astuple()}")
        C1 = _run(A_d, B_d, b_d, "gelu", dtype, c.astuple())
        C2 = _run(A_d, B_d, b_d, "gelu", dtype, c.astuple())
        torch.cuda.synchronize()
        assert torch.equal(C1, C2)
        assert_close(out_f64(C1), ref, dtype, f"padded gelu {c.astuple()}")


@pytest.mark.parametrize("M", [1, 3, 16, 17, 31, 48, 64])
def test_skinny_kernels_integer_exact(M):
    N, K = 1032, 1064
    for dtype in (wl.BF16, wl.BF16_F32OUT):
        A, B, bias = _int_inputs(M, N, K, dtype, 4)
        ref = gemm_ref.gemm(A, B, bias, "none")
        A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
        feas = [c for c in tg.enumerate_feasible(M, N, K, dtype) if c.kind == S.KIND_SKINNY]
        assert feas
        for c in feas:
            if not tg.has_kernel(dtype, c):
                continue
            mark(f"skinny M={M} dt{dtype} {c.astuple()}")
            C = _run(A_d, B_d, b_d, "none", dtype, c)
            torch.cuda.synchronize()
            _exact_check(C, ref, dtype, f"skinny M={M} {c.astuple()}")


@pytest.mark.parametrize("M", [1, 16, 40, 64])
def test_streaming_b_tiles_integer_exact(M):
    """Launches with one row of tiles read B with the non-temporal policy
    (their own instantiations): every such feasible configuration, split-K
    included, must still be exact.  N and K ragged against every tile."""
    N, K = 1000, 1064
    for dtype in (wl.BF16, wl.BF16_F32OUT):
        A, B, bias = _int_inputs(M, N, K, dtype, 6)
        ref = gemm_ref.gemm(A, B, bias, "relu")
        A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
        feas = [c for c in tg.enumerate_feasible(M, N, K, dtype)
                if c.kind == S.KIND_TILED and tg.has_kernel(dtype, c) and tg.streams_b(M, dtype, c)]
        assert len(feas) > 50
        for c in feas:
            mark(f"streaming B M={M} dt{dtype} {c.astuple()}")
            C = _run(A_d, B_d, b_d, "relu", dtype, c)
            torch.cuda.synchronize()
            _exact_check(C, ref, dtype, f"streaming B M={M} {c.astuple()}")


@pytest.mark.parametrize("act", ACT_NAMES)
def test_activations_random_inputs(act):
    M, N, K = 333, 200, 512
    for dtype in (wl.F32, wl.BF16):
        A, B, bias = wl.make_inputs(M, N, K, dtype, wl.Dist("normal", 0.1), wl.Dist("normal", 0.1),
                                    wl.Dist("normal", 0.5), 5)
        ref = gemm_ref.gemm(A, B, bias, act)
        mark(f"act {act} dt{dtype}")
        C = _run(to_dev(A), to_dev(B), to_dev(bias), act, dtype, S.default_cfg(N, K, dtype).astuple())
        torch.cuda.synchronize()
        assert_close(out_f64(C), ref, dtype, f"act {act} dtype {dtype}")


def test_gelu_epilogue_accuracy_over_its_range():
    # A = 0, so C = GELU(bias): the epilogue's GELU alone, at pre-activation
    # values across [-12, 12], against the oracle's fp64 erf, for the bf16
    # direct-to-LDS kernel, the fp32 kernel and the element-load kind
    M, N = 48, 4096
    bias = np.linspace(-12.0, 12.0, N).astype(np.float32)
    # K = 60 is not a multiple of 8: the element-load kind; M = 48 also admits the decode kernel
    cases = [(wl.BF16_F32OUT, 64, (0, 32, 128, 64, 1, 2, 2, 1)), (wl.F32, 64, (0, 32, 32, 32, 2, 2, 2, 1)),
             (wl.BF16_F32OUT, 60, None), (wl.BF16_F32OUT, 64, (1, 48, 128, 32, 2, 1, 2, 1))]
    for dtype, K, cfg in cases:
        assert cfg is None or tg.has_kernel(dtype, cfg), cfg
        A = np.zeros((M, K), np.float32 if dtype == wl.F32 else np.uint16)
        B = np.zeros((K, N), A.dtype)
        ref = gemm_ref.gemm(A, B, bias, "gelu")
        mark(f"gelu range dt{dtype} {cfg}")
        C = _run(to_dev(A), to_dev(B), to_dev(bias), "gelu", dtype, cfg)
        torch.cuda.synchronize()
        err = np.abs(out_f64(C) - ref)
        bound = 2e-6 * np.maximum(1.0, np.abs(bias.astype(np.float64)))[None, :]
        assert np.all(err <= bound), f"dt{dtype} {cfg}: worst {float(np.max(err / bound)):.3g} x the bound"


def test_empty_and_k_zero():
    for dtype in (wl.F32, wl.BF16):
        mark(f"K=0 dt{dtype}")
        A, B, bias = _int_inputs(37, 24, 0, dtype, 6)
        A_d = torch.zeros((37, 0), device="cuda", dtype=torch.float32 if dtype == wl.F32 else torch.bfloat16)
        B_d = torch.zeros((0, 24), device="cuda", dtype=A_d.dtype)
        want = np.maximum(np.broadcast_to(bias.astype(np.float64), (37, 24)), 0.0)
        C = _run(A_d, B_d, to_dev(bias), "relu", dtype)
        torch.cuda.synchronize()
        _exact_check(C, want, dtype, "K=0")
        # the sliced-K kind with no K step: every group's sums are zero
        sliced = (4, 16, 32, 64, 1, 1, 2, 4) if dtype == wl.F32 else (4, 16, 64, 128, 1, 1, 2, 4)
        assert tg.has_kernel(dtype, sliced), sliced
        C = _run(A_d, B_d, to_dev(bias), "relu", dtype, sliced)
        torch.cuda.synchronize()
        _exact_check(C, want, dtype, "K=0 sliced-K")
        # K = 0 with a ragged N: the padded path (B's copy has no rows, the
        # kernel sums nothing, the output pass adds the bias)
        A0 = torch.zeros((37, 0), device="cuda", dtype=A_d.dtype)
        B0 = torch.zeros((0, 21), device="cuda", dtype=A_d.dtype)
        want21 = np.maximum(np.broadcast_to(bias[:21].astype(np.float64), (37, 21)), 0.0)
        cfg = (0, 32, 32, 32, 1, 1, 2, 1)
        assert tg.check_cfg(37, 21, 0, dtype, cfg) == 0
        mark(f"K=0 padded dt{dtype}")
        C = _run(A0, B0, to_dev(np.ascontiguousarray(bias[:21])), "relu", dtype, cfg)
        torch.cuda.synchronize()
        _exact_check(C, want21, dtype, "K=0 padded")
        mark(f"M=0 dt{dtype}")
        C = _run(torch.zeros((0, 8), device="cuda", dtype=A_d.dtype),
                 torch.zeros((8, 16), device="cuda", dtype=A_d.dtype), None, "none", dtype)
        assert C.shape == (0, 16)


def test_split_k_deterministic_and_exact():
    M, N, K = 256, 512, 4096
    dtype = wl.BF16_F32OUT
    A, B, bias = wl.make_inputs(M, N, K, dtype, wl.Dist("normal"), wl.Dist("normal"), wl.Dist("normal"), 7)
    ref = gemm_ref.gemm(A, B, bias, "gelu")
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    for s in (1, 2, 4, 8, 16):
        cfg = (0, 128, 128, 64, 2, 2, 2, s)
        mark(f"split {s}")
        C1 = _run(A_d, B_d, b_d, "gelu", dtype, cfg)
        C2 = _run(A_d, B_d, b_d, "gelu", dtype, cfg)
        torch.cuda.synchronize()
        assert torch.equal(C1, C2), f"split {s}: two runs differ"
        assert_close(out_f64(C1), ref, dtype, f"split {s}")


def test_split_k_on_two_streams_concurrently():
    """Each stream has its own split-K workspace: split-K calls queued on two
    streams at once (different problems, different split counts) both stay
    exact."""
    M, N, K, dtype = 96, 1000, 2048, wl.BF16_F32OUT
    probs = []
    for seed, cfg in ((11, (0, 64, 128, 64, 2, 2, 2, 8)), (12, (0, 32, 256, 32, 1, 2, 4, 4))):
        A, B, bias = _int_inputs(M, N, K, dtype, seed)
        probs.append((to_dev(A), to_dev(B), to_dev(bias), gemm_ref.gemm(A, B, bias, "relu"), cfg))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty((M, N), dtype=torch.float32, device="cuda") for _ in probs]
    # first calls grow each stream's workspace
    for (A_d, B_d, b_d, _, cfg), st, C in zip(probs, streams, outs):
        with torch.cuda.stream(st):
            tg.gemm_bias_act(A_d, B_d, b_d, act="relu", out=C, cfg=cfg)
    torch.cuda.synchronize()
    mark("split-K on two streams")
    for rep in range(20):
        for (A_d, B_d, b_d, _, cfg), st, C in zip(probs, streams, outs):
            with torch.cuda.stream(st):
                tg.gemm_bias_act(A_d, B_d, b_d, act="relu", out=C, cfg=cfg)
    torch.cuda.synchronize()
    for (_, _, _, ref, cfg), C in zip(probs, outs):
        _exact_check(C, ref, dtype, f"two streams {cfg}")


def test_split_k_two_host_threads_on_the_null_stream():
    """Two host threads share the null stream's split-K workspace: each
    call's GEMM and second pass must stay adjacent on the stream, and a
    workspace that grows under one thread's call must not be freed under the
    other's.  One thread runs a small problem, the other starts small and
    switches to one that needs a larger workspace; every call writes its own
    output, and every output must be exact."""
    import threading
    dtype = wl.BF16_F32OUT
    probs = {}
    for name, (M, N, K, seed, cfg) in {
            "small": (96, 1000, 2048, 21, (0, 64, 128, 64, 2, 2, 2, 8)),
            "large": (256, 2048, 2048, 22, (0, 64, 256, 32, 2, 2, 2, 16))}.items():
        A, B, bias = _int_inputs(M, N, K, dtype, seed)
        probs[name] = (M, N, K, to_dev(A), to_dev(B), to_dev(bias), gemm_ref.gemm(A, B, bias, "relu"), cfg)
    plan = {0: ["small"] * 24, 1: ["small"] * 8 + ["large"] * 16}
    outs = {t: [torch.empty((probs[n][0], probs[n][1]), dtype=torch.float32, device="cuda") for n in names]
            for t, names in plan.items()}
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(2)

    def worker(t):
        try:
            N_ = tg._native
            N_.set_stream(None)          # the null stream, as every thread's default
            start.wait()
            for name, C in zip(plan[t], outs[t]):
                M, N, K, A_d, B_d, b_d, _, cfg = probs[name]
                st = N_.gemm_bias_act_ptr(M, N, K, A_d.data_ptr(), B_d.data_ptr(), b_d.data_ptr(), C.data_ptr(),
                                          dtype, "relu", cfg)
                if st != 0:
                    errors.append((t, st, N_.last_error()))
        except Exception as e:      # noqa: BLE001
            errors.append((t, repr(e)))

    mark("split-K from two host threads on the null stream")
    th = [threading.Thread(target=worker, args=(t,)) for t in plan]
    for x in th:
        x.start()
    for x in th:
        x.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for t, names in plan.items():
        for i, (name, C) in enumerate(zip(names, outs[t])):
            _exact_check(C, probs[name][6], dtype, f"thread {t} call {i} ({name})")


@pytest.mark.parametrize("M,N,K,cfg", [
    (2048, 2056, 520, (0, 128, 128, 64, 2, 2, 2, 1)),     # many tiles, ragged N and K
    (1000, 1000, 2048, (0, 128, 128, 128, 2, 4, 2, 4)),   # split-K
    (4352, 4224, 136, (3, 256, 256, 64, 2, 4, 2, 1)),     # a full round plus a stream-K tail
])
def test_tile_order_changes_no_result(M, N, K, cfg):
    """The scheduling order (tile rows per group) decides which workgroup
    computes which tile, never what a tile computes: every order gives the
    exact result."""
    dtype = wl.BF16_F32OUT
    A, B, bias = _int_inputs(M, N, K, dtype, 41)
    ref = gemm_ref.gemm(A, B, bias, "relu")
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    try:
        for g in (1, 3, 8, 64):
            tg.set_tile_order(g)
            mark(f"tile order {g}: {M}x{N}x{K} {cfg}")
            C = _run(A_d, B_d, b_d, "relu", dtype, cfg)
            torch.cuda.synchronize()
            _exact_check(C, ref, dtype, f"tile order {g} {cfg}")
    finally:
        tg.set_tile_order(0)


def _streamk_cfgs(M, N, K, dtype):
    return [c.astuple() for c in tg.enumerate_feasible(M, N, K, dtype) if c.kind == 3 and tg.has_kernel(dtype, c)]


@pytest.mark.parametrize("M,N,K,dtype,act", [
    (1024, 1040, 2048, wl.BF16_F32OUT, "none"),   # every tile in the tail, each cut among many workgroups
    (4352, 4224, 136, wl.BF16, "relu"),           # a full round of whole tiles plus a tail; K mod 64 = 8
    (200, 264, 64, wl.BF16, "relu"),              # one K step: every piece is a whole tile
])
def test_streamk_integer_exact(M, N, K, dtype, act):
    """Data-parallel tiles plus the stream-K tail: every stream-K configuration,
    integer-valued inputs, output equal to the exact result (fp32) or to its
    round-to-nearest-even bf16; the pieces of split tiles are added in K order
    by the second pass."""
    A, B, bias = _int_inputs(M, N, K, dtype, 31)
    ref = gemm_ref.gemm(A, B, bias, act)
    cfgs = _streamk_cfgs(M, N, K, dtype)
    assert len(cfgs) >= 12
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    for cfg in cfgs:
        mark(f"stream-K {M}x{N}x{K} dt{dtype} {cfg}")
        C = _run(A_d, B_d, b_d, act, dtype, cfg)
        torch.cuda.synchronize()
        _exact_check(C, ref, dtype, f"stream-K {cfg}")
    # the workgroup count is the plan's: full-round tiles plus the tail's workgroups
    c = cfgs[0]
    plan = S.streamk_plan(M, N, K, S.Cfg(*c))
    assert tg.grid(M, N, K, c) == (plan["tiles"], plan["blocks"])


def test_streamk_gelu_random_inputs_and_repeatable():
    M, N, K, dtype = 1024, 1040, 2048, wl.BF16
    A, B, bias = wl.make_inputs(M, N, K, dtype, wl.Dist("normal", 0.5), wl.Dist("normal", 0.5),
                                wl.Dist("normal", 0.5), 33)
    ref = gemm_ref.gemm(A, B, bias, "gelu")
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    for cfg in [(3, 256, 256, 64, 2, 4, 2, 1), (3, 128, 128, 64, 2, 2, 3, 1)]:
        mark(f"stream-K gelu {cfg}")
        C1 = _run(A_d, B_d, b_d, "gelu", dtype, cfg)
        C2 = _run(A_d, B_d, b_d, "gelu", dtype, cfg)
        torch.cuda.synchronize()
        assert torch.equal(C1, C2), "the same call gives the same bits"
        assert_close(out_f64(C1), ref, dtype, f"stream-K gelu {cfg}")


@pytest.mark.parametrize("M,N,K,dtype,act", [
    (100, 200, 1000, wl.F32, "relu"),          # ragged M, N; K not a multiple of any stage
    (256, 256, 256, wl.F32, "none"),           # the fp32 256^3 shape
    (130, 264, 1032, wl.BF16, "relu"),         # ragged M; K mod 128 = 8
    (64, 512, 4096, wl.BF16_F32OUT, "none"),   # long K: many stages per K group
    (17, 96, 40, wl.BF16, "none"),             # one partial stage
])
def test_sliced_k_integer_exact(M, N, K, dtype, act):
    """The sliced-K kind (K groups inside one workgroup, their sums added in
    LDS): every configuration, integer-valued inputs, output equal to the
    exact result (fp32) or to its round-to-nearest-even bf16, one launch."""
    A, B, bias = _int_inputs(M, N, K, dtype, 41)
    ref = gemm_ref.gemm(A, B, bias, act)
    cfgs = [c.astuple() for c in tg.enumerate_feasible(M, N, K, dtype) if c.kind == 4 and tg.has_kernel(dtype, c)]
    assert len(cfgs) >= 40
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    for cfg in cfgs:
        mark(f"sliced-K {M}x{N}x{K} dt{dtype} {cfg}")
        C = _run(A_d, B_d, b_d, act, dtype, cfg)
        torch.cuda.synchronize()
        _exact_check(C, ref, dtype, f"sliced-K {cfg}")
    c = cfgs[0]
    tiles = S.cdiv(M, c[1]) * S.cdiv(N, c[2])
    assert tg.grid(M, N, K, c) == (tiles, tiles)


def test_sliced_k_gelu_random_inputs_and_repeatable():
    for dtype, cfg in [(wl.F32, (4, 16, 32, 64, 1, 1, 2, 4)), (wl.BF16, (4, 32, 128, 128, 1, 2, 3, 4)),
                       (wl.BF16_F32OUT, (4, 64, 64, 64, 2, 2, 2, 2))]:
        M, N, K = 300, 640, 2048
        A, B, bias = wl.make_inputs(M, N, K, dtype, wl.Dist("normal", 0.5), wl.Dist("normal", 0.5),
                                    wl.Dist("normal", 0.5), 43)
        ref = gemm_ref.gemm(A, B, bias, "gelu")
        assert tg.has_kernel(dtype, cfg), cfg
        A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
        mark(f"sliced-K gelu dt{dtype} {cfg}")
        C1 = _run(A_d, B_d, b_d, "gelu", dtype, cfg)
        C2 = _run(A_d, B_d, b_d, "gelu", dtype, cfg)
        torch.cuda.synchronize()
        assert torch.equal(C1, C2), "the same call gives the same bits"
        assert_close(out_f64(C1), ref, dtype, f"sliced-K gelu {cfg}")


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32, wl.BF16_F32OUT])
def test_split_k_second_pass_edges(dtype):
    # an unaligned shape (N = 33) runs the element-load kind or the tiled kind's padded path, which
    # take any C: the second pass then writes element by element into a C shifted off 16-byte
    # alignment, and M x N = 2145 leaves a ragged tail after the four-element groups
    M, N, K = 65, 33, 630
    A, B, bias = _int_inputs(M, N, K, dtype, 8)
    ref = gemm_ref.gemm(A, B, bias, "relu")
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    feas = [c for c in tg.enumerate_feasible(M, N, K, dtype) if c.split_k > 1 and tg.has_kernel(dtype, c)]
    # the element-load kind and the tiled kind's padded path (whose output
    # pass writes C element by element too)
    assert {c.kind for c in feas} == {S.KIND_UNALIGNED, S.KIND_TILED}
    odt = torch.bfloat16 if dtype == wl.BF16 else torch.float32
    for shift in (0, 1):
        buf = torch.zeros(M * N + 1, dtype=odt, device="cuda")
        out = buf[shift:shift + M * N].view(M, N)
        for c in feas:
            mark(f"split-K second pass dt{dtype} shift {shift} {c.astuple()}")
            out.fill_(0)
            tg.gemm_bias_act(A_d, B_d, b_d, act="relu", out=out, cfg=c)
            torch.cuda.synchronize()
            _exact_check(out, ref, dtype, f"second pass dt{dtype} shift {shift} {c.astuple()}")
            if shift:
                assert float(buf[0]) == 0.0, "the second pass wrote before C"


_FULL_REF = {}


def _full_reference(index, A, B, bias, act):
    """The oracle's whole output; the 8192^3 one (about 10 s on the host's
    cores) is computed once per session."""
    if index in _FULL_REF:
        return _FULL_REF[index]
    ref = gemm_ref.gemm(A, B, bias, act)
    if wl.WORKLOADS[index].flops > 1e12:
        _FULL_REF[index] = ref
    return ref


def _workload_parity(index, cfgs, sample=None):
    w = wl.WORKLOADS[index]
    A, B, bias = wl.workload_inputs(index)
    act = ACT_NAMES[w.act]
    if sample is None:
        mark(f"workload {index}: oracle")
        ref = _full_reference(index, A, B, bias, act)
    else:
        rng = np.random.default_rng(100 + index)
        rows = np.concatenate([rng.integers(0, w.M, sample), [0, w.M - 1, w.M - 1, 0]])
        cols = np.concatenate([rng.integers(0, w.N, sample), [0, w.N - 1, 0, w.N - 1]])
        ref = gemm_ref.gemm_entries(A, B, rows, cols, bias, act)
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    for cfg in cfgs:
        mark(f"workload {index} cfg {cfg}")
        C = _run(A_d, B_d, b_d, act, w.dtype, cfg)
        torch.cuda.synchronize()
        got = out_f64(C) if sample is None else out_f64(C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()])
        assert np.all(np.isfinite(got))
        assert_close(got, ref, w.dtype, f"workload {index} cfg {cfg}")


def test_workload1_fp32_every_feasible_cfg():
    w = wl.WORKLOADS[1]
    feas = [c.astuple() for c in tg.enumerate_feasible(w.M, w.N, w.K, w.dtype) if tg.has_kernel(w.dtype, c)]
    _workload_parity(1, [None] + feas)


def test_workload2_wave_quantisation():
    w = wl.WORKLOADS[2]
    _workload_parity(2, [None, S.default_cfg(w.N, w.K, w.dtype).astuple(), (0, 64, 64, 64, 2, 2, 2, 1),
                         (0, 128, 128, 64, 2, 2, 2, 4)])


def test_workload3_square_full():
    # the whole 8192 x 8192 output, element by element
    w = wl.WORKLOADS[3]
    _workload_parity(3, [None, S.default_cfg(w.N, w.K, w.dtype).astuple()])


def test_workload4_decode():
    _workload_parity(4, [None, (0, 128, 128, 64, 2, 2, 2, 1), (1, 16, 128, 32, 4, 1, 2, 4)])


def test_workload5_ragged():
    w = wl.WORKLOADS[5]
    feas = [c.astuple() for c in tg.enumerate_feasible(w.M, w.N, w.K, w.dtype)
            if tg.has_kernel(w.dtype, c) and c.split_k == 1]
    _workload_parity(5, [None] + feas[::9])


@pytest.mark.parametrize("index", [1, 2, 3, 4, 5])
def test_persisted_tuning_launch_path(index):
    """The launch the benchmark times: the persisted tuning cache loaded into
    the library, then a call without a configuration (key lookup, cached
    entry).  Full output against the oracle."""
    import os
    path = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "tile_shape_autotuning_amd", "tuned", "mi355x.cache")
    w = wl.WORKLOADS[index]
    tg.cache_clear()
    try:
        loaded, _ = tg.cache_load(path)
        assert loaded >= 5
        key = (tg.dispatch_m(w.M), w.N, w.K, w.dtype)
        ep = dict(act=ACT_NAMES[w.act], bias=w.bias_dist is not None)
        hit = tg.cache_lookup(*key, **ep)
        assert hit is not None, "the persisted cache has an entry for this workload and epilogue"
        s0 = tg.stats()
        _workload_parity(index, [None])
        s1 = tg.stats()
        assert s1["tunes"] == s0["tunes"] and s1["cache_hits"] == s0["cache_hits"] + 1
        assert tg.cache_lookup(*key, **ep)[0] == hit[0]
    finally:
        tg.cache_clear()


def test_max_sizes():
    # K at its limit (2^21) with a skinny M; N at its limit; a tall M
    for (M, N, K, dtype) in [(16, 64, 1 << 21, wl.BF16_F32OUT), (8, 1 << 21, 64, wl.BF16),
                             (1 << 20, 64, 64, wl.BF16), (3, 1 << 20, 40, wl.F32)]:
        mark(f"max size {M}x{N}x{K} dt{dtype}")
        A, B, bias = _int_inputs(M, N, K, dtype, 8)
        rng = np.random.default_rng(9)
        rows = rng.integers(0, M, 512)
        cols = rng.integers(0, N, 512)
        ref = gemm_ref.gemm_entries(A, B, rows, cols, bias, "none")
        C = _run(to_dev(A), to_dev(B), to_dev(bias), "none", dtype)
        torch.cuda.synchronize()
        got = out_f64(C[torch.from_numpy(rows).cuda(), torch.from_numpy(cols).cuda()])
        if dtype == wl.BF16:
            want = wl.bf16_bits_to_f32(wl.f32_to_bf16_bits(ref.astype(np.float32))).astype(np.float64)
            assert np.array_equal(got, want)
        else:
            assert np.array_equal(got, ref)
    with pytest.raises(tg.TileGemmError):
        tg._native.check(tg._native.gemm_bias_act_ptr(4, 4, (1 << 21) + 8, 256, 256, 0, 256, wl.BF16, 0))
