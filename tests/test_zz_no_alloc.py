"""The entry point that allocates nothing (gemm_bias_act_noalloc), through the
C ABI, against gemm_bias_act on the same inputs: the same kernels run, so the
outputs must be identical bit for bit; both are also checked against the
oracle (integer-valued inputs make the fp32 sums exact).  Split-K
configurations put their partial sums, and the padded path its operand
copies too, in the library's fixed scratch array; two calls in a row, the
second smaller, share it."""
import numpy as np
import pytest

from oracle import gemm_ref
from tile_shape_autotuning_amd import workloads as wl

from gpu_util import mark, out_bits, out_f64, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
tg = pytest.importorskip("tile_shape_autotuning_amd")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tg._native.lib()
    tg.set_device_override(None)
    yield
    torch.cuda.synchronize()


def _problem(M, N, K, dtype, seed):
    A, B, bias = wl.make_inputs(M, N, K, dtype, wl.Dist("int", 2), wl.Dist("int", 2), wl.Dist("int", 4), seed)
    return A, B, bias, gemm_ref.gemm(A, B, bias, "relu")


def _call(fn, M, N, K, A_d, B_d, b_d, dtype, cfg):
    odt = torch.bfloat16 if dtype == wl.BF16 else torch.float32
    C = torch.full((M, N), float("nan"), dtype=odt, device="cuda")
    tg._native.set_stream(torch.cuda.current_stream().cuda_stream)
    st = fn(M, N, K, A_d.data_ptr(), B_d.data_ptr(), b_d.data_ptr(), C.data_ptr(), dtype, "relu", cfg)
    tg._native.check(st)
    torch.cuda.synchronize()
    return C


def _bits(C):
    return out_bits(C) if C.dtype == torch.bfloat16 else out_f64(C).view(np.int64)


@pytest.mark.parametrize("dtype", [wl.BF16_F32OUT, wl.BF16, wl.F32])
def test_noalloc_matches_gemm_bias_act_two_calls_second_smaller(dtype):
    N_ = tg._native
    if dtype == wl.F32:
        calls = [(300, 520, 2048, (0, 64, 64, 32, 2, 2, 2, 8)), (100, 136, 512, (0, 64, 64, 32, 2, 2, 2, 4))]
    else:
        calls = [(1000, 1000, 8192, (0, 128, 128, 128, 4, 2, 2, 4)), (16, 4096, 2048, (0, 32, 256, 32, 1, 2, 4, 2))]
    for i, (M, N, K, cfg) in enumerate(calls):
        mark(f"noalloc call {i}: {M}x{N}x{K} dt{dtype} cfg {cfg}")
        A, B, bias, ref = _problem(M, N, K, dtype, 40 + i)
        A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
        got = _call(N_.gemm_bias_act_noalloc_ptr, M, N, K, A_d, B_d, b_d, dtype, cfg)
        want = _call(N_.gemm_bias_act_ptr, M, N, K, A_d, B_d, b_d, dtype, cfg)
        assert np.array_equal(_bits(got), _bits(want)), f"call {i}: differs from gemm_bias_act"
        if dtype == wl.BF16:
            assert np.array_equal(out_bits(got), wl.f32_to_bf16_bits(ref.astype(np.float32)))
        else:
            assert np.array_equal(out_f64(got), ref)


@pytest.mark.parametrize("dtype", [wl.BF16, wl.F32])
def test_noalloc_padded_path_two_calls_second_smaller(dtype):
    # unaligned shapes on the tiled kind: the padded copies of A and B and the
    # slabs all live in the fixed scratch array
    N_ = tg._native
    if dtype == wl.F32:
        calls = [(130, 130, 258, (0, 32, 64, 32, 2, 2, 3, 2)), (65, 33, 63, (0, 32, 32, 32, 1, 1, 2, 1))]
    else:
        calls = [(513, 1001, 777, (0, 128, 64, 64, 4, 2, 3, 2)), (100, 130, 300, (0, 64, 64, 64, 2, 2, 2, 1))]
    for i, (M, N, K, cfg) in enumerate(calls):
        mark(f"noalloc padded call {i}: {M}x{N}x{K} dt{dtype} cfg {cfg}")
        A, B, bias, ref = _problem(M, N, K, dtype, 60 + i)
        A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
        got = _call(N_.gemm_bias_act_noalloc_ptr, M, N, K, A_d, B_d, b_d, dtype, cfg)
        want = _call(N_.gemm_bias_act_ptr, M, N, K, A_d, B_d, b_d, dtype, cfg)
        assert np.array_equal(_bits(got), _bits(want)), f"padded call {i}: differs from gemm_bias_act"
        if dtype == wl.BF16:
            assert np.array_equal(out_bits(got), wl.f32_to_bf16_bits(ref.astype(np.float32)))
        else:
            assert np.array_equal(out_f64(got), ref)


def test_noalloc_without_cfg_takes_the_model_choice_and_never_tunes():
    N_ = tg._native
    tg.cache_clear()
    M, N, K, dtype = 200, 1000, 4096, wl.BF16
    A, B, bias, ref = _problem(M, N, K, dtype, 50)
    A_d, B_d, b_d = to_dev(A), to_dev(B), to_dev(bias)
    s0 = tg.stats()
    mark("noalloc without cfg")
    got = _call(N_.gemm_bias_act_noalloc_ptr, M, N, K, A_d, B_d, b_d, dtype, None)
    assert tg.stats()["tunes"] == s0["tunes"] and tg.cache_size() == 0
    cfg = tg.model_choice(tg.dispatch_m(M), N, K, dtype)[0]
    want = _call(N_.gemm_bias_act_ptr, M, N, K, A_d, B_d, b_d, dtype, cfg)
    assert np.array_equal(out_bits(got), out_bits(want))
    assert np.array_equal(out_bits(got), wl.f32_to_bf16_bits(ref.astype(np.float32)))


def test_noalloc_refuses_partial_sums_beyond_its_scratch():
    N_ = tg._native
    cap = N_.noalloc_scratch_bytes()
    assert cap == 32 << 20
    M, N, K, dtype = 2048, 2048, 2048, wl.BF16_F32OUT
    cfg = (0, 128, 128, 64, 2, 2, 2, 4)          # 4 x 2048 x 2048 floats = 64 MiB > 32 MiB
    A_d = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    B_d = torch.zeros((K, N), dtype=torch.bfloat16, device="cuda")
    C = torch.full((M, N), 7.0, dtype=torch.float32, device="cuda")
    st = N_.gemm_bias_act_noalloc_ptr(M, N, K, A_d.data_ptr(), B_d.data_ptr(), 0, C.data_ptr(), dtype, "none", cfg)
    assert st == N_.TG_E_INVAL and "32" in N_.last_error()
    torch.cuda.synchronize()
    assert bool((C == 7.0).all()), "a refused call queues nothing"
