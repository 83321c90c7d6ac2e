"""The C ABI from C: include/tilegemm.h compiles as C99, and a C program
(tests/c_abi/gemm_from_c.c, built with the library) tunes, runs and refuses
through it.  The GPU test compares the program's output with the oracle."""
import os
import subprocess

import numpy as np
import pytest

from oracle import gemm_ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tile_shape_autotuning_amd", "_lib", "gemm_from_c")


def test_header_is_c99():
    r = subprocess.run(["gcc", "-x", "c", "-std=c99", "-Wall", "-Werror", "-fsyntax-only",
                        os.path.join(ROOT, "include", "tilegemm.h")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_c_program_is_built_and_checks_its_arguments():
    if not os.path.exists(EXE):
        pytest.skip("library not built")
    r = subprocess.run([EXE], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr


def _inputs(M, N, K, seed):
    """The program's closed-form integer inputs (see the C source)."""
    i = np.arange(M)[:, None]
    k = np.arange(K)[None, :]
    A = ((7 * i + 3 * k + (k * k) % 13 + (i * k) % 7 + seed) % 5 - 2).astype(np.float32)
    k2 = np.arange(K)[:, None]
    j = np.arange(N)[None, :]
    B = ((5 * k2 + 11 * j + (k2 * j) % 7 + (k2 * k2) % 11 + 2 * seed) % 5 - 2).astype(np.float32)
    bias = (np.arange(N) % 9 - 4).astype(np.float32)
    return A, B, bias


@pytest.mark.gpu
@pytest.mark.parametrize("M,N,K,seed", [(200, 136, 520, 3), (16, 1000, 1064, 5),
                                        (130, 264, 515, 9), (61, 1001, 515, 4)])   # ragged K; ragged N and K
def test_c_program_matches_oracle(tmp_path, M, N, K, seed):
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(EXE):
        pytest.fail("the C program is built with the library: run __graft_entry__.build()")
    out = tmp_path / "c.f32"
    print(f"[c-abi] gemm_from_c {M} {N} {K} {seed}", flush=True)
    r = subprocess.run([EXE, str(M), str(N), str(K), str(seed), str(out)], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "tuned cfg:" in r.stdout and "refused as expected" in r.stdout
    got = np.fromfile(out, dtype=np.float32).reshape(M, N).astype(np.float64)
    A, B, bias = _inputs(M, N, K, seed)
    ref = gemm_ref.gemm(A, B, bias, "relu")
    assert np.abs(ref).max() > 100 and (ref > 0).mean() > 0.3     # the pattern does not cancel out
    assert np.array_equal(got, ref)
