"""The RMS-normalisation oracle against closed forms and invariants (CPU only).

Each pin fails for a plausible mistake: dividing by the sum instead of the
mean (one-hot row), eps outside the square root or dropped (constant row),
a missing or transposed weight (one-hot and constant rows), normalising
columns instead of rows (rows of different scales).
"""
import numpy as np
import pytest

from oracle import rmsnorm_ref as R
from tile_shape_autotuning_amd import workloads as wl


def test_constant_row_closed_form():
    n, c, eps = 64, 3.0, 0.5
    w = np.linspace(-2.0, 2.0, n)
    y = R.rmsnorm(np.full((1, n), c), w, eps)
    assert np.allclose(y[0], c / np.sqrt(c * c + eps) * w, rtol=0, atol=1e-15)


def test_one_hot_row_is_sqrt_n():
    n, j, a = 1024, 37, -5.0
    x = np.zeros((1, n))
    x[0, j] = a
    w = np.arange(1, n + 1, dtype=np.float64)
    y = R.rmsnorm(x, w, 0.0)
    want = np.zeros(n)
    want[j] = np.sign(a) * np.sqrt(n) * w[j]
    assert np.allclose(y[0], want, rtol=1e-15, atol=0)


def test_rows_are_independent_and_scale_free():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((3, 200))
    x[1] *= 1000.0                       # rows of very different scales
    w = rng.standard_normal(200)
    y = R.rmsnorm(x, w, 0.0)
    # with eps = 0 every row of y / w has RMS 1, and scaling a row changes nothing
    assert np.allclose(np.sqrt(np.mean((y / w) ** 2, axis=1)), 1.0, rtol=1e-12)
    assert np.allclose(R.rmsnorm(x * 7.5, w, 0.0), y, rtol=1e-12)
    assert np.allclose(R.rmsnorm(x[1:2], w, 0.0), y[1:2], rtol=1e-15)


def test_bf16_inputs_are_widened_exactly():
    vals = np.array([[1.0, -2.0, 0.5, 3.0]], dtype=np.float32)
    bits = wl.f32_to_bf16_bits(vals)
    w = wl.f32_to_bf16_bits(np.ones(4, dtype=np.float32))
    y = R.rmsnorm(bits, w, 0.0)
    rms = np.sqrt(np.mean(vals.astype(np.float64) ** 2))
    assert np.allclose(y, vals / rms, rtol=1e-15)


def test_shape_errors():
    with pytest.raises(ValueError):
        R.rmsnorm(np.ones((2, 8)), np.ones(7), 0.0)
