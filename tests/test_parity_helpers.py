"""The parity tests' comparison (CPU): a per-row bound catches an error
confined to one row that the whole tensor's relative L2 lets through."""
import numpy as np
import pytest

from parity import ROW_FACTOR, assert_close, rel, rowrel


def _pair(seed=0, rows=300, cols=64, noise=2e-4):
    r = np.random.default_rng(seed)
    b = r.standard_normal((rows, cols))
    return b * (1 + noise * r.standard_normal(b.shape)), b


def test_rounding_noise_passes():
    a, b = _pair()
    assert_close(a, b, 2e-3)
    assert rowrel(a, b) < 2 * rel(a, b)


def test_one_bad_row_fails_the_row_bound_only():
    a, b = _pair()
    a[137] = b[137] * 1.01  # a 1% error in one row of 300
    assert rel(a, b) < 2e-3  # the global figure alone would pass it
    assert rowrel(a, b) > ROW_FACTOR * 2e-3
    with pytest.raises(AssertionError):
        assert_close(a, b, 2e-3)


def test_zero_rows_and_vectors():
    a, b = _pair()
    a[5] = b[5] = 0.0
    assert_close(a, b, 2e-3)
    a[6] = 0.0  # a row lost entirely
    with pytest.raises(AssertionError):
        assert_close(a, b, 2e-3)
    v = np.linspace(1, 2, 50)
    assert rowrel(v * (1 + 1e-6), v) == pytest.approx(rel(v * (1 + 1e-6), v))
