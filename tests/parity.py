"""Comparison helpers of the parity tests: the whole tensor's relative L2
and every row's own relative L2."""
import numpy as np


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-30))


# A row of 64 or more elements whose errors are independent roundings has a
# relative L2 within about 1.5x the whole tensor's; 3x leaves room for the
# spread and still catches a 1% error in one row of a 300-row tensor that
# the global figure would pass (it moves that row's figure by 1e-2).
ROW_FACTOR = 3.0


def rowrel(a, b):
    """Largest relative L2 of one row (first axis).  A row whose reference is
    nearly zero is measured against a thousandth of the typical row norm."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.ndim < 2:
        return rel(a, b)
    a, b = a.reshape(a.shape[0], -1), b.reshape(b.shape[0], -1)
    num, den = np.linalg.norm(a - b, axis=1), np.linalg.norm(b, axis=1)
    floor = max(1e-3 * float(np.sqrt(np.mean(den ** 2))), 1e-30)
    return float(np.max(num / np.maximum(den, floor)))


def assert_close(a, b, tol, row_tol=None):
    """Whole-tensor relative L2 below tol and every row's below row_tol
    (default ROW_FACTOR x tol)"""
    row_tol = ROW_FACTOR * tol if row_tol is None else row_tol
    g, r = rel(a, b), rowrel(a, b)
    assert g < tol and r < row_tol, f"rel L2 {g:.3e} (bound {tol:.1e}), worst row {r:.3e} (bound {row_tol:.1e})"
