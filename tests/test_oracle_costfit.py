"""Pins of the oracle's cost fit (CPU only): exact recovery of non-negative
coefficients, brute force over every active set, the optimality conditions of
non-negative least squares, and the fitted model's monotonicity and
convexity in n."""

import itertools

import numpy as np
import pytest

from oracle import fit_cost
from oracle.costfit import design


def _grid():
    n = np.array([1, 2, 4, 8, 16, 32, 64, 96, 128], dtype=np.float64)
    l = np.array([512, 2048, 8192, 32768], dtype=np.float64)
    nn, ll = np.meshgrid(n, l)
    return nn.ravel(), ll.ravel()


@pytest.mark.parametrize("coef", [(10.0, 0.3, 1e-3, 2e-4, 0.0), (5.0, 0.0, 2e-3, 1e-4, 1e-3),
                                  (0.0, 1.0, 0.0, 0.0, 0.0), (3.0, 0.2, 0.0, 5e-5, 2e-3),
                                  (1.0, 0.0, 0.0, 0.0, 1e-3)])
def test_exact_recovery(coef):
    n, l = _grid()
    t = design(n, l) @ np.array(coef)
    got, res = fit_cost(n, l, t)
    assert res <= 1e-18 * float(np.sum(t * t)) + 1e-24
    assert np.allclose(got, coef, rtol=1e-9, atol=1e-12)


def _brute_force(A, t):
    """Least squares on every subset of columns; the best solution whose
    coefficients are all >= 0 (the others held at 0)."""
    best = (np.inf, None)
    for r in range(0, A.shape[1] + 1):
        for S in itertools.combinations(range(A.shape[1]), r):
            x = np.zeros(A.shape[1])
            if S:
                sol, *_ = np.linalg.lstsq(A[:, S], t, rcond=None)
                if np.any(sol < 0):
                    continue
                x[list(S)] = sol
            res = float(np.sum((A @ x - t) ** 2))
            if res < best[0]:
                best = (res, x)
    return best


@pytest.mark.parametrize("seed", range(8))
def test_matches_brute_force_over_active_sets(seed):
    rng = np.random.default_rng(seed)
    n, l = _grid()
    true = rng.uniform(0, 1, 5) * np.array([20, 0.5, 2e-3, 3e-4, 2e-3]) * (rng.random(5) > 0.3)
    # latencies with noise, sometimes pulling a coefficient below zero
    t = design(n, l) @ true + rng.normal(0, 2.0, n.shape) + rng.normal(0, 5) * (n < 4)
    t = np.maximum(t, 0.0)
    got, res = fit_cost(n, l, t)
    bres, bx = _brute_force(design(n, l), t)
    assert res <= bres * (1 + 1e-9) + 1e-12
    assert np.allclose(got, bx, rtol=1e-6, atol=1e-9 * np.abs(bx).max())


@pytest.mark.parametrize("seed", range(5))
def test_kkt_conditions(seed):
    """x >= 0, gradient A^T (A x - t) zero where x > 0 and >= 0 where x = 0."""
    rng = np.random.default_rng(100 + seed)
    n, l = _grid()
    t = np.abs(rng.normal(50, 30, n.shape)) + 0.01 * n * l / 1000
    A = design(n, l)
    x, _ = fit_cost(n, l, t)
    scale = np.linalg.norm(A, axis=0)
    g = (A / scale).T @ (A @ x - t)
    assert np.all(x >= 0)
    tol = 1e-8 * np.linalg.norm(t)
    assert np.all(np.abs(g[x > 0]) <= tol)
    assert np.all(g[x == 0] >= -tol)


def test_fitted_model_is_monotone_and_convex_in_n():
    rng = np.random.default_rng(3)
    n, l = _grid()
    t = np.abs(rng.normal(100, 60, n.shape))     # arbitrary, even decreasing data
    coef, _ = fit_cost(n, l, t)
    a, b, c, e, f = coef
    for L in (0.0, 1000.0, 65536.0):
        m = np.arange(0, 129, dtype=np.float64)
        cv = a + b * m + c * m * m + e * L * m + f * L
        assert np.all(np.diff(cv) >= -1e-12)
        assert np.all(np.diff(cv, 2) >= -1e-12)


def test_rejects_too_few_points():
    with pytest.raises(ValueError):
        fit_cost([1, 2, 3, 4], [1, 1, 1, 1], [1, 2, 3, 4])
