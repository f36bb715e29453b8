"""tsv_fit_cost (host code of the C library) against the oracle's fit.  CPU:
the fit touches no device, so it runs with the other host checks."""

import numpy as np
import pytest

import oracle
import tree_structured_verification_amd as tsv
from oracle.costfit import design


def _grid(ns=(1, 2, 4, 8, 16, 24, 32, 64, 96, 128), ls=(256, 1024, 4096, 16384, 65536)):
    nn, ll = np.meshgrid(np.array(ns, np.float64), np.array(ls, np.float64))
    return nn.ravel(), ll.ravel()


def _check(n, l, t):
    c = tsv.fit_cost(n, l, t, c_d=0.5)
    got = np.array([c.a, c.b, c.c, c.e, c.f])
    ref, res = oracle.fit_cost(n, l, t)
    A = design(n, l)
    got_res = float(np.sum((A @ got - t) ** 2))
    assert np.all(got >= 0)
    assert c.c_d == 0.5
    # the same optimum: residuals equal to rounding, coefficients close
    assert got_res <= res * (1 + 1e-9) + 1e-18 * float(np.sum(t * t)) + 1e-24
    assert np.allclose(got, ref, rtol=1e-6, atol=1e-9 * max(1e-300, np.abs(ref).max()))
    return got


@pytest.mark.parametrize("coef", [(10.0, 0.3, 1e-3, 2e-4, 0.0), (0.0, 0.0, 0.0, 1e-4, 0.0),
                                  (7.0, 0.0, 0.0, 0.0, 0.0), (0.0, 2.0, 0.5, 0.0, 0.0),
                                  (0.4, 0.0, 0.0, 1e-6, 2e-3)])
def test_exact_models(coef):
    n, l = _grid()
    _check(n, l, design(n, l) @ np.array(coef))


@pytest.mark.parametrize("seed", range(10))
def test_noisy_latencies(seed):
    rng = np.random.default_rng(seed)
    n, l = _grid()
    true = rng.uniform(0, 1, 5) * np.array([30, 0.5, 3e-3, 5e-4, 2e-3]) * (rng.random(5) > 0.25)
    t = np.maximum(design(n, l) @ true + rng.normal(0, 3.0, n.shape), 0.0)
    _check(n, l, t)


def test_constraints_active():
    """Latencies falling with n: every slope is clamped at zero."""
    n, l = _grid()
    t = 100.0 - 0.5 * n
    got = _check(n, l, t)
    assert got[1] == 0 and got[2] == 0 and got[3] == 0 and got[4] == 0 and got[0] > 0


def test_single_context_length_and_few_points():
    """One context length: n and l*n are collinear, and so are 1 and l, so
    only the optimum's value is unique; it must match, with a and b carrying
    the fit (the earlier supports)."""
    n = np.array([1.0, 2.0, 3.0, 5.0, 6.0])
    l = np.full(5, 1000.0)
    t = np.array([3.0, 5.1, 7.2, 11.0, 13.3])
    c = tsv.fit_cost(n, l, t)
    got = np.array([c.a, c.b, c.c, c.e, c.f])
    _, res = oracle.fit_cost(n, l, t)
    assert np.all(got >= 0) and got[3] == 0.0 and got[4] == 0.0
    assert abs(float(np.sum((design(n, l) @ got - t) ** 2)) - res) <= 1e-12 * float(np.sum(t * t))


def test_rejects_bad_input():
    with pytest.raises(tsv.TsvError):
        tsv.fit_cost([1, 2, 3, 4], [1, 1, 1, 1], [1, 2, 3, 4])   # fewer than 5 points
    with pytest.raises(tsv.TsvError):
        tsv.fit_cost([1, 2, 3, 4, 5], [1, 1, 1, 1, 1], [1, 2, -3, 4, 5])  # negative latency
    with pytest.raises(tsv.TsvError):
        tsv.fit_cost([1, 2, 3, 4, 5], [1, 1, np.nan, 1, 1], [1, 2, 3, 4, 5])
