"""Convex, monotone verification cost from measured latencies (test
infrastructure only).

[caddtree] Methodology, item 5: the verification cost C_v(n; l) is estimated
once, offline, by convex regression on latencies measured over context
lengths and node counts, which keeps the model convex and monotone so that
the throughput objective of item 3 stays unimodal.  Item 1 gives the round
cost C = C_d + C_v(|T|; l).

Reading fixed here: the regression model is the adaptive workload's cost
family plus a term linear in l alone,
    C_v(n; l) = a + b*n + c*n^2 + e*l*n + f*l,   a, b, c, e, f >= 0,
which is non-decreasing and convex in n for every l >= 0 (and non-decreasing
in l), fitted by non-negative least squares to the measured latencies t_i at
(n_i, l_i) -- the plainest convex regression over that family.  The f*l term
is the part of a request's verification that does not grow with its tree
(reading the prefix once); without it the family cannot describe a
memory-bound attention, whose cost at fixed n grows with l.
"""

import numpy as np
from scipy.optimize import nnls


def design(n, l) -> np.ndarray:
    """Columns [1, n, n^2, l*n, l] of the cost model, fp64."""
    n = np.asarray(n, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    return np.stack([np.ones_like(n), n, n * n, l * n, l], axis=1)


def fit_cost(n, l, t):
    """Non-negative least-squares coefficients (a, b, c, e, f) of C_v, and the
    residual sum of squares."""
    A = design(n, l)
    t = np.asarray(t, dtype=np.float64)
    if A.shape[0] < A.shape[1] or not np.all(np.isfinite(A)) or not np.all(np.isfinite(t)):
        raise ValueError("need at least 5 finite measurements")
    # columns scaled to unit norm: the same non-negative solution, better conditioned
    scale = np.linalg.norm(A, axis=0)
    scale[scale == 0] = 1.0
    x, _ = nnls(A / scale, t)
    coef = x / scale
    res = float(np.sum((A @ coef - t) ** 2))
    return coef, res
