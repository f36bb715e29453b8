"""Pins of the oracle's cost-aware stop rule (CPU only)."""

import dataclasses
from fractions import Fraction

import numpy as np
import pytest

from oracle import adaptive_budget, round_cost, select_tree, topk_per_position
from workloads import Cost

CFG4 = Cost(a=1.0, b=0.02, c=1e-4, e=1e-6, c_d=0.5)


def test_single_node_closed_form():
    """One node is worth adding iff (1+s)/C(1) > 1/C(0), i.e. with these
    coefficients at l = 0: s > 0.0201 / 1.5 = 0.0134."""
    thr = 0.0201 / 1.5
    assert adaptive_budget([np.float32(thr * 1.001)], CFG4, 0, 8) == 1
    assert adaptive_budget([np.float32(thr * 0.999)], CFG4, 0, 8) == 0
    # the context term raises the bar: at l = 10**4, C(1) - C(0) = 0.0301
    thr_l = 0.0301 / (1.5 + 0.0)  # C(0) does not depend on l
    assert adaptive_budget([np.float32(thr_l * 1.001)], CFG4, 10 ** 4, 8) == 1
    assert adaptive_budget([np.float32(thr_l * 0.999)], CFG4, 10 ** 4, 8) == 0


def _exact_theta(scores, cost, l, m):
    F = Fraction
    phi = sum((F(float(s)) for s in scores[:m]), F(0))
    c = (F(cost.c_d) + F(cost.a) + F(cost.b) * m + F(cost.c) * m * m
         + F(cost.e) * l * m)
    return (1 + phi) / c


def _scores(seed, temp):
    rng = np.random.default_rng(seed)
    lg = rng.normal(0, 3, size=(16, 400)) / temp
    marg = (np.exp(lg - lg.max(-1, keepdims=True)))
    marg = (marg / marg.sum(-1, keepdims=True)).astype(np.float32)
    idx, p = topk_per_position(marg, 64)
    t = select_tree(idx, p, 64, 64)
    return [t.score[i] for i in range(t.n)]


@pytest.mark.parametrize("seed", range(10))
def test_unimodal_in_exact_arithmetic(seed):
    """With convex C_v and best-first (non-increasing) scores, Theta(m) rises
    then falls, and the greedy stop lands on its first maximiser."""
    scores = _scores(seed, temp=0.4 + 0.15 * seed)
    for l in (0, 5000, 30000):
        for cost in (CFG4, dataclasses.replace(CFG4, c=0.0),
                     dataclasses.replace(CFG4, b=0.002, c_d=4.0)):
            th = [_exact_theta(scores, cost, l, m) for m in range(len(scores) + 1)]
            peak = max(range(len(th)), key=lambda m: (th[m], -m))
            assert all(th[m] < th[m + 1] for m in range(peak))
            assert all(th[m] >= th[m + 1] for m in range(peak, len(th) - 1))
            n = adaptive_budget(scores, cost, l, len(scores))
            assert n == peak
            # the cap truncates the search
            assert adaptive_budget(scores, cost, l, max(peak - 1, 0)) == max(peak - 1, 0)


@pytest.mark.parametrize("seed", range(6))
def test_comparative_statics(seed):
    """n* falls (weakly) as l, b, c or e grow and rises as a, C_d or f (a fixed
    cost per unit of context) grow."""
    scores = _scores(seed, temp=0.5)
    base = CFG4
    def n_of(cost, l):
        return adaptive_budget(scores, cost, l, len(scores))
    ls = [0, 1000, 4000, 16000, 64000, 256000]
    ns = [n_of(base, l) for l in ls]
    assert ns == sorted(ns, reverse=True)
    for field, vals, decreasing in (("b", [0.0, 0.01, 0.02, 0.08], True),
                                    ("c", [0.0, 1e-4, 1e-3, 1e-2], True),
                                    ("e", [0.0, 1e-6, 1e-5, 1e-4], True),
                                    ("a", [0.0, 1.0, 4.0, 16.0], False),
                                    ("c_d", [0.0, 0.5, 2.0, 8.0], False),
                                    ("f", [0.0, 1e-5, 1e-4, 1e-3], False)):
        ns = [n_of(dataclasses.replace(base, **{field: v}), 8000) for v in vals]
        assert ns == sorted(ns, reverse=decreasing), (field, ns)


def test_round_cost_order_of_evaluation():
    c = Cost(a=1.0, b=0.02, c=1e-4, e=1e-6, c_d=0.5)
    assert round_cost(0, 123, c) == 1.5
    assert round_cost(3, 1000, c) == 0.5 + (((1.0 + 0.02 * 3.0) + 1e-4 * 9.0)
                                              + (1e-6 * 1000.0) * 3.0)


def test_fixed_budget_ignores_cost_and_length():
    rng = np.random.default_rng(1)
    marg = rng.dirichlet(np.ones(30), size=4).astype(np.float32)
    idx, p = topk_per_position(marg, 8)
    a = select_tree(idx, p, 8, 8, cost=None, prefix_len=0)
    b = select_tree(idx, p, 8, 8, cost=None, prefix_len=10 ** 6)
    assert a.n == b.n == 8 and np.array_equal(a.token, b.token)
    # adaptive with a huge per-token cost keeps nothing; with zero cost keeps the cap
    z = select_tree(idx, p, 8, 8, cost=Cost(1.0, 10.0, 0.0, 0.0, 0.0), prefix_len=0)
    assert z.n == 0 and (z.parent == -1).all()
    f = select_tree(idx, p, 8, 8, cost=Cost(1.0, 0.0, 0.0, 0.0, 0.0), prefix_len=0)
    assert f.n == 8


def test_stop_when_gain_is_exactly_zero():
    """The builder stops as soon as the marginal gain is not positive: with
    C(m) = 1 + 0.5 m and a first score of 0.5, Theta(1) = 1.5/1.5 = Theta(0)
    exactly, so no node is added; a slightly larger score adds it."""
    cost = Cost(a=0.75, b=0.5, c=0.0, e=0.0, c_d=0.25)
    assert adaptive_budget([np.float32(0.5)], cost, 0, 4) == 0
    assert adaptive_budget([np.float32(0.5000001)], cost, 0, 4) == 1
