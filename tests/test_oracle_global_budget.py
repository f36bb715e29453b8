"""Pins of the oracle's batch-global budget (CPU only): closed forms for a
constant table and for an engine whose step time grows linearly with the
batch, brute force over every prefix-closed selection, tie order and the
table's end."""

import itertools
from fractions import Fraction

import numpy as np
import pytest

from oracle import global_budget, global_order


def _scores(rng, R, N, quant=None):
    s = np.sort(rng.random((R, N)).astype(np.float32) ** 3, axis=1)[:, ::-1]
    if quant:
        s = (np.ceil(s * quant) / quant).astype(np.float32)
    return np.ascontiguousarray(s)


def test_constant_table_admits_every_positive_score():
    rng = np.random.default_rng(1)
    s = _scores(rng, 5, 8)
    s[2, 5:] = 0.0
    s[4, :] = 0.0
    avail = [8, 3, 8, 0, 8]
    got = global_budget(s, avail, np.full(100, 7.0))
    assert list(got) == [8, 3, 5, 0, 0]


@pytest.mark.parametrize("seed", range(6))
def test_linear_step_time_closed_form(seed):
    """SPS(B) = 1 / (alpha + beta B): admitting a raises the throughput iff
    a (alpha + beta B) > beta tau, checked in exact rationals."""
    rng = np.random.default_rng(seed)
    R, N = 6, 20
    s = _scores(rng, R, N)
    avail = rng.integers(0, N + 1, size=R)
    alpha, beta = float(rng.uniform(1, 10)), float(rng.uniform(0.01, 0.5))
    sps = 1.0 / (alpha + beta * np.arange(R + R * N + 2))
    got = global_budget(s, avail, sps)
    tau, B, want = Fraction(R), R, np.zeros(R, np.int32)
    for a, r, j in global_order(s, avail):
        if not Fraction(a) * (Fraction(alpha) + Fraction(beta) * B) > Fraction(beta) * tau:
            break
        tau += Fraction(a)
        B += 1
        want[r] += 1
    assert np.array_equal(got, want)


@pytest.mark.parametrize("seed", range(10))
def test_brute_force_over_prefix_selections(seed):
    """Every selection of a prefix per request, exact throughput: the greedy
    reaches the maximum (Theta along the global order is unimodal for an
    engine whose step time grows linearly)."""
    rng = np.random.default_rng(100 + seed)
    R, N = 3, 3
    s = _scores(rng, R, N)
    avail = rng.integers(0, N + 1, size=R)
    alpha, beta = float(rng.uniform(0.5, 4)), float(rng.uniform(0.05, 1.0))
    sps = 1.0 / (alpha + beta * np.arange(R + R * N + 2))
    theta = lambda counts: (Fraction(R) + sum(Fraction(float(s[r][j])) for r in range(R)
                                              for j in range(counts[r]))) * Fraction(float(sps[R + sum(counts)]))
    best = max(theta(c) for c in itertools.product(*[range(int(a) + 1) for a in avail]))
    got = global_budget(s, avail, sps)
    assert theta(list(got)) == best


def test_ties_go_to_the_lower_request_then_position():
    s = np.array([[0.5, 0.25], [0.5, 0.25], [0.5, 0.25]], dtype=np.float32)
    # a table that allows exactly four admissions (B from 3 to 7): the step
    # rate collapses at B = 8
    sps = np.array([1.0] * 8 + [1e-9] * 3)
    got = global_budget(s, [2, 2, 2], sps)
    assert list(got) == [2, 1, 1]       # 0.5 x3 (requests 0, 1, 2), then request 0's 0.25


def test_stops_at_the_end_of_the_table():
    s = np.full((2, 5), 0.5, dtype=np.float32)
    got = global_budget(s, [5, 5], np.ones(6))     # B can reach 5: three admissions
    assert int(got.sum()) == 3


def test_admitted_nodes_are_prefixes():
    rng = np.random.default_rng(7)
    s = _scores(rng, 8, 16, quant=6)
    avail = rng.integers(0, 17, size=8)
    sps = 1.0 / (3.0 + 0.2 * np.arange(200))
    got = global_budget(s, avail, sps)
    order = global_order(s, avail)[: int(got.sum())]
    for r in range(8):
        js = [j for _, rr, j in order if rr == r]
        assert js == list(range(got[r])) and got[r] <= avail[r]
