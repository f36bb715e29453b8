"""Pins of the oracle's per-node expansion tree (CPU only).

Pinned by: the review's toy (every expansion the page lists, including C's
children A and B, and the pruning to D = 3), a reduction to the per-position
builder (itself pinned) when every node's distribution is its depth's
marginal, brute force over the full vocabulary, the top-1 chain and the
structural invariants.
"""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import (expand_candidates, expanded_rows, select_tree, select_tree_expand,
                    topk_per_position)
from oracle.budget import adaptive_budget
from tests.conftest import GOLDEN
from workloads import Cost


def _paths(tree):
    out = []
    for i in range(tree.n):
        p, j = [], i
        while j >= 0:
            p.append(int(tree.token[j]))
            j = int(tree.parent[j])
        out.append(tuple(p[::-1]))
    return out


def _rand_rows(rng, steps, k, V, quant=None):
    rows = rng.dirichlet(np.full(V, 0.5), size=expanded_rows(steps, k)).astype(np.float32)
    if quant:
        rows = (np.round(rows * quant) / quant).astype(np.float32)
    return rows


def test_toy_example():
    g = json.load(open(os.path.join(GOLDEN, "toy_tree_expand.json")))
    V = {t: i for i, t in enumerate(g["vocab"])}
    rows = np.array(g["rows"], dtype=np.float32)
    k, s, D = g["top_k"], g["steps"], g["budget"]
    idx, p = topk_per_position(rows, k)
    cands = expand_candidates(idx, p, s)
    assert 1 + len(cands) == g["nodes_including_root"]
    # every expansion the page lists
    kids = {}
    for c in cands:
        par = () if c.parent is None else (c.parent.token,)
        kids.setdefault(par, set()).add(c.token)
    for par, want in g["children"].items():
        key = () if par == "" else (V[par],)
        assert kids[key] == {V[t] for t in want}
    tree = select_tree_expand(idx, p, s, D, 8)
    names = {tuple(V[t] for t in path): path for path in g["kept_paths"]}
    paths = _paths(tree)
    assert set(paths) == set(names)
    for i, pth in enumerate(paths):
        seen = {paths[j] for j in range(tree.n) if tree.anc_bits[i, j // 32] >> (j % 32) & 1}
        want = {tuple(V[t] for t in sq) for sq in g["sees"][" ".join(names[pth])]}
        assert seen == want


def _as_node_rows(marg, k):
    """Per-node rows that repeat the marginal of each node's depth."""
    gamma = marg.shape[0]
    return np.concatenate([np.repeat(marg[d][None], k ** d, axis=0) for d in range(gamma)])


@pytest.mark.parametrize("quant", [None, 8])
@pytest.mark.parametrize("steps,k,V,n,adaptive", [
    (2, 2, 5, 6, False), (3, 2, 8, 14, False), (3, 3, 6, 20, False), (4, 2, 7, 30, True),
    (2, 4, 9, 20, True), (5, 1, 4, 5, False), (3, 2, 4, 3, True)])
def test_reduces_to_per_position_builder(steps, k, V, n, adaptive, quant):
    """quant: probabilities in multiples of 1/quant, so that equal scores occur
    among siblings and across depths (the tie order of the per-position
    builder is pinned by its own tests)."""
    rng = np.random.default_rng(steps * 100 + k * 10 + V)
    for trial in range(5):
        if quant:
            marg = rng.integers(0, quant // 2, size=(steps, V)).astype(np.float64)
            marg[:, 0] = quant - (marg[:, 1:].sum(-1) % quant)
            marg = (marg / marg.sum(-1, keepdims=True)).astype(np.float32)
            marg[:, -1] = 0.5
        else:
            marg = rng.dirichlet(np.full(V, 0.4), size=steps).astype(np.float32)
        rows = _as_node_rows(marg, k)
        cost = Cost(a=0.3, b=0.02, c=1e-3, e=1e-5, c_d=0.2) if adaptive else None
        N_max = max(n, 1)
        pl = 500 + trial
        idx_m, p_m = topk_per_position(marg, k)
        ref = select_tree(idx_m, p_m, n, N_max, cost=cost, prefix_len=pl)
        idx_r, p_r = topk_per_position(rows, k)
        got = select_tree_expand(idx_r, p_r, steps, n, N_max, cost=cost, prefix_len=pl)
        assert got.n == ref.n
        for f in ("parent", "token", "depth", "anc_bits"):
            assert np.array_equal(getattr(got, f), getattr(ref, f)), f
        assert np.array_equal(got.score.view(np.uint32), ref.score.view(np.uint32))


def _brute_force(rows, steps, n):
    """Every token sequence of length 1..s over the full vocabulary, its
    probability found by walking the rows of its own path, best n by score
    (inputs without ties)."""
    V = rows.shape[1]
    seqs = []
    for d in range(1, steps + 1):
        for seq in itertools.product(range(V), repeat=d):
            row, s = 0, np.float32(1.0)
            for t in seq:
                s = np.float32(s * rows[row, t])
                rank = int(np.sum(rows[row] > rows[row, t]))  # distinct values
                row = V * row + 1 + rank
            seqs.append((float(s), seq))
    seqs.sort(key=lambda x: -x[0])
    return seqs[:n]


@pytest.mark.parametrize("steps,V", [(1, 6), (2, 4), (3, 3), (2, 5)])
def test_brute_force_full_vocabulary(steps, V):
    rng = np.random.default_rng(7 + steps * V)
    rows = _rand_rows(rng, steps, V, V)
    assert all(len(set(r.tolist())) == V for r in rows)
    total = sum(V ** d for d in range(1, steps + 1))
    idx, p = topk_per_position(rows, V)
    for n in range(0, total + 1, max(1, total // 7)):
        N_max = max(n, 1)
        tree = select_tree_expand(idx, p, steps, n, N_max)
        want = _brute_force(rows, steps, n)
        scores = sorted((float(tree.score[i]) for i in range(tree.n)), reverse=True)
        assert len({w[0] for w in want}) == len(want) or n == 0
        assert set(_paths(tree)) == {w[1] for w in want}
        assert scores == [w[0] for w in want]


def test_top1_is_the_argmax_chain():
    rng = np.random.default_rng(3)
    steps, V = 6, 10
    rows = _rand_rows(rng, steps, 1, V)
    idx, p = topk_per_position(rows, 1)
    tree = select_tree_expand(idx, p, steps, 4, 8)
    assert tree.n == 4
    assert list(tree.parent[:4]) == [-1, 0, 1, 2]
    assert list(tree.token[:4]) == [int(np.argmax(rows[d])) for d in range(4)]


def test_children_follow_their_own_distribution():
    # the two depth-1 nodes have disjoint favourite continuations
    V = 6
    rows = np.full((3, V), 0.01, dtype=np.float32)
    rows[0, [1, 2]] = [0.5, 0.45]
    rows[1, [3, 4]] = [0.6, 0.35]   # children of token 1
    rows[2, [0, 5]] = [0.7, 0.25]   # children of token 2
    idx, p = topk_per_position(rows, 2)
    tree = select_tree_expand(idx, p, 2, 6, 8)
    kids = {}
    for i in range(tree.n):
        if tree.parent[i] >= 0:
            kids.setdefault(int(tree.token[tree.parent[i]]), set()).add(int(tree.token[i]))
    assert kids == {1: {3, 4}, 2: {0, 5}}


@pytest.mark.parametrize("quant", [None, 16])
def test_invariants(quant):
    rng = np.random.default_rng(11)
    for steps, k in [(3, 2), (4, 3), (2, 5)]:
        rows = _rand_rows(rng, steps, k, 12, quant)
        idx, p = topk_per_position(rows, k)
        tree = select_tree_expand(idx, p, steps, 40, 64)
        assert tree.n == min(40, sum(k ** d for d in range(1, steps + 1)))
        for i in range(tree.n):
            par = tree.parent[i]
            assert -1 <= par < i
            assert tree.depth[i] == (1 if par < 0 else tree.depth[par] + 1)
            if i:
                assert tree.score[i] <= tree.score[i - 1]


def test_budget_above_candidates_and_adaptive_cap():
    rng = np.random.default_rng(5)
    rows = _rand_rows(rng, 2, 2, 5)
    idx, p = topk_per_position(rows, 2)
    assert select_tree_expand(idx, p, 2, 9, 16).n == 6
    cost = Cost(a=1.0, b=0.02, c=1e-4, e=1e-6, c_d=0.5)
    order = expand_candidates(idx, p, 2)
    t = select_tree_expand(idx, p, 2, 5, 8, cost=cost, prefix_len=1000)
    assert t.n == adaptive_budget([c.score for c in order[:5]], cost, 1000, 5)


def test_rejects_wrong_row_count():
    idx, p = topk_per_position(np.full((4, 3), 1 / 3, dtype=np.float32), 2)
    with pytest.raises(ValueError):
        expand_candidates(idx, p, 2)


def test_depth_orders_equal_scores():
    """Equal scores at different depths: the shallower node comes first even
    when the deeper one's parent scores higher (dyadic values, exact in fp32).
    Tokens 0/1; a = root's token 0 (0.75), b = token 1 (0.25); a's children
    0.5 each (0.375), b's 0.75 / 0.25; every depth-2 node's children 0.5 each.
    b's first child (0.25 * 0.75 = 0.1875, depth 2) precedes the four
    grandchildren of a (0.375 * 0.5 = 0.1875, depth 3)."""
    rows = np.array([[0.75, 0.25], [0.5, 0.5], [0.75, 0.25],
                     [0.5, 0.5], [0.5, 0.5], [0.5, 0.5], [0.5, 0.5]], dtype=np.float32)
    idx, p = topk_per_position(rows, 2)
    tree = select_tree_expand(idx, p, 3, 9, 16)
    assert _paths(tree) == [(0,), (0, 0), (0, 1), (1,), (1, 0),
                            (0, 0, 0), (0, 0, 1), (0, 1, 0), (0, 1, 1)]
    assert [float(x) for x in tree.score[:9]] == [0.75, 0.375, 0.375, 0.25] + [0.1875] * 5
