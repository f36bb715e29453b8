"""Pins of the oracle's best-first tree (CPU only)."""

import itertools
import json
import os

import numpy as np
import pytest

from oracle import select_tree, topk_per_position
from oracle.tree import best_candidates, enumerate_candidates
from tests.conftest import GOLDEN


def _paths(tree):
    """Token path (root excluded) of every selected node."""
    out = []
    for i in range(tree.n):
        p, j = [], i
        while j >= 0:
            p.append(int(tree.token[j]))
            j = int(tree.parent[j])
        out.append(tuple(p[::-1]))
    return out


def _tree_from_marginals(marg, k, n, N_max, **kw):
    idx, p = topk_per_position(marg, k)
    return select_tree(idx, p, n, N_max, **kw)


def test_toy_example():
    g = json.load(open(os.path.join(GOLDEN, "toy_tree.json")))
    V = {t: i for i, t in enumerate(g["vocab"])}
    marg = np.array(g["marginals"], dtype=np.float32)
    k, gamma, D = g["top_k"], g["gamma"], g["budget"]
    idx, p = topk_per_position(marg, k)
    # candidate count: the root plus k + k^2 drafted nodes
    assert 1 + len(enumerate_candidates(idx, p)) == g["nodes_including_root"]
    tree = select_tree(idx, p, D, 8)
    kept = {tuple(V[t] for t in path) for path in g["kept_paths"]}
    assert set(_paths(tree)) == kept
    # visibility: ancestor-or-self sets of every kept node
    names = {tuple(V[t] for t in path): path for path in g["kept_paths"]}
    paths = _paths(tree)
    for i, pth in enumerate(paths):
        seen = {paths[j] for j in range(tree.n)
                if tree.anc_bits[i, j // 32] >> (j % 32) & 1}
        want = {tuple(V[t] for t in s) for s in g["sees"][" ".join(names[pth])]}
        assert seen == want
    # chains = root-to-leaf paths
    leaves = [paths[i] for i in range(tree.n) if i not in set(tree.parent[:tree.n])]
    assert sorted(leaves) == sorted(tuple(V[t] for t in c) for c in g["chains"])


def _brute_force_top(marg, n):
    """All token sequences of length 1..gamma over the full vocabulary,
    scored by the fp32 product of their per-position marginals, best n."""
    gamma, V = marg.shape
    seqs = []
    for d in range(1, gamma + 1):
        for seq in itertools.product(range(V), repeat=d):
            s = np.float32(1.0)
            for pos, t in enumerate(seq):
                s = np.float32(s * marg[pos, t])
            seqs.append((float(s), seq))
    seqs.sort(key=lambda x: -x[0])
    # random inputs: require a strict gap at the cut so the set is unique
    assert n >= len(seqs) or seqs[n - 1][0] > seqs[n][0]
    return [s for _, s in seqs[:n]]


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_over_full_vocabulary(seed):
    rng = np.random.default_rng(100 + seed)
    V, gamma = [(4, 3), (5, 3), (6, 2), (3, 4), (16, 2), (2, 4)][seed]
    logits = rng.normal(0, 2, size=(gamma, V))
    marg = np.exp(logits) / np.exp(logits).sum(-1, keepdims=True)
    marg = marg.astype(np.float32)
    total = sum(V ** d for d in range(1, gamma + 1))
    for n in range(1, min(total, 24) + 1):
        want = _brute_force_top(marg, n)
        tree = _tree_from_marginals(marg, min(V, n), n, 32)
        assert tree.n == n
        assert _paths(tree) == want


@pytest.mark.parametrize("seed", range(8))
def test_level_pruning_equals_enumeration(seed):
    rng = np.random.default_rng(seed)
    gamma, V, k = 4, 12, 5
    if seed % 2:
        marg = (rng.integers(1, 5, size=(gamma, V)) / 8.0).astype(np.float32)  # ties
    else:
        marg = rng.dirichlet(np.ones(V), size=gamma).astype(np.float32)
    idx, p = topk_per_position(marg, k)
    full = enumerate_candidates(idx, p)
    for cap in (1, 2, 7, 31, 64):
        lv = best_candidates(idx, p, cap)
        assert [c.key for c in lv] == [c.key for c in full[:cap]]


@pytest.mark.parametrize("seed", range(6))
def test_ancestor_closed_and_scores_monotone(seed):
    rng = np.random.default_rng(seed)
    marg = rng.dirichlet(np.ones(20) * 0.3, size=6).astype(np.float32)
    tree = _tree_from_marginals(marg, 6, 40, 64)
    for i in range(tree.n):
        par = tree.parent[i]
        assert par < i
        if par >= 0:
            assert tree.depth[i] == tree.depth[par] + 1
            assert tree.score[i] <= tree.score[par]
        else:
            assert tree.depth[i] == 1
        if i:
            assert tree.score[i] <= tree.score[i - 1]
    assert (tree.parent[tree.n:] == -1).all() and (tree.token[tree.n:] == -1).all()
    assert (tree.anc_bits[tree.n:] == 0).all()


def test_linear_is_top1():
    rng = np.random.default_rng(3)
    marg = rng.dirichlet(np.ones(10), size=5).astype(np.float32)
    for n in (1, 3, 5, 8):
        tree = _tree_from_marginals(marg, 1, n, 8)
        assert tree.n == min(n, 5)
        assert tree.parent[: tree.n].tolist() == list(range(-1, tree.n - 1))
        assert tree.token[: tree.n].tolist() == np.argmax(marg, -1)[: tree.n].tolist()


@pytest.mark.parametrize("seed", range(4))
def test_k_equal_n_matches_k_equal_V(seed):
    rng = np.random.default_rng(seed)
    marg = rng.dirichlet(np.ones(9), size=3).astype(np.float32)
    for n in (1, 4, 9):
        a = _tree_from_marginals(marg, n, n, 16)
        b = _tree_from_marginals(marg, 9, n, 16)
        assert _paths(a) == _paths(b)
        assert np.array_equal(a.score, b.score)


def test_tie_order_reading():
    """Equal scores: shallower first, then the earlier parent, then the
    better-ranked sibling."""
    half = np.float32(0.5)
    marg = np.array([[half, half, 0.0], [half, half, 0.0]], dtype=np.float32)
    tree = _tree_from_marginals(marg, 2, 6, 8)
    assert _paths(tree) == [(0,), (1,), (0, 0), (0, 1), (1, 0), (1, 1)]
    # a child scoring exactly its parent's score follows the equal-scored
    # depth-1 sibling
    marg = np.array([[half, half, 0.0], [1.0, 0.0, 0.0]], dtype=np.float32)
    tree = _tree_from_marginals(marg, 2, 4, 8)
    assert _paths(tree) == [(0,), (1,), (0, 0), (1, 0)]


def test_budget_clamps_to_candidates():
    marg = np.array([[0.6, 0.4], [0.7, 0.3]], dtype=np.float32)
    tree = _tree_from_marginals(marg, 2, 8, 8)
    assert tree.n == 6
    tree = _tree_from_marginals(marg, 1, 8, 8)
    assert tree.n == 2
    assert _tree_from_marginals(marg, 2, 0, 8).n == 0
