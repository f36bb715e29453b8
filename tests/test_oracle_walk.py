"""Pins of the oracle's greedy accept walk (CPU only)."""

import json
import os

import numpy as np
import pytest

from oracle import accept_walk, row_argmax, select_tree, topk_per_position
from tests.conftest import GOLDEN


def _logits_with_argmax(rng, targets, V):
    rows = rng.normal(0, 1, size=(len(targets), V)).astype(np.float32)
    for r, t in enumerate(targets):
        rows[r, t] = rows[r].max() + 1.0
    return rows


def test_dspark_decoding_cycle():
    g = json.load(open(os.path.join(GOLDEN, "dspark_cycle.json")))
    tok = g["tokens"]
    chain = [tok[t] for t in g["chain"]]
    n = len(chain)
    parent = np.arange(-1, n - 1)
    # verified rows: root D, then E, F, G
    after = [g["root"]] + g["chain"]
    targets = [tok[g["target_argmax_after"][t]] for t in after]
    rows = _logits_with_argmax(np.random.default_rng(0), targets, g["vocab_size"])
    m, nodes, out = accept_walk(rows, n, parent, np.array(chain), gamma=4)
    assert m == g["accept_len"]
    assert nodes.tolist() == [0, 1, -1, -1]
    assert out.tolist() == [tok[t] for t in g["accepted"]] + [tok[g["bonus"]], -1, -1]


def _leading_matches(chain_tokens, argmaxes):
    m = 0
    while m < len(chain_tokens) and chain_tokens[m] == argmaxes[m]:
        m += 1
    return m


@pytest.mark.parametrize("seed", range(10))
def test_chain_equals_linear_verification(seed):
    rng = np.random.default_rng(seed)
    V, n = 6, 7
    chain = rng.integers(0, V, size=n)
    rows = rng.normal(0, 1, size=(n + 1, V)).astype(np.float32)
    # bias rows towards the chain so that long prefixes occur
    for r in range(n):
        if rng.random() < 0.8:
            rows[r, chain[r]] += 5.0
    m, nodes, out = accept_walk(rows, n, np.arange(-1, n - 1), chain, gamma=n)
    am = np.argmax(rows, -1)
    want = _leading_matches(list(chain), list(am))
    assert m == want
    assert nodes[:m].tolist() == list(range(m))
    assert out[m] == am[m]


@pytest.mark.parametrize("seed", range(10))
def test_brute_force_over_paths(seed):
    """The accepted node is the deepest node whose whole root path matches."""
    rng = np.random.default_rng(seed)
    V, gamma, k = 5, 4, 3
    marg = rng.dirichlet(np.ones(V), size=gamma).astype(np.float32)
    idx, p = topk_per_position(marg, k)
    tree = select_tree(idx, p, 20, 32)
    rows = rng.normal(0, 1, size=(1 + 32, V)).astype(np.float32)
    for r in range(1 + tree.n):
        rows[r, rng.integers(0, V)] += 3.0
    am = np.argmax(rows, -1)
    best, best_depth = -1, 0
    for i in range(tree.n):
        j, ok = i, True
        while j >= 0:
            if tree.token[j] != am[tree.parent[j] + 1]:
                ok = False
            j = tree.parent[j]
        if ok and tree.depth[i] > best_depth:
            best, best_depth = i, int(tree.depth[i])
    m, nodes, out = accept_walk(rows, tree.n, tree.parent, tree.token, gamma)
    assert m == best_depth
    if m:
        assert nodes[m - 1] == best
    assert out[m] == am[best + 1]


def test_toy_commit_path():
    g = json.load(open(os.path.join(GOLDEN, "toy_tree.json")))
    V = {t: i for i, t in enumerate(g["vocab"])}
    marg = np.array(g["marginals"], dtype=np.float32)
    idx, p = topk_per_position(marg, g["top_k"])
    tree = select_tree(idx, p, g["budget"], 8)
    rows = np.zeros((1 + 8, 3), dtype=np.float32)
    rows[0, V[g["root_argmax_for_commit"]]] = 1.0      # root row prefers C
    for r in range(1, 1 + tree.n):
        rows[r, V["A"]] = 1.0                           # no deeper match
    m, nodes, out = accept_walk(rows, tree.n, tree.parent, tree.token, 2)
    accepted = [g["vocab"][tree.token[v]] for v in nodes[:m]]
    assert accepted == g["accepted_path"]
    assert g["prefix"] + accepted == g["next_prefix"]


def test_argmax_ties_lowest_id():
    rows = np.array([[1.0, 3.0, 3.0, 2.0], [0.0, -0.0, 0.0, -1.0],
                     [-5.0, -5.0, -6.0, -5.0]], dtype=np.float32)
    assert row_argmax(rows).tolist() == [1, 0, 0]
    with pytest.raises(ValueError):
        row_argmax(np.array([[np.nan, 1.0]], dtype=np.float32))


def test_empty_tree_yields_bonus_only():
    rows = np.array([[0.0, 2.0, 1.0]], dtype=np.float32)
    m, nodes, out = accept_walk(rows, 0, np.full(4, -1), np.full(4, -1), 3)
    assert m == 0 and nodes.tolist() == [-1, -1, -1] and out.tolist() == [1, -1, -1, -1]
