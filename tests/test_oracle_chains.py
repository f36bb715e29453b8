"""Pins of the oracle's chain unfolding (CPU only): the review's toy chains,
closed forms for a chain and a star, and structural properties checked
against an independent description (every root-to-node path is a prefix of
exactly the chains through that node)."""

import json
import os

import numpy as np
import pytest

from oracle import select_tree, topk_per_position, unfold_chains
from tests.conftest import GOLDEN


def test_toy_chains():
    g = json.load(open(os.path.join(GOLDEN, "toy_tree.json")))
    V = {t: i for i, t in enumerate(g["vocab"])}
    idx, p = topk_per_position(np.array(g["marginals"], dtype=np.float32), g["top_k"])
    tree = select_tree(idx, p, g["budget"], 8)
    count, lengths, nodes = unfold_chains(tree.parent, tree.n, g["gamma"])
    chains = sorted(tuple(int(tree.token[j]) for j in nodes[c, :lengths[c]]) for c in range(count))
    assert chains == sorted(tuple(V[t] for t in ch) for ch in g["chains"])


def test_chain_tree_is_one_chain():
    count, lengths, nodes = unfold_chains([-1, 0, 1, 2, 3], 5, 8)
    assert count == 1 and list(lengths) == [5] and list(nodes[0, :5]) == [0, 1, 2, 3, 4]
    assert np.all(nodes[0, 5:] == -1)


def test_star_tree_is_one_chain_per_node():
    count, lengths, nodes = unfold_chains([-1] * 6, 6, 3)
    assert count == 6 and np.all(lengths == 1) and list(nodes[:, 0]) == list(range(6))


def test_empty_tree():
    count, lengths, nodes = unfold_chains([], 0, 4)
    assert count == 0 and lengths.shape == (0,) and nodes.shape == (0, 4)


@pytest.mark.parametrize("seed", range(6))
def test_random_trees(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 60))
    parent = [-1] + [int(rng.integers(-1, i)) for i in range(1, n)]
    depth = [0] * n
    for i in range(n):
        depth[i] = 1 if parent[i] < 0 else depth[parent[i]] + 1
    gamma = max(depth)
    count, lengths, nodes = unfold_chains(parent, n, gamma)
    leaves = [i for i in range(n) if i not in parent]
    assert count == len(leaves)
    for c in range(count):
        path = list(nodes[c, :lengths[c]])
        assert path[-1] == leaves[c] and parent[path[0]] == -1
        assert all(parent[path[t]] == path[t - 1] for t in range(1, len(path)))
    # every node lies on at least one chain, at the position of its depth
    for i in range(n):
        assert any(lengths[c] >= depth[i] and nodes[c, depth[i] - 1] == i for c in range(count))
