"""Unfolding a draft tree into its chains (test infrastructure only).

[review] "How it works", step 4 (verify preprocess): the tree is unfolded
into chains -- the toy's tree A-B, A-C, A-B-B becomes Chain1 = A-B-B and
Chain2 = A-C -- so that the prefix's state is shared while everything after
the branch point is kept per chain; step 6: after acceptance only the winning
chain's state is committed.

Readings fixed here: a chain is the path from the root to one leaf (a node
that no other node names as parent), listed root-side first; chains are
numbered by their leaf's index (best-first position); the root itself is not
part of a chain (it is the last prefix token).
"""

import numpy as np


def unfold_chains(parent, n, gamma):
    """Chains of one tree: (count, lengths int32 [count], nodes int32
    [count, gamma] padded with -1)."""
    parent = [int(x) for x in parent[:n]]
    has_child = [False] * n
    for i in range(n):
        if parent[i] >= 0:
            has_child[parent[i]] = True
    leaves = [i for i in range(n) if not has_child[i]]
    lengths = np.zeros(len(leaves), dtype=np.int32)
    nodes = np.full((len(leaves), gamma), -1, dtype=np.int32)
    for c, leaf in enumerate(leaves):
        path, j = [], leaf
        while j >= 0:
            path.append(j)
            j = parent[j]
        path.reverse()
        if len(path) > gamma:
            raise ValueError("a chain is longer than gamma")
        lengths[c] = len(path)
        nodes[c, :len(path)] = path
    return len(leaves), lengths, nodes
