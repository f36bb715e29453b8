"""Draft tree by per-node conditional expansion (test infrastructure only).

[review] "How it works", steps 1-2, and its notation paragraph: the drafter
runs s draft steps; at every step each node of the newest level branches into
the top-k tokens of its *own* next-token distribution (the toy: A expands to
{B, C}; then B to {B, C} and C to {A, B}, 1 + 2 + 4 = 7 nodes counting the
root), and the candidates are then cut to the verification budget D by score.
[review] "Our perspective": the pruning is by cumulative score.
[caddtree] Methodology, items 2-4: for a fixed node count the best tree is the
best-first one by prefix probability, and the budget may instead come from the
throughput stop rule.

Readings fixed here:
  * the expanded nodes are the root (depth 0) and every candidate of depth
    < s: a complete k-ary tree.  Their distributions are given in level order:
    row 0 is the root's, and the child of rank r of the node with row i has
    row k*i + 1 + r.  Candidates of depth s are leaves and have no row;
  * a candidate's score is the fp32 product of the conditional probabilities
    along its path (parent score times its own probability, root score 1): the
    cumulative score of the review and the prefix probability of the cost-aware
    paper;
  * selection order, budget and outputs are those of tree.select_tree: the
    nested key T(v) = (-score, depth, T(parent), rank), smallest first (every
    prefix of it is ancestor-closed), a fixed budget n = min(D, candidates) or
    the greedy throughput stop capped at D, nodes numbered in that order.
"""

import numpy as np

from .budget import adaptive_budget
from .tree import TreeResult, ancestor_bits


def expanded_rows(steps: int, k: int) -> int:
    """Number of expanded nodes (rows of distributions): 1 + k + ... + k^(s-1)."""
    return sum(k ** d for d in range(steps))


class _Node:
    __slots__ = ("score", "depth", "parent", "rank", "token", "row", "key")

    def __init__(self, score, depth, parent, rank, token, row, key):
        self.score, self.depth, self.parent = score, depth, parent
        self.rank, self.token, self.row, self.key = rank, token, row, key


def expand_candidates(tk_idx, tk_p, steps: int):
    """Every candidate of the s-step expansion, in T order.

    tk_idx / tk_p: [rows, k] top-k of each expanded node's distribution,
    rows in level order (see the module docstring).
    """
    tk_idx = np.asarray(tk_idx)
    tk_p = np.asarray(tk_p, dtype=np.float32)
    rows, k = tk_p.shape
    if rows != expanded_rows(steps, k):
        raise ValueError(f"expected {expanded_rows(steps, k)} rows for s={steps}, k={k}")
    out = []
    frontier = [(None, 0)]          # (node, row of its distribution)
    for depth in range(1, steps + 1):
        nxt = []
        for par, row in frontier:
            ps = np.float32(1.0) if par is None else par.score
            pkey = () if par is None else par.key
            for r in range(k):
                s = np.float32(ps * tk_p[row, r])
                child_row = k * row + 1 + r if depth < steps else -1
                c = _Node(s, depth, par, r, int(tk_idx[row, r]), child_row,
                          (-float(s), depth, pkey, r))
                out.append(c)
                nxt.append((c, child_row))
        frontier = nxt
    out.sort(key=lambda c: c.key)
    return out


def select_tree_expand(tk_idx, tk_p, steps: int, n_budget: int, N_max: int, cost=None,
                       prefix_len: int = 0) -> TreeResult:
    """Tree of one request from its per-node top-k lists.

    Fixed budget (cost is None): n = min(n_budget, candidates).  Adaptive:
    the greedy throughput stop over the selection order, capped at n_budget.
    """
    if not 0 <= n_budget <= N_max:
        raise ValueError("n_budget must be in [0, N_max]")
    order = expand_candidates(tk_idx, tk_p, steps)[:n_budget]
    if cost is None:
        n = len(order)
    else:
        n = adaptive_budget([c.score for c in order], cost, prefix_len, n_budget)
    nodes = order[:n]
    pos = {id(c): i for i, c in enumerate(nodes)}
    parent = np.full(N_max, -1, dtype=np.int32)
    token = np.full(N_max, -1, dtype=np.int32)
    depth = np.full(N_max, -1, dtype=np.int32)
    score = np.zeros(N_max, dtype=np.float32)
    for i, c in enumerate(nodes):
        parent[i] = -1 if c.parent is None else pos[id(c.parent)]
        token[i] = c.token
        depth[i] = c.depth
        score[i] = c.score
    return TreeResult(n, parent, token, depth, score, ancestor_bits(parent, n, N_max))
