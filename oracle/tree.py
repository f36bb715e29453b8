"""Greedy best-first draft tree by prefix probability (test infrastructure only).

[caddtree] Methodology, item 2: for any fixed node budget n the best tree is
the greedy best-first one, i.e. the n candidate nodes with the highest prefix
probability; searching over all trees reduces to a search over n.
[review] "How it works", steps 1-2: candidates are expanded from the accepted
prefix with top-k branches per drafting step and pruned to the verification
budget D by score; the toy (vocabulary {A, B, C}, top-2, two steps) has
1 + 2 + 4 = 7 nodes counting the root.

Readings fixed here:
  * the root is the last accepted token; it is not counted in n;
  * a node at depth d takes its token from the top-k list of position d-1;
    its score is the fp32 product score(parent) * q, root score 1;
  * the selection order is the nested key
        T(v) = (-score(v), depth(v), T(parent(v)), rank(v)),  T(root) = (),
    smallest first.  T grows strictly along every edge (a child's score never
    exceeds its parent's and its depth is larger), so every prefix of the
    order is ancestor-closed and the order is the pop order of a best-first
    search; nodes are numbered by their position in it, parents first;
  * ancestor sets include the node itself.
"""

import dataclasses

import numpy as np

from .budget import adaptive_budget


@dataclasses.dataclass
class _Cand:
    score: np.float32
    depth: int
    parent: "_Cand"
    rank: int
    token: int
    key: tuple


def _child(parent, depth, rank, tk_idx, tk_p):
    ps = np.float32(1.0) if parent is None else parent.score
    s = np.float32(ps * np.float32(tk_p[depth - 1, rank]))
    pkey = () if parent is None else parent.key
    return _Cand(s, depth, parent, rank, int(tk_idx[depth - 1, rank]),
                 (-float(s), depth, pkey, rank))


def _children(parent, depth, tk_idx, tk_p):
    return [_child(parent, depth, r, tk_idx, tk_p) for r in range(tk_p.shape[1])]


def enumerate_candidates(tk_idx, tk_p):
    """Every candidate node of the full top-k tree, in T order."""
    gamma = tk_p.shape[0]
    level = _children(None, 1, tk_idx, tk_p)
    allc = list(level)
    for d in range(2, gamma + 1):
        level = [c for v in level for c in _children(v, d, tk_idx, tk_p)]
        allc.extend(level)
    allc.sort(key=lambda c: c.key)
    return allc


def best_candidates(tk_idx, tk_p, cap: int):
    """The first `cap` candidates in T order, by exact level-by-level pruning.

    Any top-cap set under T is ancestor-closed, so the top-cap among depths
    <= d is contained in (top-cap among depths <= d-1) plus the children of
    its depth-(d-1) members; sorting that union and cutting at cap is exact.
    """
    gamma = tk_p.shape[0]
    if cap <= 0:
        return []
    kept = sorted(_children(None, 1, tk_idx, tk_p), key=lambda c: c.key)[:cap]
    for d in range(2, gamma + 1):
        new = [c for v in kept if v.depth == d - 1
               for c in _children(v, d, tk_idx, tk_p)]
        if not new:
            break
        kept = sorted(kept + new, key=lambda c: c.key)[:cap]
    return kept


def ancestor_bits(parent, n: int, N_max: int) -> np.ndarray:
    """uint32 [N_max, ceil(N_max/32)]: bit j of row i <=> j is i or an ancestor
    of i, found by walking parent pointers."""
    words = (N_max + 31) // 32
    bits = np.zeros((N_max, words), dtype=np.uint32)
    for i in range(n):
        j = i
        while j >= 0:
            bits[i, j // 32] |= np.uint32(1 << (j % 32))
            j = int(parent[j])
    return bits


@dataclasses.dataclass
class TreeResult:
    n: int
    parent: np.ndarray   # int32 [N_max], -1 = child of the root / padding
    token: np.ndarray    # int32 [N_max], -1 padding
    depth: np.ndarray    # int32 [N_max], 1-based, -1 padding
    score: np.ndarray    # fp32 [N_max], 0 padding
    anc_bits: np.ndarray  # uint32 [N_max, ceil(N_max/32)], 0 padding


def select_tree(tk_idx, tk_p, n_budget: int, N_max: int, cost=None,
                prefix_len: int = 0, method: str = "auto") -> TreeResult:
    """Best-first tree of one request.

    Fixed budget (cost is None): n = min(n_budget, number of candidates).
    Adaptive (cost given): n = greedy stop over the best-first scores, capped
    at n_budget.  method: "enumerate" (all candidates), "levels" (exact
    pruning) or "auto" (enumerate when there are at most 10**5 candidates).
    """
    tk_idx = np.asarray(tk_idx)
    tk_p = np.asarray(tk_p, dtype=np.float32)
    gamma, k = tk_p.shape
    if not 0 <= n_budget <= N_max:
        raise ValueError("n_budget must be in [0, N_max]")
    cap = n_budget
    total = sum(k ** d for d in range(1, gamma + 1))
    if method == "auto":
        method = "enumerate" if total <= 10 ** 5 else "levels"
    if method == "enumerate":
        order = enumerate_candidates(tk_idx, tk_p)[:cap]
    else:
        order = best_candidates(tk_idx, tk_p, cap)
    if cost is None:
        n = min(cap, len(order))
    else:
        n = adaptive_budget([c.score for c in order], cost, prefix_len, cap)
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
    return TreeResult(n, parent, token, depth, score,
                      ancestor_bits(parent, n, N_max))
