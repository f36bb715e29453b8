"""Greedy accept walk over the target's argmax (test infrastructure only).

[review] "How it works", steps 5-6: the target verifies all chains in one
pass; where the chain A-B-? fails at its second token the branch A-C can
still survive, and only the accepted path moves on.  [dspark] Problem
definition and the decoding cycle under "Architecture": verification accepts
the longest matching prefix; with draft E F G the target accepting E and F
and rejecting G yields the correction token G* after F.

Readings fixed here (greedy verification):
  * a_r = the target's argmax of verified row r, ties to the lowest token id;
    row 0 belongs to the root, row 1+i to tree node i;
  * from the root, step to the child whose token equals the argmax of the
    current node's row (siblings carry distinct tokens, so at most one does);
    stop when none does;
  * m = accepted nodes (the bonus is not counted); the round emits the m
    accepted tokens followed by the bonus a_(last accepted node or root).
"""

import numpy as np


def row_argmax(rows) -> np.ndarray:
    """First maximum of every row (np.argmax returns the lowest index)."""
    r = np.asarray(rows, dtype=np.float32)
    if np.isnan(r).any():
        raise ValueError("target logits must not be NaN")
    return np.argmax(r, axis=-1).astype(np.int32)


def accept_walk(target_rows, n: int, parent, token, gamma: int):
    """One request.  target_rows [>= 1+n, V].

    Returns (m, accept_nodes int32 [gamma] padded -1,
             out_tokens int32 [gamma+1] padded -1).
    """
    a = row_argmax(np.asarray(target_rows)[: 1 + int(n)])
    cur = -1
    path = []
    while True:
        want = a[cur + 1]
        kids = [j for j in range(int(n))
                if int(parent[j]) == cur and int(token[j]) == int(want)]
        if not kids:
            break
        if len(kids) > 1:
            raise ValueError("siblings with equal tokens")
        cur = kids[0]
        path.append(cur)
    if len(path) > gamma:
        raise ValueError("accepted path longer than gamma")
    nodes = np.full(gamma, -1, dtype=np.int32)
    toks = np.full(gamma + 1, -1, dtype=np.int32)
    for j, v in enumerate(path):
        nodes[j] = v
        toks[j] = int(token[v])
    toks[len(path)] = a[cur + 1]
    return len(path), nodes, toks
