"""Per-position top-k of the drafter's marginals (test infrastructure only).

[caddtree] Methodology: the drafter emits one marginal distribution per block
position in a single pass; the tree builder branches on the most probable
tokens of each position.  [review] "How it works" defines top-k as the number
of branches kept per drafting step.

Reading fixed here: the order is probability descending, then token id
ascending; -0.0 equals +0.0.  Inputs must be finite.
"""

import numpy as np


def topk_per_position(marginals, k: int):
    """Return (idx int32 [..., k], p fp32 [..., k]) for every row of marginals.

    A stable ascending argsort of -p puts larger probabilities first and keeps
    equal probabilities in token-id order.
    """
    m = np.asarray(marginals, dtype=np.float32)
    if not np.all(np.isfinite(m)):
        raise ValueError("marginals must be finite")
    if not 1 <= k <= m.shape[-1]:
        raise ValueError("k must be in [1, V]")
    flat = m.reshape(-1, m.shape[-1])
    idx = np.empty((flat.shape[0], k), dtype=np.int32)
    for r in range(flat.shape[0]):
        idx[r] = np.argsort(-flat[r], kind="stable")[:k]
    p = np.take_along_axis(flat, idx.astype(np.int64), axis=1)
    return (idx.reshape(m.shape[:-1] + (k,)),
            p.astype(np.float32).reshape(m.shape[:-1] + (k,)))
