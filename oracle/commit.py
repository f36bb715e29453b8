"""Accepted-path commit (test infrastructure only).

[review] "Secret weapon" and paper section 4.2 as quoted: tentative branch
state lives in a scratch pad and never goes straight into the persistent
cache; after the accepted path is chosen only its state is written back and
the rest is dropped.  "How it works", step 6: if A-C is accepted, only that
chain's KV is committed and the next round starts from prefix A-C.

Readings fixed here:
  * for j < m_b: cache row l_b + j <- scratch row accept_nodes[b][j]
    (every KV head, K and V; a latent cache copies its d_qk columns only);
    then l_b += m_b;
  * if l_b + m_b exceeds the cache capacity the request is left untouched
    and its status is 1; a node index outside [0, N_max), m_b outside
    [0, gamma] or a negative l_b gives status 2, also untouched; otherwise
    status 0.
"""

import numpy as np


def commit_path(k_cache, v_cache, prefix_len, k_tree, v_tree, accept_len,
                accept_nodes, gamma: int):
    """In place on numpy arrays.  k_cache [B, L_cap, ...]; v_cache may be None
    (latent cache).  Returns status int32 [B]."""
    B, L_cap = k_cache.shape[0], k_cache.shape[1]
    N_max = k_tree.shape[1]
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        m = int(accept_len[b])
        lb = int(prefix_len[b])
        nodes = [int(x) for x in accept_nodes[b][: max(m, 0)]]
        if m < 0 or m > gamma or lb < 0 or any(v < 0 or v >= N_max for v in nodes):
            status[b] = 2
            continue
        if lb + m > L_cap:
            status[b] = 1
            continue
        for j, v in enumerate(nodes):
            k_cache[b, lb + j] = k_tree[b, v]
            if v_cache is not None:
                v_cache[b, lb + j] = v_tree[b, v]
        prefix_len[b] = lb + m
    return status
