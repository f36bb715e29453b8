"""Branch-aware tree attention, naive and in fp64 (test infrastructure only).

[review] Difficulty 1 (paper section 3.1) and "How it works", step 3: a
candidate attends only to its own ancestors, never to another branch, so
A-B-B sees A and A-B while A-C sees only A.  Section 6 as quoted: under dense
attention the tree is a mask over the shared KV.

Readings fixed here:
  * the keys of tree node i are every persistent prefix row 0..l-1 (the root
    is the last of them) plus the scratch rows of i and of each of its
    ancestors, found by walking parent pointers;
  * grouped-query attention maps query head h to KV head h // (Hq / Hkv);
  * scores are sm_scale * q.k (inputs are already position-encoded);
  * lse is the natural-log log-sum-exp of the scaled scores.
"""

import numpy as np


def _path(parent, i):
    out = []
    j = int(i)
    while j >= 0:
        out.append(j)
        j = int(parent[j])
    return out[::-1]


def attend_node(q, k_prefix, v_prefix, k_tree, v_tree, parent, i, sm_scale):
    """Attention of tree node i for every query head.

    q [Hq, d_qk]; k_prefix [l, Hkv, d_qk]; v_prefix [l, Hkv, d_v];
    k_tree [N, Hkv, d_qk]; v_tree [N, Hkv, d_v]; parent [N].
    Returns out fp64 [Hq, d_v] and lse fp64 [Hq].
    """
    q = np.asarray(q, dtype=np.float64)
    path = _path(parent, i)
    K = np.concatenate([np.asarray(k_prefix, np.float64),
                        np.asarray(k_tree, np.float64)[path]], axis=0)
    V = np.concatenate([np.asarray(v_prefix, np.float64),
                        np.asarray(v_tree, np.float64)[path]], axis=0)
    Hq, Hkv = q.shape[0], K.shape[1]
    G = Hq // Hkv
    out = np.empty((Hq, V.shape[2]), dtype=np.float64)
    lse = np.empty(Hq, dtype=np.float64)
    for g in range(Hkv):
        heads = slice(g * G, (g + 1) * G)
        s = sm_scale * (q[heads] @ K[:, g, :].T)        # [G, keys]
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        tot = e.sum(axis=1, keepdims=True)
        out[heads] = (e @ V[:, g, :]) / tot
        lse[heads] = (mx + np.log(tot))[:, 0]
    return out, lse


def attend_request(q, k_cache, v_cache, k_tree, v_tree, prefix_len, n, parent,
                   sm_scale, nodes=None):
    """attend_node for nodes 0..n-1 (or the given subset) of one request.

    k_cache/v_cache hold at least prefix_len rows.  Returns dicts keyed by
    node index.
    """
    lp = int(prefix_len)
    outs, lses = {}, {}
    for i in (range(int(n)) if nodes is None else nodes):
        o, s = attend_node(q[i], k_cache[:lp], v_cache[:lp], k_tree, v_tree,
                           parent, i, sm_scale)
        outs[i], lses[i] = o, s
    return outs, lses


def latent_as_heads(latent, d_v):
    """View a latent cache [rows, d_qk] as one KV head: K = all d_qk columns,
    V = the first d_v columns (the latent layout shares one row for both)."""
    lat = np.asarray(latent)
    return lat[:, None, :], lat[:, None, :d_v]
