"""Helpers shared by the GPU parity tests (test code only)."""

import numpy as np
import torch

import oracle

DEV = "cuda:0"

# tolerances of the attention output and lse against the fp64 oracle
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def np32(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy; bf16 is widened to fp32 (exact)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.numpy()


def oracle_trees(marg: np.ndarray, top_k, n_budget, N_max, cost=None, prefix=None):
    idx, p = oracle.topk_per_position(marg, top_k)
    trees = [oracle.select_tree(idx[b], p[b], n_budget, N_max, cost,
                                0 if prefix is None else int(prefix[b]))
             for b in range(marg.shape[0])]
    return idx, p, trees


def stack_trees(trees, N_max):
    return dict(
        n_nodes=np.array([t.n for t in trees], dtype=np.int32),
        parent=np.stack([t.parent for t in trees]),
        token=np.stack([t.token for t in trees]),
        depth=np.stack([t.depth for t in trees]),
        score=np.stack([t.score for t in trees]),
        anc_bits=np.stack([t.anc_bits for t in trees]),
    )


def assert_tree_equal(g: dict, idx, p, trees, b_list=None, check_topk=True):
    """Bit-exact comparison of build_tree outputs with the oracle (and of the
    top-k lists of build_tree_topk unless check_topk is False)."""
    if check_topk:
        gi = g["topk_idx"].cpu().numpy()
        gp = g["topk_p"].cpu().numpy()
        assert np.array_equal(gi, idx), "top-k ids differ"
        assert np.array_equal(gp.view(np.uint32), p.view(np.uint32)), "top-k probabilities differ"
    n = g["n_nodes"].cpu().numpy()
    par = g["parent"].cpu().numpy()
    tok = g["token"].cpu().numpy()
    dep = g["depth"].cpu().numpy()
    sc = g["score"].cpu().numpy()
    anc = g["anc_bits"].cpu().numpy().view(np.uint32)
    for b in (range(len(trees)) if b_list is None else b_list):
        t = trees[b]
        assert n[b] == t.n, (b, n[b], t.n)
        assert np.array_equal(par[b], t.parent), b
        assert np.array_equal(tok[b], t.token), b
        assert np.array_equal(dep[b], t.depth), b
        assert np.array_equal(sc[b].view(np.uint32), t.score.view(np.uint32)), b
        assert np.array_equal(anc[b], t.anc_bits), b


def check_attention(out, lse, q, kc, vc, kt, vt, prefix, trees, sm_scale, tol, mla,
                    d_v, samples=None):
    """Compare rows of the GPU output with the oracle; samples: list of (b, i)
    or None for every node.  Returns the max abs error seen."""
    o = out.detach().cpu()
    o = (o.float() if o.dtype == torch.bfloat16 else o).numpy()
    ls = lse.detach().cpu().numpy()
    pairs = samples if samples is not None else [(b, i) for b in range(len(trees))
                                                  for i in range(trees[b].n)]
    worst = 0.0
    cache = {}
    for b, i in pairs:
        if b not in cache:
            lb = int(prefix[b])
            qb = np32(q[b])
            if mla:
                K, V = oracle.attention.latent_as_heads(np32(kc[b, :lb]), d_v)
                Kt, Vt = oracle.attention.latent_as_heads(np32(kt[b]), d_v)
            else:
                K, V = np32(kc[b, :lb]), np32(vc[b, :lb])
                Kt, Vt = np32(kt[b]), np32(vt[b])
            cache = {b: (qb, K, V, Kt, Vt)}
        qb, K, V, Kt, Vt = cache[b]
        ref, ref_lse = oracle.attend_node(qb[i], K, V, Kt, Vt, trees[b].parent, i, sm_scale)
        err = max(float(np.max(np.abs(o[b, i] - ref))), float(np.max(np.abs(ls[b, i] - ref_lse))))
        worst = max(worst, err)
        assert err <= tol, (b, i, err)
    return worst
