"""build_tree_expand on the GPU vs the oracle: bit-exact top-k lists and trees
of the per-node conditional expansion, and a round built on such a tree."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import tree_structured_verification_amd as tsv
from tests._helpers import DEV, TOL, assert_tree_equal, check_attention
from tests.conftest import GOLDEN
from workloads import Cost, attention_inputs, config, expand_config, node_distributions

pytestmark = pytest.mark.gpu


def _oracle(rows_np, steps, top_k, n_budget, N_max, cost=None, prefix=None):
    idx, p = oracle.topk_per_position(rows_np, top_k)
    trees = [oracle.select_tree_expand(idx[b], p[b], steps, n_budget, N_max, cost,
                                       0 if prefix is None else int(prefix[b]))
             for b in range(rows_np.shape[0])]
    return idx, p, trees


def _run(rows_np, steps, top_k, n_budget, N_max, cost=None, prefix=None):
    x = torch.from_numpy(np.ascontiguousarray(rows_np, dtype=np.float32)).to(DEV)
    pl = None if prefix is None else torch.from_numpy(np.asarray(prefix, np.int32)).to(DEV)
    g = tsv.build_tree_expand(x, steps, top_k, n_budget, N_max, cost=cost, prefix_len=pl,
                              with_topk=True)
    torch.cuda.synchronize()
    idx, p, trees = _oracle(rows_np, steps, top_k, n_budget, N_max, cost, prefix)
    assert_tree_equal(g, idx, p, trees)
    return g, trees


def test_toy_example():
    gd = json.load(open(os.path.join(GOLDEN, "toy_tree_expand.json")))
    rows = np.array(gd["rows"], dtype=np.float32)[None]
    g, trees = _run(rows, gd["steps"], gd["top_k"], gd["budget"], 8)
    assert trees[0].n == 3


@pytest.mark.parametrize("cid", [101, 102, 103])
def test_workload(cid):
    cfg = expand_config(cid)
    print(f"build_tree_expand workload {cid} {cfg.name}", flush=True)
    x = node_distributions(cfg, 0, DEV)
    _run(x.cpu().numpy(), cfg.steps, cfg.top_k, cfg.n_budget, cfg.N_max)


def _quantised(rng, shape, levels):
    x = rng.integers(0, levels, size=shape).astype(np.float64) + 1.0
    x /= x.sum(-1, keepdims=True)
    return x.astype(np.float32)


@pytest.mark.parametrize("steps,top_k", [(1, 5), (2, 2), (3, 3), (4, 4), (5, 2), (7, 2), (11, 2),
                                         (3, 7), (2, 60), (6, 1)])
def test_shapes_ties_and_budgets(steps, top_k):
    """Quantised probabilities (ties at every level), the largest list tables
    (2047 rows of top-2) and budgets on both frontier capacities."""
    rng = np.random.default_rng(steps * 131 + top_k)
    P = tsv.expanded_rows(steps, top_k)
    V = 700 if P * top_k < 1000 else 97
    rows = _quantised(rng, (3, P, V), 5)
    total = sum(top_k ** d for d in range(1, steps + 1))
    for n_budget in sorted({0, 1, 6, min(total, 64), 64, 65, 128}):
        _run(rows, steps, top_k, n_budget, 128)


@pytest.mark.parametrize("seed", range(3))
def test_adaptive_budget(seed):
    rng = np.random.default_rng(seed)
    B, steps, top_k, V = 5, 4, 3, 2000
    P = tsv.expanded_rows(steps, top_k)
    lg = rng.normal(0, 3, size=(B, P, V)) / rng.uniform(0.3, 2.0, size=(B, 1, 1))
    rows = np.exp(lg - lg.max(-1, keepdims=True))
    rows = (rows / rows.sum(-1, keepdims=True)).astype(np.float32)
    prefix = rng.integers(0, 100000, size=B).astype(np.int32)
    for cost in (Cost(a=1.0, b=0.02, c=1e-4, e=1e-6, c_d=0.5),
                 Cost(a=0.2, b=0.001, c=0.0, e=1e-7, c_d=0.1)):
        for cap in (0, 9, 100):
            _run(rows, steps, top_k, cap, 100, cost, prefix)


def test_same_as_per_position_builder_when_rows_repeat_the_marginals():
    """Both entry points give the same bits when every node's distribution is
    its depth's marginal."""
    rng = np.random.default_rng(4)
    B, steps, top_k, V = 3, 4, 3, 5000
    marg = rng.dirichlet(np.full(V, 0.3), size=(B, steps)).astype(np.float32)
    rows = np.concatenate([np.repeat(marg[:, d:d + 1], top_k ** d, axis=1) for d in range(steps)], 1)
    a = tsv.build_tree_expand(torch.from_numpy(rows).to(DEV), steps, top_k, 30, 32)
    b = tsv.build_tree(torch.from_numpy(marg).to(DEV), top_k, 30, 32)
    torch.cuda.synchronize()
    for f in ("n_nodes", "parent", "token", "depth", "score", "anc_bits"):
        assert torch.equal(a[f], b[f]), f


def test_round_on_an_expanded_tree():
    """Tree from per-node expansion -> attention -> walk -> commit, each
    against the oracle (fp32 heads of the tiny workload)."""
    cfg = config(1)
    steps, top_k, D = 3, 2, cfg.N_max
    rng = np.random.default_rng(8)
    rows = rng.dirichlet(np.full(cfg.V, 0.5), size=(cfg.B, tsv.expanded_rows(steps, top_k)))
    rows = rows.astype(np.float32)
    g, trees = _run(rows, steps, top_k, D, cfg.N_max)
    ins = attention_inputs(cfg, 0, DEV)
    out, lse = tsv.tree_verify_attn(ins["q"], ins["k_cache"], ins["v_cache"], ins["k_tree"],
                                    ins["v_tree"], ins["prefix_len"], g["n_nodes"],
                                    g["anc_bits"], cfg.Hkv, cfg.d_v, cfg.sm_scale)
    torch.cuda.synchronize()
    prefix = ins["prefix_len"].cpu().numpy()
    check_attention(out, lse, ins["q"], ins["k_cache"], ins["v_cache"], ins["k_tree"],
                    ins["v_tree"], prefix, trees, cfg.sm_scale, TOL[torch.float32], False, cfg.d_v)
    # target rows whose argmax follows the tree down to its deepest node
    t = trees[0]
    tl_np = np.random.default_rng(3).normal(size=(cfg.B, cfg.N_max + 1, cfg.V)).astype(np.float32)
    deepest = int(np.argmax(t.depth[:t.n]))
    path, j = [], deepest
    while j >= 0:
        path.append(j)
        j = int(t.parent[j])
    path = path[::-1]
    row = 0                                   # the root's row, then row 1 + node
    for node in path:
        tl_np[0, row, t.token[node]] = 10.0
        row = 1 + node
    tl = torch.from_numpy(tl_np).to(DEV)
    walk = tsv.accept_walk(tl, g["n_nodes"], g["parent"], g["token"], steps)
    kc0 = ins["k_cache"].clone()
    status = tsv.commit_path(ins["k_cache"], ins["v_cache"], ins["prefix_len"], ins["k_tree"],
                             ins["v_tree"], walk["accept_len"], walk["accept_nodes"], cfg.Hkv,
                             cfg.d_qk, cfg.d_v)
    torch.cuda.synchronize()
    m, nodes, toks = oracle.accept_walk(tl_np[0], t.n, t.parent, t.token, steps)
    assert m == len(path) >= 1
    assert int(walk["accept_len"][0]) == m
    assert np.array_equal(walk["accept_nodes"].cpu().numpy()[0], nodes)
    assert np.array_equal(walk["out_tokens"].cpu().numpy()[0], toks)
    assert int(status[0]) == 0 and int(ins["prefix_len"][0]) == prefix[0] + m
    kc, kt = kc0.cpu().numpy()[0], ins["k_tree"].cpu().numpy()[0]
    after = ins["k_cache"].cpu().numpy()[0]
    for j in range(m):
        assert np.array_equal(after[prefix[0] + j], kt[nodes[j]])
    assert np.array_equal(after[:prefix[0]], kc[:prefix[0]])


def test_invalid_arguments_return_status():
    x = torch.zeros((1, 3, 8), dtype=torch.float32, device=DEV)
    with pytest.raises(ValueError):
        tsv.build_tree_expand(x, 3, 2, 2, 4)          # 3 rows, 3 steps of top-2 need 7
    with pytest.raises(tsv.TsvError) as e:
        tsv.build_tree_expand(x, 2, 2, 5, 4)          # budget > N_max
    assert e.value.code == -1
    y = torch.zeros((1, 1365, 8), dtype=torch.float32, device=DEV)
    with pytest.raises(tsv.TsvError) as e:
        tsv.build_tree_expand(y, 6, 4, 2, 4)          # 1365 x 4 list entries > 4096
    assert e.value.code == -2


def test_depth_orders_equal_scores():
    """Equal dyadic scores across depths: the shallower node first even when
    the deeper one's parent scores higher (same rows as the oracle's pin)."""
    rows = np.array([[0.75, 0.25], [0.5, 0.5], [0.75, 0.25],
                     [0.5, 0.5], [0.5, 0.5], [0.5, 0.5], [0.5, 0.5]], dtype=np.float32)[None]
    for n in (4, 5, 6, 9, 14):
        _run(rows, 3, 2, n, 16)
