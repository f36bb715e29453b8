"""build_tree on the GPU vs the oracle: bit-exact top-k lists and trees."""

import dataclasses

import numpy as np
import pytest
import torch

import tree_structured_verification_amd as tsv
from tests._helpers import DEV, assert_tree_equal, oracle_trees
from workloads import Cost, config, marginals, prefix_lengths

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=[0, 1, 2], ids=["both", "serial", "level"])
def tree_method(request):
    """Every case under each tree selection: both methods side by side (the
    default), the serial pops alone and the level merge alone."""
    prev = tsv.set_tree_method(request.param)
    yield request.param
    tsv.set_tree_method(prev)


def _run(marg_np, top_k, n_budget, N_max, cost=None, prefix=None):
    m = torch.from_numpy(np.ascontiguousarray(marg_np, dtype=np.float32)).to(DEV)
    pl = None if prefix is None else torch.from_numpy(np.asarray(prefix, np.int32)).to(DEV)
    g = tsv.build_tree_topk(m, top_k, n_budget, N_max, cost=cost, prefix_len=pl)
    torch.cuda.synchronize()
    idx, p, trees = oracle_trees(marg_np, top_k, n_budget, N_max, cost, prefix)
    assert_tree_equal(g, idx, p, trees)
    return g, trees


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload(cid):
    cfg = config(cid)
    print(f"build_tree workload {cid} {cfg.name}", flush=True)
    marg = marginals(cfg, 0, DEV)
    pl = prefix_lengths(cfg) if cfg.cost is not None else None
    _run(marg.cpu().numpy(), cfg.top_k, cfg.n_budget, cfg.N_max, cfg.cost, pl)


def _quantised(rng, shape, levels):
    """Probabilities drawn from a few values: many exact ties."""
    x = rng.integers(0, levels, size=shape).astype(np.float64) + 1.0
    x /= x.sum(-1, keepdims=True)
    return x.astype(np.float32)


@pytest.mark.parametrize("top_k", [1, 5, 63, 64, 65, 128])
@pytest.mark.parametrize("V", [10000, 9999])
def test_ties_segments_and_vocab_tail(top_k, V):
    """Several scan segments per row, a vocabulary that is not a multiple of
    the vector width, and quantised probabilities (ties at every level)."""
    rng = np.random.default_rng(top_k * 7 + V)
    marg = _quantised(rng, (3, 5, V), 4)
    N_max = 128
    for n_budget in (0, 1, 17, 64, 65, 128):   # 64 / 65: the two frontier capacities
        _run(marg, top_k, n_budget, N_max)


def test_uniform_marginals_total_ties():
    marg = np.full((2, 4, 300), 1.0 / 300, dtype=np.float32)
    for k in (1, 3, 16):
        _run(marg, k, 40, 64)


def test_signed_zero_and_tiny_values():
    rng = np.random.default_rng(5)
    marg = rng.random((2, 3, 4000)).astype(np.float32) * 1e-38   # denormal products
    marg[:, :, ::7] = 0.0
    marg[:, :, 3::11] = -0.0
    marg[0, 0, 17] = 0.9
    _run(marg, 8, 30, 32)


@pytest.mark.parametrize("seed", range(4))
def test_adaptive_budget(seed):
    rng = np.random.default_rng(seed)
    B, gamma, V = 6, 12, 3000
    lg = rng.normal(0, 3, size=(B, gamma, V)) / rng.uniform(0.3, 2.0, size=(B, 1, 1))
    marg = np.exp(lg - lg.max(-1, keepdims=True))
    marg = (marg / marg.sum(-1, keepdims=True)).astype(np.float32)
    prefix = rng.integers(0, 200000, size=B).astype(np.int32)
    base = Cost(a=1.0, b=0.02, c=1e-4, e=1e-6, c_d=0.5)
    for cost in (base, dataclasses.replace(base, c=0.0, b=0.001),
                 dataclasses.replace(base, a=0.75, b=0.5, c=0.0, e=0.0, c_d=0.25)):
        for cap in (0, 7, 100):
            _run(marg, 32, cap, 100, cost, prefix)


def _softmax_rows(rng, shape, sigma):
    lg = rng.normal(0, sigma, size=shape)
    m = np.exp(lg - lg.max(-1, keepdims=True))
    return (m / m.sum(-1, keepdims=True)).astype(np.float32)


@pytest.mark.parametrize("sigma", [5.0, 12.0])
def test_peaked_drafter(sigma):
    """Confident drafter distributions (top-1 probability 0.4-0.8): deep trees
    whose levels re-merge many nodes, fixed and adaptive budgets, both
    frontier capacities."""
    rng = np.random.default_rng(int(sigma))
    marg = _softmax_rows(rng, (4, 16, 5000), sigma)
    for top_k, cap in ((32, 32), (128, 128), (4, 128), (8, 64)):
        _run(marg, top_k, cap, 128)
    prefix = rng.integers(0, 50000, size=4).astype(np.int32)
    cost = Cost(a=1.0, b=0.002, c=1e-5, e=1e-7, c_d=0.5)
    for top_k, cap in ((32, 32), (128, 128), (4, 100)):
        _run(marg, top_k, cap, 128, cost, prefix)


@pytest.mark.parametrize("case", range(24))
def test_random_shapes(case):
    """Seeded mix of shapes around the selection paths' boundaries: list
    lengths on both sides of the batched merge (8 / 9), caps around 64 and
    not multiples of the list length, one position, deep lists, flat and
    peaked marginals, fixed and adaptive budgets."""
    rng = np.random.default_rng(1000 + case)
    gamma = int(rng.choice([1, 2, 5, 9, 16, 24]))
    top_k = int(rng.choice([1, 2, 3, 7, 8, 9, 16, 33, 64]))
    V = int(rng.choice([top_k, 97, 2000]))
    V = max(V, top_k)
    cap = int(rng.choice([1, 5, 31, 63, 64, 65, 100, 128]))
    sigma = float(rng.choice([0.5, 3.0, 9.0]))
    marg = _softmax_rows(rng, (3, gamma, V), sigma)
    if case % 3 == 2:
        cost = Cost(a=1.0, b=float(rng.choice([1e-6, 1e-3, 0.02])), c=1e-5, e=1e-7, c_d=0.5)
        prefix = rng.integers(0, 40000, size=3).astype(np.int32)
        _run(marg, top_k, cap, 128, cost, prefix)
    else:
        _run(marg, top_k, cap, 128)


def test_adaptive_scores_below_exact_range():
    """Near-uniform marginals over a large vocabulary: depth-2 scores fall
    below 2^-23, so the throughput sums past them are taken one at a time;
    a nearly flat cost keeps the stop rule from ending early."""
    rng = np.random.default_rng(17)
    marg = _softmax_rows(rng, (3, 8, 60000), 0.05)
    prefix = np.array([10, 2000, 40000], np.int32)
    for cost in (Cost(a=1.0, b=1e-12, c=0.0, e=0.0, c_d=0.5),
                 Cost(a=1.0, b=1e-9, c=0.0, e=0.0, c_d=0.5)):
        for top_k, cap in ((4, 128), (16, 40), (128, 128)):
            _run(marg, top_k, cap, 128, cost, prefix)


def test_exact_zero_gain_stops():
    """(1 + 0.5) / (1 + 0.5) equals 1 / 1 exactly: the first node is not added."""
    marg = np.zeros((1, 2, 8), dtype=np.float32)
    marg[0, 0, 3] = 0.5
    marg[0, 1, 1] = 0.25
    cost = Cost(a=0.75, b=0.5, c=0.0, e=0.0, c_d=0.25)
    g, trees = _run(marg, 2, 4, 4, cost, [0])
    assert trees[0].n == 0 and int(g["n_nodes"][0]) == 0


def test_chain_and_small_shapes():
    rng = np.random.default_rng(9)
    marg = rng.dirichlet(np.ones(50), size=(4, 7)).astype(np.float32)
    _run(marg, 1, 5, 8)      # linear: top-1 chain
    _run(marg, 1, 8, 8)      # budget above the 7 candidates
    _run(marg[:, :1], 3, 3, 3)
    _run(marg, 50, 1, 1)     # k = V


def test_invalid_arguments_return_status():
    m = torch.zeros((1, 2, 8), dtype=torch.float32, device=DEV)
    with pytest.raises(tsv.TsvError) as e:
        tsv.build_tree(m, 9, 2, 4)       # k > V
    assert e.value.code == -1
    with pytest.raises(tsv.TsvError):
        tsv.build_tree(m, 2, 5, 4)       # budget > N_max
    with pytest.raises(tsv.TsvError) as e:
        tsv.build_tree(m, 2, 2, 129)     # N_max > 128
    assert e.value.code in (-1, -2)
    ws = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(tsv.TsvError) as e:
        tsv.build_tree(m, 2, 2, 4, ws=ws)
    assert e.value.code == -3


@pytest.mark.parametrize("adaptive", [False, True])
def test_contract_call_matches_variants(adaptive):
    """build_tree called with the boundary's exact argument list (18 arguments,
    the 40-byte cost struct) gives the oracle's trees, bit-identical to
    build_tree_topk and to build_tree_fitted with f = 0."""
    import ctypes
    rng = np.random.default_rng(31)
    B, gamma, V, top_k, cap, N_max = 5, 9, 4000, 24, 48, 64
    lg = rng.normal(0, 2, size=(B, gamma, V)) / rng.uniform(0.4, 1.5, size=(B, 1, 1))
    marg = np.exp(lg - lg.max(-1, keepdims=True))
    marg = (marg / marg.sum(-1, keepdims=True)).astype(np.float32)
    prefix = rng.integers(1000, 30000, size=B).astype(np.int32)
    cost = Cost(a=1.0, b=0.02, c=1e-4, e=1e-6, c_d=0.5) if adaptive else None
    m = torch.from_numpy(marg).to(DEV)
    pl = torch.from_numpy(prefix).to(DEV)
    L = tsv.lib()
    outs = tsv._lib._tree_outputs(B, N_max, m.device)
    for t in outs.values():
        t.fill_(0x5A)                          # every element must be overwritten
    ws = tsv.workspace(tsv.workspace_size(tsv._lib.WS_BUILD, B, gamma, V, top_k, N_max), DEV)
    c = tsv.tsv_cost(cost.a, cost.b, cost.c, cost.e, cost.c_d) if adaptive else None
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = L.build_tree(P(m), B, gamma, V, top_k, cap, ctypes.byref(c) if adaptive else None,
                      P(pl) if adaptive else None, N_max, P(outs["n_nodes"]), P(outs["parent"]),
                      P(outs["token"]), P(outs["depth"]), P(outs["score"]), P(outs["anc_bits"]),
                      P(ws), ws.numel(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0
    g_topk = tsv.build_tree_topk(m, top_k, cap, N_max, cost=cost, prefix_len=pl if adaptive else None)
    fitted = None if cost is None else dataclasses.replace(cost, f=0.0)
    g_fit = tsv.build_tree_fitted(m, top_k, cap, N_max, cost=fitted,
                                  prefix_len=pl if adaptive else None)
    torch.cuda.synchronize()
    idx, p, trees = oracle_trees(marg, top_k, cap, N_max, cost, prefix if adaptive else None)
    assert_tree_equal(g_topk, idx, p, trees)
    assert_tree_equal(outs, idx, p, trees, check_topk=False)
    for k in outs:
        assert torch.equal(outs[k], g_topk[k]), k
        assert torch.equal(outs[k], g_fit[k]), k


@pytest.mark.parametrize("top_k", [1, 2, 4, 8, 6])
def test_short_lists_deep_trees(top_k):
    """Short per-position lists (the batched level merge: list lengths that
    are powers of two take the rank-by-rank layout, 6 the full sort) in deep
    trees, with quantised scores (equal children of different parents) and
    flat and peaked marginals, capacities below, at and past 64."""
    rng = np.random.default_rng(300 + top_k)
    for sigma in (0.5, 3.0, 9.0):
        marg = _softmax_rows(rng, (3, 16, 211), sigma)
        for cap in (16, 64, 65, 128):
            _run(marg, top_k, cap, 128)
    marg = _quantised(rng, (3, 16, 211), 3)
    for cap in (40, 128):
        _run(marg, top_k, cap, 128)
