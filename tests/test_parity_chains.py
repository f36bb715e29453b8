"""unfold_chains on the GPU vs the oracle, bit-exact: the toy, the trees of
every workload, random trees, degenerate shapes and malformed parents."""

import json
import os

import numpy as np
import pytest
import torch

import oracle
import tree_structured_verification_amd as tsv
from tests._helpers import DEV
from tests.conftest import GOLDEN
from workloads import config, marginals, prefix_lengths

pytestmark = pytest.mark.gpu


def _check(n_nodes, parent, gamma, clamp=False):
    B, N = parent.shape
    tree = dict(n_nodes=torch.from_numpy(np.asarray(n_nodes, np.int32)).to(DEV),
                parent=torch.from_numpy(np.ascontiguousarray(parent, np.int32)).to(DEV))
    got = tsv.unfold_chains(tree, gamma)
    torch.cuda.synchronize()
    gc, gl, gn = (got[k].cpu().numpy() for k in ("n_chains", "chain_len", "chain_nodes"))
    for b in range(B):
        n = int(min(max(n_nodes[b], 0), N))
        par = np.array(parent[b, :n], np.int64)
        if clamp:
            par = np.where((par >= 0) & (par < np.arange(n)), par, -1)
        count, lengths, nodes = oracle.unfold_chains(par, n, 64)
        assert gc[b] == count, b
        L = np.minimum(lengths, gamma)
        assert np.array_equal(gl[b, :count], L), b
        assert np.all(gl[b, count:] == 0), b
        for c in range(count):
            assert np.array_equal(gn[b, c, :L[c]], nodes[c, :L[c]]), (b, c)
            assert np.all(gn[b, c, L[c]:] == -1), (b, c)
        assert np.all(gn[b, count:] == -1), b
    return gc


def test_toy_chains():
    g = json.load(open(os.path.join(GOLDEN, "toy_tree.json")))
    m = torch.tensor([g["marginals"]], dtype=torch.float32, device=DEV)
    tree = tsv.build_tree(m, g["top_k"], g["budget"], 8)
    torch.cuda.synchronize()
    got = tsv.unfold_chains(tree, g["gamma"])
    torch.cuda.synchronize()
    V = {t: i for i, t in enumerate(g["vocab"])}
    tok = tree["token"].cpu().numpy()[0]
    cnt = int(got["n_chains"][0])
    lens = got["chain_len"].cpu().numpy()[0]
    nodes = got["chain_nodes"].cpu().numpy()[0]
    chains = sorted(tuple(int(tok[j]) for j in nodes[c, :lens[c]]) for c in range(cnt))
    assert chains == sorted(tuple(V[t] for t in ch) for ch in g["chains"])


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload_trees(cid):
    cfg = config(cid)
    tree = tsv.build_tree(marginals(cfg, 0, DEV), cfg.top_k, cfg.n_budget, cfg.N_max,
                          cost=cfg.cost,
                          prefix_len=(torch.from_numpy(prefix_lengths(cfg)).to(DEV)
                                      if cfg.cost is not None else None))
    torch.cuda.synchronize()
    _check(tree["n_nodes"].cpu().numpy(), tree["parent"].cpu().numpy(), cfg.gamma)


@pytest.mark.parametrize("N", [1, 7, 64, 65, 128])
def test_random_and_degenerate_trees(N):
    rng = np.random.default_rng(N)
    B = 9
    parent = np.full((B, N), -1, np.int32)
    n_nodes = rng.integers(0, N + 1, size=B)
    n_nodes[0], n_nodes[1] = N, 0
    for b in range(2, B):
        for i in range(1, N):
            parent[b, i] = rng.integers(-1, i)
    parent[3, :] = np.arange(-1, N - 1)            # one chain through every node
    gc = _check(n_nodes, parent, 64)
    assert gc[0] == N and gc[1] == 0               # star; empty


def test_truncation_and_malformed_parents():
    N = 32
    chain = np.arange(-1, N - 1)[None].astype(np.int32)
    _check([N], chain, 8)                          # depth 32 > gamma 8: first 8 nodes kept
    rng = np.random.default_rng(4)
    bad = rng.integers(-40, 80, size=(4, N)).astype(np.int32)
    _check([N, 5, 0, 200], bad, 16, clamp=True)
