"""Pins of the oracle's per-chain compressed state (CPU only).

The stand-in compression (block means over c tokens, the incomplete block
kept as a running sum) is checked against what its definition fixes
independently of the oracle's incremental steps: block means of the whole
sequence computed from scratch by a reshape, closed forms (c = 1, c longer
than the sequence, conservation of the sum), the review's toy (accepting A-C
commits only that chain's blocks), and chained rounds whose committed state
must equal a from-scratch compression of the committed sequence."""

import json
import os

import numpy as np
import pytest

from oracle import (block_state, chain_entries, compress_chains, refresh_compressed,
                    select_tree, topk_per_position, unfold_chains)
from tests.conftest import GOLDEN


def scratch(rows, c):
    """Block means and tail straight from numpy, for the pins."""
    L = rows.shape[0]
    k = L // c
    ent = rows[:k * c].reshape(k, c, rows.shape[1]).mean(axis=1)
    return ent, rows[k * c:].sum(axis=0)


def test_block_state_closed_forms():
    rng = np.random.default_rng(0)
    rows = rng.standard_normal((11, 5))
    ent, tail = block_state(rows, 1)
    assert np.allclose(ent, rows) and np.allclose(tail, 0)
    ent, tail = block_state(rows, 16)
    assert ent.shape == (0, 5) and np.allclose(tail, rows.sum(axis=0))
    ent, tail = block_state(rows, 4)
    assert ent.shape == (2, 5)
    assert np.allclose(ent[1], rows[4:8].mean(axis=0))
    assert np.allclose(ent.sum(axis=0) * 4 + tail, rows.sum(axis=0))


@pytest.mark.parametrize("c", [1, 2, 4, 7, 128])
def test_chain_entries_equal_from_scratch(c):
    rng = np.random.default_rng(c)
    for l in (0, 1, c - 1, c, 3 * c + 2, 130):
        if l < 0:
            continue
        for m in (0, 1, 2, 5, 17, 64):
            P = rng.standard_normal((l, 3))
            C = rng.standard_normal((m, 3))
            _, tail = block_state(P, c)
            ent, s = chain_entries(tail, l, list(C), c)
            full_ent, full_tail = scratch(np.concatenate([P, C]), c)
            assert ent.shape[0] == full_ent.shape[0] - l // c
            assert np.allclose(ent, full_ent[l // c:], atol=1e-12)
            assert np.allclose(s, full_tail, atol=1e-12)


def random_tree(rng, n):
    parent = np.full(n, -1, dtype=np.int32)
    for i in range(1, n):
        parent[i] = rng.integers(-1, i)
    return parent


def path_to(parent, node):
    p = []
    while node >= 0:
        p.append(int(node))
        node = parent[node]
    return p[::-1]


@pytest.mark.parametrize("c", [1, 4, 5, 128])
def test_refresh_equals_from_scratch_over_rounds(c):
    rng = np.random.default_rng(10 + c)
    B, N, E, gamma, cap = 3, 12, 4, 12, 64
    hist = [rng.standard_normal((int(rng.integers(0, 9)), E)) for _ in range(B)]
    l = np.array([h.shape[0] for h in hist], dtype=np.int64)
    comp = np.zeros((B, cap, E))
    tail = np.zeros((B, E))
    for b in range(B):
        ent, t = block_state(hist[b], c)
        comp[b, :len(ent)] = ent
        tail[b] = t
    for _ in range(4):
        rows = rng.standard_normal((B, N, E))
        n_chains = np.zeros(B, dtype=np.int32)
        chain_len = np.zeros((B, N), dtype=np.int32)
        chain_nodes = np.full((B, N, gamma), -1, dtype=np.int32)
        m = np.zeros(B, dtype=np.int32)
        acc = np.full((B, gamma), -1, dtype=np.int32)
        paths = []
        for b in range(B):
            n = int(rng.integers(1, N + 1))
            parent = random_tree(rng, n)
            cnt, ln, nd = unfold_chains(parent, n, gamma)
            n_chains[b] = cnt
            chain_len[b, :cnt] = ln
            chain_nodes[b, :cnt] = nd
            path = path_to(parent, int(rng.integers(0, n)))[:int(rng.integers(0, gamma + 1))]
            m[b] = len(path)
            acc[b, :len(path)] = path
            paths.append(path)
        entries, n_ent = compress_chains(rows, tail, l, n_chains, chain_len, chain_nodes, c, gamma)
        assert np.all(n_ent[np.arange(N)[None, :] < n_chains[:, None]] >= 0)
        comp, tail, status = refresh_compressed(rows, l, m, acc, n_chains, chain_len, chain_nodes,
                                                entries, comp, tail, c, gamma)
        assert np.all(status == 0)
        for b in range(B):
            hist[b] = np.concatenate([hist[b], rows[b, paths[b]].reshape(-1, E)])
            l[b] += m[b]
            full_ent, full_tail = scratch(hist[b], c)
            assert np.allclose(comp[b, :len(full_ent)], full_ent, atol=1e-12)
            assert np.allclose(tail[b], full_tail, atol=1e-12)
            assert np.all(comp[b, len(full_ent):] == 0)


def test_toy_commits_only_the_accepted_chain():
    """The review's toy: prefix A, kept A-B, A-C, A-B-B; A-C is accepted, so
    only Chain2's compressed block reaches the persistent state (c = 2: the
    block closed by C is the mean of A and C, with nothing of B)."""
    g = json.load(open(os.path.join(GOLDEN, "toy_tree.json")))
    V = {t: i for i, t in enumerate(g["vocab"])}
    idx, p = topk_per_position(np.array(g["marginals"], dtype=np.float32), g["top_k"])
    tree = select_tree(idx, p, g["budget"], 8)
    gamma = g["gamma"]
    cnt, ln, nd = unfold_chains(tree.parent, tree.n, gamma)
    onehot = np.eye(3)
    rows = np.zeros((1, 8, 3))
    for i in range(tree.n):
        rows[0, i] = onehot[int(tree.token[i])]
    prefix = np.array([onehot[V[t]] for t in g["prefix"]])
    c = 2
    _, tail = block_state(prefix, c)
    n_chains = np.array([cnt], dtype=np.int32)
    chain_len = np.zeros((1, 8), dtype=np.int32)
    chain_len[0, :cnt] = ln
    chain_nodes = np.full((1, 8, gamma), -1, dtype=np.int32)
    chain_nodes[0, :cnt] = nd
    l = np.array([len(g["prefix"])])
    entries, n_ent = compress_chains(rows, tail[None], l, n_chains, chain_len, chain_nodes, c, gamma)
    # both chains close one block at their first node: (A + B)/2 and (A + C)/2
    firsts = sorted(tuple(entries[0, q, 0]) for q in range(cnt))
    assert firsts == sorted([(0.5, 0.5, 0.0), (0.5, 0.0, 0.5)])
    c_node = next(i for i in range(tree.n) if int(tree.token[i]) == V["C"] and tree.parent[i] < 0)
    acc = np.full((1, gamma), -1, dtype=np.int32)
    acc[0, 0] = c_node
    comp, tail2, status = refresh_compressed(rows, l, np.array([1]), acc, n_chains, chain_len,
                                             chain_nodes, entries, np.zeros((1, 4, 3)), tail[None],
                                             c, gamma)
    assert status[0] == 0
    assert np.allclose(comp[0, 0], [0.5, 0.0, 0.5]) and np.allclose(comp[0, 1:], 0)
    assert np.allclose(tail2[0], 0)
    # the next prefix is A-C: its from-scratch state is the same
    ent, t = block_state(np.array([onehot[V[x]] for x in g["next_prefix"]]), c)
    assert np.allclose(comp[0, :1], ent) and np.allclose(tail2[0], t)


def test_refresh_status_cases():
    B, N, E, gamma, c = 4, 4, 2, 3, 2
    rows = np.ones((B, N, E))
    n_chains = np.array([1, 1, 1, 1], dtype=np.int32)
    chain_len = np.zeros((B, N), dtype=np.int32)
    chain_len[:, 0] = 2
    chain_nodes = np.full((B, N, gamma), -1, dtype=np.int32)
    chain_nodes[:, 0, :2] = [0, 1]
    tail = np.zeros((B, E))
    l = np.array([0, 0, 0, 9])
    entries, _ = compress_chains(rows, tail, l, n_chains, chain_len, chain_nodes, c, gamma)
    m = np.array([4, 2, 1, 2], dtype=np.int32)         # 4 > gamma
    acc = np.full((B, gamma), -1, dtype=np.int32)
    acc[:, :2] = [0, 1]
    acc[2, 0] = 1                                      # node 1 is not a chain's first node
    comp0 = np.full((B, 4, E), 9.0)
    comp, tail2, status = refresh_compressed(rows, l, m, acc, n_chains, chain_len, chain_nodes,
                                             entries, comp0, tail, c, gamma)
    assert list(status) == [2, 0, 2, 1]                # request 3: 9 // 2 + 1 > 4 entries
    assert np.allclose(comp[1, 0], 1.0) and np.allclose(comp[1, 1:], 9.0)
    for b in (0, 2, 3):
        assert np.allclose(comp[b], 9.0) and np.allclose(tail2[b], 0)


def test_compress_marks_unreadable_chains():
    rows = np.ones((2, 4, 1))
    chain_len = np.array([[2, 0, 0, 0], [1, 0, 0, 0]], dtype=np.int32)
    chain_nodes = np.full((2, 4, 3), -1, dtype=np.int32)
    chain_nodes[0, 0, :2] = [0, 5]                     # node 5 >= N_max
    chain_nodes[1, 0, 0] = 0
    entries, n_ent = compress_chains(rows, np.zeros((2, 1)), np.array([0, -1]),
                                     np.array([1, 1]), chain_len, chain_nodes, 1, 3)
    assert n_ent[0, 0] == -1 and n_ent[1, 0] == -1 and np.all(n_ent[:, 1:] == 0)
