"""Pins of the oracle's tree attention against torch SDPA and closed forms
(CPU only)."""

import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import attend_node, attend_request
from oracle.attention import latent_as_heads
from tests.conftest import GOLDEN


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa(q, K, V, mask, scale):
    """torch SDPA in fp64 on CPU.  q [Hq, rows, d], K/V [Hq, keys, d]."""
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).double()
    m = None if mask is None else torch.from_numpy(mask)
    return F.scaled_dot_product_attention(t(q), t(K), t(V), attn_mask=m,
                                          scale=scale).numpy()


def _expand(kv, Hq):
    """[keys, Hkv, d] -> [Hq, keys, d] with head h using KV head h // G."""
    G = Hq // kv.shape[1]
    return np.repeat(kv.transpose(1, 0, 2), G, axis=0)


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (6, 1)])
def test_chain_equals_causal_attention(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    l, n, d, dv = 37, 9, 16, 12
    q = _rand(rng, n, Hq, d)
    kp, vp = _rand(rng, l, Hkv, d), _rand(rng, l, Hkv, dv)
    kt, vt = _rand(rng, n, Hkv, d), _rand(rng, n, Hkv, dv)
    parent = np.arange(-1, n - 1)
    scale = 0.31
    outs, _ = attend_request(q, kp, vp, kt, vt, l, n, parent, scale)
    K = _expand(np.concatenate([kp, kt]), Hq)
    V = _expand(np.concatenate([vp, vt]), Hq)
    mask = np.ones((n, l + n), dtype=bool)
    mask[:, l:] = np.tril(np.ones((n, n), dtype=bool))
    ref = _sdpa(q.transpose(1, 0, 2), K, V, mask, scale)   # [Hq, n, dv]
    for i in range(n):
        np.testing.assert_allclose(outs[i], ref[:, i], rtol=0, atol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_each_node_equals_attention_over_its_path(seed):
    rng = np.random.default_rng(seed)
    Hq, Hkv, l, n, d = 4, 2, 20, 12, 8
    parent = np.full(n, -1)
    for i in range(1, n):
        parent[i] = rng.integers(-1, i)
    q = _rand(rng, n, Hq, d)
    kp, vp = _rand(rng, l, Hkv, d), _rand(rng, l, Hkv, d)
    kt, vt = _rand(rng, n, Hkv, d), _rand(rng, n, Hkv, d)
    outs, lses = attend_request(q, kp, vp, kt, vt, l, n, parent, 0.5)
    for i in range(n):
        path, j = [], i
        while j >= 0:
            path.append(j)
            j = parent[j]
        K = np.concatenate([kp, kt[path[::-1]]])
        V = np.concatenate([vp, vt[path[::-1]]])
        ref = _sdpa(q[i][:, None, :], _expand(K, Hq), _expand(V, Hq), None, 0.5)
        np.testing.assert_allclose(outs[i], ref[:, 0], rtol=0, atol=1e-12)
        # lse from the definition with a library logsumexp
        s = 0.5 * np.einsum("hd,hkd->hk", q[i], _expand(K, Hq))
        np.testing.assert_allclose(lses[i], torch.logsumexp(torch.from_numpy(s), -1).numpy(),
                                   rtol=0, atol=1e-12)


def test_toy_visibility_and_sibling_isolation():
    """A-B-B attends to A (prefix) and A-B; A-C only to A: perturbing any
    non-ancestor scratch row leaves a node's output unchanged, perturbing an
    ancestor changes it."""
    g = json.load(open(os.path.join(GOLDEN, "toy_tree.json")))
    # best-first numbering of the kept nodes: 0 = A-B, 1 = A-B-B, 2 = A-C
    parent = np.array([-1, 0, -1])
    rng = np.random.default_rng(7)
    H, d = 2, 8
    q = _rand(rng, 3, H, d)
    kp, vp = _rand(rng, 1, H, d), _rand(rng, 1, H, d)    # the prefix is "A"
    kt, vt = _rand(rng, 3, H, d), _rand(rng, 3, H, d)
    base, _ = attend_request(q, kp, vp, kt, vt, 1, 3, parent, 0.4)
    sees = {1: {0, 1}, 2: {2}, 0: {0}}
    assert len(g["kept_paths"]) == 3
    for j in range(3):
        kt2, vt2 = kt.copy(), vt.copy()
        kt2[j] += 3.0
        vt2[j] -= 2.0
        pert, _ = attend_request(q, kp, vp, kt2, vt2, 1, 3, parent, 0.4)
        for i in range(3):
            same = np.array_equal(pert[i], base[i])
            assert same == (j not in sees[i])


def test_closed_forms():
    rng = np.random.default_rng(3)
    H, d = 3, 5
    q = _rand(rng, 1, H, d)
    kt, vt = _rand(rng, 1, H, d), _rand(rng, 1, H, d)
    empty = np.zeros((0, H, d))
    out, lse = attend_node(q[0], empty, empty, kt, vt, [-1], 0, 0.7)
    np.testing.assert_array_equal(out, vt[0])           # one key: its value row
    np.testing.assert_allclose(lse, 0.7 * np.sum(q[0] * kt[0], -1), rtol=0, atol=1e-14)
    # identical keys: uniform weights, output = mean of the values
    kp = np.repeat(kt, 6, axis=0)
    vp = _rand(rng, 6, H, d)
    out, lse = attend_node(q[0], kp, vp, kt, vt, [-1], 0, 0.7)
    np.testing.assert_allclose(out, np.concatenate([vp, vt]).mean(0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, 0.7 * np.sum(q[0] * kt[0], -1) + np.log(7.0),
                               rtol=0, atol=1e-13)


def test_latent_layout():
    """A latent row serves as the key (all columns) and, truncated, as the
    value; same as SDPA with V = K[:, :d_v]."""
    rng = np.random.default_rng(11)
    Hq, l, n, dqk, dv = 4, 15, 3, 10, 6
    lat = _rand(rng, l, dqk)
    latt = _rand(rng, n, dqk)
    kp, vp = latent_as_heads(lat, dv)
    kt, vt = latent_as_heads(latt, dv)
    q = _rand(rng, n, Hq, dqk)
    parent = np.array([-1, 0, 0])
    outs, _ = attend_request(q, kp, vp, kt, vt, l, n, parent, 0.2)
    for i in range(n):
        path = [0, i] if i else [0]
        K = np.concatenate([lat, latt[path]])
        ref = _sdpa(q[i][:, None, :], np.repeat(K[None], Hq, 0),
                    np.repeat(K[None, :, :dv], Hq, 0), None, 0.2)
        np.testing.assert_allclose(outs[i], ref[:, 0], rtol=0, atol=1e-12)
