"""build_tree_noalloc (the library's own per-device scratch, no workspace)
against build_tree with a workspace of the caller's: bit-identical trees on
two calls in a row, the second smaller than the first, so the second runs on
the first one's leftover table contents."""

import numpy as np
import pytest
import torch

import tree_structured_verification_amd as tsv
from tests._helpers import DEV
from workloads import Cost

pytestmark = pytest.mark.gpu


def _marginals(seed, B, gamma, V, spread=3.0):
    rng = np.random.default_rng(seed)
    lg = rng.normal(0, spread, size=(B, gamma, V)) / rng.uniform(0.5, 2.0, size=(B, 1, 1))
    m = np.exp(lg - lg.max(-1, keepdims=True))
    return torch.from_numpy((m / m.sum(-1, keepdims=True)).astype(np.float32)).to(DEV)


def _same(a, b):
    for k in ("n_nodes", "parent", "token", "depth", "anc_bits"):
        assert torch.equal(a[k], b[k]), k
    assert torch.equal(a["score"].view(torch.int32), b["score"].view(torch.int32))


def test_noalloc_matches_build_tree_twice():
    print("build_tree_noalloc: 64 x 16 x top-128 then 3 x 5 x top-8", flush=True)
    # first call: 131072 list entries (1 MiB of the 4 MiB scratch), adaptive budget
    m1 = _marginals(1, 64, 16, 20000)
    pl1 = torch.from_numpy(np.random.default_rng(2).integers(1024, 32769, 64).astype(np.int32)).to(DEV)
    cost = Cost(a=1.0, b=0.02, c=1e-4, e=1e-6, c_d=0.5)
    got1 = tsv.build_tree_noalloc(m1, 128, 128, 128, cost=cost, prefix_len=pl1)
    want1 = tsv.build_tree(m1, 128, 128, 128, cost=cost, prefix_len=pl1)
    torch.cuda.synchronize()
    _same(got1, want1)
    assert int(got1["n_nodes"].sum()) > 0
    # second call, smaller, fixed budget
    m2 = _marginals(3, 3, 5, 5000, spread=2.0)
    got2 = tsv.build_tree_noalloc(m2, 8, 20, 32)
    want2 = tsv.build_tree(m2, 8, 20, 32)
    torch.cuda.synchronize()
    _same(got2, want2)
    assert int(got2["n_nodes"].min()) == 20
    # and once more at the first size: the leftover of the small call is harmless
    got3 = tsv.build_tree_noalloc(m1, 128, 128, 128, cost=cost, prefix_len=pl1)
    torch.cuda.synchronize()
    _same(got3, want1)


def test_noalloc_rejects_tables_above_its_scratch():
    m = torch.zeros((200, 32, 256), dtype=torch.float32, device=DEV)
    with pytest.raises(tsv.TsvError) as e:
        tsv.build_tree_noalloc(m, 128, 8, 8)     # 819200 entries x 8 bytes > 4 MiB
    assert e.value.code == -2
