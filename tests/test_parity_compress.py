"""compress_chains and refresh_compressed on the GPU vs the oracle.

Counts, statuses and untouched memory are compared exactly; compressed
entries and tails are fp32 sums in sequence order on the GPU and fp64 in the
oracle, so each element is held to the forward-error bound of a recursive
fp32 sum: (terms + 1) * 2^-24 * (sum of the magnitudes of its terms), the
magnitudes taken from the oracle run on |inputs| (entries divide both sides
by c).  Copied entries must equal the GPU's own compress_chains output bit
for bit.  Cases: the grouped workload's trees (keys of 8 KV heads x 128),
random trees with ragged chains, c = 1, 4, 5, 128, bf16 and fp32 rows,
column counts that leave ragged workgroup slices, empty trees, chained
rounds against from-scratch block means of the committed sequence, and the
malformed-input statuses."""

import numpy as np
import pytest
import torch

import oracle
import tree_structured_verification_amd as tsv
from tests._helpers import DEV
from workloads import config, marginals

pytestmark = pytest.mark.gpu

U = 2.0 ** -24


def random_parents(rng, B, N, sizes):
    parent = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        for i in range(1, sizes[b]):
            parent[b, i] = rng.integers(-1, i)
    return parent


def path_to(parent, node):
    p = []
    while node >= 0:
        p.append(int(node))
        node = int(parent[node])
    return p[::-1]


def chains_of(n_nodes, parent, gamma):
    tree = dict(n_nodes=torch.from_numpy(np.asarray(n_nodes, np.int32)).to(DEV),
                parent=torch.from_numpy(np.ascontiguousarray(parent, np.int32)).to(DEV))
    ch = tsv.unfold_chains(tree, gamma)
    return ch, {k: v.cpu().numpy() for k, v in ch.items()}


def bound(abs_val, terms):
    return (terms + 1) * U * abs_val + 1e-30


def run_case(rng, B, N, E, stride, gamma, c, dtype, sizes=None, parent=None, l=None, Lc_cap=None):
    if sizes is None:
        sizes = rng.integers(0, N + 1, B)
    if parent is None:
        parent = random_parents(rng, B, N, sizes)
    ch, chn = chains_of(sizes, parent, gamma)
    rows = torch.randn(B, N, stride, generator=torch.Generator().manual_seed(int(rng.integers(1 << 30)))).to(dtype)
    rows_np = rows.float().numpy()[:, :, :E].astype(np.float64)
    rows_d = rows.to(DEV)
    if l is None:
        l = rng.integers(0, 3 * c + 5, B).astype(np.int32)
    tail = rng.standard_normal((B, E)).astype(np.float32)
    pl = torch.from_numpy(np.asarray(l, np.int32)).to(DEV)
    tail_d = torch.from_numpy(tail).to(DEV)
    ent, n_ent = tsv.compress_chains(rows_d, c, tail_d, pl, ch, gamma, E=E)
    torch.cuda.synchronize()
    ent_np, n_ent_np = ent.cpu().numpy(), n_ent.cpu().numpy()
    o_ent, o_n = oracle.compress_chains(rows_np, tail, l, chn["n_chains"], chn["chain_len"],
                                        chn["chain_nodes"], c, gamma)
    a_ent, _ = oracle.compress_chains(np.abs(rows_np), np.abs(tail), l, chn["n_chains"],
                                      chn["chain_len"], chn["chain_nodes"], c, gamma)
    assert np.array_equal(n_ent_np, o_n)
    for b in range(B):
        for q in range(int(chn["n_chains"][b])):
            k = int(o_n[b, q])
            err = np.abs(ent_np[b, q, :k] - o_ent[b, q, :k])
            assert np.all(err <= bound(a_ent[b, q, :k], c + 1)), (b, q, float(err.max()))
    # refresh along a random accepted path of every request
    m = np.zeros(B, dtype=np.int32)
    acc = np.full((B, gamma), -1, dtype=np.int32)
    for b in range(B):
        if sizes[b] > 0:
            p = path_to(parent[b], int(rng.integers(0, sizes[b])))[:int(rng.integers(0, gamma + 1))]
            m[b] = len(p)
            acc[b, :len(p)] = p
    if Lc_cap is None:
        Lc_cap = int(max(l) // c + gamma + 2)
    comp0 = rng.standard_normal((B, Lc_cap, E)).astype(np.float32)
    comp_d = torch.from_numpy(comp0).to(DEV)
    tail2_d = tail_d.clone()
    walk = dict(accept_len=torch.from_numpy(m).to(DEV), accept_nodes=torch.from_numpy(acc).to(DEV))
    st = tsv.refresh_compressed(rows_d, c, pl, walk, ch, ent, comp_d, tail2_d, gamma, E=E)
    torch.cuda.synchronize()
    st_np, comp_np, tail_np = st.cpu().numpy(), comp_d.cpu().numpy(), tail2_d.cpu().numpy()
    o_comp, o_tail, o_st = oracle.refresh_compressed(rows_np, l, m, acc, chn["n_chains"],
                                                     chn["chain_len"], chn["chain_nodes"], o_ent,
                                                     comp0, tail, c, gamma)
    _, a_tail, _ = oracle.refresh_compressed(np.abs(rows_np), l, m, acc, chn["n_chains"],
                                             chn["chain_len"], chn["chain_nodes"], a_ent,
                                             np.abs(comp0), np.abs(tail), c, gamma)
    assert np.array_equal(st_np, o_st)
    for b in range(B):
        if o_st[b] != 0 or m[b] == 0:
            assert np.array_equal(comp_np[b], comp0[b]) and np.array_equal(tail_np[b], tail[b]), b
            continue
        e = (int(l[b]) % c + int(m[b])) // c
        lo = int(l[b]) // c
        q = next(q for q in range(int(chn["n_chains"][b]))
                 if chn["chain_len"][b, q] >= m[b] and chn["chain_nodes"][b, q, m[b] - 1] == acc[b, m[b] - 1])
        assert np.array_equal(comp_np[b, lo:lo + e], ent_np[b, q, :e]), b
        assert np.array_equal(comp_np[b, :lo], comp0[b, :lo]), b
        assert np.array_equal(comp_np[b, lo + e:], comp0[b, lo + e:]), b
        err = np.abs(tail_np[b] - o_tail[b])
        assert np.all(err <= bound(a_tail[b], gamma + c + 1)), (b, float(err.max()))
    return st_np


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("c", [1, 4, 5, 128])
def test_random_trees(dtype, c):
    rng = np.random.default_rng(c * 7 + (dtype == torch.float32))
    run_case(rng, B=6, N=24, E=300, stride=320, gamma=16, c=c, dtype=dtype)


@pytest.mark.parametrize("E", [1, 1024, 1025, 2500])
def test_ragged_columns(E):
    rng = np.random.default_rng(E)
    run_case(rng, B=3, N=10, E=E, stride=E + 8, gamma=10, c=4, dtype=torch.bfloat16)


@pytest.mark.parametrize("c", [4, 128])
def test_grouped_workload_trees(c):
    """Trees built by build_tree on the grouped workload's marginals; the
    compressed rows are keys of 8 KV heads x 128 (1024 columns, bf16)."""
    cfg = config(2)
    tree = tsv.build_tree(marginals(cfg, 0, DEV), cfg.top_k, cfg.n_budget, cfg.N_max)
    n = tree["n_nodes"].cpu().numpy()
    parent = tree["parent"].cpu().numpy()
    rng = np.random.default_rng(c)
    l = rng.integers(1024, 4097, cfg.B).astype(np.int32)
    run_case(rng, B=cfg.B, N=cfg.N_max, E=cfg.Hkv * cfg.d_qk, stride=cfg.kv_stride, gamma=cfg.gamma,
             c=c, dtype=torch.bfloat16, sizes=n, parent=parent, l=l)


def test_empty_trees_and_zero_accept():
    rng = np.random.default_rng(5)
    st = run_case(rng, B=4, N=8, E=64, stride=64, gamma=8, c=4, dtype=torch.float32,
                  sizes=np.zeros(4, dtype=np.int64))
    assert np.all(st == 0)


def test_capacity_status():
    rng = np.random.default_rng(6)
    B, N = 8, 6
    sizes = np.full(B, N)
    parent = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))   # one chain of N nodes
    # l // c = 3 entries are held and the capacity is 3; l % c = 1, so the
    # first accepted token closes a block, which overflows
    st = run_case(rng, B=B, N=N, E=40, stride=40, gamma=N, c=2, dtype=torch.float32, sizes=sizes,
                  parent=parent, l=np.full(B, 7, np.int32), Lc_cap=3)
    assert np.any(st == 1)


def test_malformed_inputs():
    """Negative prefix lengths and accepted paths no chain holds give status
    2 and leave everything untouched; chains naming a node outside the tree
    are marked -1."""
    B, N, E, gamma, c = 3, 4, 16, 4, 2
    rows = torch.ones(B, N, E, device=DEV)
    ch = dict(n_chains=torch.tensor([1, 1, 1], dtype=torch.int32, device=DEV),
              chain_len=torch.tensor([[2, 0, 0, 0]] * 3, dtype=torch.int32, device=DEV),
              chain_nodes=torch.tensor([[[0, 1, -1, -1]] + [[-1] * 4] * 3,
                                        [[0, 9, -1, -1]] + [[-1] * 4] * 3,
                                        [[0, 1, -1, -1]] + [[-1] * 4] * 3],
                                       dtype=torch.int32, device=DEV))
    pl = torch.tensor([0, 0, -3], dtype=torch.int32, device=DEV)
    tail = torch.zeros(B, E, device=DEV)
    ent, n_ent = tsv.compress_chains(rows, c, tail, pl, ch, gamma)
    torch.cuda.synchronize()
    assert n_ent[:, 0].cpu().tolist() == [1, -1, -1]
    walk = dict(accept_len=torch.tensor([1, 5, 1], dtype=torch.int32, device=DEV),
                accept_nodes=torch.tensor([[1, -1, -1, -1], [0, 1, 2, 3], [0, -1, -1, -1]],
                                          dtype=torch.int32, device=DEV))
    comp = torch.full((B, 4, E), 7.0, device=DEV)
    st = tsv.refresh_compressed(rows, c, pl, walk, ch, ent, comp, tail, gamma)
    torch.cuda.synchronize()
    assert st.cpu().tolist() == [2, 2, 2]
    assert torch.all(comp == 7.0) and torch.all(tail == 0)


def test_rounds_match_from_scratch():
    """Three chained rounds (compress, refresh, then the commit's prefix
    advance) against block means of the whole committed sequence."""
    rng = np.random.default_rng(11)
    B, N, E, gamma, c, cap = 4, 16, 96, 8, 4, 64
    hist = [rng.standard_normal((int(rng.integers(0, 9)), E)).astype(np.float32) for _ in range(B)]
    l = np.array([h.shape[0] for h in hist], dtype=np.int32)
    comp = np.zeros((B, cap, E), np.float32)
    tail = np.zeros((B, E), np.float32)
    for b in range(B):
        ent, t = oracle.block_state(hist[b].astype(np.float64), c)
        comp[b, :len(ent)] = ent
        tail[b] = t
    comp_d, tail_d = torch.from_numpy(comp).to(DEV), torch.from_numpy(tail).to(DEV)
    for _ in range(3):
        sizes = rng.integers(1, N + 1, B)
        parent = random_parents(rng, B, N, sizes)
        ch, chn = chains_of(sizes, parent, gamma)
        rows = torch.from_numpy(rng.standard_normal((B, N, E)).astype(np.float32)).to(DEV)
        pl = torch.from_numpy(l).to(DEV)
        ent, _ = tsv.compress_chains(rows, c, tail_d, pl, ch, gamma)
        m = np.zeros(B, dtype=np.int32)
        acc = np.full((B, gamma), -1, dtype=np.int32)
        for b in range(B):
            p = path_to(parent[b], int(rng.integers(0, sizes[b])))[:gamma]
            m[b] = len(p)
            acc[b, :len(p)] = p
        walk = dict(accept_len=torch.from_numpy(m).to(DEV), accept_nodes=torch.from_numpy(acc).to(DEV))
        st = tsv.refresh_compressed(rows, c, pl, walk, ch, ent, comp_d, tail_d, gamma)
        torch.cuda.synchronize()
        assert np.all(st.cpu().numpy() == 0)
        rn = rows.cpu().numpy()
        for b in range(B):
            hist[b] = np.concatenate([hist[b], rn[b, acc[b, :m[b]]].reshape(-1, E)])
        l = l + m
    cn, tn = comp_d.cpu().numpy(), tail_d.cpu().numpy()
    for b in range(B):
        h = hist[b].astype(np.float64)
        ent, t = oracle.block_state(h, c)
        a_ent, a_t = oracle.block_state(np.abs(h), c)
        # every entry and the tail are sums of at most c + 1 fp32 terms
        assert np.all(np.abs(cn[b, :len(ent)] - ent) <= bound(a_ent, c + 2)), b
        assert np.all(np.abs(tn[b] - t) <= bound(a_t * 1.0, gamma + c + 2)), b


@pytest.mark.parametrize("c", [4, 128])
def test_bench_configuration(c):
    """The configuration bench.py --compressed-state times: the adaptive
    workload's trees at a fixed budget of 128 (64 requests, 7699 chains),
    its prefix lengths, 1024 bf16 columns per row."""
    from workloads import prefix_lengths
    cfg = config(4)
    tree = tsv.build_tree(marginals(cfg, 0, DEV), cfg.top_k, cfg.N_max, cfg.N_max)
    n = tree["n_nodes"].cpu().numpy()
    parent = tree["parent"].cpu().numpy()
    rng = np.random.default_rng(100 + c)
    run_case(rng, B=cfg.B, N=cfg.N_max, E=cfg.Hkv * cfg.d_qk, stride=cfg.kv_stride, gamma=cfg.gamma,
             c=c, dtype=torch.bfloat16, sizes=n, parent=parent, l=prefix_lengths(cfg, 0))
