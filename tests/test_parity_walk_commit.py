"""accept_walk and commit_path on the GPU vs the oracle (bit-exact), and
chained rounds on all five workloads."""

import numpy as np
import pytest
import torch

import oracle
import tree_structured_verification_amd as tsv
from tests._helpers import DEV, TOL, assert_tree_equal, check_attention, np32, oracle_trees, stack_trees
from workloads import attention_inputs, config, marginals, target_logits

pytestmark = pytest.mark.gpu


def _dev_tree(st):
    return {k: torch.from_numpy(np.ascontiguousarray(v).view(np.int32)
                                if v.dtype == np.uint32 else np.ascontiguousarray(v)).to(DEV)
            for k, v in st.items()}


def _check_walk(g, logits_np, trees, gamma):
    al = g["accept_len"].cpu().numpy()
    an = g["accept_nodes"].cpu().numpy()
    ot = g["out_tokens"].cpu().numpy()
    for b, t in enumerate(trees):
        m, nodes, toks = oracle.accept_walk(logits_np[b], t.n, t.parent, t.token, gamma)
        assert al[b] == m, (b, al[b], m)
        assert np.array_equal(an[b], nodes), b
        assert np.array_equal(ot[b], toks), b


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("V", [37, 4096, 50001])
def test_walk_small(dtype, V):
    rng = np.random.default_rng(V)
    B, gamma, k, N_max = 5, 6, 3, 24
    marg = rng.dirichlet(np.ones(min(V, 12)) * 0.5, size=(B, gamma)).astype(np.float32)
    marg = np.concatenate([marg, np.zeros((B, gamma, V - marg.shape[-1]), np.float32)], -1)
    budgets = [24, 0, 1, 13, 24]
    trees = []
    for b in range(B):
        idx, p = oracle.topk_per_position(marg[b:b + 1], k)
        trees.append(oracle.select_tree(idx[0], p[0], budgets[b], N_max))
    # target rows: mostly agree with the drafted tokens so long paths occur;
    # integer-valued logits force argmax ties (lowest id must win)
    lg = rng.integers(-4, 4, size=(B, 1 + N_max, V)).astype(np.float32)
    for b, t in enumerate(trees):
        for r in range(1 + t.n):
            kids = [j for j in range(t.n) if t.parent[j] == r - 1]
            if kids and rng.random() < 0.8:
                lg[b, r, t.token[kids[rng.integers(len(kids))]]] = 6.0
            elif rng.random() < 0.5:
                lg[b, r, :] = 2.0                      # full tie: id 0 wins
    st = _dev_tree(stack_trees(trees, N_max))
    logits = torch.from_numpy(lg).to(dtype).to(DEV)
    g = tsv.accept_walk(logits, st["n_nodes"], st["parent"], st["token"], gamma)
    torch.cuda.synchronize()
    _check_walk(g, np32(logits), trees, gamma)


def test_walk_workspace_reuse():
    """Calls on one workspace, with changing trees and logits, each match the
    oracle (no state survives in the workspace)."""
    B, gamma, k, N_max, V = 6, 5, 3, 20, 3001
    ws = tsv.workspace(tsv.workspace_size(2, B, gamma, V, 1, N_max, dtype=tsv.TSV_BF16), DEV)
    for call in range(3):
        rng = np.random.default_rng(100 + call)
        marg = rng.dirichlet(np.ones(10) * 0.5, size=(B, gamma)).astype(np.float32)
        marg = np.concatenate([marg, np.zeros((B, gamma, V - 10), np.float32)], -1)
        budgets = [int(x) for x in rng.integers(0, N_max + 1, size=B)]
        trees = []
        for b in range(B):
            idx, p = oracle.topk_per_position(marg[b:b + 1], k)
            trees.append(oracle.select_tree(idx[0], p[0], budgets[b], N_max))
        lg = rng.normal(0, 1, size=(B, 1 + N_max, V)).astype(np.float32)
        for b, t in enumerate(trees):
            for r in range(1 + t.n):
                kids = [j for j in range(t.n) if t.parent[j] == r - 1]
                if kids and rng.random() < 0.8:
                    lg[b, r, t.token[kids[rng.integers(len(kids))]]] = 9.0
        st = _dev_tree(stack_trees(trees, N_max))
        logits = torch.from_numpy(lg).to(torch.bfloat16).to(DEV)
        g = tsv.accept_walk(logits, st["n_nodes"], st["parent"], st["token"], gamma, ws=ws)
        torch.cuda.synchronize()
        _check_walk(g, np32(logits), trees, gamma)


def test_walk_dspark_cycle_chain():
    """Chain E F G under root D; the target agrees on E and F and prefers G*
    after F: two tokens accepted, then the correction."""
    E, F, G, H, Gs, V = 4, 5, 6, 7, 8, 9
    n, N_max, gamma = 3, 4, 4
    parent = torch.tensor([[-1, 0, 1, -1]], dtype=torch.int32, device=DEV)
    token = torch.tensor([[E, F, G, -1]], dtype=torch.int32, device=DEV)
    lg = torch.zeros(1, 1 + N_max, V, device=DEV)
    for r, t in enumerate([E, F, Gs, H]):
        lg[0, r, t] = 1.0
    g = tsv.accept_walk(lg, torch.tensor([n], dtype=torch.int32, device=DEV), parent, token, gamma)
    assert int(g["accept_len"][0]) == 2
    assert g["accept_nodes"][0].tolist() == [0, 1, -1, -1]
    assert g["out_tokens"][0].tolist() == [E, F, Gs, -1, -1]


def _commit_case(rng, B, L_cap, N_max, Hkv, d, gamma, mla, dtype):
    row = (d,) if mla else (Hkv, d)
    kc = torch.randn((B, L_cap) + row, device=DEV).to(dtype)
    kt = torch.randn((B, N_max) + row, device=DEV).to(dtype)
    vc = None if mla else torch.randn((B, L_cap) + row, device=DEV).to(dtype)
    vt = None if mla else torch.randn((B, N_max) + row, device=DEV).to(dtype)
    pl = rng.integers(0, L_cap - gamma + 1, size=B).astype(np.int32)
    pl[0] = L_cap - 1                                   # overflow when m >= 2
    alen = rng.integers(0, gamma + 1, size=B).astype(np.int32)
    alen[0] = max(alen[0], 2)
    nodes = np.full((B, gamma), -1, dtype=np.int32)
    for b in range(B):
        nodes[b, :alen[b]] = rng.permutation(N_max)[:alen[b]]
    if B > 2:
        nodes[1, 0] = N_max if alen[1] > 0 else nodes[1, 0]   # bad index -> status 2
        alen[2] = gamma + 1                                    # bad length -> status 2
    return kc, vc, kt, vt, pl, alen, nodes


def _pitched(t, pitch, fill):
    """A copy of t with rows `pitch` elements apart; the elements between rows
    hold `fill`.  Returns the copy and a view of its whole storage."""
    B, R = t.shape[:2]
    out = tsv.kv_rows(B, R, tuple(t.shape[2:]), t.dtype, DEV, pitch)
    full = out.as_strided((B, R, pitch), (R * pitch, pitch, 1))
    full.fill_(fill)
    out.copy_(t)
    return out, full


@pytest.mark.parametrize("pitched", [False, True])
@pytest.mark.parametrize("mla", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_commit_vs_oracle(mla, dtype, pitched):
    rng = np.random.default_rng(int(mla) * 2 + int(dtype == torch.float32))
    B, L_cap, N_max, Hkv, gamma = 6, 300, 20, 4, 5
    d = 576 if mla else 64
    kc, vc, kt, vt, pl, alen, nodes = _commit_case(rng, B, L_cap, N_max, Hkv, d, gamma, mla, dtype)
    fulls = []
    if pitched:
        # rows further apart than their width: only the rows' own elements move
        width = d if mla else Hkv * d
        pitch = tsv.kv_row_pitch(width, kc.element_size())
        if pitch == width:
            pitch = width + 32 // kc.element_size()
        kc, f = _pitched(kc, pitch, 7.0); fulls.append((f, width))
        kt, f = _pitched(kt, pitch, 7.0); fulls.append((f, width))
        if not mla:
            vc, f = _pitched(vc, pitch, 7.0); fulls.append((f, width))
            vt, f = _pitched(vt, pitch, 7.0); fulls.append((f, width))
    ref_k = np32(kc).copy()
    ref_v = None if mla else np32(vc).copy()
    ref_pl = pl.copy()
    st_ref = oracle.commit_path(ref_k, ref_v, ref_pl, np32(kt), None if mla else np32(vt),
                                alen, nodes, gamma)
    pl_d = torch.from_numpy(pl).to(DEV)
    st = tsv.commit_path(kc, vc, pl_d, kt, vt, torch.from_numpy(alen).to(DEV),
                         torch.from_numpy(nodes).to(DEV), 1 if mla else Hkv, d, d)
    torch.cuda.synchronize()
    assert st.tolist() == st_ref.tolist()
    assert pl_d.tolist() == ref_pl.tolist()
    assert np.array_equal(np32(kc), ref_k)
    if not mla:
        assert np.array_equal(np32(vc), ref_v)
    for f, width in fulls:
        assert bool((f[:, :, width:] == 7.0).all()), "an element between rows was written"


@pytest.mark.parametrize("cid,pitched", [(1, False), (2, False), (3, False), (4, False), (5, False),
                                         (2, True)])
def test_chained_round(cid, pitched):
    """build_tree -> tree_verify_attn -> accept_walk -> commit_path on the GPU,
    every output against the oracle (attention on a sample of nodes); once
    with cache and scratch rows at the recommended pitch."""
    cfg = config(cid)
    pitch = tsv.kv_row_pitch(cfg.Hkv * cfg.d_qk, 2) if pitched else None
    print(f"chained round workload {cid} {cfg.name}, row pitch {pitch}", flush=True)
    marg = marginals(cfg, 0, DEV)
    ins = attention_inputs(cfg, 0, DEV, row_pitch=pitch)
    pl_np = ins["prefix_len"].cpu().numpy().copy()
    g = tsv.build_tree_topk(marg, cfg.top_k, cfg.n_budget, cfg.N_max, cost=cfg.cost,
                            prefix_len=ins["prefix_len"] if cfg.cost else None)
    out, lse = tsv.tree_verify_attn(ins["q"], ins["k_cache"], ins["v_cache"], ins["k_tree"],
                                    ins["v_tree"], ins["prefix_len"], g["n_nodes"],
                                    g["anc_bits"], cfg.Hkv, cfg.d_v, cfg.sm_scale)
    idx, p, trees = oracle_trees(marg.cpu().numpy(), cfg.top_k, cfg.n_budget, cfg.N_max,
                                 cfg.cost, pl_np)
    assert_tree_equal(g, idx, p, trees)
    st = stack_trees(trees, cfg.N_max)
    tl = target_logits(cfg, 0, st["depth"], st["n_nodes"], DEV)
    w = tsv.accept_walk(tl, g["n_nodes"], g["parent"], g["token"], cfg.gamma)
    torch.cuda.synchronize()
    _check_walk(w, np32(tl), trees, cfg.gamma)
    rng = np.random.default_rng(cid)
    pairs = [(b, i) for b in range(cfg.B) for i in range(trees[b].n)]
    pick = rng.choice(len(pairs), size=min(6, len(pairs)), replace=False)
    check_attention(out, lse, ins["q"], ins["k_cache"], ins["v_cache"], ins["k_tree"],
                    ins["v_tree"], pl_np, trees, cfg.sm_scale, TOL[cfg.torch_dtype], cfg.mla,
                    cfg.d_v, sorted(pairs[j] for j in pick))
    # commit: only rows [l_b, l_b + m_b) of each request may change
    alen = w["accept_len"].cpu().numpy()
    anodes = w["accept_nodes"].cpu().numpy()
    kt_np = np32(ins["k_tree"])
    vt_np = None if cfg.mla else np32(ins["v_tree"])
    before = {b: np32(ins["k_cache"][b, max(0, pl_np[b] - 2): pl_np[b] + cfg.gamma + 2]).copy()
              for b in range(cfg.B)}
    before_v = {} if cfg.mla else {
        b: np32(ins["v_cache"][b, max(0, pl_np[b] - 2): pl_np[b] + cfg.gamma + 2]).copy()
        for b in range(cfg.B)}
    vc = None if cfg.mla else ins["v_cache"]
    vt = None if cfg.mla else ins["v_tree"]
    status = tsv.commit_path(ins["k_cache"], vc, ins["prefix_len"], ins["k_tree"], vt,
                             w["accept_len"], w["accept_nodes"], cfg.Hkv, cfg.d_qk, cfg.d_v)
    torch.cuda.synchronize()
    assert (status.cpu().numpy() == 0).all()
    assert np.array_equal(ins["prefix_len"].cpu().numpy(), pl_np + alen)
    for b in range(cfg.B):
        lo = max(0, pl_np[b] - 2)
        after = np32(ins["k_cache"][b, lo: pl_np[b] + cfg.gamma + 2])
        want = before[b].copy()
        for j in range(alen[b]):
            want[pl_np[b] - lo + j] = kt_np[b, anodes[b, j]]
        assert np.array_equal(after, want), b
        if not cfg.mla:
            after_v = np32(ins["v_cache"][b, lo: pl_np[b] + cfg.gamma + 2])
            want_v = before_v[b].copy()
            for j in range(alen[b]):
                want_v[pl_np[b] - lo + j] = vt_np[b, anodes[b, j]]
            assert np.array_equal(after_v, want_v), b
    print(f"workload {cid}: accepted {int(alen.sum())} tokens + {cfg.B} bonus over "
          f"{int(st['n_nodes'].sum())} tree nodes", flush=True)


def test_multi_round_caches_stay_equal():
    """Three rounds chained on the GPU and on the oracle (commit grows the
    prefix): caches, prefix lengths and emitted tokens stay identical."""
    cfg = config(2, B=3, V=3000, prefix=500, n_budget=12, N_max=16, top_k=6, gamma=5)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    ins = attention_inputs(cfg, 0, DEV)
    L_cap = cfg.L_cap + 3 * cfg.gamma
    kc = torch.zeros((cfg.B, L_cap, cfg.Hkv, cfg.d_qk), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    kc[:, : cfg.L_cap] = ins["k_cache"]
    vc[:, : cfg.L_cap] = ins["v_cache"]
    pl = ins["prefix_len"].clone()
    ref_k, ref_v, ref_pl = np32(kc).copy(), np32(vc).copy(), pl.cpu().numpy().copy()
    for r in range(3):
        lg = torch.randn(cfg.B, cfg.gamma, cfg.V, generator=gen, device=DEV, dtype=torch.float64)
        marg = torch.softmax(lg, -1).float()
        kt = torch.randn(cfg.B, cfg.N_max, cfg.Hkv, cfg.d_qk, generator=gen, device=DEV).bfloat16()
        vt = torch.randn(cfg.B, cfg.N_max, cfg.Hkv, cfg.d_v, generator=gen, device=DEV).bfloat16()
        g = tsv.build_tree(marg, cfg.top_k, cfg.n_budget, cfg.N_max)
        _, _, trees = oracle_trees(marg.cpu().numpy(), cfg.top_k, cfg.n_budget, cfg.N_max)
        st = stack_trees(trees, cfg.N_max)
        tl = torch.randn(cfg.B, 1 + cfg.N_max, cfg.V, generator=gen, device=DEV)
        tnp = tl.cpu().numpy()
        for b, t in enumerate(trees):          # make the target agree along one branch
            cur = -1
            for _ in range(cfg.gamma):
                kids = [j for j in range(t.n) if t.parent[j] == cur]
                if not kids:
                    break
                cur = kids[-1]
                tnp[b, t.parent[cur] + 1, t.token[cur]] = 9.0
        tl = torch.from_numpy(tnp).to(DEV)
        w = tsv.accept_walk(tl, g["n_nodes"], g["parent"], g["token"], cfg.gamma)
        tsv.commit_path(kc, vc, pl, kt, vt, w["accept_len"], w["accept_nodes"], cfg.Hkv,
                        cfg.d_qk, cfg.d_v)
        torch.cuda.synchronize()
        alen, anodes = [], []
        for b, t in enumerate(trees):
            m, nodes, _ = oracle.accept_walk(tnp[b], t.n, t.parent, t.token, cfg.gamma)
            alen.append(m)
            anodes.append(nodes)
        alen = np.array(alen, np.int32)
        assert np.array_equal(w["accept_len"].cpu().numpy(), alen)
        oracle.commit_path(ref_k, ref_v, ref_pl, np32(kt), np32(vt), alen, np.stack(anodes),
                           cfg.gamma)
        assert np.array_equal(pl.cpu().numpy(), ref_pl), r
        assert np.array_equal(np32(kc), ref_k), r
        assert np.array_equal(np32(vc), ref_v), r
    assert (ref_pl > ins["prefix_len"].cpu().numpy()).any()
