"""A request verified alone gives what it gives inside a batch.

The review page's "Performance validation: key results" (paper section 5.2,
Table 1) reports the accepted length staying flat from batch 1 to batch 64:
verification of one request must not depend on the others.  Here request b
alone (a batch of one, sliced from the same inputs) is compared with request
b inside the batch: the tree (with its top-k lists), the accepted path and
the committed cache bytes must be bit-identical; the attention output may
round differently, because the key range of a row block is cut into splits
whose sizes depend on the batch, so both are held to the oracle's tolerance
and their difference to the same bound."""

import numpy as np
import pytest
import torch

import tree_structured_verification_amd as tsv
from tests._helpers import DEV, TOL, check_attention, oracle_trees
from workloads import attention_inputs, config, marginals, prefix_lengths, target_logits

pytestmark = pytest.mark.gpu

SHAPES = {
    # grouped heads, ragged prefixes, fixed budget
    "gqa_fixed": dict(cid=4, B=8, gamma=8, V=20000, top_k=32, n_budget=32, N_max=32,
                      prefix_range=(100, 6000), cost=None),
    # grouped heads, the adaptive budget of the ragged workload
    "gqa_adaptive": dict(cid=4, B=8, gamma=8, V=20000, top_k=64, n_budget=64, N_max=64,
                         prefix_range=(100, 6000)),
    # one latent head shared by 128 query heads
    "latent": dict(cid=5, B=4, gamma=6, V=5000, top_k=4, n_budget=16, N_max=16, prefix=1500),
}


def _round(cfg, sl, marg, ins, tl):
    """One round on the requests of slice sl; returns host copies of every
    output and of the committed caches."""
    adaptive = cfg.cost is not None
    pl = ins["prefix_len"][sl].clone()
    g = tsv.build_tree_topk(marg[sl].contiguous(), cfg.top_k, cfg.n_budget, cfg.N_max,
                            cost=cfg.cost, prefix_len=pl if adaptive else None)
    kc, kt = ins["k_cache"][sl].clone(), ins["k_tree"][sl].contiguous()
    vc = kc if cfg.mla else ins["v_cache"][sl].clone()
    vt = kt if cfg.mla else ins["v_tree"][sl].contiguous()
    out, lse = tsv.tree_verify_attn(ins["q"][sl].contiguous(), kc, vc, kt, vt, pl, g["n_nodes"],
                                    g["anc_bits"], cfg.Hkv, cfg.d_v, cfg.sm_scale)
    w = tsv.accept_walk(tl[sl].contiguous(), g["n_nodes"], g["parent"], g["token"], cfg.gamma)
    st = tsv.commit_path(kc, None if cfg.mla else vc, pl, kt, None if cfg.mla else vt,
                         w["accept_len"], w["accept_nodes"], cfg.Hkv, cfg.d_qk, cfg.d_v)
    torch.cuda.synchronize()
    res = {k: v.cpu() for k, v in g.items()}
    res.update({k: v.cpu() for k, v in w.items()})
    res.update(out=out.cpu(), lse=lse.cpu(), status=st.cpu(), prefix=pl.cpu(), kc=kc.cpu(),
               vc=None if cfg.mla else vc.cpu())
    return res


@pytest.mark.parametrize("name", list(SHAPES))
def test_request_alone_equals_request_in_batch(name):
    kw = dict(SHAPES[name])
    cfg = config(kw.pop("cid"), **kw)
    print(f"batch invariance {name}", flush=True)
    marg = marginals(cfg, 0, DEV)
    ins = attention_inputs(cfg, 0, DEV)
    pl_np = prefix_lengths(cfg)
    _, _, trees = oracle_trees(marg.cpu().numpy(), cfg.top_k, cfg.n_budget, cfg.N_max, cfg.cost,
                               pl_np)
    n_np = np.array([t.n for t in trees])
    assert n_np.sum() > 0
    depth = np.stack([t.depth for t in trees])
    tl = target_logits(cfg, 0, depth, n_np, DEV)
    full = _round(cfg, slice(0, cfg.B), marg, ins, tl)
    assert (full["status"] == 0).all()
    worst = 0.0
    for b in sorted({0, int(np.argmax(n_np)), cfg.B - 1}):
        one = _round(cfg, slice(b, b + 1), marg, ins, tl)
        for k in ("n_nodes", "parent", "token", "depth", "anc_bits", "topk_idx", "accept_len",
                  "accept_nodes", "out_tokens", "status", "prefix"):
            assert torch.equal(one[k][0], full[k][b]), (name, b, k)
        for k in ("score", "topk_p"):
            assert torch.equal(one[k][0].view(torch.int32), full[k][b].view(torch.int32)), (name, b, k)
        assert torch.equal(one["kc"][0].view(torch.int16), full["kc"][b].view(torch.int16)), (name, b)
        if not cfg.mla:
            assert torch.equal(one["vc"][0].view(torch.int16), full["vc"][b].view(torch.int16)), (name, b)
        n = trees[b].n
        if n == 0:
            continue
        d_out = (one["out"][0, :n].float() - full["out"][b, :n].float()).abs().max().item()
        d_lse = (one["lse"][0, :n] - full["lse"][b, :n]).abs().max().item()
        worst = max(worst, d_out, d_lse)
        assert d_out <= TOL[cfg.torch_dtype] and d_lse <= TOL[cfg.torch_dtype], (name, b, d_out, d_lse)
        # both against the oracle, on the request's last node
        for o, l in ((one["out"], one["lse"]), (full["out"][b:b + 1], full["lse"][b:b + 1])):
            check_attention(o, l, ins["q"][b:b + 1], ins["k_cache"][b:b + 1],
                            ins["v_cache"][b:b + 1], ins["k_tree"][b:b + 1],
                            ins["v_tree"][b:b + 1], pl_np[b:b + 1], [trees[b]], cfg.sm_scale,
                            TOL[cfg.torch_dtype], cfg.mla, cfg.d_v, [(0, n - 1)])
    print(f"MARGIN batch invariance {name}: max |alone - in batch| = {worst:.3e}", flush=True)
