"""tree_verify_attn on the GPU vs the fp64 oracle (tolerance 1e-5 fp32,
2e-2 bf16), plus bitwise properties: sibling isolation and determinism."""

import ctypes
import math
import zlib

import numpy as np
import pytest
import torch

import oracle
import tree_structured_verification_amd as tsv
from tree_structured_verification_amd import _lib
from tests._helpers import DEV, TOL, check_attention, np32, oracle_trees
from workloads import attention_inputs, config, marginals

pytestmark = pytest.mark.gpu


def _random_trees(rng, B, N_max, n_list):
    """Random ancestor-closed trees (parents precede children)."""
    trees = []
    for b in range(B):
        n = n_list[b]
        parent = np.full(N_max, -1, dtype=np.int32)
        for i in range(1, n):
            parent[i] = rng.integers(-1, i)
        t = oracle.tree.TreeResult(n, parent, np.full(N_max, -1, np.int32),
                                   np.full(N_max, -1, np.int32), np.zeros(N_max, np.float32),
                                   oracle.ancestor_bits(parent, n, N_max))
        trees.append(t)
    return trees


def _inputs(rng, B, N_max, L_cap, Hq, Hkv, d_qk, d_v, dtype, prefix, mla=False):
    g = torch.Generator(device=DEV)
    g.manual_seed(int(rng.integers(1 << 30)))
    rn = lambda *s: torch.randn(*s, generator=g, device=DEV, dtype=torch.float32).to(dtype)
    q = rn(B, N_max, Hq, d_qk)
    if mla:
        kc = rn(B, L_cap, d_qk)
        kt = rn(B, N_max, d_qk)
        vc, vt = kc, kt
    else:
        kc = rn(B, L_cap, Hkv, d_qk)
        kt = rn(B, N_max, Hkv, d_qk)
        vc = rn(B, L_cap, Hkv, d_v)
        vt = rn(B, N_max, Hkv, d_v)
    pl = torch.tensor(prefix, dtype=torch.int32, device=DEV)
    return q, kc, vc, kt, vt, pl


def _run(q, kc, vc, kt, vt, pl, trees, Hkv, d_v, scale):
    B, N_max = q.shape[:2]
    n = torch.tensor([t.n for t in trees], dtype=torch.int32, device=DEV)
    anc = torch.from_numpy(np.stack([t.anc_bits for t in trees]).view(np.int32)).to(DEV)
    out = torch.full((B, N_max, q.shape[2], d_v), float("nan"), dtype=q.dtype, device=DEV)
    o, lse = tsv.tree_verify_attn(q, kc, vc, kt, vt, pl, n, anc, Hkv, d_v, scale, out=out)
    torch.cuda.synchronize()
    return o, lse, n, anc


CASES = [
    # name, B, N_max, Hq, Hkv, d_qk, d_v, dtype, prefix, n, mla
    ("fp32_mha", 2, 8, 4, 4, 64, 64, torch.float32, [100, 37], [8, 3], False),
    ("fp32_gqa_long", 1, 20, 8, 2, 32, 32, torch.float32, [3000], [20], False),
    ("bf16_gqa_mfma", 3, 40, 8, 2, 128, 128, torch.bfloat16, [700, 64, 1], [40, 5, 0], False),
    ("bf16_gqa_g4", 4, 32, 32, 8, 128, 128, torch.bfloat16, [257, 4096, 1000, 63], [32, 1, 17, 32], False),
    ("bf16_many_splits", 1, 32, 16, 4, 128, 128, torch.bfloat16, [20000], [31], False),
    ("bf16_latent_mfma", 2, 8, 16, 1, 576, 512, torch.bfloat16, [300, 33], [8, 2], True),
    ("bf16_latent_long", 1, 16, 128, 1, 576, 512, torch.bfloat16, [5000], [16], True),
    ("bf16_valu_d64", 2, 12, 6, 3, 64, 64, torch.bfloat16, [500, 9], [12, 7], False),
    ("bf16_n128_prefix0", 1, 128, 4, 1, 128, 128, torch.bfloat16, [0], [128], False),
    # ~313 splits of 16 keys: several groups of 64 in the combine, two column passes of d_v 72
    ("fp32_dv72_many_splits", 1, 8, 2, 2, 72, 72, torch.float32, [5000], [8], False),
    # 128 units x 4 splits = 512 workgroups, two per compute unit: long units take the
    # first-dispatched / second-dispatched key shares, short ones equal chunks
    ("bf16_gqa_paired_splits", 16, 32, 32, 8, 128, 128, torch.bfloat16,
     [2100, 2000, 1500, 1200, 900, 500, 64, 1, 2100, 1800, 1000, 0, 2050, 1300, 700, 2100],
     [32, 32, 17, 5, 32, 1, 0, 32, 32, 20, 32, 8, 32, 32, 3, 32], False),
    # 384 units x 3 splits = 1152 work items (more than resident): no split shorter than
    # 4096 keys, so ragged units take one, two or three splits
    ("bf16_gqa_split_floor", 48, 16, 32, 8, 128, 128, torch.bfloat16,
     [int(x) for x in np.random.default_rng(7).integers(100, 9001, 48)],
     [int(x) for x in np.random.default_rng(8).integers(0, 17, 48)], False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_small_cases(case):
    name, B, N_max, Hq, Hkv, d_qk, d_v, dtype, prefix, n_list, mla = case
    print(f"attention case {name}", flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    L_cap = max(prefix) + 16
    q, kc, vc, kt, vt, pl = _inputs(rng, B, N_max, L_cap, Hq, Hkv, d_qk, d_v, dtype, prefix, mla)
    trees = _random_trees(rng, B, N_max, n_list)
    scale = 1.0 / math.sqrt(d_qk)
    o, lse, _, _ = _run(q, kc, vc, kt, vt, pl, trees, Hkv, d_v, scale)
    check_attention(o, lse, q, kc, vc, kt, vt, prefix, trees, scale, TOL[dtype], mla, d_v)
    # rows past n_b are never written
    on = o.float().cpu().numpy()
    for b in range(B):
        assert np.isnan(on[b, n_list[b]:]).all()


def test_sibling_isolation_and_determinism():
    """Perturbing scratch rows that are not ancestors of node i leaves node i's
    output bit-identical; two identical calls give identical bits."""
    rng = np.random.default_rng(3)
    B, N_max, Hq, Hkv, d = 2, 16, 8, 2, 128
    prefix = [900, 130]
    q, kc, vc, kt, vt, pl = _inputs(rng, B, N_max, 1000, Hq, Hkv, d, d, torch.bfloat16, prefix)
    trees = _random_trees(rng, B, N_max, [16, 11])
    scale = 0.088
    o1, l1, _, _ = _run(q, kc, vc, kt, vt, pl, trees, Hkv, d, scale)
    o2, l2, _, _ = _run(q, kc, vc, kt, vt, pl, trees, Hkv, d, scale)
    bits = lambda t: t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)
    for b in range(B):      # rows past n_b are never written
        n = trees[b].n
        assert torch.equal(bits(o1[b, :n]), bits(o2[b, :n]))
        assert torch.equal(bits(l1[b, :n]), bits(l2[b, :n]))
    for b in range(B):
        for i in range(trees[b].n):
            anc = {j for j in range(N_max) if trees[b].anc_bits[i, j // 32] >> (j % 32) & 1}
            others = [j for j in range(trees[b].n) if j not in anc]
            if not others:
                continue
            kt2, vt2 = kt.clone(), vt.clone()
            kt2[b, others] = (kt2[b, others].float() * -3.0 + 1.0).to(kt.dtype)
            vt2[b, others] = (vt2[b, others].float() + 5.0).to(vt.dtype)
            o3, l3, _, _ = _run(q, kc, vc, kt2, vt2, pl, trees, Hkv, d, scale)
            assert torch.equal(bits(o3[b, i]), bits(o1[b, i]))
            assert torch.equal(bits(l3[b, i]), bits(l1[b, i]))
            if i == 0 and b == 0:
                # and an ancestor perturbation does change it
                kt3 = kt.clone()
                kt3[b, i] = (kt3[b, i].float() * -2.0).to(kt.dtype)
                o4, _, _, _ = _run(q, kc, vc, kt3, vt, pl, trees, Hkv, d, scale)
                assert not torch.equal(o4[b, i], o1[b, i])


def _structured_samples(cid, trees, rng):
    """Nodes checked at full size: for the latent workloads (one row block of
    128 rows per node) every node of the first and last request plus one node
    of every other request (3), or the first and last node of every request
    (5, about a second of oracle time per node); for the grouped workloads
    (a row block holds 32 nodes x 4 heads) one node of every request that
    verifies a tree, its last node for the longest request, and a random
    sample of the rest (2, 4)."""
    B = len(trees)
    picks = set()
    if cid == 3:
        for b in (0, B - 1):
            picks.update((b, i) for i in range(trees[b].n))
        for b in range(1, B - 1):
            if trees[b].n:
                picks.add((b, int(rng.integers(trees[b].n))))
    elif cid == 5:
        for b in range(B):
            if trees[b].n:
                picks.update({(b, 0), (b, trees[b].n - 1)})
    else:
        for b in range(B):
            if trees[b].n:
                picks.add((b, int(rng.integers(trees[b].n))))
        bl = int(np.argmax([t.n for t in trees]))
        picks.add((bl, trees[bl].n - 1))
        pairs = [(b, i) for b in range(B) for i in range(trees[b].n)]
        extra = rng.choice(len(pairs), size=min(32, len(pairs)), replace=False)
        picks.update(pairs[j] for j in extra)
    return sorted(picks)


def test_workspace_reuse_and_counter_reset():
    """Split-K arrival counters live in the workspace: repeated calls on one
    workspace give the same bits, and every call leaves the counters zero
    (the workspace contract of tree_verify_attn)."""
    rng = np.random.default_rng(11)
    B, N_max, Hq, Hkv, d = 3, 32, 16, 4, 128
    prefix = [6000, 2500, 700]
    q, kc, vc, kt, vt, pl = _inputs(rng, B, N_max, 6016, Hq, Hkv, d, d, torch.bfloat16, prefix)
    trees = _random_trees(rng, B, N_max, [32, 9, 20])
    n = torch.tensor([t.n for t in trees], dtype=torch.int32, device=DEV)
    anc = torch.from_numpy(np.stack([t.anc_bits for t in trees]).view(np.int32)).to(DEV)
    nbytes = tsv.workspace_size(1, B, 1, 1, 1, N_max, 6016, Hq, Hkv, d, d, tsv.TSV_BF16)
    ws = tsv.workspace(nbytes, DEV)
    outs = []
    for _ in range(3):
        o, l = tsv.tree_verify_attn(q, kc, vc, kt, vt, pl, n, anc, Hkv, d, 0.09, ws=ws)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).clone(), l.view(torch.int32).clone()))
        # the counters (one int per unit (request, KV head, block of 128 rows),
        # padded to a multiple of 8, at the start of the workspace) are zero again
        units = B * Hkv * ((N_max * (Hq // Hkv) + 127) // 128)
        assert int(ws[:4 * ((units + 7) // 8 * 8)].count_nonzero()) == 0
    for o, l in outs[1:]:   # rows past n_b are never written
        for b, t in enumerate(trees):
            assert torch.equal(o[b, :t.n], outs[0][0][b, :t.n])
            assert torch.equal(l[b, :t.n], outs[0][1][b, :t.n])
    check_attention(outs[0][0].view(torch.bfloat16), outs[0][1].view(torch.float32), q, kc, vc, kt, vt,
                    prefix, trees, 0.09, TOL[torch.bfloat16], False, d)


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload(cid):
    """Full-size inputs, trees built by the oracle; every node checked for
    the tiny workload, a seeded sample of nodes otherwise."""
    cfg = config(cid)
    print(f"attention workload {cid} {cfg.name}", flush=True)
    ins = attention_inputs(cfg, 0, DEV)
    pl_np = ins["prefix_len"].cpu().numpy()
    marg = marginals(cfg, 0, DEV).cpu().numpy()
    _, _, trees = oracle_trees(marg, cfg.top_k, cfg.n_budget, cfg.N_max, cfg.cost, pl_np)
    o, lse, _, _ = _run(ins["q"], ins["k_cache"], ins["v_cache"], ins["k_tree"], ins["v_tree"],
                        ins["prefix_len"], trees, cfg.Hkv, cfg.d_v, cfg.sm_scale)
    samples = None if cid == 1 else _structured_samples(cid, trees, np.random.default_rng(cid))
    worst = check_attention(o, lse, ins["q"], ins["k_cache"], ins["v_cache"], ins["k_tree"],
                            ins["v_tree"], pl_np, trees, cfg.sm_scale, TOL[cfg.torch_dtype],
                            cfg.mla, cfg.d_v, samples)
    checked = sum(t.n for t in trees) if samples is None else len(samples)
    print(f"MARGIN workload {cid} {cfg.name}: max |gpu - oracle| = {worst:.3e} over {checked} "
          f"nodes (tolerance {TOL[cfg.torch_dtype]:g})", flush=True)


def test_invalid_arguments():
    q = torch.zeros(1, 4, 4, 64, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(1, 10, 2, 64, dtype=torch.bfloat16, device=DEV)
    kt = torch.zeros(1, 4, 2, 64, dtype=torch.bfloat16, device=DEV)
    pl = torch.zeros(1, dtype=torch.int32, device=DEV)
    n = torch.zeros(1, dtype=torch.int32, device=DEV)
    anc = torch.zeros(1, 4, 1, dtype=torch.int32, device=DEV)
    with pytest.raises(tsv.TsvError) as e:
        tsv.tree_verify_attn(q, kc, kc, kt, kt, pl, n, anc, 3, 64, 0.1)   # Hq % Hkv
    assert e.value.code == -1
    with pytest.raises(tsv.TsvError) as e:
        tsv.tree_verify_attn(q, kc, kc, kt, kt, pl, n, anc, 2, 64, 0.1,
                             ws=torch.empty(64, dtype=torch.uint8, device=DEV))
    assert e.value.code == -3


def test_wide_heads_value_cache_of_its_own():
    """Head widths 576 / 512 with a value cache of its own (not the key rows,
    so not the latent path): rows padded to the key's stride and passed
    through the C entry point; the generic kernel, checked against the oracle."""
    rng = np.random.default_rng(11)
    B, N_max, Hq, dq, dv, L = 2, 6, 16, 576, 512, 160
    prefix = [130, 40]
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    rn = lambda *s: torch.randn(*s, generator=g, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    q, kc, kt = rn(B, N_max, Hq, dq), rn(B, L, dq), rn(B, N_max, dq)
    vc, vt = rn(B, L, dq), rn(B, N_max, dq)   # the value is the first dv columns
    pl = torch.tensor(prefix, dtype=torch.int32, device=DEV)
    trees = _random_trees(rng, B, N_max, [6, 3])
    n = torch.tensor([t.n for t in trees], dtype=torch.int32, device=DEV)
    anc = torch.from_numpy(np.stack([t.anc_bits for t in trees]).view(np.int32)).to(DEV)
    out = torch.full((B, N_max, Hq, dv), float("nan"), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(B, N_max, Hq, dtype=torch.float32, device=DEV)
    ws = tsv.workspace(tsv.workspace_size(1, B, 1, 1, 1, N_max, L, Hq, 1, dq, dv, tsv.TSV_BF16), DEV)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    scale = 1 / math.sqrt(dq)
    rc = _lib.lib().tree_verify_attn(P(q), P(kc), P(vc), P(kt), P(vt), dq, P(pl), P(n), P(anc),
                                     B, N_max, L, Hq, 1, dq, dv, tsv.TSV_BF16,
                                     ctypes.c_float(scale), P(out), P(lse), P(ws), ws.numel(),
                                     None)
    torch.cuda.synchronize()
    assert rc == 0
    check_attention(out, lse, q, kc.unsqueeze(2), vc[..., :dv].unsqueeze(2), kt.unsqueeze(2),
                    vt[..., :dv].unsqueeze(2), prefix, trees, scale, TOL[torch.bfloat16], False, dv)


def test_split_handoff_many_splits_sentinel():
    """One unit whose 160000 keys are cut into 500 splits of 320 keys: the
    last split to arrive combines every other split's published rows.  The
    outputs are filled with NaN before each of four launches; every row of
    every node must be written, bit-equal across launches, and within
    tolerance of the oracle on a sample of nodes."""
    rng = np.random.default_rng(17)
    B, N_max, Hq, Hkv, d = 1, 32, 4, 1, 128
    prefix = [160000]
    L_cap = prefix[0] + 16
    q, kc, vc, kt, vt, pl = _inputs(rng, B, N_max, L_cap, Hq, Hkv, d, d, torch.bfloat16, prefix)
    trees = _random_trees(rng, B, N_max, [32])
    n = torch.tensor([32], dtype=torch.int32, device=DEV)
    anc = torch.from_numpy(np.stack([t.anc_bits for t in trees]).view(np.int32)).to(DEV)
    # splits of the grouped kernel: one unit (capacity L_cap + N_max keys,
    # about 512 workgroups aimed for, at least 256 keys and at most 4096 keys
    # per split of the capacity), whose 160032 actual keys are cut into S
    # chunks rounded up to 32 keys
    cdiv = lambda x, y: -(-x // y)
    keys_max = L_cap + N_max
    cap_chunk = cdiv(max(256, cdiv(keys_max, 512)), 32) * 32
    S = max(cdiv(keys_max, cap_chunk), cdiv(keys_max, 4096))
    keys = prefix[0] + 32
    chunk = max(cdiv(cdiv(keys, S), 32) * 32, 256)
    splits = cdiv(keys, chunk)
    assert splits > 300, splits
    ws = tsv.workspace(tsv.workspace_size(1, B, 1, 1, 1, N_max, L_cap, Hq, Hkv, d, d,
                                          tsv.TSV_BF16), DEV)
    first = None
    for launch in range(4):
        out = torch.full((B, N_max, Hq, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        lse = torch.full((B, N_max, Hq), float("nan"), dtype=torch.float32, device=DEV)
        tsv.tree_verify_attn(q, kc, vc, kt, vt, pl, n, anc, Hkv, d, 0.0884, out=out, lse=lse, ws=ws)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any(), launch
        assert not torch.isnan(lse).any(), launch
        bits = (out.view(torch.int16).clone(), lse.view(torch.int32).clone())
        if first is None:
            first = bits
        else:
            assert torch.equal(bits[0], first[0]) and torch.equal(bits[1], first[1]), launch
    check_attention(out, lse, q, kc, vc, kt, vt, prefix, trees, 0.0884, TOL[torch.bfloat16],
                    False, d, [(0, i) for i in (0, 7, 19, 31)])


def test_workspace_reuse_across_dtype_and_shapes():
    """One workspace (zeroed once, sized for the largest call) serves fp32
    and bf16 calls and other prefix capacities at the same B, N_max, Hq, Hkv
    without clearing; after a call at another B it is zeroed again, as the
    header requires.  Outputs are NaN-filled before every call, and every
    row of every node must be written and match the oracle."""
    rng = np.random.default_rng(23)
    N_max, Hq, Hkv, d = 32, 16, 4, 128

    def call(B, prefix, dtype, L_cap, ws):
        q, kc, vc, kt, vt, pl = _inputs(rng, B, N_max, L_cap, Hq, Hkv, d, d, dtype, prefix)
        trees = _random_trees(rng, B, N_max, [int(rng.integers(1, N_max + 1)) for _ in range(B)])
        n = torch.tensor([t.n for t in trees], dtype=torch.int32, device=DEV)
        anc = torch.from_numpy(np.stack([t.anc_bits for t in trees]).view(np.int32)).to(DEV)
        out = torch.full((B, N_max, Hq, d), float("nan"), dtype=dtype, device=DEV)
        lse = torch.full((B, N_max, Hq), float("nan"), dtype=torch.float32, device=DEV)
        tsv.tree_verify_attn(q, kc, vc, kt, vt, pl, n, anc, Hkv, d, 0.0884, out=out, lse=lse, ws=ws)
        torch.cuda.synchronize()
        for b, t in enumerate(trees):
            assert not torch.isnan(out[b, :t.n]).any(), (B, dtype, b)
            assert not torch.isnan(lse[b, :t.n]).any(), (B, dtype, b)
        check_attention(out, lse, q, kc, vc, kt, vt, prefix, trees, 0.0884, TOL[dtype], False, d,
                        [(b, t.n - 1) for b, t in enumerate(trees)])

    need = max(tsv.workspace_size(1, B, 1, 1, 1, N_max, 9000, Hq, Hkv, d, d, dt)
               for B in (2, 3) for dt in (tsv.TSV_F32, tsv.TSV_BF16))
    ws = tsv.workspace(need, DEV)
    # same B, N_max, Hq, Hkv: dtype, path and capacity change freely
    call(2, [700, 5000], torch.float32, 5016, ws)
    call(2, [4000, 9000 - 16], torch.bfloat16, 9000, ws)
    call(2, [300, 2000], torch.float32, 2016, ws)
    call(2, [2500, 60], torch.bfloat16, 2516, ws)
    # another B: zero the workspace first
    ws.zero_()
    call(3, [5000, 128, 3000], torch.bfloat16, 5016, ws)
    call(3, [900, 4000, 33], torch.float32, 4016, ws)
    call(3, [6000, 10, 2222], torch.bfloat16, 6016, ws)
    ws.zero_()
    call(2, [1234, 4321], torch.bfloat16, 4337, ws)


def _pitched_copy(t, pitch):
    out = tsv.kv_rows(t.shape[0], t.shape[1], tuple(t.shape[2:]), t.dtype, DEV, pitch)
    out.copy_(t)
    return out


PITCH_CASES = ["fp32_mha", "bf16_gqa_g4", "bf16_latent_mfma", "bf16_valu_d64", "bf16_many_splits",
               "bf16_gqa_paired_splits"]


@pytest.mark.parametrize("name", PITCH_CASES)
def test_pitched_rows(name):
    """Cache and scratch rows further apart than their width (the recommended
    pitch, and an arbitrary 16-byte multiple): the same bits as packed rows,
    and the oracle's values."""
    case = next(c for c in CASES if c[0] == name)
    _, B, N_max, Hq, Hkv, d_qk, d_v, dtype, prefix, n_list, mla = case
    print(f"attention case {name}, pitched rows", flush=True)
    rng = np.random.default_rng(zlib.crc32(name.encode()) + 1)
    L_cap = max(prefix) + 16
    q, kc, vc, kt, vt, pl = _inputs(rng, B, N_max, L_cap, Hq, Hkv, d_qk, d_v, dtype, prefix, mla)
    trees = _random_trees(rng, B, N_max, n_list)
    scale = 1.0 / math.sqrt(d_qk)
    o0, l0, _, _ = _run(q, kc, vc, kt, vt, pl, trees, Hkv, d_v, scale)
    width = d_qk if mla else Hkv * max(d_qk, d_v)
    es = kc.element_size()
    for pitch in (tsv.kv_row_pitch(width, es), width + 48 // es):
        kc2, kt2 = _pitched_copy(kc, pitch), _pitched_copy(kt, pitch)
        vc2, vt2 = (kc2, kt2) if mla else (_pitched_copy(vc, pitch), _pitched_copy(vt, pitch))
        o, lse, _, _ = _run(q, kc2, vc2, kt2, vt2, pl, trees, Hkv, d_v, scale)
        for b, t in enumerate(trees):
            assert torch.equal(o[b, :t.n].view(torch.int16) if dtype == torch.bfloat16 else o[b, :t.n],
                               o0[b, :t.n].view(torch.int16) if dtype == torch.bfloat16 else o0[b, :t.n])
            assert torch.equal(lse[b, :t.n], l0[b, :t.n])
        check_attention(o, lse, q, kc2, vc2, kt2, vt2, prefix, trees, scale, TOL[dtype], mla, d_v)


@pytest.mark.parametrize("cid", [2, 4])
def test_workload_recommended_pitch(cid):
    """Full-size grouped workloads with rows at the recommended pitch: the
    same bits as packed rows (whose values test_workload checks against the
    oracle), and a seeded sample of nodes against the oracle."""
    cfg = config(cid)
    pitch = tsv.kv_row_pitch(cfg.Hkv * cfg.d_qk, 2)
    print(f"attention workload {cid} {cfg.name}, row pitch {pitch}", flush=True)
    dense = attention_inputs(cfg, 0, DEV)
    ins = attention_inputs(cfg, 0, DEV, row_pitch=pitch)
    assert ins["k_cache"].stride(1) == pitch
    pl_np = ins["prefix_len"].cpu().numpy()
    marg = marginals(cfg, 0, DEV).cpu().numpy()
    _, _, trees = oracle_trees(marg, cfg.top_k, cfg.n_budget, cfg.N_max, cfg.cost, pl_np)
    runs = []
    for st in (dense, ins):
        runs.append(_run(st["q"], st["k_cache"], st["v_cache"], st["k_tree"], st["v_tree"],
                         st["prefix_len"], trees, cfg.Hkv, cfg.d_v, cfg.sm_scale))
    for b, t in enumerate(trees):
        assert torch.equal(runs[0][0][b, :t.n].view(torch.int16), runs[1][0][b, :t.n].view(torch.int16))
        assert torch.equal(runs[0][1][b, :t.n], runs[1][1][b, :t.n])
    del dense
    samples = _structured_samples(cid, trees, np.random.default_rng(cid + 100))[:64]
    worst = check_attention(runs[1][0], runs[1][1], ins["q"], ins["k_cache"], ins["v_cache"],
                            ins["k_tree"], ins["v_tree"], pl_np, trees, cfg.sm_scale,
                            TOL[cfg.torch_dtype], cfg.mla, cfg.d_v, samples)
    print(f"MARGIN workload {cid} {cfg.name} (row pitch {pitch}): max |gpu - oracle| = {worst:.3e} "
          f"over {len(samples)} nodes", flush=True)
