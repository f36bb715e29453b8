"""Throughput of one tree-structured verification round on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]
                    [--no-cpu-baseline] [--no-per-workload]

A step is one round of the whole hot path -- build_tree, tree_verify_attn,
accept_walk, commit_path (one attention layer) -- over one batch of a
workload of workloads/gen.py.  The headline (`value`) is workload 2, the
grouped-query bf16 batch: 16 requests, 32 query / 8 KV heads x 128, prefix
4096, 16 drafter positions over a 151936-token vocabulary, top-32, fixed
budget 32 (synthetic, seeded).  Inputs are resident in HBM before timing;
three copies of every large input rotate across steps so the 256 MB
last-level cache cannot serve a step from the previous one (one copy when a
copy is several GB).  Each step commits into its own copy of the prefix
lengths, so every step does identical work.

Reported: verified tree tokens/s = sum_b n_b * K / wall time of K steps
(bracketed by device synchronisation) and accepted tokens/s; the attention
entry point's roofline (HBM bandwidth on its algorithmic bytes for grouped
heads, bf16 matrix throughput on its algorithmic flops for latent heads;
HIP events around the call on the launch stream in every fourth timed step,
the only events in the timed steps, recorded without a system-scope fence), against the MI355X peak and against the peaks measured in the
same run (a 1 GiB device copy, an 8192^3 bf16 GEMM); the other calls'
durations from an untimed pass with events between all calls; the HBM bytes
one attention launch actually moves (from the committed counter summary,
when it was taken on the current kernel source); and the CPU oracle on this
host's cores (all of them, and one thread) on a sample of the same round,
each step scaled to the whole batch by its own unit.  `per_workload` repeats
all of it for workloads 1-5 (fewer steps for the large ones).

    python bench.py --attention-only --copy-calibration 256 --steps 10 --warmup 2

runs only the attention calls (after three 256 MiB device copies of known
traffic), for the FETCH_SIZE / WRITE_SIZE counter runs;
--attention-workload N does the same on workload N of workloads/gen.py
(3 = mla_bf16, 5 = long_mla, ...) and prints the mean time per call with
the achieved matrix throughput and HBM bandwidth on algorithmic flops and
bytes (for the counter runs of the other kernels' shapes).

    python bench.py --expand-workload 104 --cpu-requests 4

times build_tree_expand alone (per-node conditional expansion, workloads
101..104 of workloads/gen.py) on three rotating input copies and reports its
HBM bandwidth on algorithmic bytes, with the oracle on the first requests.

    python bench.py --cost-profile

measures the grouped attention's cost over an (n, l) grid, fits the convex
monotone C_v(n; l) and reports how much perturbing the fitted coefficients by
up to 20 % changes the adaptive budgets of workload 4.

    python bench.py --global-budget

times select_global_budget (one budget across the batch) on workload 4's
trees: 64 requests x 128 candidates against a linear-step-time table, and
unfold_chains on the same trees.

    python bench.py --compressed-state

times compress_chains and refresh_compressed (the per-chain compressed state,
block means of 4 and of 128 tokens) on workload 4's trees over scratch keys
and values of 8 KV heads x 128 (bf16).
"""

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import tree_structured_verification_amd as tsv  # noqa: E402
from tree_structured_verification_amd import _lib  # noqa: E402
from workloads import Cost, attention_inputs, config, marginals, pitched, prefix_lengths, target_logits  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak
WORKLOAD = 2
ROTATE = 3
ATTN_SAMPLE = 4   # timed steps per step whose attention call is bracketed by events
ATTN_SOURCE = os.path.join(ROOT, "tree_structured_verification_amd", "csrc", "attn.hip")
TRAFFIC_PROFILE = os.path.join(ROOT, "profiles", "tree_verify_attn_gqa_bf16_traffic.md")


class TimingEvent:
    """A HIP timing event created with hipEventDisableSystemFence: recording it
    takes a timestamp on the stream without the system-scope release that a
    default event performs (a write-back of the caches that costs the stream
    several microseconds and slows the next kernel's start).  Same interface
    as TimingEvent() for record / elapsed_time; created
    through the HIP runtime that torch has loaded."""

    FLAGS = 0x20000000   # hipEventDisableSystemFence
    _hip = None

    @classmethod
    def _rt(cls):
        if cls._hip is None:
            path = os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so")
            h = ctypes.CDLL(path if os.path.exists(path) else "libamdhip64.so.7")
            h.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            h.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            h.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = h
        return cls._hip

    def __init__(self):
        self.ev = ctypes.c_void_p()
        rc = self._rt().hipEventCreateWithFlags(ctypes.byref(self.ev), self.FLAGS)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed: {rc}")

    def record(self, stream):
        rc = self._rt().hipEventRecord(self.ev, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed: {rc}")

    def elapsed_time(self, end):
        ms = ctypes.c_float()
        rc = self._rt().hipEventElapsedTime(ctypes.byref(ms), self.ev, end.ev)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return float(ms.value)

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def measured_traffic(kv_row_bytes):
    """HBM bytes per attention launch from the committed counter summary, or
    None when it is missing or was taken on another version of the kernel
    source or another cache row pitch (the summary records both)."""
    import hashlib
    try:
        text = open(TRAFFIC_PROFILE).read()
    except OSError:
        return None
    fields = {}
    for ln in text.splitlines():
        if ":" in ln and ln.strip().startswith("- "):
            k, v = ln.strip()[2:].split(":", 1)
            fields[k.strip()] = v.strip().strip("`")
    digest = hashlib.sha256(open(ATTN_SOURCE, "rb").read()).hexdigest()
    if fields.get("attn_source_sha256") != digest or fields.get("kv_row_bytes") != str(kv_row_bytes):
        return None
    try:
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def attention_bytes(cfg, prefix, n):
    """Algorithmic bytes of one tree_verify_attn launch: every prefix K/V row
    once, every tree node's Q, scratch K/V and output once, plus lse."""
    es = 2 if cfg.dtype == "bf16" else 4
    kv_row = cfg.Hkv * (cfg.d_qk + cfg.d_v) * es if not cfg.mla else cfg.d_qk * es
    live = n > 0
    prefix_bytes = int(np.sum(prefix[live].astype(np.int64))) * kv_row
    nodes = int(np.sum(n))
    per_node = cfg.Hq * cfg.d_qk * es + kv_row + cfg.Hq * cfg.d_v * es + cfg.Hq * 4
    return prefix_bytes + nodes * per_node


KV_LAYOUT = "padded"   # set from --kv-layout


def kv_pitch(cfg):
    """Elements between cache (and scratch) rows: the library's recommended
    pitch (an odd number of 128-byte lines) or the dense row width."""
    width = cfg.d_qk if cfg.mla else cfg.Hkv * max(cfg.d_qk, cfg.d_v)
    if KV_LAYOUT == "dense":
        return width
    return tsv.kv_row_pitch(width, 2 if cfg.dtype == "bf16" else 4)


def clone_rows(t):
    """A copy of a cache or scratch tensor with the same row pitch (clone()
    would pack the rows)."""
    if t.is_contiguous():
        return t.clone()
    out = pitched(t.shape[0], t.shape[1], tuple(t.shape[2:]), t.dtype, t.device, t.stride(1))
    out.copy_(t)
    return out


def attention_only(wid, K, W, dev):
    """K timed tree_verify_attn calls (after W) on workload wid, inputs in
    three rotating copies; prints one JSON line."""
    cfg = config(wid)
    print(f"[bench] attention only, workload {cfg.name}", file=sys.stderr, flush=True)
    ins = attention_inputs(cfg, 0, dev, row_pitch=kv_pitch(cfg))
    marg = marginals(cfg, 0, dev)
    pl = ins["prefix_len"]
    tree = tsv.build_tree(marg, cfg.top_k, cfg.n_budget, cfg.N_max, cost=cfg.cost,
                          prefix_len=pl if cfg.cost is not None else None)
    del marg
    keys = ("q", "k_cache", "v_cache", "k_tree", "v_tree")
    sets = [ins] + [{k: clone_rows(ins[k]) for k in keys} for _ in range(ROTATE - 1)]
    if cfg.mla:   # one latent cache serves as key and value
        for st in sets:
            st["v_cache"], st["v_tree"] = st["k_cache"], st["k_tree"]
    B, N = cfg.B, cfg.N_max
    out = torch.empty(B, N, cfg.Hq, cfg.d_v, dtype=cfg.torch_dtype, device=dev)
    lse = torch.empty(B, N, cfg.Hq, dtype=torch.float32, device=dev)
    ws = tsv.workspace(tsv.workspace_size(1, B, 1, 1, 1, N, cfg.L_cap, cfg.Hq, cfg.Hkv,
                                          cfg.d_qk, cfg.d_v, 0 if cfg.dtype == "f32" else 1), dev)
    ev = [(TimingEvent(), TimingEvent())
          for _ in range(W + K)]
    stream = torch.cuda.current_stream(dev)
    for s in range(W + K):
        st = sets[s % ROTATE]
        ev[s][0].record(stream)
        tsv.tree_verify_attn(st["q"], st["k_cache"], st["v_cache"], st["k_tree"], st["v_tree"],
                             pl, tree["n_nodes"], tree["anc_bits"], cfg.Hkv, cfg.d_v,
                             cfg.sm_scale, out=out, lse=lse, ws=ws)
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b) for a, b in ev[W:]])) / 1e3
    n = tree["n_nodes"].cpu().numpy()
    depth = tree["depth"].cpu().numpy()
    prefix = pl.cpu().numpy().astype(np.int64)
    # each node attends to the prefix and to its ancestors (depth of them)
    pairs = sum(int(n[b]) * int(prefix[b]) + int(depth[b, :n[b]].sum()) for b in range(B))
    flops = 2.0 * pairs * cfg.Hq * (cfg.d_qk + cfg.d_v)
    nbytes = attention_bytes(cfg, prefix, n)
    print(json.dumps({"attention_workload": cfg.name, "kv_row_bytes": ins["k_cache"].stride(1) * ins["k_cache"].element_size(),
                      "calls": K, "us_per_call": round(t * 1e6, 1),
                      "tflops": round(flops / t / 1e12, 1),
                      "mfma_frac_bf16": round(flops / t / 2.5e15, 4),
                      "gbs": round(nbytes / t / 1e9, 1),
                      "hbm_frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                      "algorithmic_flops": flops, "algorithmic_bytes": nbytes}), flush=True)


def expand_bytes(cfg, n_nodes):
    """Algorithmic bytes of one build_tree_expand call: every expanded node's
    distribution read once, its top-k list written and read once, the tree
    outputs written once."""
    P, k = cfg.rows, cfg.top_k
    W = (cfg.N_max + 31) // 32
    lists = cfg.B * P * k * 8 * 2
    outputs = cfg.B * (4 + cfg.N_max * (4 * 4 + 4 * W))
    return cfg.B * P * cfg.V * 4 + lists + outputs


def expand_only(wid, K, W, dev, cpu_requests):
    """K timed build_tree_expand calls (after W) on expansion workload wid,
    inputs in three rotating copies; prints one JSON line."""
    import oracle
    from workloads import expand_config, node_distributions

    cfg = expand_config(wid)
    print(f"[bench] build_tree_expand, workload {cfg.name}", file=sys.stderr, flush=True)
    x0 = node_distributions(cfg, 0, dev)
    sets = [x0] + [x0.clone() for _ in range(ROTATE - 1)]
    B, N = cfg.B, cfg.N_max
    Wd = (N + 31) // 32
    i32 = dict(dtype=torch.int32, device=dev)
    out = dict(n_nodes=torch.empty(B, **i32), parent=torch.empty(B, N, **i32),
               token=torch.empty(B, N, **i32), depth=torch.empty(B, N, **i32),
               score=torch.empty(B, N, dtype=torch.float32, device=dev),
               anc_bits=torch.empty(B, N, Wd, **i32))
    ws = tsv.workspace(tsv.workspace_size(4, B, cfg.steps, cfg.V, cfg.top_k, N), dev)
    ev = [(TimingEvent(), TimingEvent())
          for _ in range(W + K)]
    stream = torch.cuda.current_stream(dev)
    for s in range(W + K):
        ev[s][0].record(stream)
        tsv.build_tree_expand(sets[s % ROTATE], cfg.steps, cfg.top_k, cfg.n_budget, N,
                              out=out, ws=ws)
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b) for a, b in ev[W:]])) / 1e3
    nbytes = expand_bytes(cfg, out["n_nodes"])
    n_gpu = out["n_nodes"].cpu().numpy()
    # the oracle on the first requests of the same inputs
    reqs = list(range(min(cpu_requests, B)))
    host = x0[reqs].cpu().numpy()
    t0 = time.perf_counter()
    idx, p = oracle.topk_per_position(host, cfg.top_k)
    trees = [oracle.select_tree_expand(idx[j], p[j], cfg.steps, cfg.n_budget, N)
             for j in range(len(reqs))]
    dt = time.perf_counter() - t0
    if [tr.n for tr in trees] != n_gpu[reqs].tolist():
        raise RuntimeError("oracle and GPU trees differ in size")
    print(json.dumps({
        "expand_workload": cfg.name, "B": B, "steps": cfg.steps, "top_k": cfg.top_k,
        "budget": cfg.n_budget, "V": cfg.V, "rows_per_request": cfg.rows, "calls": K,
        "us_per_call": round(t * 1e6, 1),
        "tree_nodes_per_s": round(float(n_gpu.sum()) / t, 1),
        "roofline": {"bound": "hbm", "achieved": round(nbytes / t / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4),
                     "algorithmic_bytes": nbytes},
        "cpu_baseline": {"value": round(sum(tr.n for tr in trees) / dt, 2),
                         "unit": "tree nodes/s", "cores": 1, "kind": "oracle",
                         "sample": f"top-k and tree of {len(reqs)} of the {B} requests, "
                                   f"{dt:.1f} s"}}), flush=True)


def cost_profile(dev, perturbations=20):
    """Measure C_v(n; l) of the grouped-query attention on this GPU (16
    requests, 32/8 heads x 128, bf16), fit the convex monotone model, and test
    the adaptive budget's robustness to perturbed coefficients on the adaptive
    workload's marginals; prints one JSON line."""
    import dataclasses
    from tree_structured_verification_amd.profile_cost import calibrate
    from workloads import prefix_lengths

    print("[bench] measuring tree_verify_attn over an (n, l) grid", file=sys.stderr, flush=True)
    cost, (n, l, t) = calibrate(16, 32, 8, 128, c_d=0.0)
    A = np.stack([np.ones_like(n), n, n * n, l * n, l], 1)
    coef = np.array([cost.a, cost.b, cost.c, cost.e, cost.f])
    pred = A @ coef
    r2 = 1.0 - float(np.sum((pred - t) ** 2)) / float(np.sum((t - t.mean()) ** 2))
    # drafting cost: half the verification cost of one node at the median
    # prefix, the ratio C_d / C_v(1) of the adaptive workload's coefficients
    # (the drafter itself is not here)
    lmed = float(np.median(prefix_lengths(config(4))))
    cv1 = cost.a + cost.b + cost.c + cost.e * lmed + cost.f * lmed
    base = Cost(a=cost.a, b=cost.b, c=cost.c, e=cost.e, c_d=0.5 * cv1, f=cost.f)
    cfg = config(4)
    marg = marginals(cfg, 0, dev)
    pl_np = prefix_lengths(cfg)
    pl = torch.from_numpy(pl_np).to(dev)

    def run(c):
        g = tsv.build_tree_fitted(marg, cfg.top_k, cfg.n_budget, cfg.N_max, cost=c, prefix_len=pl)
        torch.cuda.synchronize()
        return g["n_nodes"].cpu().numpy(), g["score"].cpu().numpy()

    def theta(c, scores, nb, lb):
        phi = float(np.sum(scores[:nb].astype(np.float64)))
        m = float(nb)
        return (1.0 + phi) / (c.c_d + ((((c.a + c.b * m) + c.c * (m * m)) + (c.e * lb) * m) + c.f * lb))

    n0, s0 = run(base)
    # every request's scores in best-first order up to the cap (fixed budget)
    gfull = tsv.build_tree(marg, cfg.top_k, cfg.n_budget, cfg.N_max)
    torch.cuda.synchronize()
    sfull = gfull["score"].cpu().numpy()
    rng = np.random.default_rng(0)
    changed, dn, loss = [], [], []
    for _ in range(perturbations):
        f = rng.uniform(0.8, 1.2, 6)
        pc = Cost(a=base.a * f[0], b=base.b * f[1], c=base.c * f[2], e=base.e * f[3],
                  c_d=base.c_d * f[4], f=base.f * f[5])
        n1, _ = run(pc)
        changed.append(float(np.mean(n1 != n0)))
        dn.append(float(np.mean(np.abs(n1.astype(np.int64) - n0))))
        # modelled throughput (true = unperturbed cost) at the perturbed budgets
        th0 = sum(theta(base, sfull[b], n0[b], pl_np[b]) for b in range(cfg.B))
        th1 = sum(theta(base, sfull[b], n1[b], pl_np[b]) for b in range(cfg.B))
        loss.append(1.0 - th1 / th0)
    print(json.dumps({
        "cost_profile": "tree_verify_attn, 16 requests, Hq 32 / Hkv 8 x 128, bf16",
        "unit": "us per request per call", "points": int(n.size),
        "fit": {"a": cost.a, "b": cost.b, "c": cost.c, "e": cost.e, "f": cost.f, "c_d": base.c_d,
                "r2": round(r2, 5),
                "max_rel_err": round(float(np.max(np.abs(pred - t) / t)), 4)},
        "adaptive_workload_nstar": {"mean": round(float(n0.mean()), 2), "std": round(float(n0.std()), 2),
                                    "zero": int(np.sum(n0 == 0))},
        "perturbed_20pct": {"runs": perturbations, "frac_requests_changed": round(float(np.mean(changed)), 4),
                            "mean_abs_dn": round(float(np.mean(dn)), 3),
                            "mean_modelled_throughput_loss": round(float(np.mean(loss)), 6),
                            "max_modelled_throughput_loss": round(float(np.max(loss)), 6)},
        "grid": [[float(x), float(y), round(float(z), 3)] for x, y, z in zip(n, l, t)]}), flush=True)


def compressed_state_bench(dev, K, W):
    """compress_chains (keys and values) and refresh_compressed on the
    adaptive workload's trees (64 requests x 128 best-first nodes, prefix
    lengths 1024-32768) with scratch rows of 8 KV heads x 128 in bf16, for
    blocks of 4 and of 128 tokens.  The accepted path of a request is the
    first min(4, length) nodes of its first chain.  One JSON line per block
    size; algorithmic bytes = every scratch row read once, the tails read,
    the entries written (compress) or copied, the tails rewritten and the
    accepted rows read (refresh)."""
    import oracle
    cfg = config(4)
    tree = tsv.build_tree(marginals(cfg, 0, dev), cfg.top_k, cfg.N_max, cfg.N_max)
    ch = tsv.unfold_chains(tree, cfg.gamma)
    B, N, G, E = cfg.B, cfg.N_max, cfg.gamma, cfg.Hkv * cfg.d_qk
    gen = torch.Generator(device=dev).manual_seed(7)
    rows = [torch.randn(B, N, cfg.kv_stride, generator=gen, device=dev).to(torch.bfloat16)
            for _ in range(2)]
    pl_np = prefix_lengths(cfg, 0)
    pl = torch.from_numpy(pl_np).to(dev)
    tails = [torch.randn(B, E, generator=gen, device=dev) for _ in range(2)]
    chn = {k: v.cpu().numpy() for k, v in ch.items()}
    m = np.minimum(chn["chain_len"][:, 0], 4).astype(np.int32)
    acc = np.full((B, G), -1, dtype=np.int32)
    for b in range(B):
        acc[b, :m[b]] = chn["chain_nodes"][b, 0, :m[b]]
    walk = dict(accept_len=torch.from_numpy(m).to(dev), accept_nodes=torch.from_numpy(acc).to(dev))
    n_rows = int(tree["n_nodes"].sum())
    stream = torch.cuda.current_stream(dev)
    for c in (4, 128):
        M = (c - 1 + G) // c
        ent = [torch.zeros(B, N, M, E, dtype=torch.float32, device=dev) for _ in range(2)]
        n_ent = [torch.empty(B, N, dtype=torch.int32, device=dev) for _ in range(2)]
        Lc = int(pl_np.max()) // c + G + 1
        comp = [torch.zeros(B, Lc, E, dtype=torch.float32, device=dev) for _ in range(2)]
        work_tail = [t.clone() for t in tails]
        ev = [[TimingEvent() for _ in range(3)] for _ in range(W + K)]
        for s in range(W + K):
            for i in range(2):
                work_tail[i].copy_(tails[i])
            ev[s][0].record(stream)
            for i in range(2):
                tsv.compress_chains(rows[i], c, work_tail[i], pl, ch, G, E=E, entries=ent[i],
                                    n_entries=n_ent[i])
            ev[s][1].record(stream)
            for i in range(2):
                tsv.refresh_compressed(rows[i], c, pl, walk, ch, ent[i], comp[i], work_tail[i], G, E=E)
            ev[s][2].record(stream)
        torch.cuda.synchronize()
        t_c = float(np.mean([e[0].elapsed_time(e[1]) for e in ev[W:]])) * 1e3
        t_r = float(np.mean([e[1].elapsed_time(e[2]) for e in ev[W:]])) * 1e3
        ne = n_ent[0].cpu().numpy()
        n_entries = int(ne[ne > 0].sum())
        e_acc = int(np.sum((pl_np % c + m) // c))
        bytes_c = 2 * (n_rows * E * 2 + B * E * 4 + n_entries * E * 4)
        bytes_r = 2 * (2 * e_acc * E * 4 + 2 * B * E * 4 + int(m.sum()) * E * 2)
        # the oracle on a sample of 4 requests (keys only), for the CPU baseline
        smp = 4
        rows_np = rows[0][:smp].float().cpu().numpy()[:, :, :E].astype(np.float64)
        t0 = time.perf_counter()
        oracle.compress_chains(rows_np, tails[0][:smp].cpu().numpy(), pl_np[:smp],
                               chn["n_chains"][:smp], chn["chain_len"][:smp],
                               chn["chain_nodes"][:smp], c, G)
        dt = time.perf_counter() - t0
        print(json.dumps({
            "compressed_state": f"C{c}: {B} requests x {N} nodes, {int(chn['n_chains'].sum())} chains, "
                                f"keys and values of {cfg.Hkv} heads x {cfg.d_qk} (bf16)",
            "calls": K, "compress_us": round(t_c, 2), "refresh_us": round(t_r, 2),
            "entries_per_call": 2 * n_entries,
            "compress_gbs": round(bytes_c / t_c / 1e3, 1), "compress_hbm_frac": round(bytes_c / t_c / 1e3 / 8000.0, 4),
            "compress_algorithmic_bytes": bytes_c, "refresh_algorithmic_bytes": bytes_r,
            "cpu_baseline": {"value_us": round(dt * 1e6, 1), "cores": 1, "kind": "oracle",
                             "sample": f"compress_chains of the keys of {smp} of the {B} requests"}}),
            flush=True)


def global_budget_bench(dev, K, W):
    """Time select_global_budget on the adaptive workload's trees (64
    requests, 128 best-first nodes each: the largest batch of one sort),
    against a linear-step-time engine table; prints one JSON line."""
    cfg = config(4)
    marg = marginals(cfg, 0, dev)
    base = tsv.build_tree(marg, cfg.top_k, cfg.N_max, cfg.N_max)
    torch.cuda.synchronize()
    B, M = cfg.B, cfg.B * cfg.N_max
    # engine step time 1 ms + 2 us per verified token (illustrative)
    sps = (1e6 / (1000.0 + 2.0 * torch.arange(B + M + 1, dtype=torch.float64))).to(dev)
    work = {k: v.clone() for k, v in base.items()}
    ev = [(TimingEvent(), TimingEvent())
          for _ in range(W + K)]
    stream = torch.cuda.current_stream(dev)
    for s in range(W + K):
        for k, v in base.items():
            work[k].copy_(v)
        ev[s][0].record(stream)
        tsv.select_global_budget(work, sps)
        ev[s][1].record(stream)
    torch.cuda.synchronize()
    t = float(np.mean([a.elapsed_time(b) for a, b in ev[W:]])) * 1e3
    n = work["n_nodes"].cpu().numpy()
    # the oracle on the same trees
    import oracle
    host = {k: v.cpu().numpy() for k, v in base.items()}
    t0 = time.perf_counter()
    want = oracle.global_budget(host["score"], host["n_nodes"], sps.cpu().numpy())
    dt = time.perf_counter() - t0
    if not np.array_equal(want, n):
        raise RuntimeError("oracle and GPU budgets differ")
    # the same trees unfolded into their chains (per-round metadata)
    evc = [(TimingEvent(), TimingEvent())
           for _ in range(W + K)]
    for s in range(W + K):
        evc[s][0].record(stream)
        ch = tsv.unfold_chains(base, cfg.gamma)
        evc[s][1].record(stream)
    torch.cuda.synchronize()
    tc = float(np.mean([a.elapsed_time(b) for a, b in evc[W:]])) * 1e3
    print(json.dumps({"unfold_chains": f"{B} requests x {cfg.N_max} nodes (adaptive workload "
                      "trees, fixed budget 128)", "calls": K, "us_per_call": round(tc, 2),
                      "chains": int(ch["n_chains"].sum())}), flush=True)
    print(json.dumps({"global_budget": f"{B} requests x {cfg.N_max} candidates "
                      "(adaptive workload trees), engine step 1000 + 2 B us",
                      "calls": K, "us_per_call": round(t, 2), "admitted": int(n.sum()),
                      "requests_with_nodes": int(np.sum(n > 0)),
                      "cpu_baseline": {"value_us_per_call": round(dt * 1e6, 1), "cores": 1,
                                       "kind": "oracle", "sample": "the same call, once"}}),
          flush=True)


def copy_peak_gbs(dev, mib=1024, reps=8):
    """Measured device-to-device copy bandwidth (read + write bytes per
    second) of torch's copy kernel on two buffers of `mib` MiB, far larger
    than the 256 MB last-level cache; the best of `reps` copies."""
    nb = mib << 20
    src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ev = [(TimingEvent(), TimingEvent())
          for _ in range(reps)]
    stream = torch.cuda.current_stream(dev)
    for a, b in ev:
        a.record(stream)
        dst.copy_(src)
        b.record(stream)
    torch.cuda.synchronize()
    best = min(a.elapsed_time(b) for a, b in ev) / 1e3
    del src, dst
    return 2.0 * nb / best / 1e9


def read_peak_gbs(dev, mib=1024, reps=8):
    """Measured read-only bandwidth: torch's int64 sum over `mib` MiB (far
    larger than the 256 MB last-level cache; its float reductions are slower
    than the memory), the best of `reps` calls."""
    nb = mib << 20
    x = torch.ones(nb // 8, dtype=torch.int64, device=dev)
    x.sum()
    ev = [(TimingEvent(), TimingEvent())
          for _ in range(reps)]
    stream = torch.cuda.current_stream(dev)
    for a, b in ev:
        a.record(stream)
        x.sum()
        b.record(stream)
    torch.cuda.synchronize()
    best = min(a.elapsed_time(b) for a, b in ev) / 1e3
    del x
    return nb / best / 1e9


def gemm_peak_tflops(dev, n=8192, reps=5):
    """Measured dense bf16 matrix throughput of the vendor GEMM (torch.matmul,
    n x n x n), the best of `reps` calls."""
    a = torch.randn(n, n, device=dev).to(torch.bfloat16)
    b = torch.randn(n, n, device=dev).to(torch.bfloat16)
    c = a @ b
    ev = [(TimingEvent(), TimingEvent())
          for _ in range(reps)]
    stream = torch.cuda.current_stream(dev)
    for e0, e1 in ev:
        e0.record(stream)
        torch.matmul(a, b, out=c)
        e1.record(stream)
    torch.cuda.synchronize()
    best = min(e0.elapsed_time(e1) for e0, e1 in ev) / 1e3
    del a, b, c
    return 2.0 * n ** 3 / best / 1e12


def attention_flops(cfg, n, depth, prefix):
    """Algorithmic matrix flops of one attention launch: every tree node
    attends to its request's prefix and to its ancestors and itself (depth of
    them), for every query head, scores and weighted values."""
    pairs = sum(int(n[b]) * int(prefix[b]) + int(depth[b, :n[b]].sum()) for b in range(cfg.B))
    return 2.0 * pairs * cfg.Hq * (cfg.d_qk + cfg.d_v)


def round_bench(wid, K, W, dev):
    """K timed rounds (after W) of workload wid: build_tree, tree_verify_attn,
    accept_walk and commit_path on inputs resident in HBM.  Returns a dict of
    measurements and host copies the CPU baseline needs."""
    cfg = config(wid)
    L = _lib.lib()
    dt = tsv.TSV_F32 if cfg.dtype == "f32" else tsv.TSV_BF16
    adaptive = cfg.cost is not None
    print(f"[bench] generating workload {cfg.name}", file=sys.stderr, flush=True)
    marg0 = marginals(cfg, 0, dev)
    ins0 = attention_inputs(cfg, 0, dev, row_pitch=kv_pitch(cfg))
    prefix0 = ins0["prefix_len"].clone()
    # the workload's tree (deterministic) lays out the target rows
    tree0 = tsv.build_tree(marg0, cfg.top_k, cfg.n_budget, cfg.N_max, cost=cfg.cost,
                           prefix_len=prefix0 if adaptive else None)
    torch.cuda.synchronize()
    depth0 = tree0["depth"].cpu().numpy()
    n0 = tree0["n_nodes"].cpu().numpy()
    tl0 = target_logits(cfg, 0, depth0, n0, dev)
    big = [marg0, ins0["q"], ins0["k_cache"], ins0["k_tree"], tl0]
    if not cfg.mla:
        big += [ins0["v_cache"], ins0["v_tree"]]
    per_copy = sum(t.numel() * t.element_size() for t in big)   # bytes in use
    # rotating copies keep the 256 MB last-level cache from serving a step
    # from the previous one; one copy of several GB already does that
    copies = ROTATE if per_copy < (4 << 30) else 1
    sets = []
    for r in range(copies):
        c = (lambda t: t) if r == 0 else (lambda t: t.clone())
        cr = (lambda t: t) if r == 0 else clone_rows
        st = dict(marg=c(marg0), q=c(ins0["q"]), kc=cr(ins0["k_cache"]), kt=cr(ins0["k_tree"]),
                  tl=c(tl0))
        st["vc"] = st["kc"] if cfg.mla else cr(ins0["v_cache"])
        st["vt"] = st["kt"] if cfg.mla else cr(ins0["v_tree"])
        sets.append(st)
    prefixes = [prefix0.clone() for _ in range(K + W)]

    B, N, Wd = cfg.B, cfg.N_max, (cfg.N_max + 31) // 32
    i32 = dict(dtype=torch.int32, device=dev)
    tr = dict(n_nodes=torch.empty(B, **i32), parent=torch.empty(B, N, **i32),
              token=torch.empty(B, N, **i32), depth=torch.empty(B, N, **i32),
              score=torch.empty(B, N, dtype=torch.float32, device=dev),
              anc_bits=torch.empty(B, N, Wd, **i32))
    out = torch.empty(B, N, cfg.Hq, cfg.d_v, dtype=cfg.torch_dtype, device=dev)
    lse = torch.empty(B, N, cfg.Hq, dtype=torch.float32, device=dev)
    wk = dict(accept_len=torch.empty(B, **i32), accept_nodes=torch.empty(B, cfg.gamma, **i32),
              out_tokens=torch.empty(B, cfg.gamma + 1, **i32))
    status = torch.empty(B, **i32)
    ws_b = tsv.workspace(tsv.workspace_size(0, B, cfg.gamma, cfg.V, cfg.top_k, N), dev)
    ws_a = tsv.workspace(tsv.workspace_size(1, B, 1, 1, 1, N, cfg.L_cap, cfg.Hq, cfg.Hkv,
                                            cfg.d_qk, cfg.d_v, dt), dev)
    ws_w = tsv.workspace(tsv.workspace_size(2, B, cfg.gamma, cfg.V, 1, N, dtype=dt), dev)
    cost = None
    if adaptive:
        cost = tsv.tsv_cost(cfg.cost.a, cfg.cost.b, cfg.cost.c, cfg.cost.e, cfg.cost.c_d)

    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    stride = ins0["k_cache"].stride(1)
    for st in sets:
        if {st[k].stride(1) for k in ("kc", "vc", "kt", "vt")} != {stride}:
            raise RuntimeError("rotating copies lost the row pitch")

    # pre-marshalled argument tuples: the timed loop only calls the library
    def step_args(s):
        st = sets[s % copies]
        pl = prefixes[s]
        a_build = (P(st["marg"]), B, cfg.gamma, cfg.V, cfg.top_k, cfg.n_budget,
                   ctypes.byref(cost) if adaptive else None, P(pl) if adaptive else None, N,
                   P(tr["n_nodes"]), P(tr["parent"]), P(tr["token"]), P(tr["depth"]),
                   P(tr["score"]), P(tr["anc_bits"]), P(ws_b), ws_b.numel(), sp)
        a_attn = (P(st["q"]), P(st["kc"]), P(st["vc"]), P(st["kt"]), P(st["vt"]), stride,
                  P(pl), P(tr["n_nodes"]), P(tr["anc_bits"]), B, N, cfg.L_cap, cfg.Hq, cfg.Hkv,
                  cfg.d_qk, cfg.d_v, dt, ctypes.c_float(cfg.sm_scale), P(out), P(lse),
                  P(ws_a), ws_a.numel(), sp)
        a_walk = (P(st["tl"]), dt, B, N, cfg.V, cfg.gamma, P(tr["n_nodes"]),
                  P(tr["parent"]), P(tr["token"]), P(wk["accept_len"]), P(wk["accept_nodes"]),
                  P(wk["out_tokens"]), P(ws_w), ws_w.numel(), sp)
        # a latent cache commits its rows once (no separate value rows)
        a_commit = (P(st["kc"]), None if cfg.mla else P(st["vc"]), P(pl), P(st["kt"]),
                    None if cfg.mla else P(st["vt"]), stride, P(wk["accept_len"]),
                    P(wk["accept_nodes"]), B, N, cfg.L_cap, cfg.Hkv, cfg.d_qk, cfg.d_v,
                    cfg.gamma, dt, P(status), sp)
        return a_build, a_attn, a_walk, a_commit

    all_args = [step_args(s) for s in range(K + W)]
    ev = [[TimingEvent() for _ in range(5)] for _ in range(K + W)]

    # Every ATTN_SAMPLE-th timed step records the two events around the
    # attention call, the only events in the timed steps: an event marker
    # between two kernels costs the stream about 4.5 us even without a
    # system-scope fence, so the other steps run without them.  The other
    # calls' durations come from a separate, untimed pass.
    def run(s, all_events=False):
        a_build, a_attn, a_walk, a_commit = all_args[s]
        e = ev[s]
        sampled = all_events or (s - W) % ATTN_SAMPLE == 0
        if all_events:
            e[0].record(stream)
        rc = L.build_tree(*a_build)
        if sampled:
            e[1].record(stream)
        rc |= L.tree_verify_attn(*a_attn)
        if sampled:
            e[2].record(stream)
        rc |= L.accept_walk(*a_walk)
        if all_events:
            e[3].record(stream)
        rc |= L.commit_path(*a_commit)
        if all_events:
            e[4].record(stream)
        return rc

    print(f"[bench] {cfg.name}: warmup {W} steps", file=sys.stderr, flush=True)
    for s in range(W):
        if run(s) != 0:
            raise RuntimeError("library call failed during warmup")
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name}: timing {K} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    rc = 0
    for s in range(W, W + K):
        rc |= run(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if rc != 0:
        raise RuntimeError("library call failed in the timed loop")
    if not bool((status == 0).all()):
        raise RuntimeError("commit reported a non-zero status")

    ms = lambda a, b, steps: np.array([ev[s][a].elapsed_time(ev[s][b]) for s in steps])
    t_attn = ms(1, 2, range(W, W + K, ATTN_SAMPLE))
    # per-call durations of the other entry points: an untimed pass of a few
    # steps with an event between every call (the steps' inputs are reused;
    # their prefix-length copies are restored first)
    Pp = list(range(W, W + min(K, 20)))
    for s in Pp:
        prefixes[s].copy_(prefix0)
    torch.cuda.synchronize()
    for s in Pp:
        if run(s, all_events=True) != 0:
            raise RuntimeError("library call failed in the per-call timing pass")
    torch.cuda.synchronize()
    t_build, t_walk, t_commit = ms(0, 1, Pp), ms(2, 3, Pp), ms(3, 4, Pp)
    n_np = tr["n_nodes"].cpu().numpy()
    if not np.array_equal(n_np, n0):
        raise RuntimeError("the timed rounds built other trees than the workload's")
    prefix_np = prefix0.cpu().numpy().astype(np.int64)
    depth_np = tr["depth"].cpu().numpy()
    tokens = int(n_np.sum())
    accepted = int(wk["accept_len"].cpu().numpy().sum()) + B
    attn_s = float(np.mean(t_attn)) / 1e3
    res = dict(cfg=cfg, K=K, W=W, wall=wall, tokens=tokens, accepted=accepted,
               value=tokens * K / wall, accepted_per_s=accepted * K / wall,
               round_us=wall / K * 1e6, copies=copies,
               kernel_ms={"build_tree": float(np.mean(t_build)),
                          "tree_verify_attn": float(np.mean(t_attn)),
                          "accept_walk": float(np.mean(t_walk)),
                          "commit_path": float(np.mean(t_commit))},
               attn_s=attn_s, attn_bytes=attention_bytes(cfg, prefix_np, n_np),
               kv_row_bytes=stride * ins0["k_cache"].element_size(),
               attn_flops=attention_flops(cfg, n_np, depth_np, prefix_np),
               n=n_np, prefix=prefix_np, depth=depth_np)
    res["sets0"] = sets[0]
    res["marg0"] = marg0
    return res


def host_sample(res, reqs):
    """Host copies of the inputs of requests `reqs` (first rotating copy)."""
    cfg, st = res["cfg"], res["sets0"]
    f32 = lambda t: (t.float() if t.dtype == torch.bfloat16 else t).cpu().numpy()
    lmax = int(res["prefix"][reqs].max()) + cfg.gamma
    h = dict(marg=res["marg0"][reqs].cpu().numpy(), q=f32(st["q"][reqs]),
             kc=f32(st["kc"][reqs, :lmax]), kt=f32(st["kt"][reqs]), tl=f32(st["tl"][reqs]))
    h["vc"] = None if cfg.mla else f32(st["vc"][reqs, :lmax])
    h["vt"] = None if cfg.mla else f32(st["vt"][reqs])
    return h


def oracle_round(cfg, h, prefix_np, n_gpu, depth_gpu, reqs, node_cap, threads):
    """One round of the oracle over requests `reqs` of the workload (host
    copies h), with attention on the first node_cap nodes of each, BLAS on
    `threads` threads.  Every step is timed and scaled to the whole batch by
    its own unit (marginal rows, requests, node x key pairs, verified rows,
    requests); returns (tokens/s of the whole round, sample description)."""
    import oracle
    from oracle.attention import latent_as_heads
    from threadpoolctl import threadpool_limits

    r = len(reqs)
    with threadpool_limits(limits=threads):
        t0 = time.perf_counter()
        idx, p = oracle.topk_per_position(h["marg"], cfg.top_k)
        t_topk = time.perf_counter() - t0
        t0 = time.perf_counter()
        trees = [oracle.select_tree(idx[j], p[j], cfg.n_budget, cfg.N_max, cfg.cost,
                                    int(prefix_np[b])) for j, b in enumerate(reqs)]
        t_tree = time.perf_counter() - t0
        if [t.n for t in trees] != [int(n_gpu[b]) for b in reqs]:
            raise RuntimeError("oracle and GPU trees differ in size")
        pairs_s = 0
        t0 = time.perf_counter()
        for j, b in enumerate(reqs):
            t = trees[j]
            lb = int(prefix_np[b])
            nodes = list(range(min(t.n, node_cap)))
            if not nodes:
                continue
            if cfg.mla:
                Kc, Vc = latent_as_heads(h["kc"][j, :lb], cfg.d_v)
                Kt, Vt = latent_as_heads(h["kt"][j], cfg.d_v)
            else:
                Kc, Vc, Kt, Vt = h["kc"][j, :lb], h["vc"][j, :lb], h["kt"][j], h["vt"][j]
            oracle.attend_request(h["q"][j], Kc, Vc, Kt, Vt, lb, t.n, t.parent, cfg.sm_scale,
                                  nodes=nodes)
            pairs_s += sum(lb + int(t.depth[i]) for i in nodes)
        t_attn = time.perf_counter() - t0
        t0 = time.perf_counter()
        alen = np.zeros(r, np.int32)
        anodes = np.full((r, cfg.gamma), -1, np.int32)
        for j, t in enumerate(trees):
            m, nodes, _ = oracle.accept_walk(h["tl"][j], t.n, t.parent, t.token, cfg.gamma)
            alen[j], anodes[j] = m, nodes
        t_walk = time.perf_counter() - t0
        t0 = time.perf_counter()
        pl = prefix_np[reqs].copy()
        oracle.commit_path(h["kc"], h["vc"], pl, h["kt"], h["vt"], alen, anodes, cfg.gamma)
        t_commit = time.perf_counter() - t0
    B = cfg.B
    pairs_all = int(sum(int(n_gpu[b]) * int(prefix_np[b]) + int(depth_gpu[b, :n_gpu[b]].sum())
                        for b in range(B)))
    rows_s = sum(1 + t.n for t in trees)
    rows_all = int(np.sum(1 + n_gpu))
    est = (t_topk * B / r + t_tree * B / r
           + (t_attn * pairs_all / pairs_s if pairs_s else 0.0)
           + t_walk * rows_all / rows_s + t_commit * B / r)
    spent = t_topk + t_tree + t_attn + t_walk + t_commit
    desc = (f"top-k, tree, walk and commit of {r} of the {B} requests, attention of "
            f"{'all' if node_cap >= cfg.N_max else f'at most {node_cap}'} nodes of each "
            f"({pairs_s} node x key pairs of {pairs_all}); {spent:.1f} s measured, each step "
            f"scaled to the batch by its unit (rows, requests, node x key pairs, verified rows)")
    return int(n_gpu.sum()) / est, desc


# per workload: requests the oracle runs and the attention nodes per request
# (bounded so the sample costs seconds, not minutes), and timed steps
CPU_SAMPLE = {1: ([0], 8), 2: (list(range(8)), 32), 3: ([0, 1], 4), 4: (None, 3), 5: ([0], 2)}
PER_WORKLOAD_STEPS = {1: (50, 10), 2: (20, 5), 3: (10, 3), 4: (10, 3), 5: (5, 2)}


def cpu_cores():
    """Host cores the oracle may use: this process's affinity set, within the
    thread count the environment grants (OMP_NUM_THREADS)."""
    n = len(os.sched_getaffinity(0))
    try:
        n = min(n, int(os.environ.get("OMP_NUM_THREADS", n)))
    except ValueError:
        pass
    return max(1, n)


def cpu_baseline(res, cores, one_thread=True):
    cfg = res["cfg"]
    reqs, cap = CPU_SAMPLE[cfg.id]
    if reqs is None:   # ragged: the first requests that verify a tree
        reqs = [int(b) for b in np.nonzero(res["n"] > 0)[0][:2]]
    h = host_sample(res, reqs)
    value, desc = oracle_round(cfg, {k: (None if v is None else v.copy()) for k, v in h.items()},
                               res["prefix"], res["n"], res["depth"], reqs, cap, cores)
    out = {"value": round(value, 2), "unit": "tokens/s", "cores": cores, "kind": "oracle",
           "sample": desc}
    if one_thread:
        v1, _ = oracle_round(cfg, h, res["prefix"], res["n"], res["depth"], reqs, cap, 1)
        out["value_1thread"] = round(v1, 2)
    return out


def attention_roofline(res, copy_gbs, gemm_tflops, read_gbs=None):
    """Roofline of the attention launch: HBM for the grouped workloads, the
    bf16 matrix peak for the latent ones; also against the measured peaks
    (device copy and, for HBM, a read-only stream)."""
    cfg = res["cfg"]
    t = res["attn_s"]
    if cfg.mla:
        a = res["attn_flops"] / t / 1e12
        return {"bound": "mfma", "achieved": round(a, 1), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(a / MFMA_PEAK_TFLOPS, 4),
                "measured_peak": round(gemm_tflops, 1),
                "frac_of_measured": round(a / gemm_tflops, 4),
                "algorithmic_flops": res["attn_flops"]}
    a = res["attn_bytes"] / t / 1e9
    r = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
         "frac": round(a / HBM_PEAK_GBS, 4), "measured_peak": round(copy_gbs, 1),
         "frac_of_measured": round(a / copy_gbs, 4), "algorithmic_bytes": res["attn_bytes"]}
    if read_gbs:
        r["measured_read_peak"] = round(read_gbs, 1)
        r["frac_of_read_peak"] = round(a / read_gbs, 4)
    return r


def workload_desc(cfg):
    if cfg.mla:
        heads = f"{cfg.Hq} heads x latent {cfg.d_qk}/{cfg.d_v}"
    else:
        heads = f"Hq {cfg.Hq} / Hkv {cfg.Hkv} x {cfg.d_qk}"
    pre = (f"prefix {cfg.prefix_range[0]}-{cfg.prefix_range[1]}" if cfg.prefix_range
           else f"prefix {cfg.prefix}")
    bud = (f"adaptive budget (cap {cfg.n_budget})" if cfg.cost is not None
           else f"fixed budget {cfg.n_budget}")
    return (f"{cfg.name}: {cfg.B} requests, {heads}, {pre}, gamma {cfg.gamma}, V {cfg.V}, "
            f"top-{cfg.top_k}, {bud}, {cfg.dtype}")


def workload_entry(res, copy_gbs, gemm_tflops, cores, with_cpu, read_gbs=None):
    cfg = res["cfg"]
    e = {"workload": workload_desc(cfg), "steps": res["K"], "round_us": round(res["round_us"], 1),
         "tokens_per_s": round(res["value"], 1),
         "accepted_tokens_per_s": round(res["accepted_per_s"], 1),
         "tree_tokens": res["tokens"], "input_copies": res["copies"],
         "kv_row_bytes": res["kv_row_bytes"],
         "kernel_us": {k: round(v * 1e3, 1) for k, v in res["kernel_ms"].items()},
         "attention": attention_roofline(res, copy_gbs, gemm_tflops, read_gbs)}
    if with_cpu:
        print(f"[bench] timing the CPU oracle on {cfg.name}", file=sys.stderr, flush=True)
        e["cpu_baseline"] = cpu_baseline(res, cores)
    return e


def free(res):
    for k in ("sets0", "marg0"):
        res.pop(k, None)
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=WORKLOAD, metavar="N",
                    help="workload of the headline round (1..5 of workloads/gen.py)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-per-workload", action="store_true",
                    help="time only the headline workload")
    ap.add_argument("--kv-layout", choices=("padded", "dense"), default="padded",
                    help="cache and scratch rows at the library's recommended pitch (an odd "
                         "number of 128-byte lines) or packed")
    ap.add_argument("--attention-only", action="store_true",
                    help="run only the tree_verify_attn calls of the headline workload "
                         "(for counter runs)")
    ap.add_argument("--attention-workload", type=int, default=0, metavar="N",
                    help="time only tree_verify_attn on workload N (implies --attention-only)")
    ap.add_argument("--expand-workload", type=int, default=0, metavar="N",
                    help="time only build_tree_expand on expansion workload N "
                         "(101..104 of workloads/gen.py)")
    ap.add_argument("--cpu-requests", type=int, default=4,
                    help="requests of an expansion workload the CPU oracle runs")
    ap.add_argument("--global-budget", action="store_true",
                    help="time select_global_budget on the adaptive workload's trees")
    ap.add_argument("--compressed-state", action="store_true",
                    help="time compress_chains and refresh_compressed on the adaptive workload's trees")
    ap.add_argument("--cost-profile", action="store_true",
                    help="measure and fit the verification cost C_v(n; l) and test the "
                         "adaptive budget's robustness to perturbed coefficients")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first copy MIB MiB three times between device buffers, so that "
                         "byte counters can be scaled by a kernel of known traffic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the library runs on one GPU; sharding is described, not built)", file=sys.stderr)
        sys.exit(2)

    global KV_LAYOUT
    KV_LAYOUT = args.kv_layout
    dev = torch.device("cuda:0")
    if args.copy_calibration > 0:
        nb = args.copy_calibration << 20
        bufs = [torch.ones(nb, dtype=torch.uint8, device=dev) for _ in range(6)]
        for i in range(3):
            bufs[2 * i + 1].copy_(bufs[2 * i])
        torch.cuda.synchronize()
        del bufs
    if args.attention_only and not args.attention_workload:
        args.attention_workload = args.workload
    if args.attention_workload:
        attention_only(args.attention_workload, args.steps, args.warmup, dev)
        return
    if args.cost_profile:
        cost_profile(dev)
        return
    if args.global_budget:
        global_budget_bench(dev, args.steps, args.warmup)
        return
    if args.compressed_state:
        compressed_state_bench(dev, args.steps, args.warmup)
        return
    if args.expand_workload:
        expand_only(args.expand_workload, args.steps, args.warmup, dev, args.cpu_requests)
        return

    print(f"[bench] device {torch.cuda.get_device_name(dev)}", file=sys.stderr, flush=True)
    copy_gbs = copy_peak_gbs(dev)
    read_gbs = read_peak_gbs(dev)
    gemm_tflops = gemm_peak_tflops(dev)
    print(f"[bench] measured copy {copy_gbs:.0f} GB/s, read {read_gbs:.0f} GB/s, "
          f"bf16 GEMM {gemm_tflops:.0f} TFLOP/s", file=sys.stderr, flush=True)
    cores = cpu_cores()
    with_cpu = not args.no_cpu_baseline

    head = round_bench(args.workload, args.steps, args.warmup, dev)
    cfg = head["cfg"]
    roof = attention_roofline(head, copy_gbs, gemm_tflops, read_gbs)
    roof["traffic"] = measured_traffic(head["kv_row_bytes"]) if cfg.id == WORKLOAD else None
    roof["kernel"] = "tree_verify_attn"
    line = {
        "metric": "verified tree tokens/s per GPU",
        "value": round(head["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["wall"] / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if cfg.dtype == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": workload_desc(cfg), "B": cfg.B, "gamma": cfg.gamma, "V": cfg.V,
                   "top_k": cfg.top_k, "budget": cfg.n_budget, "prefix": cfg.prefix,
                   "Hq": cfg.Hq, "Hkv": cfg.Hkv, "head_dim": cfg.d_qk,
                   "kv_row_bytes": head["kv_row_bytes"]},
        "accepted_tokens_per_s": round(head["accepted_per_s"], 1),
        "kernel_ms": {k: round(v, 4) for k, v in head["kernel_ms"].items()},
        "roofline": roof,
        "measured_peaks": {"copy_gbs": round(copy_gbs, 1), "read_gbs": round(read_gbs, 1),
                           "gemm_bf16_tflops": round(gemm_tflops, 1)},
    }
    if with_cpu:
        print(f"[bench] timing the CPU oracle on {cfg.name}", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(head, cores)
    per = {}
    if not args.no_per_workload:
        per[cfg.name] = workload_entry(head, copy_gbs, gemm_tflops, cores, False, read_gbs)
        if with_cpu:
            per[cfg.name]["cpu_baseline"] = line["cpu_baseline"]
    free(head)
    if not args.no_per_workload:
        for wid in (1, 2, 3, 4, 5):
            if wid == cfg.id:
                continue
            K, W = PER_WORKLOAD_STEPS[wid]
            res = round_bench(wid, K, W, dev)
            per[res["cfg"].name] = workload_entry(res, copy_gbs, gemm_tflops, cores, with_cpu, read_gbs)
            free(res)
        line["per_workload"] = per
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
