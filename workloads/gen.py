"""Seeded synthetic workloads shaped like the pages' workloads.

No dataset or trained model is available, so every tensor of a verification
round is drawn from a seeded generator with the shapes and value
distributions of five workloads:

  1 tiny_fp32        1 request, vocabulary 16, 4 drafter positions, 8 heads x 64,
                     prefix 256, fixed budget 8, fp32
  2 gqa_bf16         Qwen3-8B-like grouped-query attention (32 query / 8 KV heads
                     x 128), 16 requests, prefix 4096, 16 positions over
                     vocabulary 151936, fixed budget 32, bf16
  3 mla_bf16         DeepSeek-style latent attention (128 heads sharing one 576-wide
                     latent, value width 512), 32 requests, prefix 8192,
                     top-2 over 8 positions, budget 16, vocabulary 129280, bf16
  4 adaptive_ragged  64 requests, GQA 32/8 x 128, prefix lengths uniform in
                     [1024, 32768], per-request temperature in [0.5, 2],
                     budget chosen per round by the cost-aware stop rule
                     (cap 128), bf16
  5 long_mla         8 requests, latent attention as in 3, prefix 65536,
                     top-4 over 16 positions, budget 128, bf16

and, for trees built by per-node conditional expansion (every expanded node
has its own next-token distribution over the 129280-token vocabulary of 3/5):

  101 s3_k2_d6       4 requests, 3 steps, top-2, budget 6
  102 s4_k2_d5       16 requests, 4 steps, top-2, budget 5
  103 s5_k2_d8       64 requests, 5 steps, top-2, budget 8
  104 s3_k2_d6_b64   64 requests, 3 steps, top-2, budget 6

Recipe (identical for every workload):
  * drafter logits ~ N(0, sigma) per (request, position, token), drawn in fp64;
    sigma is a standard deviation;
  * marginals = softmax(logits / T_b) in fp64, then rounded to fp32 (T_b = 1
    except workload 4);
  * queries, prefix keys/values and scratch (tree) keys/values ~ N(0, 1),
    drawn in fp32 and rounded to the workload dtype (bf16 round-to-nearest-even);
    cache rows at or beyond a request's prefix length are zero;
  * target logits for a verified row: the untempered drafter logits of the
    position that row predicts, plus fresh N(0, 1) noise; row 0 (the root)
    predicts position 0, row 1+i (tree node i at depth d) predicts position
    min(d, gamma-1).  The caller supplies the tree's depths, so this module
    never builds a tree itself.

Random streams: every tensor of every request has its own torch generator
seeded from numpy's SeedSequence([seed, workload, tensor id, request]), so any
request can be regenerated on its own.  Values depend on the device the
generator runs on (CPU and GPU generators differ); a test that compares the
GPU path with the oracle draws once and hands copies of the same tensors to
both sides.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Cost:
    """Round-cost coefficients: C(n; l) = c_d + a + b*n + c*n^2 + e*l*n + f*l."""

    a: float
    b: float
    c: float
    e: float
    c_d: float
    f: float = 0.0


@dataclasses.dataclass(frozen=True)
class Config:
    id: int
    name: str
    B: int
    gamma: int
    V: int
    sigma: float
    top_k: int
    n_budget: int          # fixed budget, or cap of the adaptive budget
    N_max: int
    Hq: int
    Hkv: int
    d_qk: int
    d_v: int
    kv_stride: int         # elements between consecutive token rows
    mla: bool              # one latent row serves as K (all d_qk) and V (first d_v)
    prefix: int            # fixed prefix length (ignored if prefix_range)
    prefix_range: Optional[tuple] = None
    temp_range: Optional[tuple] = None
    cost: Optional[Cost] = None
    dtype: str = "bf16"

    @property
    def L_cap(self) -> int:
        top = self.prefix_range[1] if self.prefix_range else self.prefix
        return top + self.gamma

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d_qk)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CFG4_COST = Cost(a=1.0, b=0.02, c=1e-4, e=1e-6, c_d=0.5)

CONFIGS = {
    1: Config(1, "tiny_fp32", B=1, gamma=4, V=16, sigma=2.0, top_k=8, n_budget=8,
              N_max=8, Hq=8, Hkv=8, d_qk=64, d_v=64, kv_stride=8 * 64, mla=False,
              prefix=256, dtype="f32"),
    2: Config(2, "gqa_bf16", B=16, gamma=16, V=151936, sigma=3.0, top_k=32,
              n_budget=32, N_max=32, Hq=32, Hkv=8, d_qk=128, d_v=128,
              kv_stride=8 * 128, mla=False, prefix=4096),
    3: Config(3, "mla_bf16", B=32, gamma=8, V=129280, sigma=3.0, top_k=2,
              n_budget=16, N_max=16, Hq=128, Hkv=1, d_qk=576, d_v=512,
              kv_stride=576, mla=True, prefix=8192),
    4: Config(4, "adaptive_ragged", B=64, gamma=16, V=151936, sigma=3.0,
              top_k=128, n_budget=128, N_max=128, Hq=32, Hkv=8, d_qk=128,
              d_v=128, kv_stride=8 * 128, mla=False, prefix=0,
              prefix_range=(1024, 32768), temp_range=(0.5, 2.0), cost=CFG4_COST),
    5: Config(5, "long_mla", B=8, gamma=16, V=129280, sigma=3.0, top_k=4,
              n_budget=128, N_max=128, Hq=128, Hkv=1, d_qk=576, d_v=512,
              kv_stride=576, mla=True, prefix=65536),
}

# tensor ids of the random streams
_T_DRAFT, _T_TEMP, _T_PREFIX, _T_Q, _T_K, _T_V, _T_KT, _T_VT, _T_NOISE = range(9)


def config(cfg_id: int, **overrides) -> Config:
    cfg = CONFIGS[cfg_id]
    return cfg.replace(**overrides) if overrides else cfg


def _seed(seed: int, cfg: Config, tensor: int, b: int = 0) -> int:
    ss = np.random.SeedSequence([int(seed), int(cfg.id), int(tensor), int(b)])
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def _gen(seed: int, cfg: Config, tensor: int, b: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(seed, cfg, tensor, b))
    return g


def _randn(shape, seed, cfg, tensor, b, device, dtype=torch.float32) -> torch.Tensor:
    return torch.randn(shape, generator=_gen(seed, cfg, tensor, b, device),
                       device=device, dtype=dtype)


def prefix_lengths(cfg: Config, seed: int = 0) -> np.ndarray:
    """Persistent prefix length per request (it includes the root token)."""
    if cfg.prefix_range is None:
        return np.full(cfg.B, cfg.prefix, dtype=np.int32)
    rng = np.random.default_rng(np.random.SeedSequence([seed, cfg.id, _T_PREFIX]))
    lo, hi = cfg.prefix_range
    return rng.integers(lo, hi + 1, size=cfg.B).astype(np.int32)


def temperatures(cfg: Config, seed: int = 0) -> np.ndarray:
    if cfg.temp_range is None:
        return np.ones(cfg.B, dtype=np.float64)
    rng = np.random.default_rng(np.random.SeedSequence([seed, cfg.id, _T_TEMP]))
    lo, hi = cfg.temp_range
    return rng.uniform(lo, hi, size=cfg.B)


def drafter_logits(cfg: Config, seed: int, b: int, device="cpu") -> torch.Tensor:
    """Untempered drafter logits of request b, fp64 [gamma, V], ~ N(0, sigma)."""
    x = _randn((cfg.gamma, cfg.V), seed, cfg, _T_DRAFT, b, device, torch.float64)
    return x * cfg.sigma


def marginals(cfg: Config, seed: int = 0, device="cpu") -> torch.Tensor:
    """Drafter per-position marginals, fp32 [B, gamma, V]."""
    temps = temperatures(cfg, seed)
    out = torch.empty((cfg.B, cfg.gamma, cfg.V), dtype=torch.float32, device=device)
    for b in range(cfg.B):
        lg = drafter_logits(cfg, seed, b, device) / float(temps[b])
        out[b] = torch.softmax(lg, dim=-1).to(torch.float32)
    return out


@dataclasses.dataclass(frozen=True)
class ExpandConfig:
    """Inputs of a tree built by per-node conditional expansion: s draft steps,
    top-k per node, budget D (the review's s<s>_k<k>_d<D> notation), over the
    DeepSeek-V4 vocabulary of the latent workloads.  Every expanded node (the
    root and each node of depth < s) has its own next-token distribution."""

    id: int
    name: str
    B: int
    steps: int
    top_k: int
    n_budget: int
    N_max: int
    V: int = 129280
    sigma: float = 3.0
    cost: Optional[Cost] = None

    @property
    def rows(self) -> int:
        """Expanded nodes per request: 1 + k + ... + k^(s-1)."""
        return sum(self.top_k ** d for d in range(self.steps))

    def replace(self, **kw) -> "ExpandConfig":
        return dataclasses.replace(self, **kw)


EXPAND_CONFIGS = {
    # the review's best throughput point (three steps, top-2, budget 6) at
    # batch 4, and its other named points at larger batches
    101: ExpandConfig(101, "s3_k2_d6", B=4, steps=3, top_k=2, n_budget=6, N_max=8),
    102: ExpandConfig(102, "s4_k2_d5", B=16, steps=4, top_k=2, n_budget=5, N_max=8),
    103: ExpandConfig(103, "s5_k2_d8", B=64, steps=5, top_k=2, n_budget=8, N_max=8),
    # the batch-64 end of the review's sweep, for throughput
    104: ExpandConfig(104, "s3_k2_d6_b64", B=64, steps=3, top_k=2, n_budget=6, N_max=8),
}


def expand_config(cfg_id: int, **overrides) -> ExpandConfig:
    cfg = EXPAND_CONFIGS[cfg_id]
    return cfg.replace(**overrides) if overrides else cfg


def node_distributions(cfg: ExpandConfig, seed: int = 0, device="cpu") -> torch.Tensor:
    """Next-token distributions of every expanded node, fp32 [B, rows, V], rows
    in level order (row 0 the root's; the child of rank r of the node with
    row i has row k*i + 1 + r).  Logits ~ N(0, sigma) in fp64, softmax, fp32."""
    out = torch.empty((cfg.B, cfg.rows, cfg.V), dtype=torch.float32, device=device)
    for b in range(cfg.B):
        lg = _randn((cfg.rows, cfg.V), seed, cfg, _T_DRAFT, b, device, torch.float64) * cfg.sigma
        out[b] = torch.softmax(lg, dim=-1).to(torch.float32)
    return out


def pitched(B: int, R: int, row_shape, dtype, device, pitch: Optional[int] = None) -> torch.Tensor:
    """Zeros of shape [B, R, *row_shape] whose rows lie `pitch` elements apart
    (dense when pitch is None); the elements between rows are never used."""
    width = int(np.prod(row_shape))
    if pitch is None or pitch == width:
        return torch.zeros((B, R) + tuple(row_shape), dtype=dtype, device=device)
    if pitch < width:
        raise ValueError("row pitch smaller than the row")
    base = torch.zeros((B, R, pitch), dtype=dtype, device=device)
    return base[:, :, :width].view((B, R) + tuple(row_shape))


def attention_inputs(cfg: Config, seed: int = 0, device="cpu", row_pitch: Optional[int] = None) -> dict:
    """Queries, persistent caches, scratch (tree) KV and prefix lengths.

    GQA layout: q [B, N_max, Hq, d_qk]; k_cache/v_cache [B, L_cap, Hkv, d];
    k_tree/v_tree [B, N_max, Hkv, d].  Latent layout: k_cache [B, L_cap, d_qk]
    with v_cache the same tensor (values are its first d_v columns); likewise
    k_tree/v_tree.  Cache and scratch rows lie `row_pitch` elements apart
    (dense by default); the values do not depend on it.
    """
    dt = cfg.torch_dtype
    pl = prefix_lengths(cfg, seed)
    B, L, N = cfg.B, cfg.L_cap, cfg.N_max
    row = (cfg.d_qk,) if cfg.mla else (cfg.Hkv, cfg.d_qk)
    q = torch.empty((B, N, cfg.Hq, cfg.d_qk), dtype=dt, device=device)
    kc = pitched(B, L, row, dt, device, row_pitch)
    kt = pitched(B, N, row, dt, device, row_pitch)
    vc = kc if cfg.mla else pitched(B, L, (cfg.Hkv, cfg.d_v), dt, device, row_pitch)
    vt = kt if cfg.mla else pitched(B, N, (cfg.Hkv, cfg.d_v), dt, device, row_pitch)
    for b in range(B):
        lb = int(pl[b])
        q[b] = _randn(q.shape[1:], seed, cfg, _T_Q, b, device).to(dt)
        kc[b, :lb] = _randn((lb,) + row, seed, cfg, _T_K, b, device).to(dt)
        kt[b] = _randn(kt.shape[1:], seed, cfg, _T_KT, b, device).to(dt)
        if not cfg.mla:
            vc[b, :lb] = _randn((lb, cfg.Hkv, cfg.d_v), seed, cfg, _T_V, b, device).to(dt)
            vt[b] = _randn(vt.shape[1:], seed, cfg, _T_VT, b, device).to(dt)
    return dict(q=q, k_cache=kc, v_cache=vc, k_tree=kt, v_tree=vt,
                prefix_len=torch.from_numpy(pl).to(device))


def target_row_positions(cfg: Config, depth_b: Sequence[int], n_b: int) -> list:
    """Drafter position whose logits seed each verified row of one request."""
    pos = [0] * (1 + cfg.N_max)
    for i in range(min(int(n_b), cfg.N_max)):
        pos[1 + i] = min(int(depth_b[i]), cfg.gamma - 1)
    return pos


def target_logits(cfg: Config, seed: int, depth, n_nodes, device="cpu",
                  requests: Optional[Sequence[int]] = None) -> torch.Tensor:
    """Target logits [len(requests), 1+N_max, V] in the workload dtype.

    depth [B, N_max] and n_nodes [B] describe the tree being verified (any
    array-like).  Rows beyond 1+n_b get position-0 logits plus noise; a correct
    walk never reads them.
    """
    depth = np.asarray(depth)
    n_nodes = np.asarray(n_nodes)
    reqs = list(range(cfg.B)) if requests is None else list(requests)
    out = torch.empty((len(reqs), 1 + cfg.N_max, cfg.V), dtype=cfg.torch_dtype,
                      device=device)
    for r, b in enumerate(reqs):
        base = drafter_logits(cfg, seed, b, device)
        pos = torch.tensor(target_row_positions(cfg, depth[b], n_nodes[b]),
                           device=device, dtype=torch.long)
        noise = _randn((1 + cfg.N_max, cfg.V), seed, cfg, _T_NOISE, b, device,
                       torch.float64)
        out[r] = (base[pos] + noise).to(cfg.torch_dtype)
    return out
