"""Measure the verification cost C_v(n; l) on this GPU and fit the convex,
monotone model build_tree's adaptive budget uses.

[caddtree] Methodology, item 5: C_v is estimated once, offline, by convex
regression on latencies measured over node counts and context lengths.
Here the latency of a point (n, l) is one tree_verify_attn call on B
requests that each verify n tree nodes over a prefix of l tokens, divided by
B (each request's share of a batched verification call), in microseconds;
tsv_fit_cost fits C_v(n; l) = a + b n + c n^2 + e l n + f l with every
coefficient >= 0.

    python -m tree_structured_verification_amd.profile_cost --batch 16 \\
        --heads 32 8 --dim 128 --c-d 10 --out cost.json

Inputs are random (standard normal queries and keys in the chosen dtype); the
tree is a star (every node a child of the root), whose cost equals any other
shape's up to the masking of the last tiles.
"""

from __future__ import annotations

import argparse
import json
from typing import Sequence

import numpy as np
import torch

from . import _lib

DEFAULT_N = (1, 2, 4, 8, 16, 32, 64, 96, 128)
DEFAULT_L = (512, 1024, 2048, 4096, 8192, 16384)


def measure_verify_cost(B: int, Hq: int, Hkv: int, d: int, n_grid: Sequence[int] = DEFAULT_N,
                        l_grid: Sequence[int] = DEFAULT_L, dtype=torch.bfloat16,
                        reps: int = 20, warmup: int = 3, device="cuda:0"):
    """Per-request microseconds of one tree_verify_attn call at every grid
    point.  Returns (n, l, t) as float64 arrays of one length."""
    dev = torch.device(device)
    N_max = max(n_grid)
    if N_max > 128:
        raise ValueError("node counts above 128 are not supported")
    L_cap = max(l_grid)
    W = (N_max + 31) // 32
    gen = torch.Generator(device=dev).manual_seed(1234)
    rnd = lambda *shape: torch.randn(*shape, generator=gen, device=dev, dtype=torch.float32).to(dtype)
    q = rnd(B, N_max, Hq, d)
    kc, vc = rnd(B, L_cap, Hkv, d), rnd(B, L_cap, Hkv, d)
    kt, vt = rnd(B, N_max, Hkv, d), rnd(B, N_max, Hkv, d)
    # star tree: node i sees only itself among the scratch rows
    anc = torch.zeros(B, N_max, W, dtype=torch.int32)
    for i in range(N_max):
        anc[:, i, i // 32] = np.int32(np.uint32(1 << (i % 32)).view(np.int32))
    anc = anc.to(dev)
    out = torch.empty(B, N_max, Hq, d, dtype=dtype, device=dev)
    ws = _lib.workspace(_lib.workspace_size(_lib.WS_ATTN, B, 1, 1, 1, N_max, L_cap, Hq, Hkv, d, d,
                                            _lib.dtype_code(dtype)), dev)
    stream = torch.cuda.current_stream(dev)
    ns, ls, ts = [], [], []
    for l in l_grid:
        pl = torch.full((B,), int(l), dtype=torch.int32, device=dev)
        for n in n_grid:
            nn = torch.full((B,), int(n), dtype=torch.int32, device=dev)
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(warmup + reps)]
            for r in range(warmup + reps):
                ev[r][0].record(stream)
                _lib.tree_verify_attn(q, kc, vc, kt, vt, pl, nn, anc, Hkv, d, d ** -0.5,
                                      out=out, want_lse=False, ws=ws)
                ev[r][1].record(stream)
            torch.cuda.synchronize(dev)
            us = float(np.median([a.elapsed_time(b) for a, b in ev[warmup:]])) * 1e3
            ns.append(n)
            ls.append(l)
            ts.append(us / B)
    return (np.array(ns, np.float64), np.array(ls, np.float64), np.array(ts, np.float64))


def calibrate(B: int, Hq: int, Hkv: int, d: int, c_d: float, **kw):
    """Measure and fit: returns (tsv_cost, (n, l, t))."""
    n, l, t = measure_verify_cost(B, Hq, Hkv, d, **kw)
    return _lib.fit_cost(n, l, t, c_d), (n, l, t)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--heads", type=int, nargs=2, default=(32, 8), metavar=("HQ", "HKV"))
    ap.add_argument("--dim", type=int, default=128)
    ap.add_argument("--c-d", type=float, required=True,
                    help="drafting cost per request per round, in microseconds")
    ap.add_argument("--out", default=None, help="write the fitted cost as JSON here")
    args = ap.parse_args()
    cost, (n, l, t) = calibrate(args.batch, args.heads[0], args.heads[1], args.dim, args.c_d)
    res = {"a": cost.a, "b": cost.b, "c": cost.c, "e": cost.e, "f": cost.f, "c_d": cost.c_d, "unit": "us",
           "points": [[float(x), float(y), float(z)] for x, y, z in zip(n, l, t)]}
    text = json.dumps(res)
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


if __name__ == "__main__":
    main()
