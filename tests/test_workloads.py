"""The seeded input generator: determinism, shapes and recipe (CPU only)."""

import numpy as np
import torch

from workloads import CONFIGS, attention_inputs, config, marginals, prefix_lengths, target_logits
from workloads.gen import target_row_positions


def test_configs_shapes():
    c2 = CONFIGS[2]
    assert (c2.B, c2.Hq, c2.Hkv, c2.d_qk, c2.prefix, c2.gamma, c2.V) == (16, 32, 8, 128, 4096, 16, 151936)
    c3 = CONFIGS[3]
    assert (c3.Hq, c3.Hkv, c3.d_qk, c3.d_v, c3.kv_stride, c3.mla) == (128, 1, 576, 512, 576, True)
    c4 = CONFIGS[4]
    assert c4.cost.a == 1.0 and c4.cost.c_d == 0.5 and c4.n_budget == 128
    pl = prefix_lengths(c4)
    assert pl.min() >= 1024 and pl.max() <= 32768 and len(pl) == 64
    assert c4.L_cap == 32768 + 16


def test_deterministic_and_recipe():
    cfg = config(1)
    a = marginals(cfg, 0)
    b = marginals(cfg, 0)
    assert torch.equal(a, b) and a.dtype == torch.float32
    assert torch.allclose(a.double().sum(-1), torch.ones(cfg.B, cfg.gamma, dtype=torch.float64),
                          atol=1e-6)
    assert not torch.equal(a, marginals(cfg, 1))
    ins = attention_inputs(cfg, 0)
    l = int(ins["prefix_len"][0])
    assert (ins["k_cache"][0, l:] == 0).all() and (ins["v_cache"][0, l:] == 0).all()
    assert ins["q"].shape == (1, cfg.N_max, cfg.Hq, cfg.d_qk)


def test_small_latent_config():
    cfg = config(3, B=2, prefix=40, V=50, N_max=4, n_budget=4)
    ins = attention_inputs(cfg, 0)
    assert ins["v_cache"] is ins["k_cache"]
    assert ins["k_cache"].shape == (2, 48, 576) and ins["k_cache"].dtype == torch.bfloat16


def test_target_rows_follow_depth():
    cfg = config(1)
    depth = np.array([[1, 2, 4, 4, -1, -1, -1, -1]])
    assert target_row_positions(cfg, depth[0], 4) == [0, 1, 2, 3, 3, 0, 0, 0, 0]
    t = target_logits(cfg, 0, depth, [4])
    assert t.shape == (1, 1 + cfg.N_max, cfg.V) and t.dtype == torch.float32
    assert torch.equal(t, target_logits(cfg, 0, depth, [4]))
