"""Cache and scratch row layouts accepted by the binding (host-side checks)."""

import pytest
import torch

import tree_structured_verification_amd as tsv
from workloads import attention_inputs, config, pitched


def test_recommended_pitch():
    # 8 heads x 128 bf16 = 2048 B = 16 lines -> 17 lines
    assert tsv.kv_row_pitch(8 * 128, 2) == 17 * 64
    # a 576-wide latent row is 1152 B = 9 lines already
    assert tsv.kv_row_pitch(576, 2) == 576
    # 8 heads x 64 fp32 = 2048 B -> 2176 B
    assert tsv.kv_row_pitch(8 * 64, 4) == 544
    # not a whole number of lines: 144 B -> 2 lines -> 3 lines
    assert tsv.kv_row_pitch(72, 2) == 192
    for width, es in ((1024, 2), (576, 2), (512, 4), (72, 2), (4096, 2), (100, 4)):
        p = tsv.kv_row_pitch(width, es)
        assert p >= width and (p * es) % 128 == 0 and (p * es // 128) % 2 == 1


def test_kv_rows_view_and_layout_check():
    x = tsv.kv_rows(3, 7, (8, 128), torch.bfloat16, "cpu")
    assert x.shape == (3, 7, 8, 128) and x.stride() == (7 * 1088, 1088, 128, 1)
    assert tsv.row_layout(x) == 1088
    assert tsv.row_layout(torch.zeros(2, 5, 4, 16)) == 64
    assert tsv.row_layout(torch.zeros(2, 5, 576)) == 576
    with pytest.raises(ValueError):
        tsv.row_layout(torch.zeros(2, 5, 16, 4).transpose(2, 3))   # row block not dense
    with pytest.raises(ValueError):
        tsv.row_layout(torch.zeros(5, 2, 64).transpose(0, 1))      # batches not R rows apart
    with pytest.raises(ValueError):
        tsv.row_layout(torch.zeros(4, 64))


@pytest.mark.parametrize("cid", [1, 3])
def test_pitched_inputs_hold_the_same_values(cid):
    cfg = config(cid).replace(B=2, prefix=48) if cid == 3 else config(cid)
    width = cfg.d_qk if cfg.mla else cfg.Hkv * cfg.d_qk
    dense = attention_inputs(cfg, 0, "cpu")
    padded = attention_inputs(cfg, 0, "cpu", row_pitch=width + 64)
    for k in dense:
        assert torch.equal(dense[k], padded[k]), k
    assert padded["k_cache"].stride(1) == width + 64
    assert tsv.row_layout(padded["k_tree"]) == width + 64
    assert pitched(2, 3, (4,), torch.float32, "cpu").is_contiguous()
