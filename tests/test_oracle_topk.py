"""Pins of the oracle's per-position top-k (CPU only)."""

import numpy as np
import pytest

from oracle import topk_per_position


def _repeated_max(row, k):
    """Independent selection: take the largest remaining value, the lowest
    index among equal maxima, k times."""
    row = [float(x) for x in row]
    alive = list(range(len(row)))
    out = []
    for _ in range(k):
        best = alive[0]
        for j in alive[1:]:
            if row[j] > row[best]:
                best = j
        out.append(best)
        alive.remove(best)
    return out


def test_ties_go_to_lower_id():
    p = np.array([[0.1, 0.3, 0.3, 0.05, 0.3, 0.0]], dtype=np.float32)
    idx, val = topk_per_position(p, 4)
    assert idx.tolist() == [[1, 2, 4, 0]]
    assert val[0].tolist() == pytest.approx([0.3, 0.3, 0.3, 0.1])


def test_signed_zero_is_one_value():
    p = np.array([[0.0, -0.0, 0.0, 0.5]], dtype=np.float32)
    idx, _ = topk_per_position(p, 4)
    assert idx.tolist() == [[3, 0, 1, 2]]


@pytest.mark.parametrize("seed", range(5))
def test_matches_repeated_max_with_forced_ties(seed):
    rng = np.random.default_rng(seed)
    # quantised probabilities force many equal values
    rows = (rng.integers(0, 7, size=(6, 40)) / 64.0).astype(np.float32)
    for k in (1, 3, 8, 40):
        idx, val = topk_per_position(rows, k)
        for r in range(rows.shape[0]):
            assert idx[r].tolist() == _repeated_max(rows[r], k)
            assert np.array_equal(val[r], rows[r][idx[r]])


def test_shapes_and_errors():
    p = np.random.default_rng(0).random((2, 3, 10)).astype(np.float32)
    idx, val = topk_per_position(p, 5)
    assert idx.shape == (2, 3, 5) and idx.dtype == np.int32
    assert val.shape == (2, 3, 5) and val.dtype == np.float32
    with pytest.raises(ValueError):
        topk_per_position(p, 11)
    bad = p.copy()
    bad[0, 0, 0] = np.nan
    with pytest.raises(ValueError):
        topk_per_position(bad, 2)
