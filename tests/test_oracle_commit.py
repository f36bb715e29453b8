"""Pins of the oracle's accepted-path commit (CPU only)."""

import numpy as np

from oracle import commit_path


def _setup(rng, B=3, L=12, N=5, H=2, d=4):
    kc = rng.standard_normal((B, L, H, d)).astype(np.float32)
    vc = rng.standard_normal((B, L, H, d)).astype(np.float32)
    kt = rng.standard_normal((B, N, H, d)).astype(np.float32)
    vt = rng.standard_normal((B, N, H, d)).astype(np.float32)
    return kc, vc, kt, vt


def test_copies_only_the_accepted_rows():
    rng = np.random.default_rng(0)
    kc, vc, kt, vt = _setup(rng)
    k0, v0 = kc.copy(), vc.copy()
    pl = np.array([4, 7, 0], dtype=np.int32)
    alen = np.array([2, 0, 3], dtype=np.int32)
    nodes = np.array([[3, 1, -1], [-1, -1, -1], [0, 2, 4]], dtype=np.int32)
    st = commit_path(kc, vc, pl, kt, vt, alen, nodes, gamma=3)
    assert st.tolist() == [0, 0, 0]
    assert pl.tolist() == [6, 7, 3]
    np.testing.assert_array_equal(kc[0, 4], kt[0, 3])
    np.testing.assert_array_equal(vc[0, 5], vt[0, 1])
    np.testing.assert_array_equal(kc[2, :3], kt[2, [0, 2, 4]])
    untouched = np.ones(kc.shape[:2], dtype=bool)
    untouched[0, 4:6] = False
    untouched[2, 0:3] = False
    np.testing.assert_array_equal(kc[untouched], k0[untouched])
    np.testing.assert_array_equal(vc[untouched], v0[untouched])


def test_overflow_and_bad_input_leave_request_untouched():
    rng = np.random.default_rng(1)
    kc, vc, kt, vt = _setup(rng)
    k0 = kc.copy()
    pl = np.array([11, 5, 5], dtype=np.int32)
    alen = np.array([2, 1, 4], dtype=np.int32)
    nodes = np.array([[0, 1, 2], [7, -1, -1], [0, 1, 2]], dtype=np.int32)
    st = commit_path(kc, vc, pl, kt, vt, alen, nodes, gamma=3)
    assert st.tolist() == [1, 2, 2]
    assert pl.tolist() == [11, 5, 5]
    np.testing.assert_array_equal(kc, k0)


def test_latent_cache_and_multi_round():
    rng = np.random.default_rng(2)
    B, L, N, D = 2, 20, 6, 7
    lat = np.zeros((B, L, D), dtype=np.float32)
    pl = np.array([3, 5], dtype=np.int32)
    history = [list(range(3)), list(range(5))]
    for r in range(4):
        kt = rng.standard_normal((B, N, D)).astype(np.float32)
        alen = rng.integers(0, 4, size=B).astype(np.int32)
        nodes = np.array([rng.permutation(N)[:3] for _ in range(B)], dtype=np.int32)
        before = pl.copy()
        st = commit_path(lat, None, pl, kt, None, alen, nodes, gamma=3)
        assert (st == 0).all()
        for b in range(B):
            assert pl[b] == before[b] + alen[b]
            for j in range(alen[b]):
                np.testing.assert_array_equal(lat[b, before[b] + j], kt[b, nodes[b, j]])
    assert (lat[0, pl[0]:] == 0).all() and (lat[1, pl[1]:] == 0).all()
