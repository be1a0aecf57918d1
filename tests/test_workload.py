"""Determinism and shape checks of the seeded workload generator (no GPU)."""
import numpy as np

from hierarchical_tree_indexed_04_amd import workload as W


def small():
    return W.custom("wl-small", 901, dtype=W.BF16, B=2, H_q=4, H_kv=2, d=16, T=4 ** 3 * 2 + 7,
                    C=4, L=3)


def test_same_seed_same_bytes():
    g = small()
    K1, V1 = W.make_kv(g)
    K2, V2 = W.make_kv(g)
    assert K1.dtype == np.uint16 and K1.shape == (2, 2, g.T, 16)
    np.testing.assert_array_equal(K1, K2)
    np.testing.assert_array_equal(V1, V2)
    np.testing.assert_array_equal(W.make_queries(g, K1, 3), W.make_queries(g, K2, 3))


def test_slices_generate_independently():
    g = small()
    K, V = W.make_kv(g)
    K1, V1 = W.make_kv(g, slices=[(1, 0)])
    np.testing.assert_array_equal(K[1, 0], K1[1, 0])
    np.testing.assert_array_equal(V[1, 0], V1[1, 0])
    assert not K1[0, 0].any()


def test_hierarchical_structure_of_keys():
    # Keys under the same top-level node share the sigma=1 centre: their mean differences are
    # much larger across top nodes than within one.
    g = W.custom("wl-struct", 902, dtype=W.F32, T=8 ** 3, C=8, L=3, d=64)
    K, _ = W.make_kv(g, want_v=False)
    k = K[0, 0]
    assert W.centre_spans(g) == [64, 8, 1]
    groups = k.reshape(8, 64, 64).mean(axis=1)
    within = np.var(k.reshape(8, 64, 64) - groups[:, None, :])
    across = np.var(groups)
    assert across > 0.7 and within < 0.5


def test_query_is_three_keys_plus_noise():
    g = W.custom("wl-q", 903, dtype=W.F32, T=256, C=4, L=2, d=64, H_q=2, H_kv=1)
    K, _ = W.make_kv(g, want_v=False)
    q = W.make_queries(g, K, 0)[0, 0]
    dists = np.linalg.norm(q[None, :] - 3 * K[0, 0], axis=1)
    assert dists.min() < 0.3 * 8 * 1.5  # |N(0, 0.3^2 I_64)| ~ 2.4


def test_random_chunk_sets_sorted_and_bounded():
    g = small()
    sel, cnt = W.random_chunk_sets(g, 50, 10, seed=1, cap=6)
    for h in range(50):
        ids = sel[h, :min(cnt[h], 6)]
        assert (np.diff(ids) > 0).all()
        assert ((ids >= 0) & (ids < g.n_level(1))).all()
    assert cnt.max() <= 10 and (cnt == 0).any()
