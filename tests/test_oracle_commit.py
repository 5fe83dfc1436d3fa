"""Pins of the commit oracle: the accepted path's KV rows move to L_b .. L_b+a
(an out-of-place NumPy gather), every source row is read before any write
(the hazard path 0, 2, 5 -> slots 0, 1, 2), and a chain leaves the cache
untouched while the prefix grows by a + 1."""
import numpy as np

import oracle


def _case(rng, B, Hkv, cap, D, dtype=np.float32):
    k = rng.standard_normal((B, Hkv, cap, D)).astype(dtype)
    v = rng.standard_normal((B, Hkv, cap, D)).astype(dtype)
    return k, v


def test_commit_is_a_gather():
    rng = np.random.default_rng(1)
    B, Hkv, N, D = 3, 2, 8, 4
    L = np.array([3, 0, 10], np.int32)
    cap = 10 + N
    k, v = _case(rng, B, Hkv, cap, D)
    path = np.full((B, N), -1, np.int32)
    path[0, :3] = [0, 2, 5]
    path[1, :1] = [0]
    path[2, :4] = [0, 1, 4, 7]
    acc = np.array([2, 0, 3], np.int32)
    k0, v0, L0 = k.copy(), v.copy(), L.copy()
    pl = oracle.commit(k, v, L, path, acc)
    np.testing.assert_array_equal(pl, L0 + acc + 1)
    for b in range(B):
        src = [L0[b] + path[b, d] for d in range(acc[b] + 1)]
        dst = [L0[b] + d for d in range(acc[b] + 1)]
        np.testing.assert_array_equal(k[b][:, dst], k0[b][:, src])
        np.testing.assert_array_equal(v[b][:, dst], v0[b][:, src])
        keep = np.ones(cap, bool)
        keep[dst] = False
        np.testing.assert_array_equal(k[b][:, keep], k0[b][:, keep])


def test_chain_commit_moves_nothing():
    rng = np.random.default_rng(2)
    B, Hkv, N, D = 2, 3, 6, 8
    L = np.array([5, 7], np.int32)
    k, v = _case(rng, B, Hkv, 7 + N, D, np.uint16)
    path = np.tile(np.arange(N, dtype=np.int32), (B, 1))
    acc = np.array([5, 2], np.int32)
    path[1, 3:] = -1
    k0, v0 = k.copy(), v.copy()
    pl = oracle.commit(k, v, L.copy(), path, acc)
    np.testing.assert_array_equal(pl, [11, 10])
    np.testing.assert_array_equal(k, k0)
    np.testing.assert_array_equal(v, v0)
