"""Pins of the oracle's linear-attention verification and state commit (the
SpecLA summary "SpecLA: Efficient Speculative Decoding for Linear-Attention
Models": drafts verified against a recurrent summary state, a tree mask for
branches, the state recovered afterwards from the accepted tokens' factors).
Reading: S_t = alpha_t S_{t-1} + v_t k_t^T, o_t = S_t q_t.

  * every node's output equals the recurrence replayed token by token along
    its root path (the oracle evaluates a closed form instead);
  * with alpha = 1 a chain is causal linear attention, by cumulative sums of
    outer products;
  * the commit equals replaying the accepted tokens through the recurrence;
  * a hand example with Dk = Dv = 1.
"""
import numpy as np
import pytest

import oracle


def _case(seed, B=3, N=9, H=2, Dk=5, Dv=4, tree=True, alpha=True):
    rng = np.random.default_rng(seed)
    S = rng.standard_normal((B, H, Dv, Dk)).astype(np.float32)
    q = rng.standard_normal((B, N, H, Dk)).astype(np.float32)
    k = rng.standard_normal((B, N, H, Dk)).astype(np.float32)
    v = rng.standard_normal((B, N, H, Dv)).astype(np.float32)
    al = rng.uniform(0.5, 1.0, (B, N, H)).astype(np.float32) if alpha else None
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    if tree:
        for b in range(B):
            for i in range(2, N):
                par[b, i] = rng.integers(i)
    return S, q, k, v, al, par


def _root_path(par_b, i):
    p = []
    while i >= 0:
        p.append(i)
        i = par_b[i]
    return p[::-1]


def _replay(S0, k, v, al, path, h, b):
    S = S0.astype(np.float64).copy()
    for t in path:
        a = 1.0 if al is None else float(al[b, t, h])
        S = a * S + np.outer(v[b, t, h].astype(np.float64), k[b, t, h].astype(np.float64))
    return S


@pytest.mark.parametrize("tree,alpha", [(True, True), (False, True), (True, False)])
def test_outputs_equal_the_replayed_recurrence(tree, alpha):
    S, q, k, v, al, par = _case(1 + 2 * tree + alpha, tree=tree, alpha=alpha)
    out = oracle.la_verify(S, q, k, v, al, par if tree else None, "f32")
    B, N, H, _ = q.shape
    for b in range(B):
        for h in range(H):
            for i in range(N):
                St = _replay(S[b, h], k, v, al, _root_path(par[b], i), h, b)
                np.testing.assert_allclose(out[b, i, h], St @ q[b, i, h].astype(np.float64), rtol=1e-12, atol=1e-12)


def test_chain_without_decay_is_causal_linear_attention():
    S, q, k, v, _, _ = _case(7, tree=False, alpha=False)
    out = oracle.la_verify(S, q, k, v, None, None, "f32")
    outer = np.einsum("bnhe,bnhd->bnhed", v.astype(np.float64), k.astype(np.float64))
    states = np.cumsum(outer, axis=1) + S.astype(np.float64)[:, None]
    want = np.einsum("bnhed,bnhd->bnhe", states, q.astype(np.float64))
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("tree", [True, False])
def test_commit_equals_replay_of_the_accepted_path(tree):
    S, q, k, v, al, par = _case(11 + tree, tree=tree)
    B, N, H, _ = q.shape
    rng = np.random.default_rng(5)
    path = np.full((B, N), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b in range(B):  # a random root path
        stop = int(rng.integers(N))
        rp = _root_path(par[b], stop)
        path[b, :len(rp)] = rp
        acc[b] = len(rp) - 1
    S2 = oracle.la_commit(S, k, v, al, par if tree else None, path, acc, "f32")
    for b in range(B):
        for h in range(H):
            want = _replay(S[b, h], k, v, al, path[b, :acc[b] + 1], h, b)
            np.testing.assert_allclose(S2[b, h], want, rtol=1e-6, atol=1e-6)


def test_hand_example():
    # Dk = Dv = 1: S = 2; root (alpha .5, k 1, v 3, q 1) -> S_0 = .5*2 + 3 = 4,
    # o_0 = 4; child (alpha .25, k 2, v 1, q 3) -> S_1 = .25*4 + 2 = 3, o_1 = 9.
    S = np.array([[[[2.0]]]], np.float32)
    q = np.array([[[[1.0]], [[3.0]]]], np.float32)
    k = np.array([[[[1.0]], [[2.0]]]], np.float32)
    v = np.array([[[[3.0]], [[1.0]]]], np.float32)
    al = np.array([[[0.5], [0.25]]], np.float32)
    out = oracle.la_verify(S, q, k, v, al, None, "f32")
    np.testing.assert_allclose(out[0, :, 0, 0], [4.0, 9.0], atol=1e-12)
    S2 = oracle.la_commit(S, k, v, al, None, np.array([[0, 1]], np.int32), np.array([1], np.int32), "f32")
    assert S2[0, 0, 0, 0] == 3.0
    S1 = oracle.la_commit(S, k, v, al, None, np.array([[0, -1]], np.int32), np.array([0], np.int32), "f32")
    assert S1[0, 0, 0, 0] == 4.0
