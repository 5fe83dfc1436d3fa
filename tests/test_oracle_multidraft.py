"""Pins of the oracle's multi-draft tree rejection (recursive residuals; a
reading: the "Speculative Sampling" section of the blog page "Fast Inference
from Transformers via Speculative Decoding" gives the single-draft rule, and
its MEDUSA section says tree candidates can reuse it, with no multi-draft
scheme).

  * on chains it is the single-draft rule, bit for bit;
  * at temperature 0 it is the greedy walk down the tree (first child, in
    index order, whose token is the argmax);
  * the first emitted token follows the target when a node has several
    i.i.d. drafts (chi-square over 10^6 trials), where the single-child
    residual fails the same test;
  * on a depth-2 tree whose rows depend only on the token prefix, the second
    token follows the target given the first.
"""
import numpy as np
import pytest
from scipy import special, stats

import oracle


def _draw_rows(rng, probs, size):
    """size i.i.d. draws from one distribution (inverse CDF)."""
    c = np.cumsum(probs.astype(np.float64))
    return np.minimum(np.searchsorted(c, rng.random(size) * c[-1], side="right"), len(probs) - 1)


def _chain_case(seed, B=50, N=6, V=200, T=0.8):
    rng = np.random.default_rng(seed)
    lg = (rng.standard_normal((B, N, V)) * 2).astype(np.float32)
    dp = np.zeros((B, N, V), np.float32)
    tk = np.zeros((B, N), np.int32)
    for b in range(B):
        for i in range(1, N):
            q = special.softmax((lg[b, i - 1].astype(np.float64) + rng.standard_normal(V)) / T)
            dp[b, i] = q.astype(np.float32)
            tk[b, i] = min(np.searchsorted(np.cumsum(q), rng.random() * q.sum(), side="right"), V - 1)
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    return lg, dp, tk, par, rng.random((B, N), dtype=np.float32), rng.random((B, N), dtype=np.float32)


@pytest.mark.parametrize("T", [0.8, 1.0])
def test_chain_is_the_single_draft_rule(T):
    lg, dp, tk, par, ua, us = _chain_case(5, T=T)
    a = oracle.accept("reject", lg, tk, par, T, dp, ua, us)
    m = oracle.accept_multidraft(lg, tk, par, T, dp, ua, us)
    for key in ("accept_len", "path", "out_tokens"):
        np.testing.assert_array_equal(m[key], a[key])
    assert a["accept_len"].max() >= 2


def _random_tree(rng, B, N, max_children=4):
    par = np.full((B, N), -1, np.int32)
    for b in range(B):
        nkids = np.zeros(N, int)
        for i in range(1, N):
            choices = [j for j in range(i) if nkids[j] < max_children]
            p = choices[rng.integers(len(choices))]
            par[b, i] = p
            nkids[p] += 1
    return par


def test_temperature_zero_is_the_greedy_walk():
    rng = np.random.default_rng(9)
    B, N, V = 60, 12, 7
    lg = rng.standard_normal((B, N, V)).astype(np.float32)
    par = _random_tree(rng, B, N)
    tk = rng.integers(V, size=(B, N)).astype(np.int32)
    am = lg.argmax(-1)
    for b in range(B):  # make argmax children common, with duplicates among siblings
        for i in range(1, N):
            if rng.random() < 0.6:
                tk[b, i] = am[b, par[b, i]]
    dp = np.full((B, N, V), 1.0 / V, np.float32)
    r = oracle.accept_multidraft(lg, tk, par, 0.0, dp, rng.random((B, N), dtype=np.float32),
                                 rng.random((B, N), dtype=np.float32))
    for b in range(B):
        v, walk = 0, [0]
        while True:
            kids = [c for c in range(1, N) if par[b, c] == v and tk[b, c] == am[b, v]]
            if not kids:
                break
            v = kids[0]
            walk.append(v)
        a = len(walk) - 1
        assert r["accept_len"][b] == a
        np.testing.assert_array_equal(r["path"][b][:a + 1], walk)
        want = [int(tk[b, c]) for c in walk[1:]] + [int(am[b, v])]
        np.testing.assert_array_equal(r["out_tokens"][b][:a + 1], want)


def _star(seed, m, trials, V=16, T=1.0):
    """Root with m leaf children whose tokens are i.i.d. from one draft q."""
    rng = np.random.default_rng(seed)
    N = m + 1
    base = rng.standard_normal((N, V)).astype(np.float32)
    q = special.softmax(base[0].astype(np.float64) + rng.standard_normal(V) * 1.5).astype(np.float32)
    tokens = np.zeros((trials, N), np.int32)
    c = np.cumsum(q.astype(np.float64))
    for i in range(1, N):
        tokens[:, i] = np.minimum(np.searchsorted(c, rng.random(trials) * c[-1], side="right"), V - 1)
    par = np.tile(np.array([-1] + [0] * m, np.int32), (trials, 1))
    args = (np.broadcast_to(base, (trials, N, V)), tokens, par, T, np.broadcast_to(np.tile(q, (N, 1)), (trials, N, V)),
            rng.random((trials, N), dtype=np.float32), rng.random((trials, N), dtype=np.float32))
    return args, special.softmax(base[0].astype(np.float64) / T)


@pytest.mark.slow
@pytest.mark.parametrize("m,seed", [(3, 31), (6, 32)])
def test_several_iid_drafts_keep_the_target_distribution(m, seed):
    args, p = _star(seed, m, 1_000_000)
    B = args[1].shape[0]
    r = oracle.accept_multidraft(*args)
    obs = np.bincount(r["out_tokens"][:, 0], minlength=16)
    chi2, pv = stats.chisquare(obs, p * B)
    assert pv > 1e-3, (chi2, pv)
    # the single-child residual (the plain rule over a tree) is biased here
    old = oracle.accept("reject", *args)
    chi2o, pvo = stats.chisquare(np.bincount(old["out_tokens"][:, 0], minlength=16), p * B)
    assert pvo < 1e-6, (chi2o, pvo)


@pytest.mark.slow
def test_second_token_follows_the_target_given_the_first():
    # Root -> 3 children (tokens i.i.d. from q0) -> 2 grandchildren each
    # (tokens i.i.d. from q1[token of the child]); the target row of a child
    # depends only on its token, so given the first token y the second token
    # must follow P2[y].
    rng = np.random.default_rng(41)
    V, trials = 6, 600_000
    L0 = rng.standard_normal(V).astype(np.float32)
    L1 = rng.standard_normal((V, V)).astype(np.float32) * 1.5
    q0 = special.softmax(L0.astype(np.float64) + rng.standard_normal(V)).astype(np.float32)
    q1 = special.softmax(L1.astype(np.float64) + rng.standard_normal((V, V)), axis=-1).astype(np.float32)
    par = np.array([-1, 0, 0, 0, 1, 1, 2, 2, 3, 3], np.int32)
    N = len(par)
    tokens = np.zeros((trials, N), np.int32)
    for i in (1, 2, 3):
        tokens[:, i] = _draw_rows(rng, q0, (trials,))
    for i in range(4, N):
        pt = tokens[:, par[i]]
        c = np.cumsum(q1[pt].astype(np.float64), axis=-1)
        tokens[:, i] = np.minimum((c < rng.random((trials, 1)) * c[:, -1:]).sum(-1), V - 1)
    logits = np.empty((trials, N, V), np.float32)
    logits[:, 0] = L0
    for i in range(1, N):
        logits[:, i] = L1[tokens[:, i]] if i < 4 else 0.0
    draft = np.zeros((trials, N, V), np.float32)
    draft[:, 1:4] = q0
    for i in range(4, N):
        draft[:, i] = q1[tokens[:, par[i]]]
    r = oracle.accept_multidraft(logits, tokens, np.tile(par, (trials, 1)), 1.0, draft,
                                 rng.random((trials, N), dtype=np.float32), rng.random((trials, N), dtype=np.float32))
    first = r["out_tokens"][:, 0]
    assert stats.chisquare(np.bincount(first, minlength=V), special.softmax(L0.astype(np.float64)) * trials)[1] > 1e-3
    deep = r["accept_len"] >= 1
    P2 = special.softmax(L1.astype(np.float64), axis=-1)
    for y in range(V):
        sel = deep & (first == y)
        if sel.sum() < 2000:
            continue
        obs = np.bincount(r["out_tokens"][sel, 1], minlength=V)
        assert stats.chisquare(obs, P2[y] * sel.sum())[1] > 1e-4, y
