"""Pins of the oracle's top-k / nucleus truncation before the rejection rule
(the "Speculative Sampling" section of the blog page "Fast Inference from
Transformers via Speculative Decoding" lets top-k and nucleus sampling
transform the probabilities before the rule is applied).

  * with the filters off (k = 0 or V, top_p = 1) the outputs are the plain
    rule's, bit for bit;
  * top-k with k = 1 keeps only the argmax, so the rule reduces to greedy
    matching: the outputs equal those at temperature 0;
  * hand-computed draws on 4- and 5-token vocabularies fix the readings (ties
    at the top-k boundary kept; the nucleus keeps the tokens whose larger-
    logit mass is below top_p, on the renormalised top-k distribution);
  * the emitted tokens are distributed as the truncated target (chi-square
    over 10^6 seeded trials), and the single-draft acceptance frequency is
    sum_x min(p~, q).
"""
import numpy as np
import pytest
from scipy import special, stats

import oracle


def _chain(B, N):
    return np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))


def _random_case(seed, B=40, N=6, V=300, tree=False):
    rng = np.random.default_rng(seed)
    lg = (rng.standard_normal((B, N, V)) * 2).astype(np.float32)
    dp = rng.random((B, N, V)).astype(np.float32) ** 3
    dp /= dp.sum(-1, keepdims=True)
    tk = np.empty((B, N), np.int32)
    for b in range(B):  # drafts: mostly likely tokens so that paths get long
        for i in range(N):
            pr = dp[b, i].astype(np.float64)
            tk[b, i] = rng.choice(V, p=pr / pr.sum())
    par = _chain(B, N)
    if tree:
        for b in range(B):
            for i in range(2, N):
                par[b, i] = rng.integers(i)
    ua, us = rng.random((B, N), dtype=np.float32), rng.random((B, N), dtype=np.float32)
    return lg, dp, tk, par, ua, us


@pytest.mark.parametrize("tree", [False, True])
def test_filters_off_is_the_plain_rule(tree):
    lg, dp, tk, par, ua, us = _random_case(1 + tree, tree=tree)
    V = lg.shape[2]
    ref = oracle.accept("reject", lg, tk, par, 0.9, dp, ua, us)
    for k, p in ((0, 1.0), (V, 1.0), (V + 5, 1.0)):
        r = oracle.accept("reject", lg, tk, par, 0.9, dp, ua, us, top_k=k, top_p=p)
        for key in ("accept_len", "path", "out_tokens"):
            np.testing.assert_array_equal(r[key], ref[key])


@pytest.mark.parametrize("tree", [False, True])
def test_top1_is_greedy(tree):
    lg, dp, tk, par, ua, us = _random_case(3 + tree, tree=tree)
    # make some drafts the argmax so that greedy paths are not all empty
    am = lg.argmax(-1)
    for b in range(lg.shape[0]):
        for i in range(1, lg.shape[1]):
            if (b + i) % 3:
                tk[b, i] = am[b, par[b, i]]
    greedy = oracle.accept("reject", lg, tk, par, 0.0, dp, ua, us)
    for T in (0.5, 1.0, 2.0):
        r = oracle.accept("reject", lg, tk, par, T, dp, ua, us, top_k=1)
        for key in ("accept_len", "path", "out_tokens"):
            np.testing.assert_array_equal(r[key], greedy[key])
    assert greedy["accept_len"].max() > 1


def _bonus_token(logits_row, u, **filt):
    """Final token of a request with no drafts: one draw from the (truncated)
    target row with uniform u."""
    V = len(logits_row)
    lg = np.asarray(logits_row, np.float32).reshape(1, 1, V)
    r = oracle.accept("reject", lg, np.zeros((1, 1), np.int32), None, 1.0, np.zeros((1, 1, V), np.float32),
                      np.zeros((1, 1), np.float32), np.array([[u]], np.float32), **filt)
    assert r["accept_len"][0] == 0
    return int(r["out_tokens"][0, 0])


def test_hand_draws():
    # p = (0.5, 0.3, 0.15, 0.05); inverse-CDF draw: smallest x with cum > u.
    row = np.log([0.5, 0.3, 0.15, 0.05])
    assert _bonus_token(row, 0.90) == 2 and _bonus_token(row, 0.97) == 3           # no filter
    # nucleus 0.79: masses above tokens 0..3 are 0, .5, .8, .95 -> keep {0, 1},
    # p~ = (.625, .375): u = .60 -> 0, u = .63 -> 1, u = .999 -> 1
    assert [_bonus_token(row, u, top_p=0.79) for u in (0.60, 0.63, 0.999)] == [0, 1, 1]
    # nucleus 0.81 keeps {0, 1, 2}: p~ = (.5, .3, .15) / .95, cum = .526, .842, 1
    assert [_bonus_token(row, u, top_p=0.81) for u in (0.52, 0.53, 0.85, 0.999)] == [0, 1, 2, 2]
    # top-2 = nucleus 0.79 here; top-2 then nucleus 0.6 on p' = (.625, .375)
    # keeps only token 0 (mass above token 1 is .625 >= .6)
    assert [_bonus_token(row, u, top_k=2) for u in (0.60, 0.63)] == [0, 1]
    assert [_bonus_token(row, u, top_k=2, top_p=0.6) for u in (0.0, 0.5, 0.999)] == [0, 0, 0]
    # ties at the top-k boundary are kept: logits (3, 2, 2, 2, 1), k = 2 keeps
    # tokens 0..3, p~ proportional to (e^3, e^2, e^2, e^2, 0)
    tie = [3.0, 2.0, 2.0, 2.0, 1.0]
    w = np.exp(tie[:4])
    cum = np.cumsum(w) / w.sum()
    assert _bonus_token(tie, 0.999, top_k=2) == 3
    assert _bonus_token(tie, (cum[1] + cum[2]) / 2, top_k=2) == 2
    # tokens of equal logit enter or leave the nucleus together: over the
    # whole row the mass above the tied group is p(token 0) = e^3 / (e^3 +
    # 3 e^2 + e) = .4466, so top_p = .5 keeps the group (and drops token 4,
    # whose mass above is .94) while top_p = .4 drops all three
    p0 = np.exp(3.0) / np.exp(tie).sum()
    assert 0.4 < p0 < 0.5
    assert _bonus_token(tie, 0.999, top_p=0.5) == 3
    assert _bonus_token(tie, 0.999, top_p=0.4) == 0


def test_argument_checks():
    lg = np.zeros((1, 2, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.accept("reject", lg, np.zeros((1, 2), np.int32), None, 1.0, lg, top_k=-1)
    with pytest.raises(ValueError):
        oracle.accept("reject", lg, np.zeros((1, 2), np.int32), None, 1.0, lg, top_p=0.0)
    with pytest.raises(ValueError):
        oracle.accept("typical", lg, np.zeros((1, 2), np.int32), None, 1.0, top_k=2)


def _truncated(p, logits, k, top_p):
    """p~ from the definition, for the distribution pins (independent of the
    oracle's sort and grouping)."""
    keep = np.ones(len(p), bool)
    if 0 < k < len(p):
        keep &= logits >= np.sort(logits)[::-1][k - 1]
    if top_p < 1.0:
        pk = np.where(keep, p, 0.0)
        pk /= pk.sum()
        above = np.array([pk[logits > logits[x]].sum() for x in range(len(p))])
        keep &= above < top_p
    q = np.where(keep, p, 0.0)
    return q / q.sum()


@pytest.mark.slow
@pytest.mark.parametrize("k,top_p,seed", [(6, 1.0, 11), (0, 0.7, 12), (9, 0.8, 13)])
def test_truncated_output_distribution(k, top_p, seed):
    rng = np.random.default_rng(seed)
    V, N, B = 16, 3, 1_000_000
    base = rng.standard_normal((N, V)).astype(np.float32)
    q = special.softmax(base.astype(np.float64) + rng.standard_normal((N, V)) * 1.5, axis=-1).astype(np.float32)
    tokens = np.zeros((B, N), np.int32)
    for i in range(1, N):
        c = np.cumsum(q[i].astype(np.float64))
        tokens[:, i] = np.minimum(np.searchsorted(c, rng.random(B) * c[-1], side="right"), V - 1)
    r = oracle.accept("reject", np.broadcast_to(base, (B, N, V)), tokens, None, 1.0, np.broadcast_to(q, (B, N, V)),
                      rng.random((B, N), dtype=np.float32), rng.random((B, N), dtype=np.float32),
                      top_k=k, top_p=top_p)
    pt = _truncated(special.softmax(base[0].astype(np.float64)), base[0], k, top_p)
    obs = np.bincount(r["out_tokens"][:, 0], minlength=V)
    nz = pt > 0
    assert obs[~nz].sum() == 0  # nothing outside the kept set
    chi2, pv = stats.chisquare(obs[nz], pt[nz] * B)
    assert pv > 1e-3, (chi2, pv)
    # single-draft acceptance frequency: sum_x min(p~(x), q(x))
    acc1 = (r["accept_len"] >= 1).mean()
    want = np.minimum(pt, q[1].astype(np.float64)).sum()
    assert abs(acc1 - want) < 5 * np.sqrt(want * (1 - want) / B), (acc1, want)
