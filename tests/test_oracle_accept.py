"""Pins of the fp64 acceptance oracle against facts fixed outside it.

Rejection rule ("Speculative Decoding" / "Speculative Sampling" sections of the
blog page "Fast Inference from Transformers via Speculative Decoding"):
  * the emitted tokens are distributed exactly as the target (chi-square over
    10^6 seeded trials on a 16-token vocabulary, at T = 1 and T = 0.7);
  * the single-draft acceptance frequency is sum_x min(p, q);
  * a draft equal to the target is always accepted (MEDUSA section);
  * temperature 0 is greedy longest-prefix matching plus the argmax;
  * at least one and at most depth + 1 tokens per step;
  * the worked example in tests/golden/reject_hand_example.txt.
Typical acceptance (MEDUSA section, typical-acceptance paragraph):
  * the worked example in tests/golden/typical_hand_example.txt;
  * temperature 0 is greedy; with delta < 1 the argmax child is accepted;
  * the longest accepted prefix over all candidates (brute-force enumeration).
"""
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = {}
    cases = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            if key == "case":
                cases.append([float(v) for v in vals])
            else:
                rows[key] = [float(v) for v in vals]
    return rows, cases


def _chain_parent(B, N):
    return np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))


# ---------------------------------------------------------------- hand examples
def test_reject_hand_example():
    g, cases = _read_golden("reject_hand_example.txt")
    p, q, x = np.array(g["p"]), np.array(g["q"]), int(g["x"][0])
    assert abs(p[x] / q[x] - g["ratio"][0]) < 1e-12
    np.testing.assert_allclose(np.maximum(p - q, 0), g["residual"], atol=1e-12)
    V = 3
    for u, want_len, want_tok in cases:
        for us in (0.0, 0.3, 0.77, 0.999):
            logits = np.zeros((1, 2, V), np.float32)
            logits[0, 0] = np.log(p).astype(np.float32)
            logits[0, 1] = np.log([1 / 3] * 3).astype(np.float32)
            draft = np.zeros((1, 2, V), np.float32)
            draft[0, 1] = q
            tokens = np.array([[0, x]], np.int32)
            r = oracle.accept("reject", logits, tokens, None, 1.0, draft,
                              np.array([[0.0, u]], np.float32), np.array([[us, us]], np.float32))
            assert r["accept_len"][0] == int(want_len)
            assert r["out_tokens"][0, 0] == int(want_tok)
            if want_len == 0:  # residual (0.3, 0, 0) leaves only token 0
                assert r["out_tokens"][0, 1] == -1
            else:  # bonus from the uniform row: token floor(3 us)
                assert r["out_tokens"][0, 1] == min(int(3 * us + 1e-9), 2)


def test_typical_hand_example():
    g, cases = _read_golden("typical_hand_example.txt")
    p = np.array(g["p"])
    H = -(p * np.log(p)).sum()
    assert abs(H - g["entropy_nats"][0]) < 1e-12
    assert abs(np.exp(-H) - g["exp_minus_entropy"][0]) < 1e-12
    V = 4
    for eps, delta, thr, *want in cases:
        assert abs(min(eps, delta * np.exp(-H)) - thr) < 1e-12
        for x in range(V):
            logits = np.zeros((1, 2, V), np.float32)
            logits[0, 0] = np.log(p).astype(np.float32)
            r = oracle.accept("typical", logits, np.array([[0, x]], np.int32), None, 1.0,
                              epsilon=eps, delta=delta)
            assert r["accept_len"][0] == int(want[x]), (eps, delta, x)
            # the step's last token is argmax p at the stop node: token 0 for
            # the root row p and for the uniform child row alike
            assert r["out_tokens"][0, r["accept_len"][0]] == 0


# -------------------------------------------------------------- distributions
def _chi2_first_tokens(T, seed, trials=1_000_000, V=16, K=2):
    rng = np.random.default_rng(seed)
    N = K + 1
    base = rng.standard_normal((N, V)).astype(np.float32)
    dl = base + rng.standard_normal((N, V)).astype(np.float32) * 1.5
    # draft distribution for node i: softmax of noisy logits of its parent row
    qrows = np.zeros((N, V), np.float32)
    for i in range(1, N):
        qrows[i] = special.softmax(dl[i - 1].astype(np.float64) / T).astype(np.float32)
    B = trials
    tokens = np.zeros((B, N), np.int32)
    for i in range(1, N):
        c = np.cumsum(qrows[i].astype(np.float64))
        tokens[:, i] = np.minimum(np.searchsorted(c, rng.random(B) * c[-1], side="right"), V - 1)
    logits = np.broadcast_to(base, (B, N, V))
    draft = np.broadcast_to(qrows, (B, N, V))
    r = oracle.accept("reject", logits, tokens, None, T, draft,
                      rng.random((B, N), dtype=np.float32), rng.random((B, N), dtype=np.float32))
    p = special.softmax(base.astype(np.float64) / T, axis=-1)
    return r, tokens, p


@pytest.mark.slow
@pytest.mark.parametrize("T,seed", [(1.0, 101), (0.7, 202)])
def test_rejection_output_is_target_distributed(T, seed):
    r, tokens, p = _chi2_first_tokens(T, seed)
    B = tokens.shape[0]
    first = r["out_tokens"][:, 0]
    obs = np.bincount(first, minlength=16)
    chi2, pv = stats.chisquare(obs, p[0] * B)
    assert pv > 1e-3, (chi2, pv)
    # second token, given the first draft was kept, follows the target row at node 1
    kept = r["accept_len"] >= 1
    second = r["out_tokens"][kept, 1]
    obs2 = np.bincount(second, minlength=16)
    chi2b, pv2 = stats.chisquare(obs2, p[1] * kept.sum())
    assert pv2 > 1e-3, (chi2b, pv2)
    # 1 <= emitted <= K + 1
    emitted = (r["out_tokens"] >= 0).sum(1)
    assert emitted.min() >= 1 and emitted.max() <= 3
    np.testing.assert_array_equal(emitted, r["accept_len"] + 1)


@pytest.mark.slow
def test_single_draft_acceptance_rate_closed_form():
    rng = np.random.default_rng(7)
    V, B = 16, 400_000
    p = special.softmax(rng.standard_normal(V))
    q = special.softmax(rng.standard_normal(V) * 2)
    beta = np.minimum(p, q).sum()
    logits = np.broadcast_to(np.log(p).astype(np.float32)[None, None, :], (B, 2, V)).copy()
    draft = np.zeros((1, 2, V), np.float32)
    draft[0, 1] = q
    draft = np.broadcast_to(draft, (B, 2, V))
    cq = np.cumsum(draft[0, 1].astype(np.float64))
    tokens = np.zeros((B, 2), np.int32)
    tokens[:, 1] = np.minimum(np.searchsorted(cq, rng.random(B) * cq[-1], side="right"), V - 1)
    r = oracle.accept("reject", logits, tokens, None, 1.0, draft,
                      rng.random((B, 2), dtype=np.float32), rng.random((B, 2), dtype=np.float32))
    rate = r["accept_len"].mean()
    sd = np.sqrt(beta * (1 - beta) / B)
    assert abs(rate - beta) < 5 * sd, (rate, beta)


def test_draft_equal_to_target_is_always_accepted():
    rng = np.random.default_rng(9)
    B, N, V, T = 200, 9, 64, 0.8
    for tree in ("chain", "random"):
        if tree == "chain":
            par = _chain_parent(B, N)
        else:
            par = np.full((B, N), -1, np.int32)
            for b in range(B):
                for i in range(1, N):
                    par[b, i] = rng.integers(i)
        logits = rng.standard_normal((B, N, V)).astype(np.float32) * 2
        draft = np.zeros((B, N, V), np.float32)
        tokens = np.zeros((B, N), np.int32)
        for b in range(B):
            for i in range(1, N):
                q = special.softmax(logits[b, par[b, i]].astype(np.float64) / T)
                draft[b, i] = q
                tokens[b, i] = rng.choice(V, p=q / q.sum())
        u = rng.random((B, N), dtype=np.float32) * np.float32(0.999)
        r = oracle.accept("reject", logits, tokens, par, T, draft, u, rng.random((B, N), dtype=np.float32))
        depth = np.zeros((B, N), int)
        for i in range(1, N):
            depth[:, i] = depth[np.arange(B), par[:, i]] + 1
        np.testing.assert_array_equal(r["accept_len"], depth.max(1))


def _greedy_reference(logits, tokens, par):
    B, N, V = logits.shape
    exp_len, exp_out = [], []
    for b in range(B):
        # enumerate every root path; keep nodes whose token equals the parent's argmax
        ok = {0: True}
        depth = {0: 0}
        for i in range(1, N):
            u = par[b, i]
            depth[i] = depth[u] + 1
            ok[i] = ok[u] and tokens[b, i] == int(np.argmax(logits[b, u]))
        v = max((i for i in range(N) if ok[i]), key=lambda i: (depth[i], -i))
        path = []
        n = v
        while n >= 0:
            path.append(n)
            n = par[b, n]
        path = path[::-1]
        exp_len.append(depth[v])
        exp_out.append([int(tokens[b, n]) for n in path[1:]] + [int(np.argmax(logits[b, v]))])
    return exp_len, exp_out


@pytest.mark.parametrize("rule", ["reject", "typical"])
def test_temperature_zero_is_greedy(rule):
    rng = np.random.default_rng(12)
    B, N, V = 300, 7, 12
    par = np.full((B, N), -1, np.int32)
    for b in range(B):
        for i in range(1, N):
            par[b, i] = rng.integers(i) if b % 2 else i - 1
    logits = rng.standard_normal((B, N, V)).astype(np.float32)
    tokens = np.zeros((B, N), np.int32)
    for b in range(B):
        for i in range(1, N):
            tokens[b, i] = int(np.argmax(logits[b, par[b, i]])) if rng.random() < 0.7 else rng.integers(V)
    draft = rng.random((B, N, V)).astype(np.float32)
    draft /= draft.sum(-1, keepdims=True)
    r = oracle.accept(rule, logits, tokens, par, 0.0, draft if rule == "reject" else None,
                      rng.random((B, N), dtype=np.float32), rng.random((B, N), dtype=np.float32),
                      epsilon=0.3, delta=0.5)
    exp_len, exp_out = _greedy_reference(logits, tokens, par)
    np.testing.assert_array_equal(r["accept_len"], exp_len)
    for b in range(B):
        a = exp_len[b]
        np.testing.assert_array_equal(r["out_tokens"][b, : a + 1], exp_out[b])
        assert (r["out_tokens"][b, a + 1:] == -1).all()


def test_typical_argmax_child_always_accepted():
    rng = np.random.default_rng(13)
    B, V = 500, 50
    logits = (rng.standard_normal((B, 2, V)) * rng.uniform(0.1, 4, (B, 1, 1))).astype(np.float32)
    tokens = np.zeros((B, 2), np.int32)
    tokens[:, 1] = np.argmax(logits[:, 0], axis=-1)
    for T in (0.3, 1.0, 2.0):
        for delta in (0.0, 0.5, 0.99):
            r = oracle.accept("typical", logits, tokens, None, T, epsilon=10.0, delta=delta)
            assert (r["accept_len"] == 1).all()


def _brute_tree(rule, logits, draft, tokens, par, ua, T, eps, delta):
    """Enumerate every root path; a node is on an accepted path when every node
    on its root path passes its own test.  Returns the longest such path."""
    B, N, V = logits.shape
    lens, stops = [], []
    for b in range(B):
        def passes(i):
            u = par[b, i]
            p = special.softmax(logits[b, u].astype(np.float64) / T)
            x = tokens[b, i]
            if rule == "reject":
                return float(ua[b, i]) * float(draft[b, i, x]) < p[x]
            H = -(p[p > 0] * np.log(p[p > 0])).sum()
            return p[x] > min(eps, delta * np.exp(-H))
        best, best_len = 0, 0
        for i in range(1, N):
            path = []
            n = i
            while n > 0:
                path.append(n)
                n = par[b, n]
            if all(passes(n) for n in path) and len(path) > best_len:
                best, best_len = i, len(path)
        lens.append(best_len)
        stops.append(best)
    return np.array(lens), np.array(stops)


@pytest.mark.parametrize("rule", ["reject", "typical"])
def test_longest_accepted_prefix_brute_force(rule):
    rng = np.random.default_rng(21 if rule == "reject" else 22)
    B, N, V, T = 120, 8, 10, 0.9
    par = np.full((B, N), -1, np.int32)
    for b in range(B):
        for i in range(1, N):
            par[b, i] = rng.integers(i)
    logits = (rng.standard_normal((B, N, V)) * 1.5).astype(np.float32)
    draft = rng.random((B, N, V)).astype(np.float32) ** 3
    draft /= draft.sum(-1, keepdims=True)
    tokens = rng.integers(V, size=(B, N)).astype(np.int32)
    ua = rng.random((B, N), dtype=np.float32)
    r = oracle.accept(rule, logits, tokens, par, T, draft if rule == "reject" else None, ua,
                      rng.random((B, N), dtype=np.float32), epsilon=0.12, delta=0.4)
    lens, stops = _brute_tree(rule, logits, draft, tokens, par, ua, T, 0.12, 0.4)
    np.testing.assert_array_equal(r["accept_len"], lens)
    np.testing.assert_array_equal(r["stop"], stops)
    # the path is the root path of the stop node and the tokens follow it
    for b in range(B):
        a = r["accept_len"][b]
        pth = r["path"][b]
        assert pth[0] == 0 and pth[a] == stops[b] and (pth[a + 1:] == -1).all()
        for d in range(1, a + 1):
            assert par[b, pth[d]] == pth[d - 1]
            assert r["out_tokens"][b, d - 1] == tokens[b, pth[d]]
        assert 0 <= r["out_tokens"][b, a] < V


def test_residual_draw_follows_residual_distribution():
    """Rejection at node 1 of a chain: the correction token is distributed as
    norm(max(0, p - q)) (chi-square on the rejected trials)."""
    rng = np.random.default_rng(31)
    V, B = 8, 300_000
    p = special.softmax(rng.standard_normal(V) * 1.2)
    q = special.softmax(rng.standard_normal(V) * 1.2)
    logits = np.broadcast_to(np.log(p).astype(np.float32)[None, None, :], (B, 2, V)).copy()
    draft = np.zeros((1, 2, V), np.float32)
    draft[0, 1] = q
    tokens = np.zeros((B, 2), np.int32)
    tokens[:, 1] = rng.integers(V, size=B)
    r = oracle.accept("reject", logits, tokens, None, 1.0, np.broadcast_to(draft, (B, 2, V)),
                      rng.random((B, 2), dtype=np.float32), rng.random((B, 2), dtype=np.float32))
    rej = r["accept_len"] == 0
    pf = special.softmax(np.log(p).astype(np.float32).astype(np.float64))
    res = np.maximum(pf - q.astype(np.float32).astype(np.float64), 0)
    res /= res.sum()
    obs = np.bincount(r["out_tokens"][rej, 0], minlength=V)
    nz = res > 0
    assert obs[~nz].sum() == 0
    chi2, pv = stats.chisquare(obs[nz], res[nz] * rej.sum())
    assert pv > 1e-3, (chi2, pv)


def test_chain_parent_array_equals_chain():
    rng = np.random.default_rng(41)
    B, N, V = 50, 6, 20
    logits = rng.standard_normal((B, N, V)).astype(np.float32)
    draft = rng.random((B, N, V)).astype(np.float32)
    draft /= draft.sum(-1, keepdims=True)
    tokens = rng.integers(V, size=(B, N)).astype(np.int32)
    ua, us = rng.random((B, N), dtype=np.float32), rng.random((B, N), dtype=np.float32)
    a = oracle.accept("reject", logits, tokens, None, 1.3, draft, ua, us)
    b = oracle.accept("reject", logits, tokens, _chain_parent(B, N), 1.3, draft, ua, us)
    for key in ("accept_len", "path", "out_tokens", "stop"):
        np.testing.assert_array_equal(a[key], b[key])


def test_single_node_is_a_plain_draw():
    """N = 1 (no drafts): one token drawn from p_root by inverse CDF."""
    rng = np.random.default_rng(43)
    B, V = 2000, 9
    logits = rng.standard_normal((B, 1, V)).astype(np.float32)
    us = rng.random((B, 1), dtype=np.float32)
    r = oracle.accept("reject", logits, np.zeros((B, 1), np.int32), None, 1.0, np.zeros((B, 1, V), np.float32),
                      np.zeros((B, 1), np.float32), us)
    assert (r["accept_len"] == 0).all()
    for b in range(B):
        c = np.cumsum(special.softmax(logits[b, 0].astype(np.float64)))
        assert r["out_tokens"][b, 0] == np.searchsorted(c, us[b, 0] * c[-1], side="right")


def test_margins_bracket_the_decision():
    """Moving u_accept across the ratio flips the decision; the oracle's margin
    is the distance to that flip."""
    V = 5
    p = np.array([0.1, 0.2, 0.3, 0.25, 0.15])
    q = np.array([0.3, 0.1, 0.3, 0.2, 0.1])
    x = 0  # ratio 1/3
    logits = np.log(p).astype(np.float32)[None, None, :].repeat(2, 1)
    draft = np.zeros((1, 2, V), np.float32)
    draft[0, 1] = q
    pf = special.softmax(logits[0, 0].astype(np.float64))
    ratio = pf[x] / np.float64(np.float32(q[x]))
    for du in (-1e-3, 1e-3):
        u = np.float32(ratio + du)
        r = oracle.accept("reject", logits, np.array([[0, x]], np.int32), None, 1.0, draft,
                          np.array([[0, u]], np.float32), np.array([[0.5, 0.5]], np.float32))
        assert r["accept_len"][0] == (1 if du < 0 else 0)
        assert r["margin"][0] <= abs(float(u) - ratio) + 1e-12


def test_reject_tree_hand_example():
    g, cases = _read_golden("reject_tree_hand_example.txt")
    V = 3
    p = np.array(g["p"])
    for ua1, ua2, us, want_len, want_tok in cases:
        logits = np.zeros((1, 3, V), np.float32)
        logits[0, 0] = np.log(p).astype(np.float32)
        draft = np.zeros((1, 3, V), np.float32)
        draft[0, 1], draft[0, 2] = g["q1"], g["q2"]
        tokens = np.array([[0, int(g["x1"][0]), int(g["x2"][0])]], np.int32)
        par = np.array([[-1, 0, 0]], np.int32)
        r = oracle.accept("reject", logits, tokens, par, 1.0, draft,
                          np.array([[0, ua1, ua2]], np.float32), np.array([[us, us, us]], np.float32))
        assert r["accept_len"][0] == int(want_len)
        assert r["out_tokens"][0, 0] == int(want_tok)
        # both children accepted: the smaller index is the stop node
        if ua1 < 0.6 and ua2 < 0.25:
            assert r["stop"][0] == 1
