"""Pins of the oracle's Medusa candidate tree and depth-position rotary
embedding (MEDUSA section of the blog page "Fast Inference from Transformers
via Speculative Decoding": candidates are the Cartesian product of the heads'
top predictions, arranged as a tree; positions follow tree depth).

The tree is checked against the page's node count, the Cartesian-product
structure enumerated independently, and the workload generator's own
breadth-first builder.  The rotation is checked against cos(1) and sin(1), the
identity at position 0, norm preservation, composition of positions, the
relative-position property and the use of depth rather than node index.
"""
import itertools

import numpy as np
import pytest

import oracle
from workloads import scaled
from workloads.gen import _tree


def _heads(B, widths, seed=0, V=1000):
    rng = np.random.default_rng(seed)
    W = max(widths)
    return rng.integers(V, size=(B, len(widths), W)).astype(np.int32), rng.integers(V, size=B).astype(np.int32)


@pytest.mark.parametrize("widths", [(3, 2, 2, 2), (1,), (4,), (2, 3), (1, 1, 1, 1, 1), (5, 2, 1, 3)])
def test_tree_node_count(widths):
    # The page counts the new nodes as the sum over depths of the products of
    # the head widths; (3, 2, 2, 2) is the Medusa tree with 46 nodes, 22 of
    # them with children.
    head, root = _heads(2, widths)
    parent, tokens = oracle.medusa_tree(widths, root, head)
    expect = 1 + sum(int(np.prod(widths[:d + 1])) for d in range(len(widths)))
    assert parent.shape == (2, expect)
    if tuple(widths) == (3, 2, 2, 2):
        assert expect == 46
        internal = len(set(parent[0, 1:].tolist()))
        assert internal == 22


@pytest.mark.parametrize("widths", [(3, 2, 2, 2), (2, 3), (5, 2, 1, 3), (1, 1, 1)])
def test_tree_is_the_cartesian_product(widths):
    head, root = _heads(3, widths, seed=1)
    parent, tokens = oracle.medusa_tree(widths, root, head)
    B, N = parent.shape
    for b in range(B):
        assert parent[b, 0] == -1 and tokens[b, 0] == root[b]
        paths = {}
        depth = [0] * N
        for i in range(1, N):
            p = parent[b, i]
            assert 0 <= p < i
            depth[i] = depth[p] + 1
            assert depth[i] >= depth[i - 1]  # breadth first
        # root path of every node, as candidate indices per head
        for i in range(1, N):
            ranks, n = [], i
            while n > 0:
                d = depth[n]
                ranks.append(list(head[b, d - 1, :widths[d - 1]]).index(tokens[b, n]))
                n = parent[b, n]
            paths[i] = tuple(reversed(ranks))
        for d in range(1, len(widths) + 1):
            level = [paths[i] for i in range(1, N) if depth[i] == d]
            assert level == list(itertools.product(*[range(w) for w in widths[:d]]))


@pytest.mark.parametrize("topk", [(3, 2, 2, 2), (2, 3), (4, 1, 2)])
def test_tree_matches_generator(topk):
    # The workload generator builds the same tree shape with its own code.
    cfg = scaled(3, topk=topk)
    N = 1 + sum(int(np.prod(topk[:d + 1])) for d in range(len(topk)))
    gen = _tree(cfg, 2, N, 0)
    head, root = _heads(2, topk, seed=2)
    parent, _ = oracle.medusa_tree(topk, root, head)
    np.testing.assert_array_equal(parent, gen)


@pytest.mark.parametrize("widths", [(0, 2), (4, 4, 4), (2, 7)])
def test_tree_rejects_bad_widths(widths):
    # width 0, more than 64 nodes (1 + 4 + 16 + 64), width above the array
    head = np.zeros((1, len(widths), 4), np.int32)
    with pytest.raises(ValueError):
        oracle.medusa_tree(widths, np.zeros(1, np.int32), head)


def _rope(q, k, L, parent, base=10000.0, dtype="f32"):
    return oracle.tree_rope(q, k, np.asarray(L, np.int32), parent, dtype, base)


def test_rope_hand_example():
    # D = 4, position 1: pair (x0, x2) turns by 1 rad, pair (x1, x3) by
    # 10000^(-1/2) = 0.01 rad.  q = e0 -> (cos 1, 0, sin 1, 0).
    q = np.zeros((1, 1, 1, 4), np.float32)
    q[0, 0, 0, 0] = 1.0
    q2 = np.zeros_like(q)
    q2[0, 0, 0, 1] = 1.0
    k = np.zeros((1, 1, 4, 4), np.float32)
    for qq, expect in ((q, [0.5403023058681398, 0.0, 0.8414709848078965, 0.0]),
                       (q2, [0.0, 0.9999500004166653, 0.0, 0.009999833334166664])):
        qo, _ = _rope(qq, k, [1], None)
        np.testing.assert_allclose(qo[0, 0, 0], expect, atol=1e-15)


def _rand(B, N, Hq, Hkv, D, cap, seed=3):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, N, Hq, D)).astype(np.float32),
            rng.standard_normal((B, Hkv, cap, D)).astype(np.float32))


def test_rope_identity_at_position_zero_and_norms():
    q, k = _rand(2, 5, 4, 2, 16, 20)
    qo, ko = _rope(q, k, [0, 7], None)
    np.testing.assert_allclose(qo[0, 0], q[0, 0], atol=0)  # root of a request with an empty prefix
    np.testing.assert_allclose(ko[0, :, 0], k[0, :, 0], atol=0)
    for src, out in ((q[1, 3, 2], qo[1, 3, 2]), (k[1, 1, 7 + 2], ko[1, 1, 2])):
        half = src.shape[0] // 2
        n_in = src[:half].astype(np.float64) ** 2 + src[half:].astype(np.float64) ** 2
        n_out = out[:half] ** 2 + out[half:] ** 2
        np.testing.assert_allclose(n_out, n_in, rtol=1e-12)


def test_rope_composition_and_relative_position():
    D = 32
    q, k = _rand(1, 1, 1, 1, D, 64, seed=4)
    a, b = 5, 17
    qa, _ = _rope(q, k, [a], None)
    qab, _ = _rope(qa.astype(np.float32).reshape(q.shape), k, [b], None)
    qs, _ = _rope(q, k, [a + b], None)
    np.testing.assert_allclose(qab[0, 0, 0], qs[0, 0, 0], atol=1e-6)  # input re-rounded to fp32
    # <R(m) x, R(n) y> depends on m - n only
    kk = np.zeros((1, 1, 64, D), np.float32)
    kk[0, 0, :, :] = q[0, 0, 0]
    y = np.random.default_rng(5).standard_normal((1, 1, 1, D)).astype(np.float32)
    dots = []
    for m, n in ((3, 1), (12, 10), (40, 38)):
        rm, _ = _rope(y, kk, [m], None)
        _, rn = _rope(y, kk, [n], None)
        dots.append(float(rm[0, 0, 0] @ rn[0, 0, 0]))
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)


def test_rope_uses_depth_not_index():
    # Nodes 1 and 2 are siblings (depth 1): equal inputs turn equally; node 3
    # (depth 2) turns further.
    parent = np.array([[-1, 0, 0, 1]], np.int32)
    q = np.ones((1, 4, 1, 8), np.float32)
    k = np.ones((1, 1, 10, 8), np.float32)
    qo, ko = _rope(q, k, [6], parent)
    np.testing.assert_array_equal(qo[0, 1], qo[0, 2])
    np.testing.assert_array_equal(ko[0, 0, 1], ko[0, 0, 2])
    assert not np.allclose(qo[0, 3], qo[0, 1])
    chain_q, _ = _rope(q, k, [6], None)
    np.testing.assert_array_equal(qo[0, 3], chain_q[0, 2])  # depth 2 either way
