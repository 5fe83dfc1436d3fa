"""Pins of the fp64 tree-attention oracle against facts fixed outside it.

* Brute force per root-to-leaf path: a tree node sees only itself, its
  ancestors and the prefix (MEDUSA section, tree-attention paragraph), so its
  output equals ordinary causal attention over prefix + that path.
* Chains equal PyTorch's scaled_dot_product_attention (fp64, CPU) with a
  causal mask over the draft rows - a library routine, not a retyped formula.
* Grouped-query heads equal MHA on repeat_interleave'd KV heads.
* Relabelling the tree by a topological permutation permutes the outputs.
* bf16 storage widens exactly.
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import bf16_bits, bf16_to_f32, generate, scaled


def _rand_tree(rng, N, max_depth=None):
    par = np.full(N, -1, np.int32)
    depth = [0]
    for i in range(1, N):
        cand = [j for j in range(i) if max_depth is None or depth[j] < max_depth]
        par[i] = cand[int(rng.integers(len(cand)))]
        depth.append(depth[par[i]] + 1)
    return par


def _inputs(rng, B, N, Hq, Hkv, D, L, cap):
    q = rng.standard_normal((B, N, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    pl = np.asarray(L, np.int32)
    return q, k, v, pl


def _causal_path_attention(q_rows, keys, vals, L):
    """Causal attention of the path rows over prefix + path (plain NumPy)."""
    n = q_rows.shape[0]
    D = q_rows.shape[1]
    out = np.empty_like(q_rows)
    for t in range(n):
        kk = keys[: L + t + 1]
        vv = vals[: L + t + 1]
        s = kk @ q_rows[t] / np.sqrt(D)
        w = np.exp(s - s.max())
        out[t] = (w[:, None] * vv).sum(0) / w.sum()
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_tree_equals_per_path_causal_attention(seed):
    rng = np.random.default_rng(seed)
    B, N, Hq, Hkv, D = 2, 12, 4, 2, 16
    L = [7, 0] if seed == 0 else [5, 9]
    cap = max(L) + N + 3
    q, k, v, pl = _inputs(rng, B, N, Hq, Hkv, D, L, cap)
    par = np.stack([_rand_tree(rng, N), _rand_tree(rng, N, 3)])
    out = oracle.tree_attn(q, k, v, pl, par, "f32")
    G = Hq // Hkv
    for b in range(B):
        children = {i: [j for j in range(N) if par[b, j] == i] for i in range(N)}
        leaves = [i for i in range(N) if not children[i]]
        for leaf in leaves:
            path = []
            n = leaf
            while n >= 0:
                path.append(n)
                n = par[b, n]
            path = path[::-1]
            for h in range(Hq):
                g = h // G
                Lb = int(pl[b])
                keys = np.concatenate([k[b, g, :Lb], k[b, g, [Lb + n for n in path]]]).astype(np.float64)
                vals = np.concatenate([v[b, g, :Lb], v[b, g, [Lb + n for n in path]]]).astype(np.float64)
                ref = _causal_path_attention(q[b, path, h].astype(np.float64), keys, vals, Lb)
                np.testing.assert_allclose(out[b, path, h], ref, rtol=0, atol=1e-10)


def _sdpa_chain(q, k, v, pl, Hkv):
    B, N, Hq, D = q.shape
    G = Hq // Hkv
    out = np.empty((B, N, Hq, D))
    for b in range(B):
        L = int(pl[b])
        kk = torch.from_numpy(k[b, :, : L + N].astype(np.float64)).repeat_interleave(G, dim=0)
        vv = torch.from_numpy(v[b, :, : L + N].astype(np.float64)).repeat_interleave(G, dim=0)
        qq = torch.from_numpy(q[b].astype(np.float64)).transpose(0, 1)  # [Hq][N][D]
        mask = torch.ones(N, L + N, dtype=torch.bool)
        mask[:, L:] = torch.tril(torch.ones(N, N, dtype=torch.bool))
        o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
        out[b] = o.transpose(0, 1).numpy()
    return out


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (8, 2), (6, 1)])
def test_chain_equals_library_sdpa(Hq, Hkv):
    rng = np.random.default_rng(Hq * 10 + Hkv)
    B, N, D = 3, 6, 32
    L = [0, 1, 40]
    cap = 40 + N + 1
    q, k, v, pl = _inputs(rng, B, N, Hq, Hkv, D, L, cap)
    out = oracle.tree_attn(q, k, v, pl, None, "f32")
    ref = _sdpa_chain(q, k, v, pl, Hkv)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    # an explicit chain parent array is the same tree
    par = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    np.testing.assert_array_equal(oracle.tree_attn(q, k, v, pl, par, "f32"), out)


def test_single_query_decode():
    """N = 1: plain decode attention of one query over prefix + itself."""
    rng = np.random.default_rng(5)
    q, k, v, pl = _inputs(rng, 2, 1, 2, 2, 8, [3, 17], 20)
    out = oracle.tree_attn(q, k, v, pl, None, "f32")
    ref = _sdpa_chain(q, k, v, pl, 2)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_gqa_equals_repeated_mha():
    rng = np.random.default_rng(11)
    B, N, Hq, Hkv, D, L = 2, 5, 8, 2, 16, [9, 4]
    cap = 20
    q, k, v, pl = _inputs(rng, B, N, Hq, Hkv, D, L, cap)
    par = np.stack([_rand_tree(rng, N), _rand_tree(rng, N)])
    gqa = oracle.tree_attn(q, k, v, pl, par, "f32")
    mha = oracle.tree_attn(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), pl, par, "f32")
    np.testing.assert_allclose(gqa, mha, rtol=0, atol=1e-13)


def test_relabelling_permutes_outputs():
    rng = np.random.default_rng(3)
    B, N, Hq, Hkv, D, L = 1, 10, 2, 1, 8, [6]
    cap = L[0] + N
    q, k, v, pl = _inputs(rng, B, N, Hq, Hkv, D, L, cap)
    par = _rand_tree(rng, N)[None]
    out = oracle.tree_attn(q, k, v, pl, par, "f32")
    # a random topological relabelling: reverse-sorted by (depth, random key)
    depth = np.zeros(N, int)
    for i in range(1, N):
        depth[i] = depth[par[0, i]] + 1
    order = sorted(range(N), key=lambda i: (depth[i], rng.random()))
    new_of = {old: new for new, old in enumerate(order)}
    par2 = np.array([[-1 if par[0, old] < 0 else new_of[par[0, old]] for old in order]], np.int32)
    assert all(par2[0, i] < i for i in range(1, N))
    q2 = q[:, order]
    k2, v2 = k.copy(), v.copy()
    k2[0, :, L[0]: L[0] + N] = k[0, :, [L[0] + o for o in order]].transpose(1, 0, 2)
    v2[0, :, L[0]: L[0] + N] = v[0, :, [L[0] + o for o in order]].transpose(1, 0, 2)
    out2 = oracle.tree_attn(q2, k2, v2, pl, par2, "f32")
    np.testing.assert_allclose(out2, out[:, order], rtol=0, atol=1e-13)


def test_bf16_storage_widens_exactly():
    rng = np.random.default_rng(8)
    q, k, v, pl = _inputs(rng, 1, 4, 2, 1, 16, [5], 12)
    qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    a = oracle.tree_attn(qb, kb, vb, pl, None, "bf16")
    b = oracle.tree_attn(bf16_to_f32(qb), bf16_to_f32(kb), bf16_to_f32(vb), pl, None, "f32")
    np.testing.assert_array_equal(a, b)
    # and the bf16 rounding is round-to-nearest-even on the bit pattern
    x = np.array([1.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8, -2.5, 0.0], np.float32)
    np.testing.assert_array_equal(bf16_to_f32(bf16_bits(x)), np.array([1.0, 1.0, 1.0 + 2**-6, -2.5, 0.0], np.float32))


def test_row_selection_matches_full():
    w = generate(scaled(5, batch=2, num_q_heads=4, num_kv_heads=2, prefix_len=30, nodes=9, vocab=16),
                 with_accept=False)
    full = oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.prefix_len, w.parent, w.dtype)
    rows = np.array([[1, 8, 3], [0, 0, 0], [1, 4, 2]], np.int32)
    part = oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.prefix_len, w.parent, w.dtype, rows=rows)
    for j, (b, i, h) in enumerate(rows):
        np.testing.assert_array_equal(part[j], full[b, i, h])
    assert np.isfinite(full).all(), "poisoned rows beyond L_b + N must never be read"
