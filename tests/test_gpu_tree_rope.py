"""GPU parity of the Medusa candidate tree and the depth-position rotary
embedding (MEDUSA section of the blog page "Fast Inference from Transformers
via Speculative Decoding"), through the C ABI, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_tree_amd as sv
from workloads.gen import bf16_bits, bf16_to_f32
from tests.gpu_helpers import announce, check_attention, dev_kv, host_f64

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("widths", [(3, 2, 2, 2), (1,), (10,), (2, 3), (1, 1, 1, 1, 1, 1, 1), (5, 2, 1, 3), (63 * [1])])
def test_medusa_tree_matches_oracle(widths):
    widths = list(widths)
    announce(f"medusa tree widths={widths[:8]}{'...' if len(widths) > 8 else ''}")
    B, K, W = 3, len(widths), max(widths) + 1
    rng = np.random.default_rng(len(widths) * 7 + sum(widths))
    head = rng.integers(128256, size=(B, K, W)).astype(np.int32)
    root = rng.integers(128256, size=B).astype(np.int32)
    ref_p, ref_t = oracle.medusa_tree(widths, root, head)
    par, tok = sv.spec_medusa_tree(widths, torch.from_numpy(root).cuda(), torch.from_numpy(head).cuda())
    torch.cuda.synchronize()
    np.testing.assert_array_equal(par.cpu().numpy(), ref_p)
    np.testing.assert_array_equal(tok.cpu().numpy(), ref_t)
    assert sv.spec_medusa_tree_nodes(widths, W) == ref_p.shape[1]


def test_medusa_tree_empty_batch():
    announce("medusa tree B=0")
    head = torch.empty(0, 2, 3, dtype=torch.int32, device="cuda")
    par, tok = sv.spec_medusa_tree([3, 2], torch.empty(0, dtype=torch.int32, device="cuda"), head)
    assert par.shape == (0, 10)


def _random_parent(rng, B, N, max_depth):
    par = np.full((B, N), -1, np.int32)
    for b in range(B):
        depth = [0]
        for i in range(1, N):
            cand = [j for j in range(i) if depth[j] < max_depth]
            p = cand[int(rng.integers(len(cand)))]
            par[b, i] = p
            depth.append(depth[p] + 1)
    return par


def _rope_case(dtype, D, B, N, Hq, Hkv, L, tree, seed, base=10000.0):
    rng = np.random.default_rng(seed)
    L = np.asarray(L, np.int32)
    cap = int(L.max()) + N + 3
    q = rng.standard_normal((B, N, Hq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, cap, D)).astype(np.float32)
    if dtype == "bf16":
        q, k = bf16_bits(q), bf16_bits(k)
    parent = _random_parent(rng, B, N, 6) if tree else None
    return q, k, L, parent, base


@pytest.mark.parametrize("dtype,D,B,N,Hq,Hkv,L,tree", [
    ("bf16", 128, 3, 46, 32, 32, [0, 700, 4096], True),     # Medusa-shaped, MHA
    ("bf16", 128, 2, 6, 32, 8, [2048, 31], False),          # Llama-3-8B chain
    ("bf16", 128, 2, 64, 64, 8, [32768, 1000], True),       # long context, 64 nodes
    ("bf16", 64, 2, 20, 8, 2, [5, 129], True),
    ("f32", 128, 2, 9, 4, 4, [77, 0], True),
    ("f32", 64, 1, 5, 4, 1, [128], False),
])
def test_tree_rope_matches_oracle(dtype, D, B, N, Hq, Hkv, L, tree):
    announce(f"tree rope {dtype} D={D} B={B} N={N} Hq={Hq} Hkv={Hkv} L={L} tree={tree}")
    q, k, Lp, parent, base = _rope_case(dtype, D, B, N, Hq, Hkv, L, tree, seed=D + N + B)
    ref_q, ref_k = oracle.tree_rope(q, k, Lp, parent, dtype, base)
    qd, kd = dev_kv(q, dtype), dev_kv(k, dtype)
    k_before = host_f64(kd)
    sv.spec_tree_rope(qd, kd, torch.from_numpy(Lp).cuda(), None if parent is None else torch.from_numpy(parent).cuda(),
                      base)
    torch.cuda.synchronize()
    gq, gk = host_f64(qd), host_f64(kd)
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -22
    err_q = np.abs(gq - ref_q)
    assert (err_q <= rel * np.abs(ref_q) + 1e-6).all(), f"q: max err {err_q.max():.3e}"
    for b in range(B):
        tree_rows = gk[b, :, Lp[b]:Lp[b] + N]
        err_k = np.abs(tree_rows - ref_k[b])
        assert (err_k <= rel * np.abs(ref_k[b]) + 1e-6).all(), f"k: max err {err_k.max():.3e}"
        # the prefix and the spare rows are untouched
        np.testing.assert_array_equal(gk[b, :, :Lp[b]], k_before[b, :, :Lp[b]])
        np.testing.assert_array_equal(gk[b, :, Lp[b] + N:], k_before[b, :, Lp[b] + N:])


def test_tree_then_rope_then_attention():
    # End to end: the candidate tree built on the GPU, its rotation, then tree
    # attention, against the oracle's tree, rotation (rounded to bf16) and
    # attention.
    announce("medusa tree -> rope -> attention")
    rng = np.random.default_rng(11)
    widths, B, Hq, Hkv, D, base = [3, 2, 2], 2, 16, 4, 128, 500000.0
    N = 1 + 3 + 6 + 12
    L = np.array([300, 1200], np.int32)
    cap = int(L.max()) + N
    head = rng.integers(32000, size=(B, 3, 3)).astype(np.int32)
    root = rng.integers(32000, size=B).astype(np.int32)
    q = bf16_bits(rng.standard_normal((B, N, Hq, D)).astype(np.float32))
    k = bf16_bits(rng.standard_normal((B, Hkv, cap, D)).astype(np.float32))
    v = bf16_bits(rng.standard_normal((B, Hkv, cap, D)).astype(np.float32))
    ref_par, _ = oracle.medusa_tree(widths, root, head)
    rq, rk = oracle.tree_rope(q, k, L, ref_par, "bf16", base)
    q_rot = bf16_bits(rq.astype(np.float32))
    k_rot = k.copy()
    for b in range(B):
        k_rot[b, :, L[b]:L[b] + N] = bf16_bits(rk[b].astype(np.float32))
    ref = oracle.tree_attn(q_rot, k_rot, v, L, ref_par, "bf16")

    par, _ = sv.spec_medusa_tree(widths, torch.from_numpy(root).cuda(), torch.from_numpy(head).cuda())
    qd, kd, vd = dev_kv(q, "bf16"), dev_kv(k, "bf16"), dev_kv(v, "bf16")
    pl = torch.from_numpy(L).cuda()
    sv.spec_tree_rope(qd, kd, pl, par, base)
    out = sv.spec_verify_attn(qd, kd, vd, pl, par, int(L.max()))
    torch.cuda.synchronize()
    check_attention(host_f64(out), ref, "tree -> rope -> attention")


def _fused_case(dtype, D, B, N, Hq, Hkv, L, tree, seed):
    q, k, Lp, parent, base = _rope_case(dtype, D, B, N, Hq, Hkv, L, tree, seed, base=500000.0)
    rng = np.random.default_rng(seed + 1)
    v = rng.standard_normal(k.shape).astype(np.float32)
    if dtype == "bf16":
        v = bf16_bits(v)
    return q, k, v, Lp, parent, base


def _rounded(x, dtype):
    return bf16_bits(x.astype(np.float32)) if dtype == "bf16" else x.astype(np.float32)


@pytest.mark.parametrize("dtype,D,B,N,Hq,Hkv,L,tree", [
    ("bf16", 128, 2, 6, 32, 8, [2048, 31], False),          # Llama-3-8B chain: one-wave kernel, R = 24
    ("bf16", 128, 3, 46, 32, 32, [0, 700, 4096], True),     # Medusa-shaped tree, MHA: R = 46
    ("bf16", 128, 2, 64, 64, 8, [3000, 1000], True),        # 64-node tree, R = 512: shared-KV kernel
    ("bf16", 128, 5, 8, 32, 8, [512, 8000, 77, 1, 4000], False),  # ragged chains
    ("bf16", 64, 2, 20, 8, 2, [5, 129], True),              # D = 64
    ("bf16", 64, 2, 40, 16, 4, [300, 90], True),            # D = 64, R = 160: shared-KV kernel
    ("bf16", 64, 4, 6, 16, 4, [3000, 100, 2900, 1], True),  # D = 64, R = 24, 1.5k blocks: key-split waves
    ("f32", 128, 2, 9, 4, 4, [77, 0], True),                # fp32 VALU kernel
    ("f32", 64, 1, 5, 4, 1, [128], False),
])
def test_fused_rope_attention_matches_oracle(dtype, D, B, N, Hq, Hkv, L, tree):
    """spec_verify_attn with rope_base > 0 against the oracle's depth-position
    rotation (rounded to the dtype) followed by its tree attention; q and the
    cache are read, not written."""
    announce(f"fused rope attention {dtype} D={D} B={B} N={N} Hq={Hq} Hkv={Hkv} L={L} tree={tree}")
    q, k, v, Lp, parent, base = _fused_case(dtype, D, B, N, Hq, Hkv, L, tree, seed=3 * D + N + B)
    rq, rk = oracle.tree_rope(q, k, Lp, parent, dtype, base)
    q_rot = _rounded(rq, dtype)
    k_rot = k.copy()
    for b in range(B):
        k_rot[b, :, Lp[b]:Lp[b] + N] = _rounded(rk[b], dtype)
    ref = oracle.tree_attn(q_rot, k_rot, v, Lp, parent, dtype)
    qd, kd, vd = dev_kv(q, dtype), dev_kv(k, dtype), dev_kv(v, dtype)
    q0, k0 = qd.clone(), kd.clone()
    out = sv.spec_verify_attn(qd, kd, vd, torch.from_numpy(Lp).cuda(),
                              None if parent is None else torch.from_numpy(parent).cuda(), int(Lp.max()),
                              rope_base=base)
    torch.cuda.synchronize()
    check_attention(host_f64(out), ref, f"fused rope {dtype} D={D}")
    assert torch.equal(qd, q0) and torch.equal(kd, k0), "the fused call must not write q or the cache"


@pytest.mark.parametrize("dtype,D,tree", [("bf16", 128, False), ("bf16", 128, True), ("bf16", 64, True),
                                          ("f32", 128, True)])
def test_fused_rope_commit_matches_oracle(dtype, D, tree):
    """spec_commit_kv with rope_base > 0: the accepted K rows land rotated at
    their new positions (the oracle: rotate the tree rows at their depth
    positions, then commit); V rows move unchanged; the prefix is untouched."""
    B, N, Hkv = 4, 12, 2
    L = [40, 0, 333, 7]
    announce(f"fused rope commit {dtype} D={D} tree={tree}")
    q, k, v, Lp, parent, base = _fused_case(dtype, D, B, N, 4, Hkv, L, tree, seed=D + 17 * tree)
    par = parent if parent is not None else np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    rng = np.random.default_rng(5)
    path = np.full((B, N), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b in range(B):  # a random root path of each tree
        node, p = 0, [0]
        while True:
            kids = [i for i in range(N) if par[b, i] == node]
            if not kids or rng.random() < 0.15:
                break
            node = kids[int(rng.integers(len(kids)))]
            p.append(node)
        path[b, :len(p)] = p
        acc[b] = len(p) - 1
    _, rk = oracle.tree_rope(q, k, Lp, parent, dtype, base)
    k_ref, v_ref = k.copy(), v.copy()
    for b in range(B):
        k_ref[b, :, Lp[b]:Lp[b] + N] = _rounded(rk[b], dtype)
    pl_ref = oracle.commit(k_ref, v_ref, Lp.copy(), path, acc)
    kd, vd = dev_kv(k, dtype), dev_kv(v, dtype)
    pl = torch.from_numpy(Lp.copy()).cuda()
    sv.spec_commit_kv(kd, vd, pl, torch.from_numpy(path).cuda(), torch.from_numpy(acc).cuda(), rope_base=base)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pl.cpu().numpy(), pl_ref)
    gk, gv = host_f64(kd), host_f64(vd)
    rk_ref, rv_ref = host_f64(dev_kv(k_ref, dtype)), host_f64(dev_kv(v_ref, dtype))
    rel = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -22
    for b in range(B):
        n = int(pl_ref[b])  # the grown prefix
        err = np.abs(gk[b, :, :n] - rk_ref[b, :, :n])
        assert (err <= rel * np.abs(rk_ref[b, :, :n]) + 1e-6).all(), f"K b={b}: max err {err.max():.3e}"
        np.testing.assert_array_equal(gv[b, :, :n], rv_ref[b, :, :n])
