"""GPU parity of the multi-draft tree rejection (recursive residuals over the
children of each node, in index order; the "Speculative Sampling" and
MEDUSA sections of the blog page "Fast Inference from Transformers via
Speculative Decoding" give the single-draft rule and its reuse over trees),
through the C ABI, against the oracle on the same seeded inputs."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_tree_amd as sv
from workloads import scaled, generate
from tests.gpu_helpers import announce, check_accept, f32

pytestmark = pytest.mark.gpu


def _run(w, T=None):
    T = w.temperature if T is None else T
    d = dict(lg=torch.from_numpy(w.target_logits).cuda(), dp=torch.from_numpy(w.draft_probs).cuda(),
             tk=torch.from_numpy(w.tokens).cuda(), ua=torch.from_numpy(w.u_accept).cuda(),
             us=torch.from_numpy(w.u_sample).cuda(), par=None if w.is_chain else torch.from_numpy(w.parent).cuda())
    al, path, out = sv.spec_accept_multidraft(d["lg"], d["dp"], d["tk"], d["par"], d["ua"], d["us"], T)
    torch.cuda.synchronize()
    return dict(accept_len=al.cpu().numpy(), path=path.cpu().numpy(), out_tokens=out.cpu().numpy()), d


def _ref(w, T=None):
    T = w.temperature if T is None else T
    return oracle.accept_multidraft(w.target_logits, w.tokens, w.parent, f32(T), w.draft_probs, w.u_accept,
                                    w.u_sample)


CASES = [
    (dict(batch=16, vocab=300, prefix_len=(0, 8)), None),         # random 64-node trees, small vocabulary
    (dict(batch=6, prefix_len=(0, 8)), None),                     # V = 128256
    (dict(batch=8, vocab=1001, nodes=20, prefix_len=(0, 8)), None),   # V % 4 != 0
    (dict(batch=8, vocab=2000, nodes=64, max_depth=63, prefix_len=(0, 8)), None),  # deep tree
    (dict(batch=12, vocab=500, prefix_len=(0, 8)), 0.0),          # T = 0: greedy walk
    (dict(batch=8, vocab=700, nodes=1, prefix_len=(0, 8)), None), # N = 1: bonus only
]


@pytest.mark.parametrize("over,T", CASES)
def test_multidraft_matches_oracle(over, T):
    w = generate(scaled(5, **over), with_attention=False)
    announce(f"multidraft accept cfg5 {over} T={T} B={w.B} N={w.N} V={w.V}")
    gpu, d = _run(w, T)
    ref = _ref(w, T)
    excl = check_accept(w, gpu, ref)
    announce(f"  near-tie requests excluded: {excl} of {w.B}")
    assert excl <= max(2, w.B // 6), excl
    again, _ = _run(w, T)
    for key in gpu:
        np.testing.assert_array_equal(again[key], gpu[key])


def test_multidraft_on_chains_is_the_plain_rule():
    w = generate(scaled(4, batch=24, prefix_len=(10, 40)), with_attention=False)
    announce("multidraft on chains vs spec_accept_reject")
    gpu, d = _run(w)
    al, path, out = sv.spec_accept_reject(d["lg"], d["dp"], d["tk"], d["par"], d["ua"], d["us"], w.temperature)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(gpu["accept_len"], al.cpu().numpy())
    np.testing.assert_array_equal(gpu["path"], path.cpu().numpy())
    np.testing.assert_array_equal(gpu["out_tokens"], out.cpu().numpy())


def test_multidraft_cartesian_tree():
    # Medusa-shaped tree (3, 2, 2) whose siblings share one draft distribution.
    w = generate(scaled(3, batch=6, vocab=3000, rule="reject"), with_attention=False)
    if w.draft_probs is None:  # the Medusa workload draws its candidates from heads: give it drafts
        rng = np.random.default_rng(3)
        B, N, V = w.target_logits.shape
        dp = np.zeros((B, N, V), np.float32)
        for b in range(B):
            for i in range(1, N):
                q = rng.random(V) ** 4
                dp[b, i] = (q / q.sum()).astype(np.float32)
        for b in range(B):  # siblings share their parent's first child's q
            for i in range(1, N):
                sib = [j for j in range(1, N) if w.parent[b, j] == w.parent[b, i]]
                dp[b, i] = dp[b, sib[0]]
        w.draft_probs = dp
        w.u_accept = rng.random((B, N), dtype=np.float32)
        w.u_sample = rng.random((B, N), dtype=np.float32)
    announce(f"multidraft accept on a Medusa tree B={w.B} N={w.N}")
    gpu, _ = _run(w, 1.0)
    excl = check_accept(w, gpu, _ref(w, 1.0))
    assert excl <= 1, excl
