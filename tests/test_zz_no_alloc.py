"""GPU: spec_accept_reject_noalloc (the library's per-GPU scratch in place of
a workspace) returns exactly what spec_accept_reject returns, on two calls in
a row, the second smaller than the first (the scratch keeps the first call's
contents), and a third call repeats the first."""
import numpy as np
import pytest
import torch

import speculative_decoding_verification_tree_amd as sv
from workloads import generate, scaled
from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu


def _inputs(w):
    par = None if w.is_chain else torch.from_numpy(w.parent).cuda()
    return (torch.from_numpy(w.target_logits).cuda(), torch.from_numpy(w.draft_probs).cuda(),
            torch.from_numpy(w.tokens).cuda(), par, torch.from_numpy(w.u_accept).cuda(),
            torch.from_numpy(w.u_sample).cuda(), w.temperature)


def _outs(B, N):
    return (torch.full((B,), -7, dtype=torch.int32, device="cuda"),
            torch.full((B, N), -7, dtype=torch.int32, device="cuda"),
            torch.full((B, N), -7, dtype=torch.int32, device="cuda"))


def _both(w, what):
    announce(f"no-alloc acceptance: {what} B={w.B} N={w.N} V={w.V}")
    args = _inputs(w)
    ref = sv.spec_accept_reject(*args)
    got = sv.spec_accept_reject_noalloc(*args, *_outs(w.B, w.N))
    torch.cuda.synchronize()
    for r, g, n in zip(ref, got, ("accept_len", "path", "out_tokens")):
        assert torch.equal(r, g), f"{what}: {n} differs from spec_accept_reject"
    return [t.cpu().numpy() for t in got]


def test_noalloc_matches_workspace_entry_point():
    big = generate(scaled(4, batch=64), with_attention=False)       # the ragged batch's acceptance shape
    small = generate(scaled(5, batch=3, nodes=40, vocab=9000), with_attention=False)  # a tree, fewer chunks
    first = _both(big, "ragged batch, full vocabulary")
    _both(small, "64-node trees, small vocabulary, after a larger call")
    again = _both(big, "ragged batch again")
    for a, b in zip(first, again):
        assert np.array_equal(a, b)


def test_noalloc_rejects_oversized_shapes():
    # Host-side check before any launch: the workspace this shape needs is
    # above the scratch array's size.
    B, N, V = 4096, 64, 128256
    assert sv.spec_accept_workspace_bytes(B, N, V) > (8 << 20)
    dummy = torch.empty(16, dtype=torch.float32, device="cuda")
    i32 = torch.empty(16, dtype=torch.int32, device="cuda")
    rc = sv.lib().spec_accept_reject_noalloc(B, N, V, dummy.data_ptr(), dummy.data_ptr(), i32.data_ptr(), None,
                                             dummy.data_ptr(), dummy.data_ptr(), 1.0, i32.data_ptr(),
                                             i32.data_ptr(), i32.data_ptr(), None)
    assert rc == -3  # SPEC_EWORKSPACE
