"""Shared helpers of the GPU parity tests: move a seeded workload to the device,
run the HIP path through the C-ABI binding, run the oracle on the same inputs
and compare to the stated bar.

Bars
  attention : |gpu - oracle| <= 2e-2 + 1e-2 * |oracle| elementwise (the oracle
              is fp64 on the bf16-rounded inputs; the GPU output is stored in
              the input dtype)
  acceptance: accept_len, path and out_tokens identical, except requests whose
              oracle margin (distance of any output-deciding comparison from
              its threshold) is below 1e-6; those are counted and only checked
              for validity
"""
import sys

import numpy as np
import torch

import oracle
import speculative_decoding_verification_tree_amd as sv

ATOL, RTOL = 2e-2, 1e-2
NEAR_TIE = 1e-6


def announce(msg):
    sys.__stderr__.write(f"[gpu-case] {msg}\n")
    sys.__stderr__.flush()


def dev_kv(arr, dtype):
    """NumPy (uint16 bf16 bits or float32) -> device tensor of the matching dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).cuda()


def host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def f32(x):
    """The value a float parameter has once it crosses the C ABI."""
    return float(np.float32(x))


def run_attention(w, max_prefix_len=None, stream=None, kv_split_keys=0):
    q = dev_kv(w.q, w.dtype)
    k = dev_kv(w.k_cache, w.dtype)
    v = dev_kv(w.v_cache, w.dtype)
    pl = torch.from_numpy(w.prefix_len).cuda()
    par = None if w.is_chain else torch.from_numpy(w.parent).cuda()
    mpl = w.max_prefix_len if max_prefix_len is None else max_prefix_len
    out = sv.spec_verify_attn(q, k, v, pl, par, mpl, stream=stream, kv_split_keys=kv_split_keys)
    torch.cuda.synchronize()
    return host_f64(out)


def check_attention(gpu, ref, what=""):
    assert np.isfinite(gpu).all(), f"{what}: non-finite attention output"
    err = np.abs(gpu - ref)
    bound = ATOL + RTOL * np.abs(ref)
    bad = err > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {bad.size} outside 2e-2 + 1e-2|ref|; "
                           f"max err {err.max():.3e}")
    return float(err.max())


def run_accept(w):
    lg = torch.from_numpy(w.target_logits).cuda()
    tk = torch.from_numpy(w.tokens).cuda()
    par = None if w.is_chain else torch.from_numpy(w.parent).cuda()
    if w.rule == "reject":
        dp = torch.from_numpy(w.draft_probs).cuda() if w.draft_probs is not None else None
        ua = torch.from_numpy(w.u_accept).cuda()
        us = torch.from_numpy(w.u_sample).cuda()
        al, path, out = sv.spec_accept_reject(lg, dp, tk, par, ua, us, w.temperature)
    else:
        al, path, out = sv.spec_accept_typical(lg, tk, par, w.temperature, w.epsilon, w.delta)
    torch.cuda.synchronize()
    return dict(accept_len=al.cpu().numpy(), path=path.cpu().numpy(), out_tokens=out.cpu().numpy())


def oracle_accept(w):
    par = None if w.is_chain else w.parent
    return oracle.accept(w.rule, w.target_logits, w.tokens, par, f32(w.temperature), w.draft_probs,
                         w.u_accept, w.u_sample, f32(w.epsilon), f32(w.delta))


def check_accept(w, gpu, ref):
    """Bit-exact on every request whose oracle margin is >= 1e-6; validity on
    the rest.  Returns the number of excluded near-tie requests."""
    B, N = w.B, w.N
    excluded = 0
    for b in range(B):
        a = int(gpu["accept_len"][b])
        pth = gpu["path"][b]
        out = gpu["out_tokens"][b]
        # validity (always)
        assert 0 <= a < N, (b, a)
        assert pth[0] == 0 and (pth[a + 1:] == -1).all() and (out[a + 1:] == -1).all(), b
        for d in range(1, a + 1):
            p = pth[d - 1]
            assert (w.parent[b, pth[d]] == p), (b, d)
            assert out[d - 1] == w.tokens[b, pth[d]], (b, d)
        assert 0 <= out[a] < w.V, (b, out[a])
        if ref["margin"][b] < NEAR_TIE:
            excluded += 1
            continue
        assert a == ref["accept_len"][b], (b, a, ref["accept_len"][b], ref["margin"][b])
        np.testing.assert_array_equal(pth, ref["path"][b], err_msg=f"path b={b}")
        np.testing.assert_array_equal(out, ref["out_tokens"][b], err_msg=f"out_tokens b={b}")
    # A case whose every request is a near-tie would pass without comparing
    # anything bit for bit.
    assert B == 0 or excluded < B, f"all {B} requests are near-ties: nothing was compared"
    return excluded
