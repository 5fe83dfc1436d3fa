"""Thin PyTorch binding of the C ABI in include/spec_verify.h.

Each function has the name of the C entry point it calls and only marshals
arguments: it checks that the tensors are contiguous device tensors of the
right dtype, passes their data pointers and the current HIP stream, and raises
on a non-zero status.  All arithmetic runs in the HIP kernels.  Output and
workspace tensors may be passed in (no allocation) or are created with
``torch.empty`` when omitted (no workspace needs initialisation: every call
writes what it later reads).
"""
import ctypes

import torch

from . import _native
from ._native import AttnDesc, LaDesc, LaFactors, SPEC_BF16, SPEC_F32


class SpecError(RuntimeError):
    def __init__(self, fn, rc):
        super().__init__(f"{fn}: {_native.status_string(rc)} ({rc})")
        self.status = rc


def _check(fn, rc):
    if rc != 0:
        raise SpecError(fn, rc)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dev(t, name, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(dt):
    if dt == torch.bfloat16:
        return SPEC_BF16
    if dt == torch.float32:
        return SPEC_F32
    raise ValueError(f"unsupported dtype {dt}")


def attn_desc(batch, num_nodes, num_q_heads, num_kv_heads, head_dim, kv_capacity, dtype, softmax_scale=0.0,
              kv_split_keys=0, rope_base=0.0):
    return AttnDesc(batch, num_nodes, num_q_heads, num_kv_heads, head_dim, kv_capacity,
                    _dtype_code(dtype) if isinstance(dtype, torch.dtype) else int(dtype), float(softmax_scale),
                    int(kv_split_keys), float(rope_base))


def spec_verify_attn_workspace_bytes(desc, max_prefix_len):
    return int(_native.lib().spec_verify_attn_workspace_bytes(ctypes.byref(desc), int(max_prefix_len)))


def spec_verify_attn(q, k_cache, v_cache, prefix_len, parent, max_prefix_len, out=None, workspace=None,
                     softmax_scale=0.0, stream=None, kv_split_keys=0, rope_base=0.0):
    """Tree-verify attention.  q [B][N][Hq][D]; caches [B][Hkv][cap][D] (same
    dtype, bf16 or fp32); prefix_len [B] int32; parent [B][N] int32 or None
    (chain); max_prefix_len: host int >= every prefix length; kv_split_keys:
    least keys per KV range (0: automatic); rope_base > 0: q and the tree's K
    rows are rotated at their depth positions as they are read."""
    B, N, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    for t, n in ((q, "q"), (k_cache, "k_cache"), (v_cache, "v_cache")):
        _dev(t, n, q.dtype)
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(parent, "parent", torch.int32)
    desc = attn_desc(B, N, Hq, Hkv, D, cap, q.dtype, softmax_scale, kv_split_keys, rope_base)
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out", q.dtype)
    need = spec_verify_attn_workspace_bytes(desc, max_prefix_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = _native.lib().spec_verify_attn(ctypes.byref(desc), int(max_prefix_len), _ptr(q), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(prefix_len), _ptr(parent), _ptr(out),
                                        _ptr(workspace), nbytes, _stream(stream))
    _check("spec_verify_attn", rc)
    return out


def spec_accept_workspace_bytes(batch, num_nodes, vocab):
    return int(_native.lib().spec_accept_workspace_bytes(int(batch), int(num_nodes), int(vocab)))


def spec_accept_filtered_workspace_bytes(batch, num_nodes, vocab):
    return int(_native.lib().spec_accept_filtered_workspace_bytes(int(batch), int(num_nodes), int(vocab)))


def _accept_outputs(B, N, dev, accept_len, path, out_tokens):
    if accept_len is None:
        accept_len = torch.empty(B, dtype=torch.int32, device=dev)
    if path is None:
        path = torch.empty(B, N, dtype=torch.int32, device=dev)
    if out_tokens is None:
        out_tokens = torch.empty(B, N, dtype=torch.int32, device=dev)
    for t, n in ((accept_len, "accept_len"), (path, "path"), (out_tokens, "out_tokens")):
        _dev(t, n, torch.int32)
    return accept_len, path, out_tokens


def spec_accept_reject(target_logits, draft_probs, tokens, parent, u_accept, u_sample, temperature,
                       accept_len=None, path=None, out_tokens=None, workspace=None, stream=None):
    """Rejection-rule acceptance; returns (accept_len, path, out_tokens)."""
    B, N, V = target_logits.shape
    _dev(target_logits, "target_logits", torch.float32)
    _dev(draft_probs, "draft_probs", torch.float32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parent, "parent", torch.int32)
    _dev(u_accept, "u_accept", torch.float32)
    _dev(u_sample, "u_sample", torch.float32)
    accept_len, path, out_tokens = _accept_outputs(B, N, target_logits.device, accept_len, path, out_tokens)
    if workspace is None:
        workspace = torch.empty(max(spec_accept_workspace_bytes(B, N, V), 1), dtype=torch.uint8,
                                device=target_logits.device)
    rc = _native.lib().spec_accept_reject(B, N, V, _ptr(target_logits), _ptr(draft_probs), _ptr(tokens),
                                          _ptr(parent), _ptr(u_accept), _ptr(u_sample), float(temperature),
                                          _ptr(accept_len), _ptr(path), _ptr(out_tokens), _ptr(workspace),
                                          workspace.numel(), _stream(stream))
    _check("spec_accept_reject", rc)
    return accept_len, path, out_tokens


def spec_accept_reject_noalloc(target_logits, draft_probs, tokens, parent, u_accept, u_sample, temperature,
                               accept_len, path, out_tokens, stream=None):
    """spec_accept_reject with the library's per-GPU scratch instead of a
    workspace; the outputs must be passed in (nothing is allocated)."""
    B, N, V = target_logits.shape
    _dev(target_logits, "target_logits", torch.float32)
    _dev(draft_probs, "draft_probs", torch.float32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parent, "parent", torch.int32)
    _dev(u_accept, "u_accept", torch.float32)
    _dev(u_sample, "u_sample", torch.float32)
    for t, n in ((accept_len, "accept_len"), (path, "path"), (out_tokens, "out_tokens")):
        if t is None:
            raise ValueError(f"{n} must be passed in")
        _dev(t, n, torch.int32)
    rc = _native.lib().spec_accept_reject_noalloc(B, N, V, _ptr(target_logits), _ptr(draft_probs), _ptr(tokens),
                                                  _ptr(parent), _ptr(u_accept), _ptr(u_sample), float(temperature),
                                                  _ptr(accept_len), _ptr(path), _ptr(out_tokens), _stream(stream))
    _check("spec_accept_reject_noalloc", rc)
    return accept_len, path, out_tokens


def spec_accept_reject_filtered(target_logits, draft_probs, tokens, parent, u_accept, u_sample, temperature,
                                top_k=0, top_p=1.0, accept_len=None, path=None, out_tokens=None, workspace=None,
                                stream=None):
    """Rejection-rule acceptance on the top-k / nucleus truncated target;
    returns (accept_len, path, out_tokens)."""
    B, N, V = target_logits.shape
    _dev(target_logits, "target_logits", torch.float32)
    _dev(draft_probs, "draft_probs", torch.float32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parent, "parent", torch.int32)
    _dev(u_accept, "u_accept", torch.float32)
    _dev(u_sample, "u_sample", torch.float32)
    accept_len, path, out_tokens = _accept_outputs(B, N, target_logits.device, accept_len, path, out_tokens)
    if workspace is None:
        workspace = torch.empty(max(spec_accept_filtered_workspace_bytes(B, N, V), 1), dtype=torch.uint8,
                                device=target_logits.device)
    rc = _native.lib().spec_accept_reject_filtered(B, N, V, _ptr(target_logits), _ptr(draft_probs), _ptr(tokens),
                                                   _ptr(parent), _ptr(u_accept), _ptr(u_sample), float(temperature),
                                                   int(top_k), float(top_p), _ptr(accept_len), _ptr(path),
                                                   _ptr(out_tokens), _ptr(workspace), workspace.numel(),
                                                   _stream(stream))
    _check("spec_accept_reject_filtered", rc)
    return accept_len, path, out_tokens


def spec_accept_multidraft_workspace_bytes(batch, vocab):
    return int(_native.lib().spec_accept_multidraft_workspace_bytes(int(batch), int(vocab)))


def spec_accept_multidraft(target_logits, draft_probs, tokens, parent, u_accept, u_sample, temperature,
                           accept_len=None, path=None, out_tokens=None, workspace=None, stream=None):
    """Multi-draft tree rejection by recursive residuals; returns
    (accept_len, path, out_tokens)."""
    B, N, V = target_logits.shape
    _dev(target_logits, "target_logits", torch.float32)
    _dev(draft_probs, "draft_probs", torch.float32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parent, "parent", torch.int32)
    _dev(u_accept, "u_accept", torch.float32)
    _dev(u_sample, "u_sample", torch.float32)
    accept_len, path, out_tokens = _accept_outputs(B, N, target_logits.device, accept_len, path, out_tokens)
    if workspace is None:
        workspace = torch.empty(max(spec_accept_multidraft_workspace_bytes(B, V), 1), dtype=torch.uint8,
                                device=target_logits.device)
    rc = _native.lib().spec_accept_multidraft(B, N, V, _ptr(target_logits), _ptr(draft_probs), _ptr(tokens),
                                              _ptr(parent), _ptr(u_accept), _ptr(u_sample), float(temperature),
                                              _ptr(accept_len), _ptr(path), _ptr(out_tokens), _ptr(workspace),
                                              workspace.numel(), _stream(stream))
    _check("spec_accept_multidraft", rc)
    return accept_len, path, out_tokens


def spec_accept_typical(target_logits, tokens, parent, temperature, epsilon, delta, accept_len=None,
                        path=None, out_tokens=None, workspace=None, stream=None):
    """Typical acceptance; returns (accept_len, path, out_tokens)."""
    B, N, V = target_logits.shape
    _dev(target_logits, "target_logits", torch.float32)
    _dev(tokens, "tokens", torch.int32)
    _dev(parent, "parent", torch.int32)
    accept_len, path, out_tokens = _accept_outputs(B, N, target_logits.device, accept_len, path, out_tokens)
    if workspace is None:
        workspace = torch.empty(max(spec_accept_workspace_bytes(B, N, V), 1), dtype=torch.uint8,
                                device=target_logits.device)
    rc = _native.lib().spec_accept_typical(B, N, V, _ptr(target_logits), _ptr(tokens), _ptr(parent),
                                           float(temperature), float(epsilon), float(delta), _ptr(accept_len),
                                           _ptr(path), _ptr(out_tokens), _ptr(workspace), workspace.numel(),
                                           _stream(stream))
    _check("spec_accept_typical", rc)
    return accept_len, path, out_tokens


def spec_commit_kv(k_cache, v_cache, prefix_len, path, accept_len, stream=None, rope_base=0.0):
    """In-place commit of the accepted path's KV rows; advances prefix_len.
    rope_base > 0: the accepted K rows are written rotated at their new
    positions (the fused-RoPE attention's convention)."""
    B, Hkv, cap, D = k_cache.shape
    N = path.shape[1]
    _dev(k_cache, "k_cache")
    _dev(v_cache, "v_cache", k_cache.dtype)
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(path, "path", torch.int32)
    _dev(accept_len, "accept_len", torch.int32)
    desc = attn_desc(B, N, Hkv, Hkv, D, cap, k_cache.dtype, rope_base=rope_base)
    rc = _native.lib().spec_commit_kv(ctypes.byref(desc), _ptr(k_cache), _ptr(v_cache), _ptr(prefix_len),
                                      _ptr(path), _ptr(accept_len), _stream(stream))
    _check("spec_commit_kv", rc)


def spec_tree_positions(prefix_len, parent, num_nodes, positions=None, stream=None):
    B = prefix_len.shape[0]
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(parent, "parent", torch.int32)
    if positions is None:
        positions = torch.empty(B, num_nodes, dtype=torch.int32, device=prefix_len.device)
    _dev(positions, "positions", torch.int32)
    rc = _native.lib().spec_tree_positions(B, int(num_nodes), _ptr(prefix_len), _ptr(parent), _ptr(positions),
                                           _stream(stream))
    _check("spec_tree_positions", rc)
    return positions


def spec_validate_tree(parent, status=None, stream=None):
    B, N = parent.shape
    _dev(parent, "parent", torch.int32)
    if status is None:
        status = torch.empty(B, dtype=torch.int32, device=parent.device)
    _dev(status, "status", torch.int32)
    rc = _native.lib().spec_validate_tree(B, N, _ptr(parent), _ptr(status), _stream(stream))
    _check("spec_validate_tree", rc)
    return status


def spec_medusa_tree_nodes(widths, max_width=None):
    """Node count N of the Medusa candidate tree for head widths s_1..s_K (0 if invalid)."""
    w = (ctypes.c_int32 * len(widths))(*[int(x) for x in widths])
    mw = max(int(x) for x in widths) if max_width is None else int(max_width)
    return int(_native.lib().spec_medusa_tree_nodes(len(widths), w, mw))


def spec_medusa_tree(widths, root_tokens, head_tokens, parent=None, tokens=None, stream=None):
    """Cartesian-product candidate tree: head_tokens [B][K][max_width] int32 (top-s_k
    candidates of head k in rank order), root_tokens [B]; returns (parent, tokens) [B][N]."""
    B, K, W = head_tokens.shape
    if len(widths) != K:
        raise ValueError("one width per head")
    _dev(root_tokens, "root_tokens", torch.int32)
    _dev(head_tokens, "head_tokens", torch.int32)
    N = spec_medusa_tree_nodes(widths, W)
    if N == 0:
        raise SpecError("spec_medusa_tree", _native.SPEC_EINVAL)
    if parent is None:
        parent = torch.empty(B, N, dtype=torch.int32, device=head_tokens.device)
    if tokens is None:
        tokens = torch.empty(B, N, dtype=torch.int32, device=head_tokens.device)
    _dev(parent, "parent", torch.int32)
    _dev(tokens, "tokens", torch.int32)
    w = (ctypes.c_int32 * K)(*[int(x) for x in widths])
    rc = _native.lib().spec_medusa_tree(B, K, w, W, _ptr(root_tokens), _ptr(head_tokens), _ptr(parent),
                                        _ptr(tokens), _stream(stream))
    _check("spec_medusa_tree", rc)
    return parent, tokens


def spec_tree_rope(q, k_cache, prefix_len, parent, rope_base, stream=None):
    """In-place depth-position rotary embedding of q [B][N][Hq][D] and the tree rows of
    k_cache [B][Hkv][cap][D] (positions L_b + depth)."""
    B, N, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    _dev(q, "q")
    _dev(k_cache, "k_cache", q.dtype)
    _dev(prefix_len, "prefix_len", torch.int32)
    _dev(parent, "parent", torch.int32)
    desc = attn_desc(B, N, Hq, Hkv, D, cap, q.dtype)
    rc = _native.lib().spec_tree_rope(ctypes.byref(desc), _ptr(q), _ptr(k_cache), _ptr(prefix_len), _ptr(parent),
                                      float(rope_base), _stream(stream))
    _check("spec_tree_rope", rc)


def _la_factors(k, v, alpha, parent, path, accept_len):
    for t, n in ((path, "path"), (accept_len, "accept_len")):
        _dev(t, n, torch.int32)
    _dev(parent, "parent", torch.int32)
    _dev(alpha, "alpha", torch.float32)
    return LaFactors(k.shape[1], _ptr(k), _ptr(v), _ptr(alpha), _ptr(parent), _ptr(path), _ptr(accept_len))


def spec_la_verify(state, q, k, v, alpha=None, parent=None, out=None, pending=None, stream=None):
    """Linear-attention verification of a tree (or chain) of drafts: returns
    out [B][N][H][Dv].  state [B][H][Dv][Dk] fp32 (advanced in place first by
    ``pending`` = (k, v, alpha, parent, path, accept_len) of the previous
    step, the deferred commit); q, k [B][N][H][Dk], v [B][N][H][Dv] (fp32 or
    bf16); alpha [B][N][H] fp32 decays or None; parent [B][N] or None."""
    B, N, H, Dk = q.shape
    Dv = v.shape[3]
    _dev(state, "state", torch.float32)
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n, q.dtype)
    _dev(alpha, "alpha", torch.float32)
    _dev(parent, "parent", torch.int32)
    if out is None:
        out = torch.empty(B, N, H, Dv, dtype=q.dtype, device=q.device)
    desc = LaDesc(B, N, H, Dk, Dv, _dtype_code(q.dtype))
    f = _la_factors(*pending) if pending is not None else None
    rc = _native.lib().spec_la_verify(ctypes.byref(desc), _ptr(state), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                                      _ptr(parent), _ptr(out), ctypes.byref(f) if f is not None else None,
                                      _stream(stream))
    _check("spec_la_verify", rc)
    return out


def spec_la_commit(state, k, v, alpha, parent, path, accept_len, stream=None):
    """Commit of the accepted path into the linear-attention state, in place,
    from the step's factors (k, v, alpha, parent) and its accepted path."""
    B, Np, H, Dk = k.shape
    Dv = v.shape[3]
    _dev(state, "state", torch.float32)
    desc = LaDesc(B, Np, H, Dk, Dv, _dtype_code(k.dtype))
    f = _la_factors(k, v, alpha, parent, path, accept_len)
    rc = _native.lib().spec_la_commit(ctypes.byref(desc), _ptr(state), ctypes.byref(f), _stream(stream))
    _check("spec_la_commit", rc)
    return state
