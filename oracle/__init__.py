"""fp64 CPU oracle of the verification step (tree attention, acceptance, commit).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg use it; the product path (the HIP library and its binding)
never imports it.  The arithmetic lives in ``oracle.c`` (plain C, double
precision); this module only builds it and marshals NumPy arrays through ctypes.

Every function here is pinned by the CPU test-suite against facts the pages and
the mathematics fix (brute-force per-path causal attention, library attention,
closed forms, the chi-square test of the output distribution, worked examples).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force=True):
    """Compile oracle.c into liboracle.so with gcc (OpenMP, no fast-math).

    ORACLE_CC and ORACLE_CFLAGS replace the compiler and add flags (the CPU
    sanitizer run, tests/sanitize_cpu.sh, builds it with clang and
    address/undefined-behaviour checks)."""
    cc = os.environ.get("ORACLE_CC", "gcc")
    extra = os.environ.get("ORACLE_CFLAGS", "").split()
    cmd = [cc, "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", *extra, _SRC, "-o", _LIB + ".tmp", "-lm"]
    if force or not os.path.exists(_LIB):
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        D = ctypes.c_double
        lib.oracle_tree_attn.argtypes = [I, I, I, I, I, I, I, D, P, P, P, P, P, I, P, P]
        lib.oracle_tree_attn.restype = I
        lib.oracle_accept.argtypes = [I, I, I, I, P, P, P, P, P, P, D, D, D, P, P, P, P, P]
        lib.oracle_accept.restype = I
        lib.oracle_accept_ex.argtypes = [I, I, I, I, P, P, P, P, P, P, D, D, D, I, D, P, P, P, P, P]
        lib.oracle_accept_ex.restype = I
        lib.oracle_accept_multidraft.argtypes = [I, I, I, P, P, P, P, P, P, D, P, P, P, P, P]
        lib.oracle_accept_multidraft.restype = I
        lib.oracle_la_verify.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P]
        lib.oracle_la_verify.restype = I
        lib.oracle_la_commit.argtypes = [I, I, I, I, I, I, P, P, P, P, P, P, P]
        lib.oracle_la_commit.restype = I
        lib.oracle_commit.argtypes = [I, I, I, I, I, P, P, P, P, P]
        lib.oracle_commit.restype = I
        lib.oracle_medusa_tree.argtypes = [I, I, P, I, I, P, P, P, P]
        lib.oracle_medusa_tree.restype = I
        lib.oracle_tree_rope.argtypes = [I, I, I, I, I, I, I, P, P, P, P, D, P, P]
        lib.oracle_tree_rope.restype = I
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = I
        lib.oracle_set_num_threads.argtypes = [I]
        lib.oracle_set_num_threads.restype = I
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def tree_attn(q, k_cache, v_cache, prefix_len, parent, dtype, scale=None, rows=None):
    """Tree attention in fp64.

    q [B][N][Hq][D], k_cache/v_cache [B][Hkv][cap][D] (float32, or uint16
    bf16 bits when dtype == "bf16"), prefix_len [B], parent [B][N] or None for
    a chain.  rows: optional (n, 3) int array of (b, node, q-head); the result
    is then [n][D], else [B][N][Hq][D] (float64).
    """
    B, N, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    dt = 1 if dtype == "bf16" else 0
    store = np.uint16 if dt else np.float32
    q, k, v = _c(q, store), _c(k_cache, store), _c(v_cache, store)
    pl = _c(prefix_len, np.int32)
    par = _c(parent, np.int32)
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    if rows is None:
        out = np.empty((B, N, Hq, D), dtype=np.float64)
        sel, nsel = None, 0
    else:
        sel = _c(rows, np.int32).reshape(-1, 3)
        nsel = sel.shape[0]
        out = np.empty((nsel, D), dtype=np.float64)
    rc = _load().oracle_tree_attn(B, N, Hq, Hkv, D, cap, dt, float(scale), _ptr(q), _ptr(k), _ptr(v),
                                  _ptr(pl), _ptr(par), nsel, _ptr(sel), _ptr(out))
    if rc != 0:
        raise ValueError("oracle_tree_attn rejected its arguments")
    return out


def accept(rule, target_logits, tokens, parent, temperature, draft_probs=None, u_accept=None,
           u_sample=None, epsilon=0.0, delta=0.0, top_k=0, top_p=1.0):
    """Acceptance in fp64 ("reject" or "typical").  top_k / top_p truncate
    the target distribution before the rejection rule (0 and 1.0: off).

    Returns dict(accept_len [B], path [B][N], out_tokens [B][N], margin [B],
    stop [B]).
    """
    B, N, V = target_logits.shape
    r = {"reject": 0, "typical": 1}[rule]
    lg = _c(target_logits, np.float32)
    dp = _c(draft_probs, np.float32)
    tk = _c(tokens, np.int32)
    par = _c(parent, np.int32)
    ua = _c(u_accept, np.float32) if u_accept is not None else np.zeros((B, N), np.float32)
    us = _c(u_sample, np.float32) if u_sample is not None else np.zeros((B, N), np.float32)
    acc = np.empty(B, np.int32)
    path = np.empty((B, N), np.int32)
    out = np.empty((B, N), np.int32)
    margin = np.empty(B, np.float64)
    stop = np.empty(B, np.int32)
    rc = _load().oracle_accept_ex(B, N, V, r, _ptr(lg), _ptr(dp), _ptr(tk), _ptr(par), _ptr(ua), _ptr(us),
                                  float(temperature), float(epsilon), float(delta), int(top_k), float(top_p),
                                  _ptr(acc), _ptr(path), _ptr(out), _ptr(margin), _ptr(stop))
    if rc != 0:
        raise ValueError("oracle_accept rejected its arguments")
    return dict(accept_len=acc, path=path, out_tokens=out, margin=margin, stop=stop)


def accept_multidraft(target_logits, tokens, parent, temperature, draft_probs, u_accept, u_sample):
    """Rejection over a tree by recursive residuals (children tested in index
    order, each against the residual of its rejected elder siblings); fp64.

    Returns dict(accept_len, path, out_tokens, margin, stop) as accept().
    """
    B, N, V = target_logits.shape
    lg = _c(target_logits, np.float32)
    dp = _c(draft_probs, np.float32)
    tk = _c(tokens, np.int32)
    par = _c(parent, np.int32)
    ua = _c(u_accept, np.float32)
    us = _c(u_sample, np.float32)
    acc = np.empty(B, np.int32)
    path = np.empty((B, N), np.int32)
    out = np.empty((B, N), np.int32)
    margin = np.empty(B, np.float64)
    stop = np.empty(B, np.int32)
    rc = _load().oracle_accept_multidraft(B, N, V, _ptr(lg), _ptr(dp), _ptr(tk), _ptr(par), _ptr(ua), _ptr(us),
                                          float(temperature), _ptr(acc), _ptr(path), _ptr(out), _ptr(margin),
                                          _ptr(stop))
    if rc != 0:
        raise ValueError("oracle_accept_multidraft rejected its arguments")
    return dict(accept_len=acc, path=path, out_tokens=out, margin=margin, stop=stop)


def _dt(dtype):
    return {"f32": 0, "bf16": 1}[dtype]


def la_verify(state, q, k, v, alpha, parent, dtype):
    """Linear-attention tree verification in fp64: out [B][N][H][Dv].
    state [B][H][Dv][Dk] fp32; q, k [B][N][H][Dk] and v [B][N][H][Dv] as
    float32 or bf16 bits (uint16); alpha [B][N][H] or None; parent or None."""
    B, N, H, Dk = q.shape
    Dv = v.shape[3]
    st = _c(state, np.float32)
    el = np.uint16 if dtype == "bf16" else np.float32
    out = np.empty((B, N, H, Dv), np.float64)
    rc = _load().oracle_la_verify(B, N, H, Dk, Dv, _dt(dtype), _ptr(st), _ptr(_c(q, el)), _ptr(_c(k, el)),
                                  _ptr(_c(v, el)), _ptr(_c(alpha, np.float32)), _ptr(_c(parent, np.int32)),
                                  _ptr(out))
    if rc != 0:
        raise ValueError("oracle_la_verify rejected its arguments")
    return out


def la_commit(state, k, v, alpha, parent, path, accept_len, dtype):
    """The state after committing the accepted path (a new fp32 array)."""
    B, N, H, Dk = k.shape
    Dv = v.shape[3]
    st = np.array(state, np.float32, copy=True, order="C")
    el = np.uint16 if dtype == "bf16" else np.float32
    rc = _load().oracle_la_commit(B, N, H, Dk, Dv, _dt(dtype), _ptr(st), _ptr(_c(k, el)), _ptr(_c(v, el)),
                                  _ptr(_c(alpha, np.float32)), _ptr(_c(parent, np.int32)),
                                  _ptr(_c(path, np.int32)), _ptr(_c(accept_len, np.int32)))
    if rc != 0:
        raise ValueError("oracle_la_commit rejected its arguments")
    return st


def commit(k_cache, v_cache, prefix_len, path, accept_len):
    """In-place commit of the accepted path's KV rows (NumPy arrays, modified).

    Returns the updated prefix_len (also written in place when it is an int32
    contiguous array).
    """
    B, Hkv, cap, D = k_cache.shape
    assert k_cache.flags.c_contiguous and v_cache.flags.c_contiguous
    N = path.shape[1]
    pl = prefix_len if (prefix_len.dtype == np.int32 and prefix_len.flags.c_contiguous) else _c(prefix_len, np.int32)
    pa = _c(path, np.int32)
    al = _c(accept_len, np.int32)
    rc = _load().oracle_commit(B, N, Hkv, cap, D * k_cache.itemsize, _ptr(k_cache), _ptr(v_cache), _ptr(pl),
                               _ptr(pa), _ptr(al))
    if rc != 0:
        raise ValueError("oracle_commit rejected its arguments")
    return pl


def medusa_tree(widths, root_tokens, head_tokens, max_nodes=64):
    """Cartesian-product candidate tree of the Medusa heads.

    widths: s_1..s_K; root_tokens [B]; head_tokens [B][K][max_width].
    Returns (parent [B][N], tokens [B][N]) int32.
    """
    w = _c(widths, np.int32)
    root = _c(root_tokens, np.int32)
    head = _c(head_tokens, np.int32)
    B, K, W = head.shape
    n = 1
    level = 1
    for s in w:
        level *= int(s)
        n += level
    parent = np.empty((B, max(n, 1)), np.int32)
    tokens = np.empty((B, max(n, 1)), np.int32)
    N = _load().oracle_medusa_tree(B, K, _ptr(w), W, int(max_nodes), _ptr(root), _ptr(head), _ptr(parent),
                                   _ptr(tokens))
    if N < 0:
        raise ValueError("oracle_medusa_tree rejected its arguments")
    return parent, tokens


def tree_rope(q, k_cache, prefix_len, parent, dtype, base):
    """Depth-position rotary embedding of q and the tree's K rows (fp64, unrounded).

    Returns (q_out [B][N][Hq][D], k_out [B][Hkv][N][D]) float64.
    """
    B, N, Hq, D = q.shape
    Hkv, cap = k_cache.shape[1], k_cache.shape[2]
    dt = 1 if dtype == "bf16" else 0
    q_ = np.ascontiguousarray(q)
    k_ = np.ascontiguousarray(k_cache)
    pl = _c(prefix_len, np.int32)
    par = _c(parent, np.int32)
    q_out = np.empty((B, N, Hq, D), np.float64)
    k_out = np.empty((B, Hkv, N, D), np.float64)
    rc = _load().oracle_tree_rope(B, N, Hq, Hkv, D, cap, dt, _ptr(q_), _ptr(k_), _ptr(pl), _ptr(par), float(base),
                                  _ptr(q_out), _ptr(k_out))
    if rc != 0:
        raise ValueError("oracle_tree_rope rejected its arguments")
    return q_out, k_out


def num_threads():
    """OpenMP threads the oracle runs with."""
    return int(_load().oracle_num_threads())


def set_num_threads(n):
    """Sets the oracle's OpenMP thread count; returns the count in effect."""
    return int(_load().oracle_set_num_threads(int(n)))


def run_workload(w, rows=None, attention=True, accept_=True):
    """Oracle outputs for a workloads.Workload (attention and/or acceptance)."""
    res = {}
    par = None if w.is_chain else w.parent
    if attention:
        res["attn"] = tree_attn(w.q, w.k_cache, w.v_cache, w.prefix_len, par, w.dtype, rows=rows)
    if accept_:
        res["accept"] = accept(w.rule, w.target_logits, w.tokens, par, w.temperature, w.draft_probs,
                               w.u_accept, w.u_sample, w.epsilon, w.delta)
    return res
