"""Seeded input generation (NumPy PCG64, one stream per tensor).

Everything here is input synthesis: it draws the tensors a verification step is
handed (queries, KV cache, a draft tree, target logits, the draft distributions
the draft tokens were sampled from, and the caller's uniforms).  The draft side
is simulated, because drafting is outside the verification step.  No part of
the verification arithmetic (tree attention, acceptance tests, resampling,
commit) lives here.

Stream ids (``seed = [config_id, stream, variant]``)::

    0 Q   1 K   2 V   3 target logits   4 draft noise   5 draft tokens
    6 u_accept   7 u_sample   8 tree   9 prefix lengths   10 per-request sigma
    11 boosted ids   12 Medusa head noise
"""
from dataclasses import dataclass, field

import numpy as np

from .configs import num_nodes

S_Q, S_K, S_V, S_LOGITS, S_NOISE, S_TOKENS, S_UACC, S_USMP, S_TREE, S_LEN, S_SIGMA, S_BOOST, S_HEAD = range(13)

BF16_NAN = np.uint16(0x7FC0)


def bf16_bits(x):
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Worked in slices of 4M elements with in-place uint32 arithmetic (the same
    operations on every element as one whole-array expression, without its
    full-size temporaries)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.reshape(-1).view(np.uint32)
    out = np.empty(u.size, dtype=np.uint16)
    step = 1 << 22
    for s in range(0, u.size, step):
        c = u[s:s + step]
        t = c >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        t += c
        t >>= np.uint32(16)
        out[s:s + step] = t
    return out.reshape(x.shape)


def bf16_to_f32(b):
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Workload:
    """One seeded verification-step input.

    Layouts (row-major):
      q            [B][N][Hq][D]     float32, or uint16 bf16 bits
      k_cache      [B][Hkv][cap][D]  rows [0, L_b) verified prefix, rows
      v_cache      [B][Hkv][cap][D]  [L_b, L_b+N) the N tree nodes; the rest
                                     is filled with NaN (never to be read)
      prefix_len   [B] int32
      parent       [B][N] int32, parent[b][0] = -1, parent[b][i] < i
      tokens       [B][N] int32 (tokens[b][0], the root token, is not tested)
      target_logits[B][N][V] float32, row i = target logits at node i
      draft_probs  [B][N][V] float32, row i = distribution node i's token was
                   drawn from (row 0 unused); None for typical acceptance
      u_accept, u_sample [B][N] float32 in [0, 1)
    """
    cfg: dict
    B: int
    N: int
    Hq: int
    Hkv: int
    D: int
    V: int
    cap: int
    dtype: str
    q: np.ndarray
    k_cache: np.ndarray
    v_cache: np.ndarray
    prefix_len: np.ndarray
    parent: np.ndarray
    is_chain: bool
    tokens: np.ndarray
    target_logits: np.ndarray
    draft_probs: object
    u_accept: np.ndarray
    u_sample: np.ndarray
    temperature: float
    rule: str
    epsilon: float
    delta: float
    extra: dict = field(default_factory=dict)

    @property
    def max_prefix_len(self):
        return int(self.prefix_len.max()) if self.B else 0


def _rng(cid, stream, variant):
    return np.random.default_rng([int(cid), int(stream), int(variant)])


def _normal_f32(rng, shape, std=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def _softmax_rows_f64(x, temperature):
    """Row-wise softmax of x / T in float64 (draft-side simulation only)."""
    z = x.astype(np.float64) / temperature
    z -= z.max(axis=-1, keepdims=True)
    np.exp(z, out=z)
    z /= z.sum(axis=-1, keepdims=True)
    return z


def _draw_from(rng, probs_f64):
    """One token per row of probs by inverse CDF on a seeded uniform."""
    c = np.cumsum(probs_f64, axis=-1)
    u = rng.random(size=probs_f64.shape[:-1]) * c[..., -1]
    out = np.empty(probs_f64.shape[:-1], dtype=np.int32)
    flat_c = c.reshape(-1, c.shape[-1])
    flat_u = u.reshape(-1)
    flat_o = out.reshape(-1)
    for r in range(flat_c.shape[0]):
        flat_o[r] = min(int(np.searchsorted(flat_c[r], flat_u[r], side="right")), c.shape[-1] - 1)
    return out


def _tree(cfg, B, N, variant):
    par = np.full((B, N), -1, dtype=np.int32)
    if cfg["tree"] == "chain":
        par[:, 1:] = np.arange(N - 1, dtype=np.int32)
        return par
    if cfg["tree"] == "cartesian":
        # Breadth-first Cartesian product of per-depth top-s_k candidates.
        frontier, nxt = [0], 1
        for s in cfg["topk"]:
            new = []
            for p in frontier:
                for _ in range(s):
                    par[:, nxt] = p
                    new.append(nxt)
                    nxt += 1
            frontier = new
        assert nxt == N
        return par
    rng = _rng(cfg["id"], S_TREE, variant)
    cap = cfg["max_depth"]
    for b in range(B):
        depth = [0]
        for i in range(1, N):
            cand = [j for j in range(i) if depth[j] < cap]
            p = cand[int(rng.integers(len(cand)))]
            par[b, i] = p
            depth.append(depth[p] + 1)
    return par


def generate(cfg, variant=0, poison=True, with_attention=True, with_accept=True, capacity=None):
    """Draw one seeded input for workload ``cfg`` (see workloads.configs)."""
    cid = cfg["id"]
    B, Hq, Hkv, D, V = cfg["batch"], cfg["num_q_heads"], cfg["num_kv_heads"], cfg["head_dim"], cfg["vocab"]
    N = num_nodes(cfg)
    T = float(cfg["temperature"])
    rule = cfg["rule"]

    pl = cfg["prefix_len"]
    if isinstance(pl, (tuple, list)):
        prefix_len = _rng(cid, S_LEN, variant).integers(pl[0], pl[1] + 1, size=B).astype(np.int32)
    else:
        prefix_len = np.full(B, int(pl), dtype=np.int32)
    cap = int(capacity) if capacity is not None else (int(prefix_len.max()) + N if B else N)

    parent = _tree(cfg, B, N, variant)
    is_chain = cfg["tree"] == "chain"

    q = k_cache = v_cache = None
    if with_attention:
        bf16 = cfg["dtype"] == "bf16"
        conv = bf16_bits if bf16 else (lambda a: a)
        q = conv(_normal_f32(_rng(cid, S_Q, variant), (B, N, Hq, D)))
        et = np.uint16 if bf16 else np.float32
        fill = (BF16_NAN if poison else np.uint16(0)) if bf16 else (np.float32(np.nan) if poison else np.float32(0))
        k_cache = np.empty((B, Hkv, cap, D), dtype=et)
        v_cache = np.empty((B, Hkv, cap, D), dtype=et)
        rk, rv = _rng(cid, S_K, variant), _rng(cid, S_V, variant)
        for b in range(B):  # per request: the same draws, converted as they come
            rows = int(prefix_len[b]) + N
            k_cache[b, :, :rows] = conv(_normal_f32(rk, (Hkv, rows, D)))
            v_cache[b, :, :rows] = conv(_normal_f32(rv, (Hkv, rows, D)))
            k_cache[b, :, rows:] = fill
            v_cache[b, :, rows:] = fill

    tokens = np.zeros((B, N), dtype=np.int32)
    logits = draft = u_acc = u_smp = None
    extra = {}
    if with_accept:
        logits = _normal_f32(_rng(cid, S_LOGITS, variant), (B, N, V), cfg["logit_std"])
        nboost = int(round(cfg.get("boost_frac", 0.0) * V))
        if nboost:
            ids = _rng(cid, S_BOOST, variant).choice(V, size=nboost, replace=False)
            logits[:, :, ids] += np.float32(cfg["boost"])
            extra["boost_ids"] = np.sort(ids)
        trng = _rng(cid, S_TOKENS, variant)
        if cfg["tree"] == "cartesian":
            # Head k proposes the same top-s_k tokens under every depth-(k-1)
            # node; its logits follow the first-child path's target row.
            hrng = _rng(cid, S_HEAD, variant)
            depth_nodes, d_first = [], 0
            frontier = [0]
            first_path = [0]
            for s in cfg["topk"]:
                nxt = [i for i in range(N) if parent[0, i] in frontier]
                depth_nodes.append(nxt)
                first_path.append(nxt[0])
                frontier = nxt
            for b in range(B):
                for k, s in enumerate(cfg["topk"]):
                    head = logits[b, first_path[k]] + _normal_f32(hrng, (V,), cfg["head_noise"])
                    top = np.argsort(-head.astype(np.float64), kind="stable")[:s].astype(np.int32)
                    for i in depth_nodes[k]:
                        sib = [j for j in range(N) if parent[b, j] == parent[b, i]]
                        tokens[b, i] = top[sib.index(i)]
            tokens[:, 0] = trng.integers(V, size=B)
        else:
            nrng = _rng(cid, S_NOISE, variant)
            sig = cfg["draft_noise"]
            if len(sig) > 1:
                sigma = np.asarray(sig, dtype=np.float64)[_rng(cid, S_SIGMA, variant).integers(len(sig), size=B)]
            else:
                sigma = np.full(B, float(sig[0]))
            extra["sigma"] = sigma
            if rule == "reject":
                draft = np.zeros((B, N, V), dtype=np.float32)
            for b in range(B):
                parents = sorted(set(int(p) for p in parent[b, 1:]))
                for p in parents:
                    dl = logits[b, p] + _normal_f32(nrng, (V,), float(sigma[b]))
                    qd = _softmax_rows_f64(dl[None, :], T if T > 0 else 1.0)[0]
                    kids = [i for i in range(1, N) if parent[b, i] == p]
                    qf32 = qd.astype(np.float32)
                    toks = _draw_from(trng, np.broadcast_to(qf32.astype(np.float64), (len(kids), V)).copy())
                    for j, i in enumerate(kids):
                        tokens[b, i] = toks[j]
                        if draft is not None:
                            draft[b, i] = qf32
            tokens[:, 0] = trng.integers(V, size=B)
        u_acc = _rng(cid, S_UACC, variant).random(size=(B, N), dtype=np.float32)
        u_smp = _rng(cid, S_USMP, variant).random(size=(B, N), dtype=np.float32)

    return Workload(
        cfg=cfg, B=B, N=N, Hq=Hq, Hkv=Hkv, D=D, V=V, cap=cap, dtype=cfg["dtype"],
        q=q, k_cache=k_cache, v_cache=v_cache, prefix_len=prefix_len, parent=parent,
        is_chain=is_chain, tokens=tokens, target_logits=logits, draft_probs=draft,
        u_accept=u_acc, u_sample=u_smp, temperature=T, rule=rule,
        epsilon=float(cfg.get("epsilon", 0.0)), delta=float(cfg.get("delta", 0.0)), extra=extra,
    )
