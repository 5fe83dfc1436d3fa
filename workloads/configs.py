"""The five verification-step workloads, as parameter dictionaries.

Shapes and value distributions follow the workload list of the verification
step: a tiny fp32 chain, a Llama-3-8B-shaped chain, a Medusa-style Cartesian
tree with typical acceptance, a ragged serving batch and a long-context random
tree.  Every distribution parameter written ``N(0, s)`` below is read as mean 0
and standard deviation ``s``.

Keys
----
batch, num_q_heads, num_kv_heads, head_dim, dtype ("f32" | "bf16")
prefix_len            int, or (lo, hi) for a per-request uniform integer draw
tree                  "chain" | "cartesian" | "random"
drafts                chain length K (chain trees: N = K + 1 query rows)
topk                  per-head top-s_k widths (cartesian trees)
nodes, max_depth      node count including the root, depth cap (random trees)
vocab, logit_std      target logits ~ N(0, logit_std)
boost_frac, boost     a fixed seeded subset of round(boost_frac * vocab) ids
                      gets +boost on every row
draft_noise           draft logits = target logits of the parent row + N(0, s);
                      a list means s is drawn per request from the list
head_noise            cartesian trees: head-k logits = target logits of the
                      first-child path node at depth k-1 + N(0, head_noise)
temperature, rule ("reject" | "typical"), epsilon, delta, commit
"""
import copy

CONFIGS = {
    1: dict(
        name="tiny_chain", batch=1, num_q_heads=4, num_kv_heads=1, head_dim=64,
        dtype="f32", prefix_len=128, tree="chain", drafts=4, vocab=1000,
        logit_std=2.0, boost_frac=0.0, boost=0.0, draft_noise=[1.0],
        temperature=1.0, rule="reject", epsilon=0.0, delta=0.0, commit=False,
    ),
    2: dict(
        name="llama3_8b_chain", batch=1, num_q_heads=32, num_kv_heads=8,
        head_dim=128, dtype="bf16", prefix_len=2048, tree="chain", drafts=5,
        vocab=128256, logit_std=3.0, boost_frac=0.01, boost=8.0,
        draft_noise=[1.5], temperature=1.0, rule="reject", epsilon=0.0,
        delta=0.0, commit=False,
    ),
    3: dict(
        name="medusa_tree", batch=8, num_q_heads=32, num_kv_heads=32,
        head_dim=128, dtype="bf16", prefix_len=4096, tree="cartesian",
        topk=(3, 2, 2, 2), vocab=32000, logit_std=3.0, boost_frac=0.0,
        boost=0.0, head_noise=1.0, temperature=0.7, rule="typical",
        epsilon=0.09, delta=0.3, commit=False,
    ),
    4: dict(
        name="ragged_serving", batch=64, num_q_heads=32, num_kv_heads=8,
        head_dim=128, dtype="bf16", prefix_len=(512, 8192), tree="chain",
        drafts=7, vocab=128256, logit_std=3.0, boost_frac=0.0, boost=0.0,
        draft_noise=[0.5, 1.0, 2.0], temperature=0.8, rule="reject",
        epsilon=0.0, delta=0.0, commit=True,
    ),
    5: dict(
        name="long_ctx_tree", batch=4, num_q_heads=64, num_kv_heads=8,
        head_dim=128, dtype="bf16", prefix_len=32768, tree="random", nodes=64,
        max_depth=6, vocab=128256, logit_std=3.0, boost_frac=0.0, boost=0.0,
        draft_noise=[1.0], temperature=1.0, rule="reject", epsilon=0.0,
        delta=0.0, commit=False,
    ),
}


def config(cid):
    """A fresh copy of workload ``cid`` (1..5)."""
    c = copy.deepcopy(CONFIGS[cid])
    c["id"] = cid
    return c


def scaled(cid, **overrides):
    """Workload ``cid`` with some parameters replaced (smaller test sizes)."""
    c = config(cid)
    for k, v in overrides.items():
        if k not in c and k not in ("topk", "nodes", "max_depth", "drafts", "head_noise"):
            raise KeyError(k)
        c[k] = v
    return c


def num_nodes(c):
    """N, the number of query rows per request including the root."""
    if c["tree"] == "chain":
        return c["drafts"] + 1
    if c["tree"] == "cartesian":
        n, width = 1, 1
        for s in c["topk"]:
            width *= s
            n += width
        return n
    return c["nodes"]
