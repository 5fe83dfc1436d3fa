"""Benchmark of the speculative-decoding verification step on one MI355X.

A step is the whole hot path over one batch: tree-verify attention
(spec_verify_attn), acceptance (spec_accept_reject / spec_accept_typical) and
the KV commit (spec_commit_kv).  Every step runs all three on the same fixed
workload: the commit moves the accepted rows and advances its own copy of the
prefix lengths inside spare cache capacity, while attention keeps reading the
workload's prefix lengths.

The headline workload is the largest one that fits one GPU, the ragged serving
batch (64 requests, 32 query / 8 KV heads, head dim 128, bf16 KV prefixes
512..8192, K = 7 chain drafts, vocabulary 128256, T = 0.8, rejection rule and
commit).  By default every one of the five workloads is measured as well and
reported under "configs"; --only measures the headline alone.

Inputs are seeded synthetic tensors, generated once and copied to the GPU;
enough copies are rotated that consecutive reuses of one copy are more than
512 MB of traffic apart, so the 256 MB Infinity Cache cannot serve them.

Timing: each phase (the step, and each call alone) is captured in a HIP graph
of at least 32 steps; the graph is replayed at least 5 times and at least 100
steps in total, each replay bracketed by HIP events on the launch stream, and
the median per-step time over the replays is reported (with min and max).

Prints ONE JSON line: the metric (verified draft tokens per second =
B * (N - 1) / step time, every non-root node of the tree counted as one
adjudicated draft), the dominant kernel's roofline fraction, and the fp64 CPU
oracle timed on a bounded sample of the same step (all host threads, and one
thread).
"""
import argparse
import hashlib
import json
import math
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
ROTATE_BYTES = 640 << 20
HEADLINE = 4
READ_PEAK_FILE = os.path.join(ROOT, "profiles", "hbm_read_peak.json")
READ_PROBE = os.path.join(ROOT, "hbm_read_probe")
CSRC = os.path.join(ROOT, "speculative_decoding_verification_tree_amd", "csrc")

# What the stored counter files describe: the kernels of one call, compiled
# from these sources.
ATTN_SOURCES = ("attn.hip", "spec_common.h", "spec_internal.h")
ACCEPT_SOURCES = ("accept.hip", "spec_common.h", "spec_internal.h")
# The calls beside the path (truncated and multi-draft acceptance, linear
# attention): one stored counter file per workload, keyed by these sources.
EXTRA_SOURCES = ("accept.hip", "multidraft.hip", "linattn.hip", "spec_common.h", "spec_internal.h")


def traffic_file(kind, name):
    """Stored HBM counters of one call (kind 'attn' | 'accept') on the named workload."""
    return os.path.join(ROOT, "profiles", f"{kind}_{name}_traffic.json")


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100, help="least number of timed steps (at least 100 are timed)")
    ap.add_argument("--warmup", type=int, default=10, help="eager warm-up steps (at least 10)")
    ap.add_argument("--config", type=int, default=HEADLINE, help="headline workload id 1..5 (default: the ragged batch)")
    ap.add_argument("--only", action="store_true", help="measure the headline workload alone (no 'configs' map)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the calls beside the path (truncated / multi-draft acceptance, RoPE, linear attention)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-baseline sample budget (all threads)")
    ap.add_argument("--rotate-mb", type=int, default=ROTATE_BYTES >> 20,
                    help="input bytes cycled between reuses of one copy (default beats the 256 MB Infinity Cache; "
                         "0 keeps two copies, i.e. cache-warm)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--read-peak", action="store_true",
                    help="only run the streaming-read calibration program (measured HBM read bandwidth)")
    return ap.parse_args(argv)


def source_hash(names):
    """Hash of kernel sources: stored counters stay valid while these are unchanged."""
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def kernel_source_hash():
    return source_hash(ATTN_SOURCES)


def accept_source_hash():
    return source_hash(ACCEPT_SOURCES)


def extra_source_hash():
    return source_hash(EXTRA_SOURCES)


def stored_extra_traffic(name, cid):
    """Per-call HBM bytes of the calls beside the path ({call: bytes}) from
    the stored counter file, or {} when it is missing or stale."""
    path = traffic_file("extras", name)
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        tr = json.load(f)
    if tr.get("kernel_source_hash") != extra_source_hash() or tr.get("config") != cid:
        return {}
    return {k: v["bytes_per_call"] for k, v in tr.get("calls", {}).items()}


def attn_bytes(w):
    """Algorithmic bytes of one attention launch: every K and V row of the
    prefix plus the tree read once, Q read once, O written once."""
    es = 2 if w.dtype == "bf16" else 4
    kv = sum(int(L) + w.N for L in w.prefix_len) * w.Hkv * w.D * es * 2
    qo = 2 * w.B * w.N * w.Hq * w.D * es
    return kv + qo


def node_depths(parent_row):
    d = [0] * len(parent_row)
    for i in range(1, len(parent_row)):
        d[i] = d[int(parent_row[i])] + 1
    return d


def attn_flops(w):
    """Algorithmic FLOPs of one attention launch: 4 * D per (query row, key),
    a node's keys being the prefix and its root path (itself included)."""
    import numpy as np

    par = w.parent if not w.is_chain else np.tile(np.arange(-1, w.N - 1, dtype=np.int32), (w.B, 1))
    keys = 0
    for b in range(w.B):
        keys += sum(int(w.prefix_len[b]) + d + 1 for d in node_depths(par[b]))
    return 4 * w.D * w.Hq * keys


def accept_bytes(w, accept_len, path):
    """Algorithmic bytes of one acceptance call with the given outcome: the
    logits row of every node with children read once, the stop row when it is
    a leaf, and for the rejection rule the draft row of the stop node's first
    child when it has one; plus the per-node gathers and the outputs."""
    import numpy as np

    B, N, V = w.B, w.N, w.V
    par = w.parent if w.parent is not None else np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    rows = 0
    for b in range(B):
        has_child = np.zeros(N, dtype=bool)
        has_child[par[b][1:]] = True
        rows += int(has_child.sum())
        v = int(path[b][int(accept_len[b])])
        if not has_child[v]:
            rows += 1
        elif w.rule == "reject":
            rows += 1
    gathers = B * (N - 1) * (4 + 4 + 4 + 4 + 4)  # token, parent, u, draft prob and logit at the token
    outputs = B * (1 + 2 * N) * 4
    return rows * V * 4 + gathers + outputs


def multidraft_bytes(w, accept_len, path):
    """Algorithmic bytes of one multi-draft call with the given outcome: one
    read of the target row of every node on the accepted path (its
    statistics), three row passes per rejected child (the residual or target
    row and the child's draft row read, the new residual written), and one
    read of the row the last token is drawn from (T > 0)."""
    import numpy as np

    B, N, V = w.B, w.N, w.V
    par = w.parent if w.parent is not None else np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    rows = 0
    for b in range(B):
        a = int(accept_len[b])
        nodes = [int(x) for x in path[b][:a + 1]]
        for d, v in enumerate(nodes):
            rows += 1
            kids = [c for c in range(1, N) if int(par[b][c]) == v]
            nxt = nodes[d + 1] if d < a else None
            rej = sum(1 for c in kids if nxt is None or c < nxt)
            if w.temperature > 0:
                rows += 3 * rej
        if w.temperature > 0:
            rows += 1
    return rows * V * 4


def stored_traffic(kind, name, cid, khash):
    """Per-call HBM bytes from the stored counter file, or None when the file
    is missing or describes other kernel sources."""
    path = traffic_file(kind, name)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        tr = json.load(f)
    if tr.get("kernel_source_hash") == khash and tr.get("config") == cid:
        return tr.get("bytes_per_launch")
    return None


def oracle_step(oracle, w, kk, vv, zero_len):
    """One full oracle step: attention of every row, acceptance, and the
    commit of the accepted path.  The commit moves rows of the tree region
    only, so it runs on a compact copy of that region (kk, vv: the N tree rows
    of every (request, KV head), prefix lengths 0): the same row moves as on
    the whole cache, without copying the prefix."""
    import numpy as np

    par = None if w.is_chain else w.parent
    T32 = float(np.float32(w.temperature))
    oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.prefix_len, par, w.dtype)
    r = oracle.accept(w.rule, w.target_logits, w.tokens, par, T32, w.draft_probs, w.u_accept, w.u_sample,
                      float(np.float32(w.epsilon)), float(np.float32(w.delta)))
    oracle.commit(kk, vv, zero_len.copy(), r["path"], r["accept_len"])


def request_slice(w, nreq):
    """The first nreq requests of a workload (a bounded sample of it)."""
    import copy

    s = copy.copy(w)
    s.B = nreq
    for f in ("q", "k_cache", "v_cache", "prefix_len", "parent", "tokens", "target_logits", "draft_probs",
              "u_accept", "u_sample"):
        a = getattr(w, f)
        if a is not None:
            setattr(s, f, a[:nreq])
    return s


def cpu_sample(w, budget_s, nreq):
    """Time oracle steps on the first nreq requests until budget_s has passed
    (at least one step).  Returns (steps, seconds, requests)."""
    import numpy as np

    import oracle

    s = request_slice(w, nreq) if nreq < w.B else w
    # the tree region of the caches, outside the timed region
    rows = np.stack([np.arange(int(L), int(L) + s.N) for L in s.prefix_len])  # [B][N]
    kk = np.ascontiguousarray(np.stack([s.k_cache[b][:, rows[b]] for b in range(s.B)]))
    vv = np.ascontiguousarray(np.stack([s.v_cache[b][:, rows[b]] for b in range(s.B)]))
    zero_len = np.zeros(s.B, dtype=np.int32)
    n, t = 0, 0.0
    while n == 0 or t < budget_s:
        t0 = time.perf_counter()
        oracle_step(oracle, s, kk, vv, zero_len)
        t += time.perf_counter() - t0
        n += 1
        if n >= 1000:
            break
    return n, t, s.B


def cpu_baseline(w, budget_s):
    """The oracle on the host: all threads on whole steps, and one thread on
    the first requests of the workload."""
    import oracle

    per_req = w.N - 1
    nth = oracle.num_threads()
    n, t, b = cpu_sample(w, budget_s, w.B)
    res = {"value": per_req * b * n / t, "unit": "verified draft tokens/s", "cores": nth, "kind": "oracle",
           "sample": f"{n} full step(s) of the same workload ({b} requests: attention of every row, acceptance, "
                     f"commit), {t:.1f} s on the host with {nth} OpenMP threads"}
    # one thread: as many leading requests as fit the budget at the measured rate
    nreq = max(1, min(w.B, int(budget_s / max(t / n / b * nth, 1e-9))))
    oracle.set_num_threads(1)
    try:
        n1, t1, b1 = cpu_sample(w, budget_s, nreq)
    finally:
        oracle.set_num_threads(nth)
    res["single_thread"] = {"value": per_req * b1 * n1 / t1, "unit": "verified draft tokens/s", "cores": 1,
                            "sample": f"{n1} step(s) of the first {b1} request(s) of the workload, "
                                      f"{t1:.1f} s on one host thread"}
    return res


class Timer:
    """Median per-step time of graph replays, HIP events on the launch stream."""

    def __init__(self, torch, spg, reps):
        self.torch, self.spg, self.reps = torch, spg, reps

    def __call__(self, g):
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(self.reps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record()
            g.replay()
            e1.record()
        torch.cuda.synchronize()
        per = sorted(e0.elapsed_time(e1) / self.spg for e0, e1 in ev)
        m = len(per) // 2
        med = per[m] if len(per) % 2 else 0.5 * (per[m - 1] + per[m])
        return {"median_ms": med, "min_ms": per[0], "max_ms": per[-1]}


def measure(cid, args, dev, with_extras):
    """Everything measured on workload cid; returns the per-workload record."""
    import numpy as np
    import torch

    import speculative_decoding_verification_tree_amd as sv
    from workloads import config, generate

    cfg = config(cid)
    w = generate(cfg, poison=False)
    B, N, V = w.B, w.N, w.V
    touched = attn_bytes(w) + (N * V * 4) * (2 if w.draft_probs is not None else 1)
    ncopies = max(2, math.ceil((args.rotate_mb << 20) / max(touched, 1)))
    # One graph replay runs spg steps over the copies in rotation (at least 32
    # so the per-replay launch cost is amortised); at least 5 replays and at
    # least max(--steps, 100) timed steps.
    spg = ncopies * math.ceil(32 / ncopies)
    reps = max(5, math.ceil(max(args.steps, 100) / spg))
    warmup = max(args.warmup, 10)
    # The commit advances its own copy of the prefix lengths by at most N rows
    # per use (attention keeps reading the fixed workload's lengths), so the
    # cache gets headroom for every use: eager warm-up, then one warm and reps
    # timed replays of the step and commit graphs.
    uses = math.ceil(max(warmup, ncopies) / ncopies) + 2 * (reps + 1) * (spg // ncopies) + 1
    mpl = int(w.prefix_len.max())
    cap = mpl + (uses + 1) * N

    def to_dev(arr, bf16):
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16) if bf16 else np.ascontiguousarray(arr))
        t = t.to(dev)
        return t.view(torch.bfloat16) if bf16 else t

    bf16 = w.dtype == "bf16"
    kd = torch.zeros((B, w.Hkv, cap, w.D), dtype=torch.bfloat16 if bf16 else torch.float32, device=dev)
    vd = torch.zeros_like(kd)
    kd[:, :, : w.cap] = to_dev(w.k_cache, bf16)
    vd[:, :, : w.cap] = to_dev(w.v_cache, bf16)
    base = dict(
        q=to_dev(w.q, bf16), k=kd, v=vd,
        logits=torch.from_numpy(w.target_logits).to(dev),
        draft=torch.from_numpy(w.draft_probs).to(dev) if w.draft_probs is not None else None,
        tokens=torch.from_numpy(w.tokens).to(dev),
        parent=None if w.is_chain else torch.from_numpy(w.parent).to(dev),
        ua=torch.from_numpy(w.u_accept).to(dev), us=torch.from_numpy(w.u_sample).to(dev),
    )
    copies = []
    for i in range(ncopies):
        c = {k: (t.clone() if (t is not None and i > 0) else t) for k, t in base.items()}
        c["pl"] = torch.from_numpy(w.prefix_len.copy()).to(dev)        # read by attention
        c["pl_commit"] = torch.from_numpy(w.prefix_len.copy()).to(dev)  # advanced by the commit
        c["out"] = torch.empty_like(c["q"])
        c["al"] = torch.empty(B, dtype=torch.int32, device=dev)
        c["path"] = torch.empty(B, N, dtype=torch.int32, device=dev)
        c["otok"] = torch.empty(B, N, dtype=torch.int32, device=dev)
        copies.append(c)
    del base, kd, vd
    desc = sv.attn_desc(B, N, w.Hq, w.Hkv, w.D, cap, torch.bfloat16 if bf16 else torch.float32)
    attn_ws = torch.empty(max(sv.spec_verify_attn_workspace_bytes(desc, mpl), 16), dtype=torch.uint8, device=dev)
    acc_ws = torch.empty(max(sv.spec_accept_workspace_bytes(B, N, V), 16), dtype=torch.uint8, device=dev)

    def attn(c):
        sv.spec_verify_attn(c["q"], c["k"], c["v"], c["pl"], c["parent"], mpl, out=c["out"], workspace=attn_ws)

    def accept(c):
        if w.rule == "reject":
            sv.spec_accept_reject(c["logits"], c["draft"], c["tokens"], c["parent"], c["ua"], c["us"],
                                  w.temperature, c["al"], c["path"], c["otok"], workspace=acc_ws)
        else:
            sv.spec_accept_typical(c["logits"], c["tokens"], c["parent"], w.temperature, w.epsilon, w.delta,
                                   c["al"], c["path"], c["otok"], workspace=acc_ws)

    def commit(c):
        sv.spec_commit_kv(c["k"], c["v"], c["pl_commit"], c["path"], c["al"])

    # eager warm-up (also checks every call returns SPEC_OK)
    for i in range(max(warmup, ncopies)):
        c = copies[i % ncopies]
        attn(c)
        accept(c)
        commit(c)
    torch.cuda.synchronize()

    def capture(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(spg):
                for fn in fns:
                    fn(copies[i % ncopies])
        return g

    timer = Timer(torch, spg, reps)
    phases = {"step": [attn, accept, commit], "attn_accept": [attn, accept], "attention": [attn],
              "accept": [accept], "commit": [commit]}
    graphs = {k: capture(f) for k, f in phases.items()}
    for g in graphs.values():
        g.replay()
    torch.cuda.synchronize()
    t = {k: timer(g) for k, g in graphs.items()}
    del graphs

    al = copies[0]["al"].cpu().numpy()
    path = copies[0]["path"].cpu().numpy()
    step_ms = t["step"]["median_ms"]
    attn_ms, acc_ms = t["attention"]["median_ms"], t["accept"]["median_ms"]
    verified = B * (N - 1)
    emitted = int(al.sum()) + B

    a_bytes = attn_bytes(w)
    a_flops = attn_flops(w)
    acc_b = accept_bytes(w, al, path)
    khash, ahash = kernel_source_hash(), accept_source_hash()
    attn_traffic = stored_traffic("attn", cfg["name"], cid, khash)
    acc_traffic = stored_traffic("accept", cfg["name"], cid, ahash)
    read_peak = None
    if os.path.exists(READ_PEAK_FILE):
        with open(READ_PEAK_FILE) as f:
            read_peak = json.load(f).get("kv_read_GBs")
    attn_gbs = a_bytes / (attn_ms * 1e-3) / 1e9
    attn_roof = {"bound": "hbm", "kernel": "spec_verify_attn", "achieved": attn_gbs, "peak": HBM_PEAK_GBS,
                 "unit": "GB/s", "frac": attn_gbs / HBM_PEAK_GBS, "traffic": attn_traffic,
                 "algorithmic_bytes_per_launch": a_bytes, "kernel_source_hash": khash,
                 "measured_read_peak": read_peak,
                 "frac_of_measured_read_peak": None if read_peak is None else attn_gbs / read_peak}
    tflops = a_flops / (attn_ms * 1e-3) / 1e12
    mfma_roof = {"bound": "mfma", "kernel": "spec_verify_attn", "achieved": tflops, "peak": BF16_MFMA_PEAK_TFLOPS,
                 "unit": "TFLOP/s", "frac": tflops / BF16_MFMA_PEAK_TFLOPS, "traffic": attn_traffic,
                 "algorithmic_flops_per_launch": a_flops, "kernel_source_hash": khash,
                 "hbm_GBs": attn_gbs, "hbm_frac": attn_gbs / HBM_PEAK_GBS}
    acc_gbs = acc_b / (acc_ms * 1e-3) / 1e9
    acc_roof = {"bound": "hbm", "calls": "spec_accept_reject" if w.rule == "reject" else "spec_accept_typical",
                "achieved": acc_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": acc_gbs / HBM_PEAK_GBS,
                "traffic": acc_traffic, "algorithmic_bytes_per_call": acc_b, "kernel_source_hash": ahash}
    # Attention of the many-row tree workload is bound by the matrix cores
    # (512 FLOP per KV byte); the others by HBM.
    mfma_bound = cid == 5
    rec = {
        "workload": f"{cfg['name']}: B={B}, Hq={w.Hq}/Hkv={w.Hkv}, D={w.D}, {w.dtype} KV prefix "
                    f"{int(w.prefix_len.min())}..{int(w.prefix_len.max())}, N={N} nodes "
                    f"({'chain' if w.is_chain else 'tree'}), V={V}, T={w.temperature}, {w.rule} rule",
        "us_per_step": step_ms * 1e3,
        "us_per_step_min": t["step"]["min_ms"] * 1e3,
        "us_per_step_max": t["step"]["max_ms"] * 1e3,
        "verified_tok_s": verified / (step_ms * 1e-3),
        "emitted_tok_s": emitted / (step_ms * 1e-3),
        "verified_per_step": verified,
        "emitted_per_step": emitted,
        "breakdown_us": {"attention": attn_ms * 1e3, "accept": acc_ms * 1e3,
                         "commit": t["commit"]["median_ms"] * 1e3,
                         "attention_plus_accept": t["attn_accept"]["median_ms"] * 1e3},
        "roofline": mfma_roof if mfma_bound else attn_roof,
        "attn_hbm_roofline": attn_roof,
        "accept_roofline": acc_roof,
        "timing": {"replays": reps, "steps_per_replay": spg, "timed_steps": reps * spg, "warmup_steps": warmup,
                   "rotated_copies": ncopies, "mb_between_reuses": ncopies * touched / 2 ** 20},
        "accept_len_first": al.tolist()[:8],
    }
    if with_extras:
        rec["extras"] = measure_extras(cfg, w, copies, acc_ws, Timer(torch, spg, reps), spg, dev)
        # counter-measured bytes of each call (when stored for these sources)
        ex_tr = stored_extra_traffic(cfg["name"], cid)
        for call, key in (("filtered_accept", "filtered_accept"), ("multidraft_accept", "multidraft_accept"),
                          ("la_verify", "linear_attention")):
            ent = rec["extras"].get(key)
            if ent is None:
                continue
            ent["traffic" if call != "la_verify" else "verify_traffic"] = ex_tr.get(call)
    del copies, attn_ws, acc_ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, w


def measure_extras(cfg, w, copies, acc_ws, timer, spg, dev):
    """The calls beside the path, each timed on its own on the same workload."""
    import torch

    import speculative_decoding_verification_tree_amd as sv

    B, N, V = w.B, w.N, w.V
    ncopies = len(copies)
    bf16 = w.dtype == "bf16"

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(spg):
                fn(copies[i % ncopies])
        g.replay()
        torch.cuda.synchronize()
        return g

    out = {}
    # The step before the path: the Medusa candidate tree (Cartesian trees) and
    # the depth-position rotary embedding of q and the tree's K rows, in place.
    rope_base = 500000.0
    cartesian = cfg["tree"] == "cartesian"
    if cartesian:
        widths = list(cfg["topk"])
        head_tok = torch.randint(0, V, (B, len(widths), max(widths)), dtype=torch.int32, device=dev)
        root_tok = torch.randint(0, V, (B,), dtype=torch.int32, device=dev)
        tree_par = torch.empty(B, N, dtype=torch.int32, device=dev)
        tree_tok = torch.empty(B, N, dtype=torch.int32, device=dev)

    def tree_rope(c):
        if cartesian:
            sv.spec_medusa_tree(widths, root_tok, head_tok, tree_par, tree_tok)
            sv.spec_tree_rope(c["q"], c["k"], c["pl"], tree_par, rope_base)
        else:
            sv.spec_tree_rope(c["q"], c["k"], c["pl"], c["parent"], rope_base)

    tree_rope(copies[0])
    ms = timer(capture(tree_rope))["median_ms"]
    esz = 2 if bf16 else 4
    rb = 2 * (B * N * w.Hq * w.D + B * w.Hkv * N * w.D) * esz  # read + write, q and tree K rows
    out["tree_rope"] = {"us": ms * 1e3, "bytes": rb, "achieved_GBs": rb / (ms * 1e-3) / 1e9,
                        "calls": ("spec_medusa_tree + " if cartesian else "") + "spec_tree_rope"}

    # Depth-position RoPE fused into the attention (q and the tree's K rows
    # turned as they are read) against the separate rotation pass followed by
    # the plain attention.
    mpl = int(w.prefix_len.max())
    desc = sv.attn_desc(B, N, w.Hq, w.Hkv, w.D, copies[0]["k"].shape[2], copies[0]["q"].dtype)
    rws = torch.empty(max(sv.spec_verify_attn_workspace_bytes(desc, mpl), 16), dtype=torch.uint8, device=dev)

    def attn_fused(c):
        sv.spec_verify_attn(c["q"], c["k"], c["v"], c["pl"], c["parent"], mpl, out=c["out"], workspace=rws,
                            rope_base=rope_base)

    def attn_unfused(c):
        sv.spec_tree_rope(c["q"], c["k"], c["pl"], c["parent"], rope_base)
        sv.spec_verify_attn(c["q"], c["k"], c["v"], c["pl"], c["parent"], mpl, out=c["out"], workspace=rws)

    attn_fused(copies[0])
    fused_ms = timer(capture(attn_fused))["median_ms"]
    attn_unfused(copies[0])
    unfused_ms = timer(capture(attn_unfused))["median_ms"]
    out["rope_attention"] = {"fused_us": fused_ms * 1e3, "unfused_us": unfused_ms * 1e3,
                             "calls": "spec_verify_attn with rope_base, against spec_tree_rope + spec_verify_attn"}

    if w.rule == "reject" and w.temperature > 0:
        fk, fp = 50, 0.9
        filt_ws = torch.empty(max(sv.spec_accept_filtered_workspace_bytes(B, N, V), 16), dtype=torch.uint8,
                              device=dev)

        def accept_filtered(c):
            sv.spec_accept_reject_filtered(c["logits"], c["draft"], c["tokens"], c["parent"], c["ua"], c["us"],
                                           w.temperature, fk, fp, c["al"], c["path"], c["otok"], workspace=filt_ws)

        for c in copies:
            accept_filtered(c)
        ms = timer(capture(accept_filtered))["median_ms"]
        fb = (B * N * V + 2 * B * V) * 4  # every target row, the stop row and one draft row per request
        out["filtered_accept"] = {"us": ms * 1e3, "top_k": fk, "top_p": fp, "bytes": fb,
                                  "achieved_GBs": fb / (ms * 1e-3) / 1e9, "calls": "spec_accept_reject_filtered"}

    if w.rule == "reject" and not w.is_chain:
        md_ws = torch.empty(max(sv.spec_accept_multidraft_workspace_bytes(B, V), 16), dtype=torch.uint8, device=dev)

        def accept_multidraft(c):
            sv.spec_accept_multidraft(c["logits"], c["draft"], c["tokens"], c["parent"], c["ua"], c["us"],
                                      w.temperature, c["al"], c["path"], c["otok"], workspace=md_ws)

        for c in copies:
            accept_multidraft(c)
        ms = timer(capture(accept_multidraft))["median_ms"]
        mb = multidraft_bytes(w, copies[0]["al"].cpu().numpy(), copies[0]["path"].cpu().numpy())
        out["multidraft_accept"] = {"us": ms * 1e3, "bytes": mb, "achieved_GBs": mb / (ms * 1e-3) / 1e9,
                                    "frac": mb / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), "calls": "spec_accept_multidraft"}

    if cfg["id"] == HEADLINE:
        # A short multi-head (Hq = Hkv) chain: 6 query rows per slab, a third
        # of one 16-row matrix tile; the KV stream bounds it all the same.
        mB, mH, mD, mL, mN = 16, 32, 128, 4096, 6
        mq = torch.randn(mB, mN, mH, mD, device=dev).to(torch.bfloat16)
        mk = torch.randn(mB, mH, mL + mN, mD, device=dev).to(torch.bfloat16)
        mv = torch.randn(mB, mH, mL + mN, mD, device=dev).to(torch.bfloat16)
        mpl_t = torch.full((mB,), mL, dtype=torch.int32, device=dev)
        mo = torch.empty_like(mq)
        mdesc = sv.attn_desc(mB, mN, mH, mH, mD, mL + mN, torch.bfloat16)
        mws = torch.empty(max(sv.spec_verify_attn_workspace_bytes(mdesc, mL), 16), dtype=torch.uint8, device=dev)

        def mha(c):
            sv.spec_verify_attn(mq, mk, mv, mpl_t, None, mL, out=mo, workspace=mws)

        mha(None)
        ms = timer(capture(mha))["median_ms"]
        mbytes = (mB * mH * (mL + mN) * mD * 2 * 2) + 2 * mB * mN * mH * mD * 2
        out["mha_short_chain"] = {
            "workload": f"B={mB}, Hq=Hkv={mH}, D={mD}, bf16 KV prefix {mL}, K={mN - 1} chain (6 query rows per slab)",
            "us": ms * 1e3, "bytes": mbytes, "achieved_GBs": mbytes / (ms * 1e-3) / 1e9,
            "frac": mbytes / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), "calls": "spec_verify_attn",
            "note": "one copy of the 1.07 GB KV, larger than the 256 MB Infinity Cache"}

    # Linear-attention verification of the same trees (16 heads, Dk = Dv =
    # 128, bf16 q/k/v, fp32 state), its factor commit, and both fused.
    LH, LD = 16, 128
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    la_state = torch.randn(B, LH, LD, LD, device=dev, generator=g) / LD ** 0.5
    la_q = (torch.randn(B, N, LH, LD, device=dev, generator=g) / LD ** 0.5).to(torch.bfloat16)
    la_k = torch.randn(B, N, LH, LD, device=dev, generator=g).to(torch.bfloat16)
    la_v = torch.randn(B, N, LH, LD, device=dev, generator=g).to(torch.bfloat16)
    la_alpha = torch.rand(B, N, LH, device=dev, generator=g) * 0.4 + 0.6
    la_out = torch.empty_like(la_v)
    pend = (la_k, la_v, la_alpha, copies[0]["parent"], copies[0]["path"], copies[0]["al"])
    fns = {
        "verify": lambda c: sv.spec_la_verify(la_state, la_q, la_k, la_v, la_alpha, c["parent"], out=la_out),
        "commit": lambda c: sv.spec_la_commit(la_state, *pend),
        "fused": lambda c: sv.spec_la_verify(la_state, la_q, la_k, la_v, la_alpha, c["parent"], out=la_out,
                                             pending=pend),
    }
    st = B * LH * LD * LD * 4
    io = B * N * LH * LD * 2 * 4
    la_b = {"verify": st + io, "commit": 2 * st, "fused": 2 * st + io}
    la = {"heads": LH, "key_dim": LD, "value_dim": LD}
    for k, fn in fns.items():
        fn(copies[0])
        ms = timer(capture(fn))["median_ms"]
        la[f"{k}_us"] = ms * 1e3
        la[f"{k}_GBs"] = la_b[k] / (ms * 1e-3) / 1e9
    la["calls"] = "spec_la_verify, spec_la_commit, spec_la_verify with pending factors"
    out["linear_attention"] = la
    out["note"] = "beside the path, each timed alone; not part of the step"
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); runs on several GPUs are not part of "
              "this path's measurement", file=sys.stderr)
        sys.exit(2)

    if args.read_peak:
        # A child process of its own (nothing here has touched the GPU yet).
        if not os.path.exists(READ_PROBE):
            sys.exit(f"{READ_PROBE} is not built (run __graft_entry__.build())")
        res = subprocess.run([READ_PROBE], capture_output=True, text=True)
        sys.stderr.write(res.stderr)
        print(res.stdout.strip(), flush=True)
        sys.exit(res.returncode)

    import torch

    import speculative_decoding_verification_tree_amd as sv

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sv.lib()  # fails loudly if the HIP library is not built

    if args.copy_calibration:
        n = 256 << 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n}))
        return

    from workloads import config

    head = args.config
    order = [head] if args.only else [head] + [c for c in (1, 2, 3, 4, 5) if c != head]
    recs = {}
    cpu = None
    for cid in order:
        t0 = time.time()
        rec, w = measure(cid, args, dev, with_extras=not args.no_extras)
        recs[cid] = rec
        if cid == head and not args.no_cpu_baseline:
            cpu = cpu_baseline(w, args.cpu_seconds)
        del w
        print(f"[bench] {config(cid)['name']}: {rec['us_per_step']:.1f} us/step "
              f"({time.time() - t0:.0f} s)", file=sys.stderr, flush=True)

    h = recs[head]
    hc = config(head)
    line = {
        "metric": "verified draft tokens/s per verify step (attn+accept); % of HBM peak",
        "value": h["verified_tok_s"],
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": h["timing"]["timed_steps"],
        "warmup": h["timing"]["warmup_steps"],
        "ms_per_step": h["us_per_step"] * 1e-3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": hc["dtype"],
        "data": f"synthetic (seeded; inputs resident in HBM, rotated over {h['timing']['rotated_copies']} copies, "
                f"{h['timing']['mb_between_reuses']:.0f} MB between reuses of one copy)",
        "config": {"workload": h["workload"], "global_batch": hc["batch"], "parallelism": "single GPU"},
        "step_includes": "spec_verify_attn + spec_accept_* + spec_commit_kv (the whole verification step); "
                         "breakdown_us.attention_plus_accept times the first two alone",
        "verified_definition": "B * (N - 1) per step: every non-root node of the chain or tree is a draft the "
                               "step adjudicates; emitted_tok_s counts the tokens the step outputs "
                               "(accepted drafts plus the final token)",
        "ms_per_step_min": h["us_per_step_min"] * 1e-3,
        "ms_per_step_max": h["us_per_step_max"] * 1e-3,
        "emitted_tok_s": h["emitted_tok_s"],
        "breakdown_us": h["breakdown_us"],
        "roofline": h["roofline"],
        "accept_roofline": h["accept_roofline"],
        "cpu_baseline": cpu,
        "timing": h["timing"],
        "configs": {config(c)["name"]: recs[c] for c in sorted(recs)},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
