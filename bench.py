"""Benchmark of one speculative-decoding verification step on one MI355X.

A step is the whole hot path over one batch: tree-verify attention
(spec_verify_attn), acceptance (spec_accept_reject / spec_accept_typical) and
the KV commit (spec_commit_kv).  Every step runs all three on the same fixed
workload: the commit moves the accepted rows and advances its own copy of the
prefix lengths inside spare cache capacity, while attention keeps reading the
workload's prefix lengths.  The default workload is the Llama-3-8B-shaped
chain (batch 1, 32 query / 8 KV heads, head dim 128, bf16 KV prefix 2048,
K = 5 drafts, vocabulary 128256, T = 1, rejection rule).

Inputs are seeded synthetic tensors, generated once and copied to the GPU;
enough copies are rotated that consecutive reuses of one copy are more than
512 MB of traffic apart, so the 256 MB Infinity Cache cannot serve them.

Prints ONE JSON line: the metric (verified draft tokens per second =
B * (N - 1) / step time), the attention kernel's achieved algorithmic HBM
bandwidth against the 8 TB/s peak (timed live with HIP events on the launch
stream), and the fp64 CPU oracle timed on a bounded sample of the same step.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 640 << 20
def traffic_file(name):
    """Stored HBM counters of one attention call on the named workload."""
    return os.path.join(ROOT, "profiles", f"attn_{name}_traffic.json")
READ_PEAK_FILE = os.path.join(ROOT, "profiles", "hbm_read_peak.json")
READ_PROBE = os.path.join(ROOT, "speculative_decoding_verification_tree_amd", "hbm_read_probe")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2, help="workload id 1..5 (default: the Llama-3-8B chain)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU-baseline sample budget")
    ap.add_argument("--rotate-mb", type=int, default=ROTATE_BYTES >> 20,
                    help="input bytes cycled between reuses of one copy (default beats the 256 MB Infinity Cache; "
                         "0 keeps two copies, i.e. cache-warm)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (counter calibration)")
    ap.add_argument("--read-peak", action="store_true",
                    help="only run the streaming-read calibration program (measured HBM read bandwidth)")
    return ap.parse_args()


ATTN_SOURCES = ("attn.hip", "spec_common.h", "spec_internal.h")  # what the spec_verify_attn kernels compile from


def kernel_source_hash():
    """Hash of the attention kernels' sources: the stored traffic counters
    describe a spec_verify_attn call and stay valid while these are unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "speculative_decoding_verification_tree_amd", "csrc")
    for name in ATTN_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def attn_bytes(w):
    """Algorithmic bytes of one attention launch: every K and V row of the
    prefix plus the tree read once, Q read once, O written once."""
    es = 2 if w.dtype == "bf16" else 4
    kv = sum(int(L) + w.N for L in w.prefix_len) * w.Hkv * w.D * es * 2
    qo = 2 * w.B * w.N * w.Hq * w.D * es
    return kv + qo


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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); multi-GPU runs are not part of this "
              "build", file=sys.stderr)
        sys.exit(2)

    if args.read_peak:
        # A child process of its own (nothing here has touched the GPU yet).
        import subprocess
        if not os.path.exists(READ_PROBE):
            sys.exit(f"{READ_PROBE} is not built (run __graft_entry__.build())")
        res = subprocess.run([READ_PROBE], capture_output=True, text=True)
        sys.stderr.write(res.stderr)
        print(res.stdout.strip(), flush=True)
        sys.exit(res.returncode)

    import numpy as np
    import torch

    import speculative_decoding_verification_tree_amd as sv
    from workloads import config, generate

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

    cfg = config(args.config)
    w = generate(cfg, poison=False)
    B, N, V = w.B, w.N, w.V
    touched = attn_bytes(w) + (N * V * 4) * (2 if w.draft_probs is not None else 1)
    ncopies = max(2, math.ceil((args.rotate_mb << 20) / max(touched, 1)))
    # One graph replay runs `spg` steps over the copies in rotation; at least
    # 32 steps per replay so the per-replay launch cost is amortised.
    spg = ncopies * math.ceil(32 / ncopies)
    reps = max(1, math.ceil(args.steps / spg))
    # The commit advances its own copy of the prefix lengths by at most N rows
    # per use (attention keeps reading the fixed workload's lengths), so the
    # cache gets headroom for every use: eager warm-up, then (1 + reps)
    # replays each of the step and commit graphs.
    uses = math.ceil(max(args.warmup, ncopies) / ncopies) + 2 * (reps + 1) * (spg // ncopies) + 1
    mpl = int(w.prefix_len.max())
    cap = mpl + (uses + 1) * N

    def to_dev(arr, bf16):
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16) if bf16 else np.ascontiguousarray(arr))
        t = t.to(dev)
        return t.view(torch.bfloat16) if bf16 else t

    bf16 = w.dtype == "bf16"
    kpad = np.zeros((B, w.Hkv, cap, w.D), dtype=w.k_cache.dtype)
    vpad = np.zeros_like(kpad)
    kpad[:, :, : w.cap] = w.k_cache
    vpad[:, :, : w.cap] = w.v_cache
    base = dict(
        q=to_dev(w.q, bf16), k=to_dev(kpad, bf16), v=to_dev(vpad, bf16),
        logits=torch.from_numpy(w.target_logits).to(dev),
        draft=torch.from_numpy(w.draft_probs).to(dev) if w.draft_probs is not None else None,
        tokens=torch.from_numpy(w.tokens).to(dev),
        parent=None if w.is_chain else torch.from_numpy(w.parent).to(dev),
        ua=torch.from_numpy(w.u_accept).to(dev), us=torch.from_numpy(w.u_sample).to(dev),
    )
    del kpad, vpad
    copies = []
    for _ in range(ncopies):
        c = {k: (t.clone() if t is not None else None) for k, t in base.items()}
        c["pl"] = torch.from_numpy(w.prefix_len.copy()).to(dev)        # read by attention
        c["pl_commit"] = torch.from_numpy(w.prefix_len.copy()).to(dev)  # advanced by the commit
        c["out"] = torch.empty_like(c["q"])
        c["al"] = torch.empty(B, dtype=torch.int32, device=dev)
        c["path"] = torch.empty(B, N, dtype=torch.int32, device=dev)
        c["otok"] = torch.empty(B, N, dtype=torch.int32, device=dev)
        copies.append(c)
    desc = sv.attn_desc(B, N, w.Hq, w.Hkv, w.D, cap, torch.bfloat16 if bf16 else torch.float32)
    attn_ws = torch.zeros(max(sv.spec_verify_attn_workspace_bytes(desc, mpl), 1), dtype=torch.uint8, device=dev)
    acc_ws = torch.zeros(max(sv.spec_accept_workspace_bytes(B, N, V), 1), dtype=torch.uint8, device=dev)

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

    def step(c):
        attn(c)
        accept(c)
        commit(c)

    # The step before the path, timed on its own: the Medusa candidate tree
    # (tree workloads built as a Cartesian product) and the depth-position
    # rotary embedding of q and the tree's K rows, in place.
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

    # The rejection rule on a truncated target (top-k, then nucleus), timed on
    # its own for rejection-rule workloads.
    filt_k, filt_p = 50, 0.9

    def accept_filtered(c):
        sv.spec_accept_reject_filtered(c["logits"], c["draft"], c["tokens"], c["parent"], c["ua"], c["us"],
                                       w.temperature, filt_k, filt_p, c["al"], c["path"], c["otok"],
                                       workspace=acc_ws)

    # Multi-draft tree rejection (recursive residuals), timed on its own for
    # rejection-rule tree workloads.
    md_ws = None
    if w.rule == "reject" and not w.is_chain:
        md_ws = torch.empty(max(sv.spec_accept_multidraft_workspace_bytes(B, V), 1), dtype=torch.uint8, device=dev)

    def accept_multidraft(c):
        sv.spec_accept_multidraft(c["logits"], c["draft"], c["tokens"], c["parent"], c["ua"], c["us"],
                                  w.temperature, c["al"], c["path"], c["otok"], workspace=md_ws)

    # Linear-attention verification of the same trees (16 heads, Dk = Dv =
    # 128, bf16 q/k/v, fp32 state), its factor commit, and the two fused (the
    # deferred commit), timed on their own.
    LH, LD = 16, 128
    la_state = torch.randn(B, LH, LD, LD, device=dev) / LD ** 0.5
    la_q = (torch.randn(B, N, LH, LD, device=dev) / LD ** 0.5).to(torch.bfloat16)
    la_k = torch.randn(B, N, LH, LD, device=dev).to(torch.bfloat16)
    la_v = torch.randn(B, N, LH, LD, device=dev).to(torch.bfloat16)
    la_alpha = torch.rand(B, N, LH, device=dev) * 0.4 + 0.6
    la_out = torch.empty_like(la_v)
    la_path = copies[0]["path"]
    la_acc = copies[0]["al"]
    la_pending = (la_k, la_v, la_alpha, copies[0]["parent"], la_path, la_acc)

    def la_verify(c):
        sv.spec_la_verify(la_state, la_q, la_k, la_v, la_alpha, c["parent"], out=la_out)

    def la_commit(c):
        sv.spec_la_commit(la_state, *la_pending)

    def la_fused(c):
        sv.spec_la_verify(la_state, la_q, la_k, la_v, la_alpha, c["parent"], out=la_out, pending=la_pending)

    # eager warm-up (also checks every call returns SPEC_OK)
    for i in range(max(args.warmup, ncopies)):
        step(copies[i % ncopies])
    torch.cuda.synchronize()

    # One HIP graph per phase covering every rotated copy once: replaying it
    # launches the kernels back to back without per-call host overhead.
    def capture(fns):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(spg):
                for fn in fns:
                    fn(copies[i % ncopies])
        return g

    g_step = capture([attn, accept, commit])
    g_attn = capture([attn])
    g_acc = capture([accept])
    g_commit = capture([commit])
    g_rope = capture([tree_rope])
    graphs = [g_step, g_attn, g_acc, g_commit, g_rope]
    g_filt = None
    if w.rule == "reject" and w.temperature > 0:
        for i in range(ncopies):
            accept_filtered(copies[i])
        g_filt = capture([accept_filtered])
        graphs.append(g_filt)
    for fn in (la_verify, la_commit, la_fused):
        fn(copies[0])
    torch.cuda.synchronize()
    g_lav, g_lac, g_laf = capture([la_verify]), capture([la_commit]), capture([la_fused])
    graphs += [g_lav, g_lac, g_laf]
    g_md = None
    if md_ws is not None:
        for i in range(ncopies):
            accept_multidraft(copies[i])
        g_md = capture([accept_multidraft])
        graphs.append(g_md)
    for g in graphs:
        g.replay()
    torch.cuda.synchronize()

    def timed(g, reps):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record()
        for _ in range(reps):
            g.replay()
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / (reps * spg)

    K = reps * spg
    ms_step = timed(g_step, reps)
    attn_ms = timed(g_attn, reps)
    accept_ms = timed(g_acc, reps)
    commit_ms = timed(g_commit, reps)
    rope_ms = timed(g_rope, reps)
    filt_ms = timed(g_filt, reps) if g_filt is not None else None
    md_ms = timed(g_md, reps) if g_md is not None else None
    lav_ms, lac_ms, laf_ms = timed(g_lav, reps), timed(g_lac, reps), timed(g_laf, reps)
    la_state_b = B * LH * LD * LD * 4
    la_io_b = B * N * LH * LD * 2 * 4  # q, k, v in and out, bf16
    la_verify_b = la_state_b + la_io_b
    la_commit_b = 2 * la_state_b  # the state read and written (the path's factors are small)
    # every target row once (leaf rows too: the stop row may be one), plus the
    # stop row and one draft row per request for the residual
    filt_bytes = (B * N * V + 2 * B * V) * 4
    esz = 2 if bf16 else 4
    rope_bytes = 2 * (B * N * w.Hq * w.D + B * w.Hkv * N * w.D) * esz  # read + write, q and tree K rows

    a_bytes = attn_bytes(w)
    achieved = a_bytes / (attn_ms * 1e-3) / 1e9
    acc_bytes = accept_bytes(w, copies[0]["al"].cpu().numpy(), copies[0]["path"].cpu().numpy())
    read_peak = None
    if os.path.exists(READ_PEAK_FILE):
        with open(READ_PEAK_FILE) as f:
            read_peak = json.load(f).get("kv_read_GBs")
    traffic = None
    khash = kernel_source_hash()
    if os.path.exists(traffic_file(cfg["name"])):
        with open(traffic_file(cfg["name"])) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == khash and tr.get("config") == args.config:
            traffic = tr.get("bytes_per_launch")

    verified = B * (N - 1)
    value = verified / (ms_step * 1e-3)
    al = copies[0]["al"].cpu().numpy()

    cpu = None
    if not args.no_cpu_baseline:
        import oracle

        par = None if w.is_chain else w.parent
        n_done, t_cpu = 0, 0.0
        T32 = float(np.float32(w.temperature))
        while n_done == 0 or t_cpu < args.cpu_seconds:
            s0 = time.perf_counter()
            oracle.tree_attn(w.q, w.k_cache, w.v_cache, w.prefix_len, par, w.dtype)
            r = oracle.accept(w.rule, w.target_logits, w.tokens, par, T32, w.draft_probs, w.u_accept,
                              w.u_sample, float(np.float32(w.epsilon)), float(np.float32(w.delta)))
            kk, vv = w.k_cache.copy(), w.v_cache.copy()
            oracle.commit(kk, vv, w.prefix_len.copy(), r["path"], r["accept_len"])
            t_cpu += time.perf_counter() - s0
            n_done += 1
            if n_done >= 1000:
                break
        cpu = {"value": verified * n_done / t_cpu, "unit": "verified draft tokens/s", "cores": oracle.num_threads(),
               "kind": "oracle",
               "sample": f"{n_done} full steps (attention all rows, acceptance, commit) of the same workload, "
                         f"{t_cpu:.1f} s on the host"}

    name = cfg["name"]
    line = {
        "metric": "verified draft tokens/s per verify step (attn+accept)",
        "value": value,
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": f"synthetic (seeded; inputs resident in HBM, rotated over {ncopies} copies, "
                f"{ncopies * touched / 2**20:.0f} MB between reuses of one copy)",
        "config": {
            "workload": f"{name}: B={B}, Hq={w.Hq}/Hkv={w.Hkv}, D={w.D}, {w.dtype} KV prefix "
                        f"{int(w.prefix_len.min())}..{int(w.prefix_len.max())}, N={N} nodes "
                        f"({'chain' if w.is_chain else 'tree'}), V={V}, T={w.temperature}, {w.rule} rule",
            "global_batch": B,
            "parallelism": "single GPU",
        },
        "breakdown_us": {"attention": attn_ms * 1e3, "accept": accept_ms * 1e3, "commit": commit_ms * 1e3,
                         "tree_rope": rope_ms * 1e3},
        "tree_rope": {"us": rope_ms * 1e3, "bytes": rope_bytes,
                      "achieved_GBs": rope_bytes / (rope_ms * 1e-3) / 1e9,
                      "calls": ("spec_medusa_tree + " if cartesian else "") + "spec_tree_rope",
                      "note": "before the path; not part of ms_per_step"},
        "filtered_accept": None if filt_ms is None else {
            "us": filt_ms * 1e3, "top_k": filt_k, "top_p": filt_p, "bytes": filt_bytes,
            "achieved_GBs": filt_bytes / (filt_ms * 1e-3) / 1e9, "calls": "spec_accept_reject_filtered",
            "note": "the rejection rule on the top-k / nucleus truncated target; not part of ms_per_step"},
        "linear_attention": {
            "heads": LH, "key_dim": LD, "value_dim": LD,
            "verify_us": lav_ms * 1e3, "verify_GBs": la_verify_b / (lav_ms * 1e-3) / 1e9,
            "commit_us": lac_ms * 1e3, "commit_GBs": la_commit_b / (lac_ms * 1e-3) / 1e9,
            "fused_us": laf_ms * 1e3, "fused_GBs": (la_verify_b + la_state_b) / (laf_ms * 1e-3) / 1e9,
            "calls": "spec_la_verify, spec_la_commit, spec_la_verify with pending factors",
            "note": "same trees as the workload, bf16 q/k/v, fp32 state; not part of ms_per_step"},
        "multidraft_accept": None if md_ms is None else {
            "us": md_ms * 1e3, "calls": "spec_accept_multidraft",
            "note": "tree rejection by recursive residuals over each node's children; not part of ms_per_step"},
        "roofline": {
            "bound": "hbm",
            "kernel": "spec_verify_attn",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
            "algorithmic_bytes_per_launch": a_bytes,
            "kernel_source_hash": khash,
            "measured_read_peak": read_peak,
            "frac_of_measured_read_peak": None if read_peak is None else achieved / read_peak,
        },
        "accept_roofline": {
            "bound": "hbm",
            "calls": "spec_accept_reject" if w.rule == "reject" else "spec_accept_typical",
            "achieved": acc_bytes / (accept_ms * 1e-3) / 1e9,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": acc_bytes / (accept_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes_per_call": acc_bytes,
        },
        "cpu_baseline": cpu,
        "accept_len_last_step": al.tolist()[:8],
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
