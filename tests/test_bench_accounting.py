"""Host-side byte accounting that bench.py's roofline fractions rest on (no
GPU): the algorithmic bytes of the attention and acceptance calls, on shapes
small enough to count by hand."""
import os
import sys
from types import SimpleNamespace

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def _w(rule="reject", parent=None, B=1, N=3, V=10):
    return SimpleNamespace(B=B, N=N, V=V, rule=rule, parent=parent)


GATHERS = 1 * 2 * 20        # B (N - 1) nodes x (token, parent, u, draft prob, logit)
OUTPUTS = 1 * (1 + 2 * 3) * 4  # accept_len, path, out_tokens


def test_reject_first_draft_rejected():
    # chain 0-1-2: rows 0 and 1 have children; stop at the root, which has a
    # child, so its first child's draft row is read too
    path = np.array([[0, -1, -1]], dtype=np.int32)
    got = bench.accept_bytes(_w(), np.array([0]), path)
    assert got == 3 * 10 * 4 + GATHERS + OUTPUTS


def test_reject_all_accepted_reads_the_leaf_row():
    path = np.array([[0, 1, 2]], dtype=np.int32)
    got = bench.accept_bytes(_w(), np.array([2]), path)
    assert got == 3 * 10 * 4 + GATHERS + OUTPUTS  # two internal rows + the leaf stop row


def test_typical_stop_inside_reads_no_extra_row():
    path = np.array([[0, 1, -1]], dtype=np.int32)
    got = bench.accept_bytes(_w(rule="typical"), np.array([1]), path)
    assert got == 2 * 10 * 4 + GATHERS + OUTPUTS


def test_tree_internal_rows_counted_once():
    # root with children 1 and 2; node 1 with child 3 (N = 4): internal rows 0, 1
    parent = np.array([[-1, 0, 0, 1]], dtype=np.int32)
    path = np.array([[0, 2, -1, -1]], dtype=np.int32)  # stops at leaf 2
    w = _w(parent=parent, N=4)
    got = bench.accept_bytes(w, np.array([1]), path)
    gathers = 1 * 3 * 20
    outputs = 1 * (1 + 2 * 4) * 4
    assert got == 3 * 10 * 4 + gathers + outputs  # rows 0, 1 and the leaf stop row 2


def test_attention_bytes_count_each_kv_row_once():
    w = SimpleNamespace(dtype="bf16", prefix_len=np.array([5, 9]), N=3, Hkv=2, D=4, B=2, Hq=4)
    kv = (5 + 3 + 9 + 3) * 2 * 4 * 2 * 2  # rows x heads x D x bf16 x (K and V)
    qo = 2 * 2 * 3 * 4 * 4 * 2            # q read and out written, bf16
    assert bench.attn_bytes(w) == kv + qo


def test_stored_traffic_matches_each_workload():
    # Every stored traffic file (attention and acceptance calls) names the
    # configuration it was measured on, and the bench looks it up by that
    # workload's name.
    from workloads.configs import config
    import json
    found = 0
    for kind in ("attn", "accept", "extras"):
        for cid in (1, 2, 3, 4, 5):
            path = bench.traffic_file(kind, config(cid)["name"])
            if not os.path.exists(path):
                continue
            found += 1
            with open(path) as f:
                tr = json.load(f)
            assert tr["config"] == cid
            if kind == "extras":
                assert all(v["bytes_per_call"] > 0 for v in tr["calls"].values())
            else:
                assert tr["bytes_per_launch"] > 0
            assert len(tr["kernel_source_hash"]) == len(bench.kernel_source_hash())
    assert found >= 1


def test_attention_flops_follow_root_paths():
    # chain of 3 over prefixes 5 and 9: node i sees L + i + 1 keys
    w = SimpleNamespace(dtype="bf16", prefix_len=np.array([5, 9]), N=3, Hkv=2, D=4, B=2, Hq=4, is_chain=True,
                        parent=None)
    keys = (5 + 1) + (5 + 2) + (5 + 3) + (9 + 1) + (9 + 2) + (9 + 3)
    assert bench.attn_flops(w) == 4 * 4 * 4 * keys
    # tree 0 <- 1, 0 <- 2, 1 <- 3: depths 0, 1, 1, 2
    t = SimpleNamespace(dtype="bf16", prefix_len=np.array([7]), N=4, Hkv=1, D=8, B=1, Hq=2, is_chain=False,
                        parent=np.array([[-1, 0, 0, 1]]))
    assert bench.attn_flops(t) == 4 * 8 * 2 * (4 * 7 + 1 + 2 + 2 + 3)


def test_multidraft_bytes_count_passes():
    # chain 0-1-2: the child of 0 passes, the child of 1 is rejected: two
    # statistics passes, three row passes for the rejection, one draw pass
    w = SimpleNamespace(B=1, N=3, V=10, parent=None, temperature=1.0)
    got = bench.multidraft_bytes(w, np.array([1]), np.array([[0, 1, -1]], dtype=np.int32))
    assert got == (2 + 3 + 1) * 10 * 4
    # tree 0 <- 1, 0 <- 2, 0 <- 3: children 1 and 2 rejected, 3 passes, 3 a leaf
    t = SimpleNamespace(B=1, N=4, V=10, parent=np.array([[-1, 0, 0, 0]], dtype=np.int32), temperature=1.0)
    got = bench.multidraft_bytes(t, np.array([1]), np.array([[0, 3, -1, -1]], dtype=np.int32))
    assert got == (2 + 3 * 2 + 1) * 10 * 4
    # greedy: statistics passes only
    g = SimpleNamespace(B=1, N=4, V=10, parent=np.array([[-1, 0, 0, 0]], dtype=np.int32), temperature=0.0)
    assert bench.multidraft_bytes(g, np.array([1]), np.array([[0, 3, -1, -1]], dtype=np.int32)) == 2 * 10 * 4
