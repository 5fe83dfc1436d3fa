"""The C ABI on the CPU: the library loads, exports every entry point that
include/spec_verify.h declares (with a binding signature for each), and
rejects invalid arguments with the documented status before launching
anything (no GPU is touched by these calls)."""
import ctypes
import os
import re

import pytest

import speculative_decoding_verification_tree_amd as sv
from speculative_decoding_verification_tree_amd._native import AttnDesc, SIGNATURES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "spec_verify.h")
OK, EINVAL, EUNSUPPORTED, EWORKSPACE = 0, -1, -2, -3
FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) == 19, names
    lib = sv.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in SIGNATURES, n
    assert set(SIGNATURES) == set(names)


def test_struct_layout_matches_header():
    assert ctypes.sizeof(AttnDesc) == 40


def _desc(**kw):
    d = dict(batch=1, num_nodes=6, num_q_heads=32, num_kv_heads=8, head_dim=128, kv_capacity=2054, dtype=1,
             softmax_scale=0.0, kv_split_keys=0, rope_base=0.0)
    d.update(kw)
    return AttnDesc(**d)


def _attn(desc, mpl=2048, ws_bytes=1 << 30, ws=FAKE):
    return sv.lib().spec_verify_attn(ctypes.byref(desc) if desc is not None else None, mpl, FAKE, FAKE, FAKE,
                                     FAKE, None, FAKE, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,want", [
    (dict(num_nodes=0), EINVAL),
    (dict(num_nodes=65), EINVAL),
    (dict(num_q_heads=30), EINVAL),
    (dict(num_kv_heads=0), EINVAL),
    (dict(head_dim=96), EUNSUPPORTED),
    (dict(head_dim=0), EINVAL),
    (dict(dtype=7), EUNSUPPORTED),
    (dict(kv_capacity=2053), EINVAL),
    (dict(batch=-1), EINVAL),
    (dict(softmax_scale=float("nan")), EINVAL),
    (dict(kv_split_keys=-1), EINVAL),
    (dict(rope_base=-1.0), EINVAL),
    (dict(rope_base=float("nan")), EINVAL),
    (dict(rope_base=float("inf")), EINVAL),
])
def test_attention_argument_errors(kw, want):
    assert _attn(_desc(**kw)) == want


def test_attention_null_and_workspace_errors():
    lib = sv.lib()
    assert _attn(None) == EINVAL
    d = _desc()
    need = lib.spec_verify_attn_workspace_bytes(ctypes.byref(d), 2048)
    assert need > 0
    assert _attn(d, ws_bytes=need - 1) == EWORKSPACE
    assert _attn(d, ws=None) == EWORKSPACE
    assert lib.spec_verify_attn(ctypes.byref(d), 2048, None, FAKE, FAKE, FAKE, None, FAKE, FAKE, need, None) == EINVAL
    assert _attn(d, mpl=-1) == EINVAL
    # 16-byte vectors: every tensor and the workspace must be 16-byte aligned
    odd = ctypes.c_void_p(0x10000 + 8)
    call = lambda q=FAKE, k=FAKE, v=FAKE, o=FAKE, ws=FAKE: lib.spec_verify_attn(
        ctypes.byref(d), 2048, q, k, v, FAKE, None, o, ws, need, None)
    assert call(q=odd) == EINVAL
    assert call(k=odd) == EINVAL
    assert call(v=odd) == EINVAL
    assert call(o=odd) == EINVAL
    assert call(ws=odd) == EINVAL
    # empty batch: nothing to do, nothing launched
    assert _attn(_desc(batch=0)) == OK
    assert lib.spec_verify_attn_workspace_bytes(ctypes.byref(_desc(head_dim=96)), 10) == 0


def test_attention_split_granularity_sizes_workspace():
    # Finer KV ranges mean more partials: the workspace grows, and one
    # 32-key block per range is the finest split.
    lib = sv.lib()
    auto = lib.spec_verify_attn_workspace_bytes(ctypes.byref(_desc(batch=4)), 2048)
    fine = lib.spec_verify_attn_workspace_bytes(ctypes.byref(_desc(batch=4, kv_split_keys=32)), 2048)
    one = lib.spec_verify_attn_workspace_bytes(ctypes.byref(_desc(batch=4, kv_split_keys=1)), 2048)
    assert fine >= auto > 0
    assert one == fine


def _rej(B=2, N=6, V=1000, T=1.0, ws_bytes=1 << 30, ws=FAKE, draft=FAKE, us=FAKE):
    return sv.lib().spec_accept_reject(B, N, V, FAKE, draft, FAKE, None, FAKE, us, T, FAKE, FAKE, FAKE, ws,
                                       ws_bytes, None)


def _typ(B=2, N=6, V=1000, T=1.0, eps=0.1, delta=0.2, ws_bytes=1 << 30):
    return sv.lib().spec_accept_typical(B, N, V, FAKE, FAKE, None, T, eps, delta, FAKE, FAKE, FAKE, FAKE, ws_bytes,
                                        None)


def test_accept_argument_errors():
    lib = sv.lib()
    assert _rej(V=0) == EINVAL
    assert _rej(N=0) == EINVAL
    assert _rej(N=65) == EINVAL
    assert _rej(B=-1) == EINVAL
    assert _rej(T=-0.5) == EINVAL
    assert _rej(T=float("nan")) == EINVAL
    assert _rej(T=float("inf")) == EINVAL
    assert _rej(draft=None) == EINVAL
    assert _rej(us=None) == EINVAL
    need = lib.spec_accept_workspace_bytes(2, 6, 1000)
    assert need > 0
    assert _rej(ws_bytes=need - 1) == EWORKSPACE
    assert _rej(ws=None) == EWORKSPACE
    assert _typ(eps=-1.0) == EINVAL
    assert _typ(delta=float("nan")) == EINVAL
    assert _typ(T=-1.0) == EINVAL
    assert _typ(ws_bytes=lib.spec_accept_workspace_bytes(2, 6, 1000) - 8) == EWORKSPACE
    assert _rej(B=0) == OK and _typ(B=0) == OK
    assert lib.spec_accept_workspace_bytes(0, 6, 10) == 0


def _filt(B=2, N=6, V=1000, T=1.0, k=5, p=0.9, ws_bytes=1 << 30):
    return sv.lib().spec_accept_reject_filtered(B, N, V, FAKE, FAKE, FAKE, None, FAKE, FAKE, T, k, p, FAKE, FAKE,
                                                FAKE, FAKE, ws_bytes, None)


def test_noalloc_accept_errors():
    # Host-side checks only: none of these reach a device call.
    lib = sv.lib()
    call = lambda B=2, N=6, V=1000, T=1.0, us=FAKE: lib.spec_accept_reject_noalloc(
        B, N, V, FAKE, FAKE, FAKE, None, FAKE, us, T, FAKE, FAKE, FAKE, None)
    assert call(B=-1) == EINVAL
    assert call(B=0) == OK
    assert call(N=65) == EINVAL
    assert call(T=float("nan")) == EINVAL
    assert call(us=None) == EINVAL
    # a shape whose workspace exceeds the library's scratch array
    assert sv.spec_accept_workspace_bytes(4096, 64, 128256) > (8 << 20)
    assert call(B=4096, N=64, V=128256) == EWORKSPACE


def test_filtered_accept_errors():
    assert _filt(k=-1) == EINVAL
    assert _filt(p=0.0) == EINVAL
    assert _filt(p=1.5) == EINVAL
    assert _filt(p=float("nan")) == EINVAL
    assert _filt(T=-1.0) == EINVAL
    assert _filt(V=0) == EINVAL
    assert _filt(N=65) == EINVAL
    assert _filt(ws_bytes=sv.lib().spec_accept_workspace_bytes(2, 6, 1000) - 1) == EWORKSPACE
    assert _filt(B=0) == OK


def test_filtered_workspace_extends_the_plain_one():
    lib = sv.lib()
    for B, N, V in ((2, 6, 1000), (1, 6, 128256), (64, 8, 128256), (4, 64, 128256)):
        plain = lib.spec_accept_workspace_bytes(B, N, V)
        filt = lib.spec_accept_filtered_workspace_bytes(B, N, V)
        # per (row, chunk), at least one chunk a row: a 16-byte record, 64 digit counts, 256 keys
        assert filt >= plain + B * N * (16 + 64 * 4 + 256 * 4), (B, N, V)
    assert lib.spec_accept_filtered_workspace_bytes(0, 6, 1000) == 0
    assert lib.spec_accept_filtered_workspace_bytes(2, 65, 1000) == 0
    assert lib.spec_accept_filtered_workspace_bytes(2, 6, 0) == 0


def test_multidraft_errors():
    lib = sv.lib()
    need = lib.spec_accept_multidraft_workspace_bytes(2, 1000)
    up = lambda n: (n + 255) // 256 * 256  # noqa: E731
    # two residual rows per request, two rounds of 64 16-byte records per
    # request, each region 256-byte aligned
    assert need == up(2 * 2 * 1000 * 4) + up(2 * 2 * 64 * 16)
    assert lib.spec_accept_multidraft_workspace_bytes(0, 1000) == 0
    assert lib.spec_accept_multidraft_workspace_bytes(2, 0) == 0

    def md(B=2, N=6, V=1000, T=1.0, ws_bytes=need, draft=FAKE):
        return lib.spec_accept_multidraft(B, N, V, FAKE, draft, FAKE, None, FAKE, FAKE, T, FAKE, FAKE, FAKE, FAKE,
                                          ws_bytes, None)
    assert md(ws_bytes=need - 1) == EWORKSPACE
    assert md(T=-1.0) == EINVAL
    assert md(N=65) == EINVAL
    assert md(draft=None) == EINVAL
    assert md(B=-1) == EINVAL
    assert md(B=0) == OK


def test_linear_attention_errors():
    from speculative_decoding_verification_tree_amd._native import LaDesc, LaFactors
    lib = sv.lib()

    def d(**kw):
        x = dict(batch=2, num_nodes=6, num_heads=4, key_dim=128, value_dim=128, dtype=0)
        x.update(kw)
        return LaDesc(**x)

    def ver(desc, state=FAKE, pending=None):
        return lib.spec_la_verify(ctypes.byref(desc), state, FAKE, FAKE, FAKE, None, None, FAKE,
                                  ctypes.byref(pending) if pending is not None else None, None)
    assert ver(d(key_dim=96)) == EUNSUPPORTED
    assert ver(d(value_dim=256)) == EUNSUPPORTED
    assert ver(d(key_dim=0)) == EINVAL
    assert ver(d(dtype=5)) == EUNSUPPORTED
    assert ver(d(num_nodes=65)) == EINVAL
    assert ver(d(num_heads=0)) == EINVAL
    assert ver(d(batch=-1)) == EINVAL
    assert ver(d(), state=None) == EINVAL
    assert ver(d(), pending=LaFactors(0, FAKE, FAKE, None, None, FAKE, FAKE)) == EINVAL
    assert ver(d(batch=0), state=None) == OK
    assert lib.spec_la_verify(None, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, None) == EINVAL
    good = LaFactors(6, FAKE, FAKE, None, None, FAKE, FAKE)
    assert lib.spec_la_commit(ctypes.byref(d()), None, ctypes.byref(good), None) == EINVAL
    assert lib.spec_la_commit(ctypes.byref(d()), FAKE, None, None) == EINVAL
    assert lib.spec_la_commit(ctypes.byref(d(key_dim=32)), FAKE, ctypes.byref(good), None) == EUNSUPPORTED
    odd = ctypes.c_void_p(0x10000 + 4)  # the state moves in 16-byte vectors
    assert ver(d(), state=odd) == EINVAL
    assert lib.spec_la_commit(ctypes.byref(d()), odd, ctypes.byref(good), None) == EINVAL


def test_commit_and_helper_errors():
    lib = sv.lib()
    assert lib.spec_commit_kv(ctypes.byref(_desc(head_dim=80)), FAKE, FAKE, FAKE, FAKE, FAKE, None) == EUNSUPPORTED
    assert lib.spec_commit_kv(ctypes.byref(_desc()), None, FAKE, FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.spec_commit_kv(ctypes.byref(_desc(batch=0)), None, None, None, None, None, None) == OK
    assert lib.spec_tree_positions(2, 0, FAKE, None, FAKE, None) == EINVAL
    assert lib.spec_tree_positions(2, 4, None, None, FAKE, None) == EINVAL
    assert lib.spec_validate_tree(2, 65, FAKE, FAKE, None) == EINVAL
    assert lib.spec_validate_tree(2, 4, None, FAKE, None) == EINVAL
    for rc in (0, -1, -2, -3, -4, 5):
        assert sv.status_string(rc)


def test_medusa_tree_and_rope_errors():
    lib = sv.lib()
    W = ctypes.c_int32 * 8
    assert lib.spec_medusa_tree_nodes(4, W(3, 2, 2, 2), 3) == 46
    assert lib.spec_medusa_tree_nodes(1, W(1), 1) == 2
    assert lib.spec_medusa_tree_nodes(3, W(4, 4, 4), 4) == 0   # 85 nodes
    assert lib.spec_medusa_tree_nodes(2, W(2, 3), 2) == 0      # width above max_width
    assert lib.spec_medusa_tree_nodes(2, W(0, 3), 3) == 0
    assert lib.spec_medusa_tree_nodes(0, W(1), 1) == 0
    assert lib.spec_medusa_tree_nodes(2, None, 3) == 0
    assert lib.spec_medusa_tree(2, 3, W(4, 4, 4), 4, FAKE, FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.spec_medusa_tree(-1, 1, W(2), 2, FAKE, FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.spec_medusa_tree(2, 1, W(2), 2, None, FAKE, FAKE, FAKE, None) == EINVAL
    assert lib.spec_medusa_tree(0, 1, W(2), 2, None, None, None, None, None) == OK
    d = _desc()
    assert lib.spec_tree_rope(ctypes.byref(d), FAKE, FAKE, FAKE, None, 0.0, None) == EINVAL
    assert lib.spec_tree_rope(ctypes.byref(d), FAKE, FAKE, FAKE, None, float("inf"), None) == EINVAL
    assert lib.spec_tree_rope(ctypes.byref(d), FAKE, FAKE, None, None, 10000.0, None) == EINVAL
    assert lib.spec_tree_rope(ctypes.byref(_desc(head_dim=96)), FAKE, FAKE, FAKE, None, 1e4, None) == EUNSUPPORTED
    assert lib.spec_tree_rope(ctypes.byref(_desc(batch=0)), None, None, None, None, 1e4, None) == OK
