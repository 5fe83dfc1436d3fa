"""MI355X (gfx950) speculative-decoding verification step.

Tree-verify attention, rejection / typical acceptance over the vocabulary
(also on a top-k / nucleus truncated target, and by recursive residuals over
multi-draft trees), the in-place KV commit, the Medusa candidate tree with its
depth-position rotary embedding, and linear-attention verification with its
factor commit, as hand-written HIP kernels behind the C ABI of
include/spec_verify.h.  This package is the thin PyTorch binding of that ABI.
"""
from .api import (
    SpecError,
    attn_desc,
    spec_accept_multidraft,
    spec_accept_multidraft_workspace_bytes,
    spec_accept_reject,
    spec_accept_reject_noalloc,
    spec_accept_reject_filtered,
    spec_accept_filtered_workspace_bytes,
    spec_accept_typical,
    spec_accept_workspace_bytes,
    spec_commit_kv,
    spec_la_commit,
    spec_la_verify,
    spec_medusa_tree,
    spec_medusa_tree_nodes,
    spec_tree_positions,
    spec_tree_rope,
    spec_validate_tree,
    spec_verify_attn,
    spec_verify_attn_workspace_bytes,
)
from ._native import LIB_PATH, SIGNATURES, lib, status_string

__all__ = [
    "SpecError", "attn_desc", "spec_accept_multidraft", "spec_accept_multidraft_workspace_bytes", "spec_accept_reject", "spec_accept_reject_noalloc",
    "spec_accept_reject_filtered", "spec_accept_filtered_workspace_bytes", "spec_accept_typical", "spec_accept_workspace_bytes",
    "spec_commit_kv", "spec_la_commit", "spec_la_verify", "spec_medusa_tree", "spec_medusa_tree_nodes", "spec_tree_positions", "spec_tree_rope",
    "spec_validate_tree", "spec_verify_attn",
    "spec_verify_attn_workspace_bytes", "LIB_PATH", "SIGNATURES", "lib", "status_string",
]
