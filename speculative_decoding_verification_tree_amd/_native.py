"""ctypes loader of libspecverify.so (the gfx950 HIP library).

Loading fails loudly when the library has not been built: there is no
fallback implementation of any entry point.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libspecverify.so")

# Every symbol declared in include/spec_verify.h, with its ctypes signature.
_P = ctypes.c_void_p
_I = ctypes.c_int32
_F = ctypes.c_float
_Z = ctypes.c_size_t
SIGNATURES = {
    "spec_verify_attn_workspace_bytes": (_Z, [_P, _I]),
    "spec_verify_attn": (ctypes.c_int, [_P, _I, _P, _P, _P, _P, _P, _P, _P, _Z, _P]),
    "spec_accept_workspace_bytes": (_Z, [_I, _I, _I]),
    "spec_accept_filtered_workspace_bytes": (_Z, [_I, _I, _I]),
    "spec_accept_reject": (ctypes.c_int, [_I, _I, _I, _P, _P, _P, _P, _P, _P, _F, _P, _P, _P, _P, _Z, _P]),
    "spec_accept_reject_noalloc": (ctypes.c_int, [_I, _I, _I, _P, _P, _P, _P, _P, _P, _F, _P, _P, _P, _P]),
    "spec_accept_multidraft_workspace_bytes": (ctypes.c_size_t, [_I, _I]),
    "spec_accept_multidraft": (ctypes.c_int, [_I, _I, _I, _P, _P, _P, _P, _P, _P, _F, _P, _P, _P, _P, _Z, _P]),
    "spec_accept_reject_filtered": (ctypes.c_int,
                                    [_I, _I, _I, _P, _P, _P, _P, _P, _P, _F, _I, _F, _P, _P, _P, _P, _Z, _P]),
    "spec_accept_typical": (ctypes.c_int, [_I, _I, _I, _P, _P, _P, _F, _F, _F, _P, _P, _P, _P, _Z, _P]),
    "spec_commit_kv": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P]),
    "spec_tree_positions": (ctypes.c_int, [_I, _I, _P, _P, _P, _P]),
    "spec_validate_tree": (ctypes.c_int, [_I, _I, _P, _P, _P]),
    "spec_medusa_tree_nodes": (_I, [_I, _P, _I]),
    "spec_medusa_tree": (ctypes.c_int, [_I, _I, _P, _I, _P, _P, _P, _P, _P]),
    "spec_tree_rope": (ctypes.c_int, [_P, _P, _P, _P, _P, _F, _P]),
    "spec_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "spec_la_verify": (ctypes.c_int, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P]),
    "spec_la_commit": (ctypes.c_int, [_P, _P, _P, _P]),
}

SPEC_OK, SPEC_EINVAL, SPEC_EUNSUPPORTED, SPEC_EWORKSPACE, SPEC_EHIP = 0, -1, -2, -3, -4
SPEC_F32, SPEC_BF16 = 0, 1


class AttnDesc(ctypes.Structure):
    """Mirror of spec_attn_desc."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_nodes", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_capacity", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("kv_split_keys", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
    ]


class LaDesc(ctypes.Structure):
    """Mirror of spec_la_desc."""
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_nodes", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("key_dim", ctypes.c_int32),
        ("value_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
    ]


class LaFactors(ctypes.Structure):
    """Mirror of spec_la_factors."""
    _fields_ = [
        ("num_nodes", ctypes.c_int32),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("alpha", ctypes.c_void_p),
        ("parent", ctypes.c_void_p),
        ("path", ctypes.c_void_p),
        ("accept_len", ctypes.c_void_p),
    ]


_lib = None


def lib():
    """The loaded library (raises if libspecverify.so is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is not built; run speculative_decoding_verification_tree_amd/build.py "
                "(or __graft_entry__.build()) first -- there is no fallback path")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def status_string(rc):
    return lib().spec_status_string(int(rc)).decode()
