"""GPU parity of linear-attention verification and its factor commit (SpecLA
paragraphs of the summary "SpecLA: Efficient Speculative Decoding for
Linear-Attention Models"; recurrence S_t = alpha_t S_{t-1} + v_t k_t^T,
o_t = S_t q_t), through the C ABI, against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import speculative_decoding_verification_tree_amd as sv
from workloads.gen import bf16_bits, bf16_to_f32
from tests.gpu_helpers import announce

pytestmark = pytest.mark.gpu


def _case(seed, B, N, H, Dk, Dv, dtype, tree, decay):
    rng = np.random.default_rng(seed)
    S = (rng.standard_normal((B, H, Dv, Dk)) / np.sqrt(Dk)).astype(np.float32)
    q = (rng.standard_normal((B, N, H, Dk)) / np.sqrt(Dk)).astype(np.float32)
    k = rng.standard_normal((B, N, H, Dk)).astype(np.float32)
    v = rng.standard_normal((B, N, H, Dv)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = bf16_bits(q), bf16_bits(k), bf16_bits(v)
    al = rng.uniform(0.6, 1.0, (B, N, H)).astype(np.float32) if decay else None
    par = None
    if tree:
        par = np.full((B, N), -1, np.int32)
        for b in range(B):
            for i in range(1, N):
                par[b, i] = rng.integers(i)
    return S, q, k, v, al, par


def _dev(x, dtype=None):
    if x is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _check(got, ref, dtype, what):
    rms = np.sqrt(np.mean(ref ** 2)) + 1e-30
    rel = 2.0 ** -8 if dtype == "bf16" else 1e-5
    err = np.abs(got - ref)
    bound = rel * np.abs(ref) + 1e-4 * rms
    assert (err <= bound).all(), f"{what}: max err {err.max():.3e}, worst ratio {(err / bound).max():.2f}"


def _random_paths(rng, par, B, N):
    path = np.full((B, N), -1, np.int32)
    acc = np.zeros(B, np.int32)
    for b in range(B):
        i = int(rng.integers(N))
        rp = []
        while i >= 0:
            rp.append(i)
            i = -1 if par is None and i == 0 else (i - 1 if par is None else int(par[b, i]))
        rp = rp[::-1]
        path[b, :len(rp)] = rp
        acc[b] = len(rp) - 1
    return path, acc


CASES = [
    (3, 6, 4, 128, 128, "f32", False, True),
    (3, 64, 4, 128, 128, "f32", True, True),
    (2, 33, 3, 64, 128, "f32", True, False),
    (2, 20, 2, 128, 64, "bf16", True, True),
    (4, 8, 8, 64, 64, "bf16", False, True),
    (1, 1, 2, 128, 128, "f32", False, True),
    # 512 (request, head) pairs and more: one workgroup per pair, the whole state
    (64, 8, 8, 128, 128, "bf16", False, True),
    (32, 20, 16, 64, 64, "f32", True, True),
    # about a hundred pairs of a large tree: on a 256-CU device, slices of 64
    # state rows (32-row slices would not all run at once)
    (8, 46, 12, 128, 128, "bf16", True, True),
    (8, 46, 12, 128, 128, "f32", True, False),
    # 512 pairs of 24-node trees: the whole state per workgroup, the large-tree instance
    (32, 24, 16, 128, 128, "bf16", True, True),
]


@pytest.mark.parametrize("B,N,H,Dk,Dv,dtype,tree,decay", CASES)
def test_la_verify_and_commit_match_oracle(B, N, H, Dk, Dv, dtype, tree, decay):
    announce(f"linear attention B={B} N={N} H={H} Dk={Dk} Dv={Dv} {dtype} tree={tree} decay={decay}")
    S, q, k, v, al, par = _case(B * 100 + N, B, N, H, Dk, Dv, dtype, tree, decay)
    st = _dev(S)
    out = sv.spec_la_verify(st, _dev(q, dtype), _dev(k, dtype), _dev(v, dtype), _dev(al), _dev(par))
    torch.cuda.synchronize()
    ref = oracle.la_verify(S, q, k, v, al, par, dtype)
    _check(out.float().cpu().numpy().astype(np.float64), ref, dtype, "verify")
    np.testing.assert_array_equal(st.cpu().numpy(), S)  # verification alone leaves the state unchanged
    # commit of a random accepted root path
    path, acc = _random_paths(np.random.default_rng(N), par, B, N)
    sv.spec_la_commit(st, _dev(k, dtype), _dev(v, dtype), _dev(al), _dev(par), _dev(path), _dev(acc))
    torch.cuda.synchronize()
    want = oracle.la_commit(S, k, v, al, par, path, acc, dtype).astype(np.float64)
    rms = np.sqrt(np.mean(want ** 2))
    err = np.abs(st.cpu().numpy().astype(np.float64) - want)
    assert (err <= 1e-5 * np.abs(want) + 1e-5 * rms).all(), err.max()


@pytest.mark.parametrize("B,H,Np,Nv", [
    (3, 4, 24, 24),
    (3, 4, 64, 8),   # a large committed tree before a small verified one
    (3, 4, 8, 8),    # both within the small-tree launch
    (2, 4, 16, 40),
    (64, 8, 8, 8),   # one workgroup per (head, request), the whole state
    (64, 8, 24, 20),  # the same with the large-tree instance
])
def test_la_deferred_commit_equals_commit_then_verify(B, H, Np, Nv):
    announce(f"linear attention: deferred commit folded into the next verification B={B} H={H} "
             f"committed tree {Np} verified tree {Nv}")
    Dk, Dv = 128, 128
    S, q, k, v, al, par = _case(5, B, Np, H, Dk, Dv, "f32", True, True)
    _, q2, k2, v2, al2, par2 = _case(6, B, Nv, H, Dk, Dv, "f32", True, True)
    path, acc = _random_paths(np.random.default_rng(1), par, B, Np)
    f = (_dev(k), _dev(v), _dev(al), _dev(par), _dev(path), _dev(acc))
    # two launches
    s1 = _dev(S)
    sv.spec_la_commit(s1, *f)
    o1 = sv.spec_la_verify(s1, _dev(q2), _dev(k2), _dev(v2), _dev(al2), _dev(par2))
    # one launch
    s2 = _dev(S)
    o2 = sv.spec_la_verify(s2, _dev(q2), _dev(k2), _dev(v2), _dev(al2), _dev(par2), pending=f)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(s2.cpu().numpy(), s1.cpu().numpy())
    np.testing.assert_array_equal(o2.cpu().numpy(), o1.cpu().numpy())
    # and both against the oracle
    S1 = oracle.la_commit(S, k, v, al, par, path, acc, "f32")
    _check(o1.cpu().numpy().astype(np.float64), oracle.la_verify(S1, q2, k2, v2, al2, par2, "f32"), "f32", "deferred")


def test_la_chain_parent_array_equals_null():
    B, N, H = 2, 7, 2
    S, q, k, v, al, _ = _case(8, B, N, H, 128, 128, "f32", False, True)
    chain = np.tile(np.arange(-1, N - 1, dtype=np.int32), (B, 1))
    a = sv.spec_la_verify(_dev(S), _dev(q), _dev(k), _dev(v), _dev(al), None)
    b = sv.spec_la_verify(_dev(S), _dev(q), _dev(k), _dev(v), _dev(al), _dev(chain))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(a.cpu().numpy(), b.cpu().numpy())


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_la_rows_not_16_byte_aligned(dtype):
    """q, k and v starting off a 16-byte boundary take the element-wise loads; the
    values reaching the arithmetic are the same, so the results are bit-identical."""
    B, N, H, Dk, Dv = 3, 20, 4, 128, 128
    announce(f"linear attention: rows off a 16-byte boundary ({dtype})")
    S, q, k, v, al, par = _case(11, B, N, H, Dk, Dv, dtype, True, True)

    def shifted(x):
        t = _dev(x, dtype)
        flat = t.reshape(-1)
        buf = torch.empty(flat.numel() + 1, dtype=t.dtype, device=t.device)
        buf[1:] = flat
        out = buf[1:].view(t.shape)
        assert out.data_ptr() % 16 != 0
        return out

    path, acc = _random_paths(np.random.default_rng(3), par, B, N)
    outs, states = [], []
    for make in (lambda x: _dev(x, dtype), shifted):
        st = _dev(S)
        f = (make(k), make(v), _dev(al), _dev(par), _dev(path), _dev(acc))
        o = sv.spec_la_verify(st, make(q), make(k), make(v), _dev(al), _dev(par), pending=f)
        torch.cuda.synchronize()
        outs.append(o.float().cpu().numpy())
        states.append(st.cpu().numpy())
    np.testing.assert_array_equal(outs[1], outs[0])
    np.testing.assert_array_equal(states[1], states[0])
