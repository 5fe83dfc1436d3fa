// Candidate-tree construction and depth-position rotary embedding for gfx950
// (MEDUSA section of the blog page "Fast Inference from Transformers via
// Speculative Decoding": the candidates are the Cartesian product of the
// heads' top predictions, arranged as a tree, and positions follow tree
// depth).
#include "spec_common.h"
#include "spec_internal.h"

namespace specv {

static_assert(kTreeMaxNodes == kMaxNodes, "tree arguments sized for the node limit");

// ---------------------------------------------------------------------------
// Cartesian-product tree.  Level d (d = 1..K) holds prod_{k<=d} s_k nodes
// starting at off[d]; node off[d] + f*s_d + c is child c of the f-th node of
// level d-1 and carries head d's candidate of rank c.  One wavefront per
// request, one lane per node.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void medusa_tree(MedusaTreeArgs a) {
    const int b = blockIdx.x, i = threadIdx.x;
    if (i >= a.N) return;
    const size_t o = static_cast<size_t>(b) * a.N + i;
    if (i == 0) {
        a.parent[o] = -1;
        a.tokens[o] = a.root[b];
        return;
    }
    int d = 1;
    while (d < a.K && i >= a.off[d + 1]) ++d;
    const int s = a.widths[d - 1];
    const int j = i - a.off[d];
    const int f = j / s, c = j - f * s;
    a.parent[o] = (d == 1 ? 0 : a.off[d - 1]) + f;
    a.tokens[o] = a.head[(static_cast<size_t>(b) * a.K + (d - 1)) * a.W + c];
}

int launch_medusa_tree(const MedusaTreeArgs& a, int B, hipStream_t stream) {
    hipLaunchKernelGGL(medusa_tree, dim3(B), dim3(64), 0, stream, a);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

// ---------------------------------------------------------------------------
// Rotary embedding at pos = L_b + depth(i), in place.  One workgroup per
// (request, node); a thread owns pair j of every row it visits (q heads,
// then kv heads' tree rows), so its angle is computed once.  Depths come
// from root-path masks built by pointer doubling over the parent array in
// one wavefront.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ double rope_load(const T* p, size_t i);
template <>
__device__ __forceinline__ double rope_load<float>(const float* p, size_t i) {
    return p[i];
}
template <>
__device__ __forceinline__ double rope_load<uint16_t>(const uint16_t* p, size_t i) {
    return bf16_bits_to_f32(p[i]);
}
template <typename T>
__device__ __forceinline__ void rope_store(T* p, size_t i, double v);
template <>
__device__ __forceinline__ void rope_store<float>(float* p, size_t i, double v) {
    p[i] = static_cast<float>(v);
}
template <>
__device__ __forceinline__ void rope_store<uint16_t>(uint16_t* p, size_t i, double v) {
    p[i] = static_cast<uint16_t>(f32_to_bf16_bits(static_cast<float>(v)));
}

template <typename T>
__global__ __launch_bounds__(256) void tree_rope(TreeRopeArgs a) {
    __shared__ int s_depth;
    const int b = blockIdx.x / a.N, i = blockIdx.x % a.N;
    const int tid = threadIdx.x;
    const int L = a.prefix_len[b];
    if (L < 0 || L + a.N > a.cap) return;  // outside the contract: untouched
    if (tid < 64) {
        const int lane = tid;
        const int me = lane < a.N ? lane : 0;
        int up = tree_parent(a.parent, a.N, b, me);
        uint64_t anc = 1ull << me;
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            const int src = up >= 0 ? up : 0;
            const uint32_t lo = __shfl(static_cast<uint32_t>(anc), src), hi = __shfl(static_cast<uint32_t>(anc >> 32), src);
            const int upup = __shfl(up, src);
            if (up >= 0) {
                anc |= static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
                up = upup;
            }
        }
        if (lane == i) s_depth = __popcll(anc) - 1;
    }
    __syncthreads();
    const int half = a.D / 2;
    const int j = tid % half;
    const double pos = static_cast<double>(L) + s_depth;
    const double theta = pos * exp2(-2.0 * j / a.D * a.log2_base);
    double sn, cs;
    sincos(theta, &sn, &cs);
    T* q = static_cast<T*>(a.q);
    T* k = static_cast<T*>(a.k);
    const int rows = a.Hq + a.Hkv, step = 256 / half, r0 = tid / half;
    if (r0 >= rows) return;
    const int nr = (rows - r0 + step - 1) / step;  // rows of this thread: r0, r0 + step, ...
    // Rounds of kRopeBatch rows: every load of a round issued before its
    // first store (rows never overlap, so no store feeds a later load).
    constexpr int kRopeBatch = 8;
    for (int it0 = 0; it0 < nr; it0 += kRopeBatch) {
        T* ptr[kRopeBatch];
        double x[kRopeBatch], y[kRopeBatch];
#pragma unroll
        for (int u = 0; u < kRopeBatch; ++u) {
            const int r = r0 + min(it0 + u, nr - 1) * step;  // past the end: this thread's last row, reloaded
            T* p = r < a.Hq ? q + ((static_cast<size_t>(b) * a.N + i) * a.Hq + r) * a.D
                            : k + ((static_cast<size_t>(b) * a.Hkv + (r - a.Hq)) * a.cap + L + i) * a.D;
            ptr[u] = p;
            x[u] = rope_load(p, j);
            y[u] = rope_load(p, j + half);
        }
#pragma unroll
        for (int u = 0; u < kRopeBatch; ++u) {
            if (it0 + u < nr) {
                rope_store(ptr[u], j, x[u] * cs - y[u] * sn);
                rope_store(ptr[u], j + half, x[u] * sn + y[u] * cs);
            }
        }
    }
}

int launch_tree_rope(const TreeRopeArgs& a, int B, bool bf16, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(B) * a.N);
    if (bf16)
        hipLaunchKernelGGL(tree_rope<uint16_t>, grid, dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(tree_rope<float>, grid, dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // namespace specv
