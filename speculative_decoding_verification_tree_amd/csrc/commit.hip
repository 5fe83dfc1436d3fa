// KV commit of the accepted path, depth positions and the parent-array check.
//
// Commit: the speculative-decoding loop keeps the accepted drafts and drops
// the rest ("Speculative Decoding" section of the blog page "Fast Inference
// from Transformers via Speculative Decoding").  In cache terms the rows
// L_b + path[d] (d = 0..a) move to L_b + d and the verified prefix grows by
// a + 1 (the root and the a accepted drafts).
//
// In-place safety: path is strictly increasing with path[d] >= d, so for
// d' > d the source L_b + path[d'] lies above the destination L_b + d.  One
// thread owns one 16-byte column of every row of a (request, kv head,
// K-or-V) slab and walks d upwards, reading each source before the write that
// could cover it; columns never overlap between threads.  A chain
// (path[d] == d) moves nothing.
#include "spec_common.h"
#include "spec_internal.h"

namespace specv {

__global__ __launch_bounds__(256) void commit_kv(void* k, void* v, int32_t* prefix_len, const int32_t* path,
                                                 const int32_t* accept_len, int N, int Hkv, int cap,
                                                 int row_bytes) {
    const int b = blockIdx.x;
    const int L = prefix_len[b];
    int acount = accept_len[b];
    __shared__ int s_src[kMaxNodes];
    __shared__ int s_ok;
    if (threadIdx.x == 0) {
        s_ok = (L >= 0 && L + N <= cap && acount >= 0 && acount < N) ? 1 : 0;
    }
    __syncthreads();
    if (!s_ok) return;
    if (threadIdx.x <= acount) {
        int p = path[static_cast<size_t>(b) * N + threadIdx.x];
        s_src[threadIdx.x] = (p >= 0 && p < N) ? p : static_cast<int>(threadIdx.x);
    }
    __syncthreads();
    const int cols = row_bytes / 16;
    const int total = 2 * Hkv * cols;
    for (int col = threadIdx.x; col < total; col += blockDim.x) {
        const int which = col / (Hkv * cols);
        const int g = (col / cols) % Hkv;
        const int cc = col % cols;
        unsigned char* base = static_cast<unsigned char*>(which ? v : k) +
                              (static_cast<size_t>(b) * Hkv + g) * cap * static_cast<size_t>(row_bytes) + cc * 16;
        for (int d = 1; d <= acount; ++d) {
            const int s = s_src[d];
            if (s == d) continue;
            const u32x4 x = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(L + s) * row_bytes);
            *reinterpret_cast<u32x4*>(base + static_cast<size_t>(L + d) * row_bytes) = x;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) prefix_len[b] = L + acount + 1;
}

__global__ __launch_bounds__(64) void tree_positions(const int32_t* prefix_len, const int32_t* parent, int N,
                                                     int32_t* pos) {
    const int b = blockIdx.x, i = threadIdx.x;
    if (i >= N) return;
    int depth = 0;
    for (int n = i; n > 0 && depth < kMaxNodes;) {
        n = tree_parent(parent, N, b, n);
        if (n < 0) break;
        ++depth;
    }
    pos[static_cast<size_t>(b) * N + i] = prefix_len[b] + depth;
}

__global__ __launch_bounds__(64) void validate_tree(const int32_t* parent, int N, int32_t* status) {
    const int b = blockIdx.x, i = threadIdx.x;
    bool bad = false;
    if (i < N) {
        const int p = parent[static_cast<size_t>(b) * N + i];
        bad = i == 0 ? p != -1 : (p < 0 || p >= i);
    }
    const unsigned long long m = __ballot(bad);
    if (i == 0) status[b] = m ? __ffsll(static_cast<long long>(m)) : 0;  // 1 + first bad node
}

int launch_commit(const spec_attn_desc& d, void* k, void* v, int32_t* prefix_len, const int32_t* path,
                  const int32_t* accept_len, hipStream_t stream) {
    const int es = d.dtype == SPEC_BF16 ? 2 : 4;
    hipLaunchKernelGGL(commit_kv, dim3(d.batch), dim3(256), 0, stream, k, v, prefix_len, path, accept_len,
                       d.num_nodes, d.num_kv_heads, d.kv_capacity, d.head_dim * es);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

int launch_positions(int B, int N, const int32_t* prefix_len, const int32_t* parent, int32_t* pos,
                     hipStream_t stream) {
    hipLaunchKernelGGL(tree_positions, dim3(B), dim3(64), 0, stream, prefix_len, parent, N, pos);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

int launch_validate(int B, int N, const int32_t* parent, int32_t* status, hipStream_t stream) {
    hipLaunchKernelGGL(validate_tree, dim3(B), dim3(64), 0, stream, parent, N, status);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // namespace specv
