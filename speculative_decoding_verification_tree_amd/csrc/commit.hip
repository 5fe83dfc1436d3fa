// KV commit of the accepted path, depth positions and the parent-array check.
//
// Commit: the speculative-decoding loop keeps the accepted drafts and drops
// the rest ("Speculative Decoding" section of the blog page "Fast Inference
// from Transformers via Speculative Decoding").  In cache terms the rows
// L_b + path[d] (d = 0..a) move to L_b + d and the verified prefix grows by
// a + 1 (the root and the a accepted drafts).
//
// In-place safety: path is strictly increasing with path[d] >= d, so for
// d' > d the source L_b + path[d'] lies above the destination L_b + d: no
// source is ever a destination of a smaller d.  One workgroup per request;
// a thread owns 16-byte columns of the (kv head, K-or-V) slabs and takes
// each column's moves d = 1..a in ascending batches, every load of a batch
// issued before its first store (the loads of a batch are in flight
// together instead of one dependent round trip per row; a batch past d = a
// re-reads row a, never stored).  Columns never overlap between threads.  A
// chain (path[d] == d) moves nothing.
#include <algorithm>

#include "spec_common.h"
#include "spec_internal.h"

namespace specv {

constexpr int kCommitThreads = 1024;
constexpr int kCommitBatch = 8;

__global__ __launch_bounds__(kCommitThreads) void commit_kv(void* k, void* v, int32_t* prefix_len, const int32_t* path,
                                                            const int32_t* accept_len, int N, int Hkv, int cap,
                                                            int row_bytes) {
    const int b = blockIdx.x;
    const int L = prefix_len[b];
    const int acount = accept_len[b];
    __shared__ int s_src[kMaxNodes];
    __shared__ int s_nmove;
    if (!(L >= 0 && L + N <= cap && acount >= 0 && acount < N)) return;  // uniform across the workgroup
    if (threadIdx.x == 0) s_nmove = 0;
    __syncthreads();
    if (threadIdx.x <= acount) {
        const int p = path[static_cast<size_t>(b) * N + threadIdx.x];
        const int src = (p >= 0 && p < N) ? p : static_cast<int>(threadIdx.x);
        s_src[threadIdx.x] = src;
        if (src != static_cast<int>(threadIdx.x)) atomicAdd(&s_nmove, 1);
    }
    __syncthreads();
    if (s_nmove > 0) {
        const int cols = row_bytes / 16;
        const int total = 2 * Hkv * cols;
        for (int col = threadIdx.x; col < total; col += blockDim.x) {
            const int which = col / (Hkv * cols);
            const int g = (col / cols) % Hkv;
            unsigned char* base = static_cast<unsigned char*>(which ? v : k) +
                                  (static_cast<size_t>(b) * Hkv + g) * cap * static_cast<size_t>(row_bytes) +
                                  (col % cols) * 16;
            for (int d0 = 1; d0 <= acount; d0 += kCommitBatch) {
                u32x4 x[kCommitBatch];
#pragma unroll
                for (int j = 0; j < kCommitBatch; ++j) {
                    const int d = min(d0 + j, acount);
                    x[j] = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(L + s_src[d]) * row_bytes);
                }
#pragma unroll
                for (int j = 0; j < kCommitBatch; ++j) {
                    const int d = d0 + j;
                    if (d <= acount && s_src[d] != d)
                        *reinterpret_cast<u32x4*>(base + static_cast<size_t>(L + d) * row_bytes) = x[j];
                }
            }
        }
    }
    __syncthreads();  // every thread has read L before it changes
    if (threadIdx.x == 0) prefix_len[b] = L + acount + 1;
}

// The commit of a fused-RoPE step: the accepted path's K rows are written
// rotated at their new positions L + d (every d = 0..a, moved or not), V rows
// moved as above.  A thread owns the pair of 16-byte K columns D/2 apart
// that hold its rotary pairs (or one V column), and takes the rows d = 0..a
// in ascending batches with every load of a batch before its first store:
// the sources L + path[d'] of later rows lie above every destination written.
template <typename T>
__global__ __launch_bounds__(kCommitThreads) void commit_kv_rope(T* k, T* v, int32_t* prefix_len, const int32_t* path,
                                                                 const int32_t* accept_len, int N, int Hkv, int cap,
                                                                 int D, RopeTable tab) {
    constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte column
    const int b = blockIdx.x;
    const int L = prefix_len[b];
    const int acount = accept_len[b];
    __shared__ int s_src[kMaxNodes];
    __shared__ double s_rev[kRopeMaxPairs];
    if (!(L >= 0 && L + N <= cap && acount >= 0 && acount < N)) return;  // uniform across the workgroup
    if (threadIdx.x <= acount) {
        const int p = path[static_cast<size_t>(b) * N + threadIdx.x];
        s_src[threadIdx.x] = (p >= 0 && p < N) ? p : static_cast<int>(threadIdx.x);
    }
    if (threadIdx.x < kRopeMaxPairs) {
        double r = 0.0;
#pragma unroll
        for (int j = 0; j < kRopeMaxPairs; ++j) r = static_cast<int>(threadIdx.x) == j ? tab.rev[j] : r;
        s_rev[threadIdx.x] = r;
    }
    __syncthreads();
    const int cols = D / EPC, half = cols / 2;
    const int ktasks = Hkv * half, total = ktasks + Hkv * cols;
    for (int task = threadIdx.x; task < total; task += blockDim.x) {
        if (task < ktasks) {
            const int g = task / half, c = task % half;
            T* base = k + (static_cast<size_t>(b) * Hkv + g) * cap * static_cast<size_t>(D);
            for (int d0 = 0; d0 <= acount; d0 += kCommitBatch) {
                u32x4 lo[kCommitBatch], hi[kCommitBatch];
#pragma unroll
                for (int j = 0; j < kCommitBatch; ++j) {
                    const size_t row = static_cast<size_t>(L + s_src[min(d0 + j, acount)]) * D;
                    lo[j] = *reinterpret_cast<const u32x4*>(base + row + c * EPC);
                    hi[j] = *reinterpret_cast<const u32x4*>(base + row + c * EPC + D / 2);
                }
#pragma unroll
                for (int j = 0; j < kCommitBatch; ++j) {
                    const int d = d0 + j;
                    if (d <= acount) {
                        if constexpr (sizeof(T) == 2) rope_bf16x8(lo[j], hi[j], L + d, s_rev, c * EPC);
                        else rope_f32x4(lo[j], hi[j], L + d, s_rev, c * EPC);
                        const size_t row = static_cast<size_t>(L + d) * D;
                        *reinterpret_cast<u32x4*>(base + row + c * EPC) = lo[j];
                        *reinterpret_cast<u32x4*>(base + row + c * EPC + D / 2) = hi[j];
                    }
                }
            }
        } else {
            const int vt = task - ktasks;
            const int g = vt / cols, c = vt % cols;
            T* base = v + (static_cast<size_t>(b) * Hkv + g) * cap * static_cast<size_t>(D) + c * EPC;
            for (int d0 = 1; d0 <= acount; d0 += kCommitBatch) {
                u32x4 x[kCommitBatch];
#pragma unroll
                for (int j = 0; j < kCommitBatch; ++j)
                    x[j] = *reinterpret_cast<const u32x4*>(base + static_cast<size_t>(L + s_src[min(d0 + j, acount)]) * D);
#pragma unroll
                for (int j = 0; j < kCommitBatch; ++j) {
                    const int d = d0 + j;
                    if (d <= acount && s_src[d] != d) *reinterpret_cast<u32x4*>(base + static_cast<size_t>(L + d) * D) = x[j];
                }
            }
        }
    }
    __syncthreads();  // every thread has read L before it changes
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
    if (d.rope_base > 0.f) {
        RopeTable tab;
        fill_rope_table(tab, d.head_dim, d.rope_base);
        const int cols = d.head_dim * es / 16;
        const long tasks = static_cast<long>(d.num_kv_heads) * (cols / 2 + cols);
        const int threads = static_cast<int>(std::min<long>(kCommitThreads, std::max<long>(64, (tasks + 63) / 64 * 64)));
        if (d.dtype == SPEC_BF16)
            hipLaunchKernelGGL(commit_kv_rope<uint16_t>, dim3(d.batch), dim3(threads), 0, stream, static_cast<uint16_t*>(k),
                               static_cast<uint16_t*>(v), prefix_len, path, accept_len, d.num_nodes, d.num_kv_heads,
                               d.kv_capacity, d.head_dim, tab);
        else
            hipLaunchKernelGGL(commit_kv_rope<float>, dim3(d.batch), dim3(threads), 0, stream, static_cast<float*>(k),
                               static_cast<float*>(v), prefix_len, path, accept_len, d.num_nodes, d.num_kv_heads,
                               d.kv_capacity, d.head_dim, tab);
        return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
    }
    // One thread per 16-byte column of the request's slabs, up to 1024.
    const long cols = 2L * d.num_kv_heads * (d.head_dim * es / 16);
    const int threads = static_cast<int>(std::min<long>(kCommitThreads, std::max<long>(64, (cols + 63) / 64 * 64)));
    hipLaunchKernelGGL(commit_kv, dim3(d.batch), dim3(threads), 0, stream, k, v, prefix_len, path, accept_len,
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
