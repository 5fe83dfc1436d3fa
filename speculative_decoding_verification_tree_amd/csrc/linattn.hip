// Linear-attention verification and state commit for gfx950 (SpecLA
// paragraphs of the summary "SpecLA: Efficient Speculative Decoding for
// Linear-Attention Models": drafts are verified against the recurrent summary
// state kept on chip, branches under a tree mask, and the state is recovered
// afterwards from the accepted tokens' compact factors, the final update
// deferred to the next step).  Recurrence (a reading; the summary gives
// none): S_t = alpha_t S_{t-1} + v_t k_t^T, o_t = S_t q_t, per (request,
// head), S [Dv][Dk] fp32.
//
// One 256-thread workgroup per (head, request, slice of state rows): the
// rows e of S (the output dims) are independent in both phases, so when
// (head, request) pairs are too few to fill the chip a pair is spread over
// Dv / 32 workgroups, each recomputing the small N x N score matrix.  Two
// optional phases:
//   commit: S <- A(-> v] S + sum_{j on the accepted path} A(j -> v] v_j k_j^T,
//           the path's k, v and decay weights in LDS, every state element
//           written once (in place; the workgroup owns its slab);
//   verify: o_i = A(-> i] S q_i + sum_{j in anc(i)} A(j -> i] (q_i . k_j) v_j
//           with Q, K, V in LDS, the N x N decayed, masked scores in LDS and
//           the state streamed through LDS in 32-column chunks.
// Both phases in one launch are the deferred update: the previous step's
// commit folded into this step's verification (one state read and write).
// Decay products are exp2 of differences of log2 prefix sums along root paths.
#include "spec_common.h"
#include "spec_internal.h"

namespace specv {

constexpr int kLaThreads = 256;
constexpr int kLaMaxD = 128;
constexpr int kLaChunk = 32;
// State rows (output dims) per workgroup: a slice of 32 when (head, request)
// pairs are few, else the whole state (kLaMaxD).
constexpr int kLaSliceRows = 32;

// Rows [0, rows) of `cols` elements (bf16 or fp32, row t at global element
// offset row_off(t)) into LDS dst[t * ldst + c], in rounds of kLaBatch
// elements per thread: every load of a round issued before its first LDS
// store (a load followed by its store in one loop body costs one round trip
// per element).
constexpr int kLaBatch = 8;

template <class RowOff>
__device__ __forceinline__ void la_rows_to_lds(const void* src, bool bf16, int rows, int cols, RowOff row_off, float* dst,
                                               int ldst) {
    const int tid = threadIdx.x, n = rows * cols;
    for (int base = 0; base < n; base += kLaBatch * kLaThreads) {
        float v[kLaBatch];
        if (bf16) {
#pragma unroll
            for (int j = 0; j < kLaBatch; ++j) {
                const int x = min(base + tid + j * kLaThreads, n - 1), t = x / cols;
                v[j] = __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(src)[row_off(t) + (x - t * cols)])
                                       << 16);
            }
        } else {
#pragma unroll
            for (int j = 0; j < kLaBatch; ++j) {
                const int x = min(base + tid + j * kLaThreads, n - 1), t = x / cols;
                v[j] = static_cast<const float*>(src)[row_off(t) + (x - t * cols)];
            }
        }
#pragma unroll
        for (int j = 0; j < kLaBatch; ++j) {
            const int x = base + tid + j * kLaThreads;
            if (x < n) {
                const int t = x / cols;
                dst[t * ldst + (x - t * cols)] = v[j];
            }
        }
    }
}

// Root-path structure of request b's tree of N nodes: L[i] = log2 of the
// decay product over the path root .. i, anc[i] = the path's node mask.
// One lane per node (wave 0) and pointer doubling: after round r a lane
// holds the sum and mask over its 2^r nearest path nodes and the node 2^r
// above it, so six rounds cover 64 levels (a walk from the root would be
// one dependent LDS round trip per node).
__device__ __forceinline__ void la_tree(const int32_t* parent, const float* alpha, int b, int N, int H, int h,
                                        float* s_L, uint64_t* s_anc) {
    const int i = threadIdx.x;
    if (i < 64) {
        int up = -1;
        float Ls = 0.f;
        if (i < N) {
            const int p = tree_parent(parent, N, b, i);
            up = p >= 0 && p < i ? p : -1;  // out-of-contract parents read as roots
            Ls = alpha ? __log2f(alpha[(static_cast<size_t>(b) * N + i) * H + h]) : 0.f;
        }
        uint64_t anc = 1ull << i;
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            const int u = up >= 0 ? up : i;
            const float Lu = __shfl(Ls, u);
            const uint32_t alo = __shfl(static_cast<uint32_t>(anc), u), ahi = __shfl(static_cast<uint32_t>(anc >> 32), u);
            const int uu = __shfl(up, u);
            if (up >= 0) {
                Ls += Lu;
                anc |= static_cast<uint64_t>(alo) | (static_cast<uint64_t>(ahi) << 32);
                up = uu;
            }
        }
        if (i < N) {
            s_L[i] = Ls;
            s_anc[i] = anc;
        }
    }
    __syncthreads();
}

// LDS floats for trees of at most NMAX nodes: commit (path factors k, v)
// or verify (Q and K rows padded by one, V, the scores W, a 32-column chunk
// of the state), whichever is larger.
template <int NMAX, bool COMMIT, bool VERIFY, int ROWS>
constexpr int la_lds_floats() {
    constexpr int commit = COMMIT ? NMAX * (kLaMaxD + ROWS) : 0;
    constexpr int verify = VERIFY ? 2 * NMAX * (kLaMaxD + 1) + NMAX * ROWS + NMAX * NMAX + ROWS * (kLaChunk + 1) : 0;
    return commit > verify ? commit : verify;
}

// COMMIT: the launch may commit (alone or before verifying); without it the
// LDS is sized for verification only.
template <int NMAX, bool COMMIT, bool VERIFY, int ROWS>
__global__ __launch_bounds__(kLaThreads) void la_kernel(LaArgs a) {
    constexpr int kLaRows = ROWS;
    const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int Dk = a.Dk, Dv = a.Dv, H = a.H;
    const int es0 = blockIdx.z * kLaRows, ne = min(kLaRows, Dv - es0);  // this workgroup's state rows
    const bool bf16 = a.bf16 != 0;
    __shared__ __attribute__((aligned(16))) float lds[la_lds_floats<NMAX, COMMIT, VERIFY, ROWS>()];
    __shared__ float s_L[kMaxNodes];
    __shared__ uint64_t s_anc[kMaxNodes];
    __shared__ float s_c[kMaxNodes];
    __shared__ int s_j[kMaxNodes];
    __shared__ int s_off[kMaxNodes + 1];
    float* S = a.state + (static_cast<size_t>(b) * H + h) * Dv * Dk;

    if (COMMIT && a.do_commit) {
        const int N = a.pN;
        la_tree(a.pparent, a.palpha, b, N, H, h, s_L, s_anc);
        // (device data: out-of-range entries are clamped into the tree)
        const int acc = min(max(a.pacc[b], 0), N - 1);
        const int vstop = min(max(a.ppath[static_cast<size_t>(b) * N + acc], 0), N - 1);
        if (tid <= acc) {
            const int j = min(max(a.ppath[static_cast<size_t>(b) * N + tid], 0), N - 1);
            s_j[tid] = j;
            s_c[tid] = exp2f(s_L[vstop] - s_L[j]);
        }
        __syncthreads();
        float* kf = lds;                 // [acc + 1][Dk]
        float* vf = lds + (acc + 1) * Dk;  // [acc + 1][ne]: this slice's dims of v
        la_rows_to_lds(a.pk, bf16, acc + 1, Dk,
                              [&](int t) { return ((static_cast<size_t>(b) * N + s_j[t]) * H + h) * Dk; }, kf, Dk);
        la_rows_to_lds(a.pv, bf16, acc + 1, ne,
                              [&](int t) { return ((static_cast<size_t>(b) * N + s_j[t]) * H + h) * Dv + es0; }, vf,
                              ne);
        __syncthreads();
        // This thread's four columns d4 .. d4 + 3 of slice rows e0, e0 + estep,
        // ...: 16-byte loads, every one issued before the first update (rows
        // past the slice read its last row and are not stored).  The path's
        // terms then go in order t = 0 .. acc, each k row's four values read
        // once for all of the thread's rows.
        const float Av = exp2f(s_L[vstop]);
        const int tpr = Dk / 4, d4 = 4 * (tid % tpr), e0 = tid / tpr, estep = kLaThreads / tpr;
        constexpr int kRows4 = kLaRows * kLaMaxD / 4 / kLaThreads;  // row slots a thread may hold
        float4 sv[kRows4];
#pragma unroll
        for (int r = 0; r < kRows4; ++r) {
            const int e = min(e0 + r * estep, ne - 1);
            sv[r] = *reinterpret_cast<const float4*>(S + static_cast<size_t>(es0 + e) * Dk + d4);
        }
#pragma unroll
        for (int r = 0; r < kRows4; ++r) {
            sv[r].x *= Av;
            sv[r].y *= Av;
            sv[r].z *= Av;
            sv[r].w *= Av;
        }
        for (int t = 0; t <= acc; ++t) {
            const float4 k4 = *reinterpret_cast<const float4*>(kf + t * Dk + d4);
            const float ct = s_c[t];
#pragma unroll
            for (int r = 0; r < kRows4; ++r) {
                const float w = ct * vf[t * ne + min(e0 + r * estep, ne - 1)];
                sv[r].x = fmaf(w, k4.x, sv[r].x);
                sv[r].y = fmaf(w, k4.y, sv[r].y);
                sv[r].z = fmaf(w, k4.z, sv[r].z);
                sv[r].w = fmaf(w, k4.w, sv[r].w);
            }
        }
#pragma unroll
        for (int r = 0; r < kRows4; ++r) {
            const int e = e0 + r * estep;
            if (e < ne) *reinterpret_cast<float4*>(S + static_cast<size_t>(es0 + e) * Dk + d4) = sv[r];
        }
        __syncthreads();  // the workgroup's own state writes before its reads below
    }
    if (!VERIFY || !a.do_verify) return;

    const int N = a.N;
    la_tree(a.parent, a.alpha, b, N, H, h, s_L, s_anc);
    const int DkP = Dk + 1;               // padded rows: lanes on different rows hit different banks
    float* Qs = lds;                      // [N][Dk + 1]
    float* Ks = Qs + NMAX * (kLaMaxD + 1);
    float* Vs = Ks + NMAX * (kLaMaxD + 1);  // [N][ne]: this slice's dims of v
    float* W = Vs + NMAX * kLaRows;         // [N][N]
    float* Sc = W + NMAX * NMAX;            // [ne][kLaChunk + 1]
    {
        auto rk = [&](int i) { return ((static_cast<size_t>(b) * N + i) * H + h) * Dk; };
        auto rv = [&](int i) { return ((static_cast<size_t>(b) * N + i) * H + h) * Dv + es0; };
        la_rows_to_lds(a.q, bf16, N, Dk, rk, Qs, DkP);
        la_rows_to_lds(a.k, bf16, N, Dk, rk, Ks, DkP);
        la_rows_to_lds(a.v, bf16, N, ne, rv, Vs, ne);
    }
    __syncthreads();
    // W[i][j] = A(j -> i] (q_i . k_j) for j on i's root path (the other
    // entries are never read).  The (node, ancestor) pairs are numbered
    // node by node, s_off[i] the first pair of node i, and dealt out one per
    // thread: a tree has far fewer pairs than N * N entries.
    if (tid < 64) {
        int v = tid < N ? __popcll(s_anc[tid]) : 0;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int t = __shfl_up(v, o);
            if (tid >= o) v += t;
        }
        s_off[tid + 1] = v;
        if (tid == 0) s_off[0] = 0;
    }
    __syncthreads();
    for (int pr = tid; pr < s_off[N]; pr += kLaThreads) {
        int lo = 0, hi = N - 1;  // node i: the last with s_off[i] <= pr
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_off[mid] <= pr) lo = mid;
            else hi = mid - 1;
        }
        const int i = lo;
        uint64_t m = s_anc[i];
        for (int r = pr - s_off[i]; r > 0; --r) m &= m - 1ull;  // drop the lower ancestors
        const int j = __ffsll(static_cast<long long>(m)) - 1;
        // four independent partial sums, eight LDS reads per round in
        // flight (one wave per SIMD here: a single dependent chain waited
        // out every read's latency)
        float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
        const float* qi = Qs + i * DkP;
        const float* kj = Ks + j * DkP;
#pragma unroll 4
        for (int d = 0; d < Dk; d += 4) {
            d0 = fmaf(qi[d], kj[d], d0);
            d1 = fmaf(qi[d + 1], kj[d + 1], d1);
            d2 = fmaf(qi[d + 2], kj[d + 2], d2);
            d3 = fmaf(qi[d + 3], kj[d + 3], d3);
        }
        W[i * N + j] = exp2f(s_L[i] - s_L[j]) * ((d0 + d1) + (d2 + d3));
    }
    // Thread (e, group g): slice row e, nodes g, g + G, ... with G = 256 /
    // kLaRows groups (threads of rows past ne idle).
    const int e = tid % kLaRows, g = tid / kLaRows, G = kLaThreads / kLaRows;
    constexpr int kPer = NMAX / (kLaThreads / kLaRows) > 1 ? NMAX / (kLaThreads / kLaRows) : 1;  // nodes per thread
    float acc[kPer];
#pragma unroll
    for (int n = 0; n < kPer; ++n) acc[n] = 0.f;
    // The slice's 32-column chunks of the state as 16-byte loads (one per
    // thread), the next chunk loaded while the current one is used.
    constexpr int kS4 = (kLaRows * kLaChunk / 4 + kLaThreads - 1) / kLaThreads;
    const int n4 = ne * (kLaChunk / 4);
    float4 sreg[kS4];
    auto load_chunk = [&](int c0) {
#pragma unroll
        for (int j = 0; j < kS4; ++j) {
            const int x = min(tid + j * kLaThreads, n4 - 1), r = x / (kLaChunk / 4), c4 = x - r * (kLaChunk / 4);
            sreg[j] = *reinterpret_cast<const float4*>(S + static_cast<size_t>(es0 + r) * Dk + c0 + 4 * c4);
        }
    };
    load_chunk(0);
    for (int c0 = 0; c0 < Dk; c0 += kLaChunk) {
        __syncthreads();  // the previous chunk is consumed (and W is complete)
#pragma unroll
        for (int j = 0; j < kS4; ++j) {
            const int x = tid + j * kLaThreads;
            if (x < n4) {
                const int r = x / (kLaChunk / 4), c4 = x - r * (kLaChunk / 4);
                float* dst = Sc + r * (kLaChunk + 1) + 4 * c4;
                dst[0] = sreg[j].x;
                dst[1] = sreg[j].y;
                dst[2] = sreg[j].z;
                dst[3] = sreg[j].w;
            }
        }
        if (c0 + kLaChunk < Dk) load_chunk(c0 + kLaChunk);
        __syncthreads();
        if (e >= ne) {  // a row past the slice (Dv not a multiple of kLaRows): nothing to add
        } else if constexpr (NMAX > 16) {
            // Large trees, column by column: one state value feeds this
            // thread's kPer nodes as independent chains (a per-node branch
            // kept each node's 32-step chain apart, every step waiting out
            // its LDS reads).  Rows past N hold stale LDS; their sums are
            // never used.
#pragma unroll 4
            for (int cc = 0; cc < kLaChunk; ++cc) {
                const float sv = Sc[e * (kLaChunk + 1) + cc];
#pragma unroll
                for (int n = 0; n < kPer; ++n) {
                    const int i = min(g + n * G, NMAX - 1);
                    acc[n] = fmaf(sv, Qs[i * DkP + c0 + cc], acc[n]);
                }
            }
        } else {  // small trees: only the nodes that exist
#pragma unroll
            for (int n = 0; n < kPer; ++n) {
                const int i = g + n * G;
                if (i < N) {
                    float s = acc[n];
                    for (int cc = 0; cc < kLaChunk; ++cc)
                        s = fmaf(Sc[e * (kLaChunk + 1) + cc], Qs[i * DkP + c0 + cc], s);
                    acc[n] = s;
                }
            }
        }
    }
#pragma unroll
    for (int n = 0; n < kPer; ++n) {
        const int i = g + n * G;
        if (i < N && e < ne) {
            float o = exp2f(s_L[i]) * acc[n];
            for (uint64_t m = s_anc[i]; m != 0ull; m &= m - 1ull) {  // the ancestors j, ascending
                const int j = __ffsll(static_cast<long long>(m)) - 1;
                o = fmaf(W[i * N + j], Vs[j * ne + e], o);
            }
            const size_t oi = ((static_cast<size_t>(b) * N + i) * H + h) * Dv + es0 + e;
            if (bf16)
                static_cast<uint16_t*>(a.out)[oi] = static_cast<uint16_t>(f32_to_bf16_bits(o));
            else
                static_cast<float*>(a.out)[oi] = o;
        }
    }
}

template <int NMAX, int ROWS>
static void launch_la_n(const LaArgs& a, const dim3& grid, hipStream_t stream) {
    if (a.do_commit && a.do_verify)
        hipLaunchKernelGGL((la_kernel<NMAX, true, true, ROWS>), grid, dim3(kLaThreads), 0, stream, a);
    else if (a.do_commit)
        hipLaunchKernelGGL((la_kernel<NMAX, true, false, ROWS>), grid, dim3(kLaThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((la_kernel<NMAX, false, true, ROWS>), grid, dim3(kLaThreads), 0, stream, a);
}

template <int ROWS>
static void launch_la_rows(const LaArgs& a, hipStream_t stream) {
    const dim3 grid(a.H, a.B, (a.Dv + ROWS - 1) / ROWS);
    // NMAX bounds both trees: the one verified and the one whose path is
    // committed (LDS is sized for the phases the launch runs).
    const bool small = (!a.do_verify || a.N <= 16) && (!a.do_commit || a.pN <= 16);
    if (small)
        launch_la_n<16, ROWS>(a, grid, stream);
    else
        launch_la_n<kMaxNodes, ROWS>(a, grid, stream);
}

int launch_la(const LaArgs& a, hipStream_t stream) {
    // Slices only when the pairs leave most CUs idle (the slices recompute
    // the score matrix, which costs more than it spreads once the chip is
    // full: 64 requests x 16 heads ran slower sliced).
    if (static_cast<long>(a.B) * a.H < 512)
        launch_la_rows<kLaSliceRows>(a, stream);
    else if (a.Dv <= 64)
        launch_la_rows<64>(a, stream);
    else
        launch_la_rows<kLaMaxD>(a, stream);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // namespace specv
