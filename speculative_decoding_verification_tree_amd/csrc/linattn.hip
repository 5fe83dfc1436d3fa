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
#include <type_traits>

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

// The same as 16-byte pieces (8 bf16 or 4 fp32 elements; the source's row
// starts 16-byte aligned, cols a multiple of 8): every piece of the row set
// is loaded first, MAXP per thread (spare slots re-read the last piece and
// are not stored), so a row set costs one round trip and its loads can be
// issued ahead of other work.
template <bool BF, int MAXP>
struct LaPieces {
    static constexpr int EPP = BF ? 8 : 4;  // elements per piece
    u32x4 r[MAXP];
    template <class RowOff>
    __device__ __forceinline__ void load(const void* src, int rows, int cols, RowOff row_off) {
        const int ppr = cols / EPP, n = rows * ppr;
#pragma unroll
        for (int j = 0; j < MAXP; ++j) {
            const int p = min(static_cast<int>(threadIdx.x) + j * kLaThreads, n - 1), t = p / ppr;
            const size_t el = row_off(t) + static_cast<size_t>(p - t * ppr) * EPP;
            r[j] = *reinterpret_cast<const u32x4*>(static_cast<const char*>(src) + el * (BF ? 2 : 4));
        }
    }
    __device__ __forceinline__ void store(int rows, int cols, float* dst, int ldst) const {
        const int ppr = cols / EPP, n = rows * ppr;
#pragma unroll
        for (int j = 0; j < MAXP; ++j) {
            const int p = static_cast<int>(threadIdx.x) + j * kLaThreads;
            if (p < n) {
                const int t = p / ppr;
                float* d = dst + t * ldst + (p - t * ppr) * EPP;
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    if constexpr (BF) {
                        d[2 * w] = __uint_as_float(r[j][w] << 16);
                        d[2 * w + 1] = __uint_as_float(r[j][w] & 0xFFFF0000u);
                    } else {
                        d[w] = __uint_as_float(r[j][w]);
                    }
                }
            }
        }
    }
};

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
    constexpr int ks_sc = NMAX * (kLaMaxD + 4) > ROWS * (kLaChunk + 4) ? NMAX * (kLaMaxD + 4) : ROWS * (kLaChunk + 4);
    constexpr int verify = VERIFY ? NMAX * (kLaMaxD + 4) + ks_sc + NMAX * ROWS + NMAX * NMAX : 0;
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
        // This thread's four columns d4 .. d4 + 3 of slice rows e0, e0 + estep,
        // ...: 16-byte loads, issued first (no address depends on the path;
        // rows past the slice read its last row and are not stored).
        const int tpr = Dk / 4, d4 = 4 * (tid % tpr), e0 = tid / tpr, estep = kLaThreads / tpr;
        constexpr int kRows4 = kLaRows * kLaMaxD / 4 / kLaThreads;  // row slots a thread may hold
        float4 sv[kRows4];
#pragma unroll
        for (int r = 0; r < kRows4; ++r) {
            const int e = min(e0 + r * estep, ne - 1);
            sv[r] = *reinterpret_cast<const float4*>(S + static_cast<size_t>(es0 + e) * Dk + d4);
        }
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
        auto pko = [&](int t) { return ((static_cast<size_t>(b) * N + s_j[t]) * H + h) * Dk; };
        auto pvo = [&](int t) { return ((static_cast<size_t>(b) * N + s_j[t]) * H + h) * Dv + es0; };
        auto path_rows = [&](auto bfc) {
            constexpr bool BF = decltype(bfc)::value;
            constexpr int EPP = LaPieces<BF, 1>::EPP;
            LaPieces<BF, (NMAX * kLaMaxD / EPP + kLaThreads - 1) / kLaThreads> pk;
            LaPieces<BF, (NMAX * kLaRows / EPP + kLaThreads - 1) / kLaThreads> pv;
            pk.load(a.pk, acc + 1, Dk, pko);
            pv.load(a.pv, acc + 1, ne, pvo);
            pk.store(acc + 1, Dk, kf, Dk);
            pv.store(acc + 1, ne, vf, ne);
        };
        if (!a.vec) {
            la_rows_to_lds(a.pk, bf16, acc + 1, Dk, pko, kf, Dk);
            la_rows_to_lds(a.pv, bf16, acc + 1, ne, pvo, vf, ne);
        } else if (bf16) {
            path_rows(std::true_type{});
        } else {
            path_rows(std::false_type{});
        }
        __syncthreads();
        // The path's terms in order t = 0 .. acc, each k row's four values
        // read once for all of the thread's rows.
        const float Av = exp2f(s_L[vstop]);
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
    // Rows padded by four floats: 16-byte aligned for vector reads, and the
    // 16-byte reads of eight lanes on consecutive rows fall on distinct banks.
    const int DkP = Dk + 4;
    constexpr int kScP = kLaChunk + 4;
    // K is read only for the scores W, so the state's chunks reuse its space.
    constexpr int kKsSc = NMAX * (kLaMaxD + 4) > kLaRows * kScP ? NMAX * (kLaMaxD + 4) : kLaRows * kScP;
    float* Qs = lds;                      // [N][Dk + 4]
    float* Ks = Qs + NMAX * (kLaMaxD + 4);
    float* Sc = Ks;                       // [ne][kLaChunk + 4], after W is complete
    float* Vs = Ks + kKsSc;               // [N][ne]: this slice's dims of v
    float* W = Vs + NMAX * kLaRows;       // [N][N]
    // Every load of the phase goes first: the slice's state, all of its
    // 32-column chunks as 16-byte loads (one per thread and chunk), then
    // the rows of Q, K and the slice's V; the tree's parents and decays
    // follow, and the LDS stores wait for all of them together.
    constexpr int kNC = kLaMaxD / kLaChunk;
    constexpr int kS4 = (kLaRows * kLaChunk / 4 + kLaThreads - 1) / kLaThreads;
    const int n4 = ne * (kLaChunk / 4);
    float4 sreg[kNC * kS4];
#pragma unroll
    for (int c = 0; c < kNC; ++c) {
        const int c0 = min(c * kLaChunk, Dk - kLaChunk);  // Dk = 64: the spare chunks re-read the last
#pragma unroll
        for (int j = 0; j < kS4; ++j) {
            const int x = min(tid + j * kLaThreads, n4 - 1), r = x / (kLaChunk / 4), c4 = x - r * (kLaChunk / 4);
            sreg[c * kS4 + j] = *reinterpret_cast<const float4*>(S + static_cast<size_t>(es0 + r) * Dk + c0 + 4 * c4);
        }
    }
    auto rk = [&](int i) { return ((static_cast<size_t>(b) * N + i) * H + h) * Dk; };
    auto rv = [&](int i) { return ((static_cast<size_t>(b) * N + i) * H + h) * Dv + es0; };
    auto qkv_rows = [&](auto bfc) {
        constexpr bool BF = decltype(bfc)::value;
        constexpr int EPP = LaPieces<BF, 1>::EPP;
        LaPieces<BF, (NMAX * kLaMaxD / EPP + kLaThreads - 1) / kLaThreads> lq, lk;
        LaPieces<BF, (NMAX * kLaRows / EPP + kLaThreads - 1) / kLaThreads> lv;
        lq.load(a.q, N, Dk, rk);
        lk.load(a.k, N, Dk, rk);
        lv.load(a.v, N, ne, rv);
        la_tree(a.parent, a.alpha, b, N, H, h, s_L, s_anc);
        lq.store(N, Dk, Qs, DkP);
        lk.store(N, Dk, Ks, DkP);
        lv.store(N, ne, Vs, ne);
    };
    if (!a.vec) {
        la_tree(a.parent, a.alpha, b, N, H, h, s_L, s_anc);
        la_rows_to_lds(a.q, bf16, N, Dk, rk, Qs, DkP);
        la_rows_to_lds(a.k, bf16, N, Dk, rk, Ks, DkP);
        la_rows_to_lds(a.v, bf16, N, ne, rv, Vs, ne);
    } else if (bf16) {
        qkv_rows(std::true_type{});
    } else {
        qkv_rows(std::false_type{});
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
        // four independent partial sums over 16-byte reads
        float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
        const float4* qi = reinterpret_cast<const float4*>(Qs + i * DkP);
        const float4* kj = reinterpret_cast<const float4*>(Ks + j * DkP);
#pragma unroll 4
        for (int d4 = 0; d4 < Dk / 4; ++d4) {
            const float4 x = qi[d4], y = kj[d4];
            d0 = fmaf(x.x, y.x, d0);
            d1 = fmaf(x.y, y.y, d1);
            d2 = fmaf(x.z, y.z, d2);
            d3 = fmaf(x.w, y.w, d3);
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
    // Chunk C: columns 32C .. 32C + 31 (a compile-time index, so the
    // state's registers are never addressed dynamically).
    auto chunk = [&](auto cidx) {
        constexpr int C = decltype(cidx)::value;
        const int c0 = C * kLaChunk;
        __syncthreads();  // the previous chunk is consumed (and W is complete)
#pragma unroll
        for (int j = 0; j < kS4; ++j) {
            const int x = tid + j * kLaThreads;
            if (x < n4) {
                const int r = x / (kLaChunk / 4), c4 = x - r * (kLaChunk / 4);
                // (four scalar stores: a 16-byte store of the register
                // array's element made the compiler keep the array in
                // scratch memory)
                float* dst = Sc + r * kScP + 4 * c4;
                dst[0] = sreg[C * kS4 + j].x;
                dst[1] = sreg[C * kS4 + j].y;
                dst[2] = sreg[C * kS4 + j].z;
                dst[3] = sreg[C * kS4 + j].w;
            }
        }
        __syncthreads();
        const float4* srow = reinterpret_cast<const float4*>(Sc + min(e, ne - 1) * kScP);
        if (e >= ne) {  // a row past the slice (Dv not a multiple of kLaRows): nothing to add
        } else if constexpr (NMAX > 16) {
            // Large trees, four columns at a time: one 16-byte state read
            // feeds this thread's kPer nodes as independent chains.  Rows
            // past N hold stale LDS; their sums are never used.
#pragma unroll 2
            for (int c4 = 0; c4 < kLaChunk / 4; ++c4) {
                const float4 s4 = srow[c4];
#pragma unroll
                for (int n = 0; n < kPer; ++n) {
                    const int i = min(g + n * G, NMAX - 1);
                    const float4 q4 = *reinterpret_cast<const float4*>(Qs + i * DkP + c0 + 4 * c4);
                    float t = fmaf(s4.x, q4.x, acc[n]);
                    t = fmaf(s4.y, q4.y, t);
                    t = fmaf(s4.z, q4.z, t);
                    acc[n] = fmaf(s4.w, q4.w, t);
                }
            }
        } else {  // small trees: only the nodes that exist
#pragma unroll
            for (int n = 0; n < kPer; ++n) {
                const int i = g + n * G;
                if (i < N) {
                    const float4* qrow = reinterpret_cast<const float4*>(Qs + i * DkP + c0);
                    float t = acc[n];
#pragma unroll
                    for (int c4 = 0; c4 < kLaChunk / 4; ++c4) {
                        const float4 s4 = srow[c4], q4 = qrow[c4];
                        t = fmaf(s4.x, q4.x, t);
                        t = fmaf(s4.y, q4.y, t);
                        t = fmaf(s4.z, q4.z, t);
                        t = fmaf(s4.w, q4.w, t);
                    }
                    acc[n] = t;
                }
            }
        }
    };
    static_assert(kNC == 4, "Dk is 64 or 128: two or four chunks");
    chunk(std::integral_constant<int, 0>{});
    chunk(std::integral_constant<int, 1>{});
    if (Dk > 2 * kLaChunk) {  // workgroup-uniform
        chunk(std::integral_constant<int, 2>{});
        chunk(std::integral_constant<int, 3>{});
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

// Workgroups of the instance that run at once on the current device
// (queried once per device and phase combination).
template <int NMAX, int ROWS>
static long la_resident(const LaArgs& a) {
    static long cache[64][3];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
    const int kind = a.do_commit && a.do_verify ? 0 : a.do_commit ? 1 : 2;
    if (dev >= 0 && cache[dev][kind] > 0) return cache[dev][kind];
    int n = 0;
    hipError_t e;
    if (a.do_commit && a.do_verify)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, la_kernel<NMAX, true, true, ROWS>, kLaThreads, 0);
    else if (a.do_commit)
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, la_kernel<NMAX, true, false, ROWS>, kLaThreads, 0);
    else
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, la_kernel<NMAX, false, true, ROWS>, kLaThreads, 0);
    if (e != hipSuccess || n < 1) n = 1;
    int cus = 0;
    if (dev < 0 || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        cus = 256;
    const long r = static_cast<long>(n) * cus;
    if (dev >= 0) cache[dev][kind] = r;
    return r;
}

template <int NMAX>
static void launch_la_nmax(const LaArgs& a, hipStream_t stream) {
    // Slices of state rows only when the (head, request) pairs leave most
    // CUs idle (the slices recompute the score matrix, which costs more than
    // it spreads once the chip is full: 64 requests x 16 heads ran slower
    // sliced), and no more of them than run at once: a second round of
    // workgroups costs more than a slice twice as tall.
    const long pairs = static_cast<long>(a.B) * a.H;
    int rows = a.Dv <= 64 ? 64 : kLaMaxD;
    if (pairs < 512) {
        rows = kLaSliceRows;
        if (pairs * (a.Dv / kLaSliceRows) > la_resident<NMAX, kLaSliceRows>(a) && a.Dv > 64 &&
            pairs * (a.Dv / 64) <= la_resident<NMAX, 64>(a))
            rows = 64;
    }
    const dim3 grid(a.H, a.B, (a.Dv + rows - 1) / rows);
    if (rows == kLaSliceRows)
        launch_la_n<NMAX, kLaSliceRows>(a, grid, stream);
    else if (rows == 64)
        launch_la_n<NMAX, 64>(a, grid, stream);
    else
        launch_la_n<NMAX, kLaMaxD>(a, grid, stream);
}

static bool la_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int launch_la(const LaArgs& args, hipStream_t stream) {
    LaArgs a = args;
    a.vec = (!a.do_verify || (la_aligned16(a.q) && la_aligned16(a.k) && la_aligned16(a.v))) &&
            (!a.do_commit || (la_aligned16(a.pk) && la_aligned16(a.pv)));
    // NMAX bounds both trees: the one verified and the one whose path is
    // committed (LDS is sized for the phases the launch runs).
    const bool small = (!a.do_verify || a.N <= 16) && (!a.do_commit || a.pN <= 16);
    if (small)
        launch_la_nmax<16>(a, stream);
    else
        launch_la_nmax<kMaxNodes>(a, stream);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // namespace specv
