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
//           S q_i on the matrix cores (fp32), the state's tiles loaded
//           straight into operand registers.
// Both phases in one launch are the deferred update: the previous step's
// commit folded into this step's verification (one state read and write).
// Decay products are exp2 of differences of log2 prefix sums along root paths.
#include <atomic>
#include <type_traits>

#include "spec_common.h"
#include "spec_internal.h"

namespace specv {

constexpr int kLaThreads = 256;
constexpr int kLaMaxD = 128;
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
// or verify (Q and K rows padded by four, V, the scores W), whichever is
// larger.
template <int NMAX, bool COMMIT, bool VERIFY, int ROWS>
constexpr int la_lds_floats() {
    constexpr int commit = COMMIT ? NMAX * (kLaMaxD + ROWS) : 0;
    constexpr int verify = VERIFY ? 2 * NMAX * (kLaMaxD + 4) + NMAX * ROWS + NMAX * NMAX : 0;
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

    // The slice of the state lives in registers, in the matrix-core operand
    // layout of the verification's S q_i (v_mfma_f32_16x16x4_f32, C[e][i] =
    // sum_d S[e][d] Q[i][d] per 16-row tile and 16-node tile): lane (r, g) =
    // (lane % 16, lane / 16) holds S[e0 + r][16j + 4g .. 16j + 4g + 3] for
    // every 16-column group j (16-byte loads, issued first: no address
    // depends on the tree or the path).  Component c of group j is the A
    // operand of one product, whose contraction index g stands for column
    // 16j + 4g + c; the B operand (Q[node][that column]) comes from LDS the
    // same way, and the result lands as C[e0 + 4g + c][node tile + r].  The
    // commit updates these registers in place, so a launch that commits and
    // verifies reads the state once.
    // Waves: with four or more row tiles each wave takes every fourth tile
    // and all node tiles; with two, two waves per row tile split the node
    // tiles (both update the tile; the first stores it).
    constexpr int kRT = kLaRows / 16;
    constexpr int kRowW = kRT >= 4 ? 4 : kRT;
    constexpr int kNodeW = 4 / kRowW;
    constexpr int kTPW = kRT / kRowW;       // row tiles per wave
    constexpr int kJ = kLaMaxD / 16;        // 16-column groups (Dk = 64: the spare ones re-read the last)
    static_assert(kRT * 16 == kLaRows && kRowW * kNodeW == 4 && kTPW * kRowW == kRT, "row tiles over four waves");
    // A launch that only commits 32-row slices keeps the row-major layout
    // below instead (two waves per tile would duplicate the update).
    constexpr bool kTiled = VERIFY || kNodeW == 1;
    const int wave = tid >> 6, lr = tid & 15, lg = (tid >> 4) & 3;
    const int rsel = wave % kRowW, nsel = wave / kRowW;
    float4 sreg[kTiled ? kTPW * kJ : 1];
    if constexpr (kTiled) {
#pragma unroll
        for (int t = 0; t < kTPW; ++t) {
            const int row = min((rsel + kRowW * t) * 16 + lr, ne - 1);
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
                const int jj = min(j, Dk / 16 - 1);
                sreg[t * kJ + j] =
                    *reinterpret_cast<const float4*>(S + static_cast<size_t>(es0 + row) * Dk + 16 * jj + 4 * lg);
            }
        }
    }
    // Row-major: this thread's four columns d4 .. d4 + 3 of slice rows e0,
    // e0 + estep, ... (rows past the slice read its last row and are not
    // stored).
    const int tpr = Dk / 4, d4 = 4 * (tid % tpr), e0 = tid / tpr, estep = kLaThreads / tpr;
    constexpr int kRows4 = kTiled ? 1 : kLaRows * kLaMaxD / 4 / kLaThreads;
    float4 sv[kRows4];
    if constexpr (!kTiled) {
#pragma unroll
        for (int r = 0; r < kRows4; ++r) {
            const int e = min(e0 + r * estep, ne - 1);
            sv[r] = *reinterpret_cast<const float4*>(S + static_cast<size_t>(es0 + e) * Dk + d4);
        }
    }

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
        // S <- A(-> v] S + sum_t c_t v_t[e] k_t^T, the path's terms in order
        // t = 0 .. acc.
        const float Av = exp2f(s_L[vstop]);
        if constexpr (!kTiled) {
#pragma unroll
            for (int r = 0; r < kRows4; ++r) {
                sv[r].x *= Av;
                sv[r].y *= Av;
                sv[r].z *= Av;
                sv[r].w *= Av;
            }
            for (int t = 0; t <= acc; ++t) {  // each k row's four values read once for all rows
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
        }
#pragma unroll
        for (int t = 0; t < (kTiled ? kTPW : 0); ++t) {
            const int r0 = (rsel + kRowW * t) * 16;
            if (r0 >= ne) continue;  // wave-uniform
            const int row = r0 + lr;
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
                float4& x = sreg[t * kJ + j];
                x.x *= Av;
                x.y *= Av;
                x.z *= Av;
                x.w *= Av;
            }
            for (int tt = 0; tt <= acc; ++tt) {
                const float w = s_c[tt] * vf[tt * ne + row];
                const float* kr = kf + tt * Dk + 4 * lg;
#pragma unroll
                for (int j = 0; j < kJ; ++j) {
                    const float4 k4 = *reinterpret_cast<const float4*>(kr + 16 * min(j, Dk / 16 - 1));
                    float4& x = sreg[t * kJ + j];
                    x.x = fmaf(w, k4.x, x.x);
                    x.y = fmaf(w, k4.y, x.y);
                    x.z = fmaf(w, k4.z, x.z);
                    x.w = fmaf(w, k4.w, x.w);
                }
            }
            if (nsel == 0) {  // wave-uniform: one writer per tile
#pragma unroll
                for (int j = 0; j < kJ; ++j)
                    if (16 * j < Dk)
                        *reinterpret_cast<float4*>(S + static_cast<size_t>(es0 + row) * Dk + 16 * j + 4 * lg) =
                            sreg[t * kJ + j];
            }
        }
        __syncthreads();  // the path rows in LDS are read before the verification's stores
    }
    if (!VERIFY || !a.do_verify) return;

    const int N = a.N;
    // Rows padded by four floats: 16-byte aligned for vector reads, and the
    // 16-byte reads of eight lanes on consecutive rows fall on distinct banks.
    const int DkP = Dk + 4;
    float* Qs = lds;                      // [N][Dk + 4]
    float* Ks = Qs + NMAX * (kLaMaxD + 4);
    float* Vs = Ks + NMAX * (kLaMaxD + 4);  // [N][ne]: this slice's dims of v
    float* W = Vs + NMAX * kLaRows;         // [N][N]
    // The rows of Q, K and the slice's V are loaded next; the tree's parents
    // and decays follow, and the LDS stores wait for all of them together.
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
    __syncthreads();  // W is complete
    const int ntiles = (N + 15) / 16;
#pragma unroll
    for (int t = 0; t < kTPW; ++t) {
        const int r0 = (rsel + kRowW * t) * 16;
        if (r0 >= ne) continue;  // wave-uniform
        for (int nt = nsel; nt < ntiles; nt += kNodeW) {
            const int node = nt * 16 + lr;
            const float* qrow = Qs + min(node, N - 1) * DkP;
            // two independent accumulator chains, added at the end
            f32x4 ca = {0.f, 0.f, 0.f, 0.f}, cb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < kJ; ++j) {
                if (16 * j < Dk) {  // workgroup-uniform
                    const float4 q4 = *reinterpret_cast<const float4*>(qrow + 16 * j + 4 * lg);
                    const float4 s4 = sreg[t * kJ + j];
                    ca = __builtin_amdgcn_mfma_f32_16x16x4f32(s4.x, q4.x, ca, 0, 0, 0);
                    cb = __builtin_amdgcn_mfma_f32_16x16x4f32(s4.y, q4.y, cb, 0, 0, 0);
                    ca = __builtin_amdgcn_mfma_f32_16x16x4f32(s4.z, q4.z, ca, 0, 0, 0);
                    cb = __builtin_amdgcn_mfma_f32_16x16x4f32(s4.w, q4.w, cb, 0, 0, 0);
                }
            }
            if (node < N) {
                // rows e = r0 + 4g + c of node `node`: the decayed state term,
                // then the tree's own terms over the ancestors j, ascending
                const int e0 = r0 + 4 * lg;
                const float base = exp2f(s_L[node]);
                float o[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) o[c] = base * (ca[c] + cb[c]);
                for (uint64_t m = s_anc[node]; m != 0ull; m &= m - 1ull) {
                    const int j = __ffsll(static_cast<long long>(m)) - 1;
                    const float w = W[node * N + j];
                    const float4 v4 = *reinterpret_cast<const float4*>(Vs + j * ne + e0);
                    o[0] = fmaf(w, v4.x, o[0]);
                    o[1] = fmaf(w, v4.y, o[1]);
                    o[2] = fmaf(w, v4.z, o[2]);
                    o[3] = fmaf(w, v4.w, o[3]);
                }
                const size_t oi = ((static_cast<size_t>(b) * N + node) * H + h) * Dv + es0 + e0;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    if (bf16)
                        static_cast<uint16_t*>(a.out)[oi + c] = static_cast<uint16_t>(f32_to_bf16_bits(o[c]));
                    else
                        static_cast<float*>(a.out)[oi + c] = o[c];
                }
            }
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
    static std::atomic<long> cache[64][3];  // host threads may race to fill it (same value)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
    const int kind = a.do_commit && a.do_verify ? 0 : a.do_commit ? 1 : 2;
    if (dev >= 0) {
        const long c = cache[dev][kind].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
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
    if (dev >= 0) cache[dev][kind].store(r, std::memory_order_relaxed);
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
