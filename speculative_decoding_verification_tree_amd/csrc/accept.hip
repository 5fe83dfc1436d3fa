// Acceptance over the vocabulary for gfx950: the rejection rule and the
// typical-acceptance rule.
//
// Rejection rule ("Speculative Decoding" / "Speculative Sampling" sections of
// the blog page "Fast Inference from Transformers via Speculative Decoding"):
// node i with parent u and token x passes when u_accept[i] * q_i(x) < p_u(x),
// p_u = softmax(logits_u / T); the first rejection is replaced by a draw from
// norm(max(0, p - q)), and when every draft passes one bonus token is drawn
// from the target at the last node.  Typical acceptance (MEDUSA section of the
// same page): x passes when p_u(x) > min(eps, delta * exp(-H(p_u))); the last
// token is the greedy one.  Over a tree the output is the longest accepted
// root path.
//
// Three launches per call; kernel boundaries are the only cross-workgroup
// synchronisation (a device-scope fence inside a kernel costs an L2 write-back
// and invalidate on this chip):
//   accept_rowstats grid (chunks, N, B): every node row with children, per
//                   vocabulary chunk: max logit (+ lowest argmax),
//                   sum exp((l - max)/T) and sum t*exp(t) (entropy).
//   accept_sample   grid (chunks, B): every workgroup combines the chunk
//                   statistics of its request and runs the node tests (fp64,
//                   from the gathered logit and draft probability) -- cheap
//                   and identical in every workgroup, so no workgroup waits
//                   for another; chunk 0 writes the path, the accepted tokens
//                   and the decision.  Then each workgroup reduces its chunk
//                   of the stop row: residual mass, bonus mass or argmax.
//   accept_select   grid B: scan the chunk masses in token order, find the
//                   chunk that holds u * total and the token inside it
//                   (wavefront scans, ascending token ids).
#include "spec_common.h"
#include "spec_internal.h"

namespace specv {

struct RowStat {  // per (request, node row, chunk)
    double S;     // sum 2^t2 over the chunk, t2 = (l - M) * log2(e) / T
    double A;     // sum t2 * 2^t2 (so sum t * exp(t) = ln2 * A for t = (l - M) / T)
    float M;      // chunk max logit
    int arg;      // lowest index of the chunk max
};

enum { MODE_DONE = 0, MODE_RESID = 1, MODE_BONUS = 2, MODE_ARGMAX = 3 };

struct Decision {  // per request
    double S;      // stop row: sum exp((l - M)/T) over the whole row (over its kept tokens when truncated)
    float M;       // stop row: max logit
    float u;       // u_sample at the stop node
    int mode, v, c, a;
    uint32_t tau;  // stop row: key of its smallest kept logit (0: every token kept)
};

struct RowRec {    // per (request, node row), truncated target (top-k / nucleus)
    double S;      // sum over the kept tokens of 2^((l - M) * log2(e) / T)
    float M;       // max logit
    uint32_t tau;  // a token is kept iff logit_key(l) >= tau
    int arg;       // lowest index of the max
    int pad;
};

// Order-preserving 32-bit key of a float (-0 and +0 share the key of +0):
// a < b as floats iff logit_key(a) < logit_key(b), for non-NaN values.
__device__ __forceinline__ uint32_t logit_key(float f) {
    uint32_t u = __float_as_uint(f);
    u = u == 0x80000000u ? 0u : u;
    return u ^ (static_cast<uint32_t>(static_cast<int32_t>(u) >> 31) | 0x80000000u);
}

struct ChunkStat {  // per (request, chunk) of the stop row
    double m1;      // residual mass | bonus mass relative to the chunk max
    double m2;      // plain target mass (residual fallback)
    float M;        // chunk max logit (bonus / argmax)
    int arg;
};

struct AcceptArgs {
    const float* logits;
    const float* draft;
    const int32_t* tokens;
    const int32_t* parent;
    const float* u_acc;
    const float* u_smp;
    int32_t* accept_len;
    int32_t* path;
    int32_t* out_tokens;
    RowStat* rowstat;
    RowRec* rowrec;  // truncated rows (aliases rowstat's space)
    Decision* dec;
    ChunkStat* cstat;
    // [B][nchunk][kSubMax]: per 1024-token slice of each stop-row chunk of
    // four or more slices, the residual (or bonus) mass
    double* cslice;
    int B, N, V, chunk, nchunk, rule;  // rule 0 = rejection, 1 = typical
    int lg_seg;                        // log2 of the lanes per row in the decision: 2^lg_seg >= min(nchunk, 64)
    int vec4;                          // rows are 16-byte aligned: 16-byte loads
    float T, eps, delta;
    int top_k;    // 0: off
    float top_p;  // 1: off
    // Truncation split over the chunks of each row (top_k > 0 and a
    // workspace of spec_accept_filtered_workspace_bytes), else null.
    struct ChunkRec* frec;  // [B*N][nchunk] per chunk: max, digit and key counts
    uint32_t* fbins;        // [B*N][nchunk][kFBinCap] (digit << 20 | count) of the chunk's top digits
    uint32_t* fkeys;        // [B*N][nchunk][kFKeyCap] the keys of those digits
};

struct ChunkRec {  // one chunk of a row, split truncation
    float M;       // chunk max logit
    int arg;       // not computed (0x7fffffff): the truncated rule runs at T > 0, where no argmax is read
    int nbins;     // non-empty first digits at or above the chunk's top-k digit (> kFBinCap: too many)
    int nkeys;     // keys of those digits (> kFKeyCap: too many)
};

// Per chunk: the non-empty first digits at or above the chunk's own top-k
// digit, and their keys; a row with a chunk over either bound is redone
// whole by its finishing workgroup.
constexpr int kFBinCap = 64;  // (one a lane when gathered)
constexpr int kFKeyCap = 256;
static_assert(kFBinCap == 64 && kFKeyCap % 64 == 0, "the split finish gathers whole waves of entries");
// Candidate keys the split finish holds in LDS (more: the row is redone whole).
constexpr int kFCandRow = 4096;
// (row, chunk) pairs of a split truncation: a bound on its grid and workspace.
constexpr long kFMaxSlots = 65536;

constexpr int kThreads = 256;
// Slices of a chunk for the token search: four entries of every thread
// (1024 tokens, contiguous in both load layouts); at most 8 per chunk.
constexpr int kSubTokens = 4 * kThreads;
constexpr int kSubMax = 8;

// Helpers that take LDS arrays by pointer are force-inlined: called out of
// line they receive generic pointers, whose LDS-aperture test this compiler
// fails to select.
constexpr int kRowsPerWave = kMaxNodes / 4;
constexpr int kMaxChunks = 1024;

__device__ __forceinline__ double block_sum_d(double v, double* s_red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) s_red[wv] = v;
    __syncthreads();
    return s_red[0] + s_red[1] + s_red[2] + s_red[3];
}

// Block sums of NS per-slice values and, with TWO, one more value (s_sl:
// 4 * (NS + 1) doubles); every thread gets the totals, the waves added in a
// fixed order.
template <int NS, bool TWO>
__device__ __forceinline__ void block_sum_slices(double (&x)[NS], double& y, double* s_sl) {
    constexpr int W = NS + 1;
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < NS; ++j) x[j] = wave_sum(x[j]);
    if constexpr (TWO) y = wave_sum(y);
    if (lane == 0) {
#pragma unroll
        for (int j = 0; j < NS; ++j) s_sl[wv * W + j] = x[j];
        if constexpr (TWO) s_sl[wv * W + NS] = y;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NS; ++j) x[j] = ((s_sl[j] + s_sl[W + j]) + s_sl[2 * W + j]) + s_sl[3 * W + j];
    if constexpr (TWO) y = ((s_sl[NS] + s_sl[W + NS]) + s_sl[2 * W + NS]) + s_sl[3 * W + NS];
}

__device__ __forceinline__ void block_argmax(float& v, int& i, float* s_v, int* s_i) {
    wave_argmax(v, i);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) {
        s_v[wv] = v;
        s_i[wv] = i;
    }
    __syncthreads();
    v = s_v[0];
    i = s_i[0];
    for (int k = 1; k < 4; ++k)
        if (s_v[k] > v || (s_v[k] == v && s_i[k] < i)) {
            v = s_v[k];
            i = s_i[k];
        }
}

// The same over the workgroup: one LDS exchange.
__device__ __forceinline__ void block_min_max_i(int& mn, int& mx, int* s_mn, int* s_mx) {
    wave_min_max_i(mn, mx);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) {
        s_mn[wv] = mn;
        s_mx[wv] = mx;
    }
    __syncthreads();
    mn = min(min(s_mn[0], s_mn[1]), min(s_mn[2], s_mn[3]));
    mx = max(max(s_mx[0], s_mx[1]), max(s_mx[2], s_mx[3]));
}

// Reductions over aligned segments of 2^lg lanes (lg wave-uniform, 0..6):
// the butterfly of the wave reductions cut after lg levels.
__device__ __forceinline__ double seg_sum(double v, int lg) {
    if (lg >= 1) v += move_d<dpp_xor1>(v);
    if (lg >= 2) v += move_d<dpp_xor2>(v);
    if (lg >= 3) v += move_d<dpp_mirror8>(v);
    if (lg >= 4) v += move_d<dpp_mirror16>(v);
    if (lg >= 5) {
        const uint64_t u = __builtin_bit_cast(uint64_t, v);
        const auto x = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(u), static_cast<uint32_t>(u), false, false);
        const auto y =
            __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(u >> 32), static_cast<uint32_t>(u >> 32), false, false);
        v = __builtin_bit_cast(double, static_cast<uint64_t>(x[0]) | (static_cast<uint64_t>(y[0]) << 32)) +
            __builtin_bit_cast(double, static_cast<uint64_t>(x[1]) | (static_cast<uint64_t>(y[1]) << 32));
    }
    if (lg >= 6) {
        const uint64_t u = __builtin_bit_cast(uint64_t, v);
        const auto x = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(u), static_cast<uint32_t>(u), false, false);
        const auto y =
            __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(u >> 32), static_cast<uint32_t>(u >> 32), false, false);
        v = __builtin_bit_cast(double, static_cast<uint64_t>(x[0]) | (static_cast<uint64_t>(y[0]) << 32)) +
            __builtin_bit_cast(double, static_cast<uint64_t>(x[1]) | (static_cast<uint64_t>(y[1]) << 32));
    }
    return v;
}

// (value, index) argmax over aligned segments of 2^lg lanes: largest value,
// lowest index on ties.
__device__ __forceinline__ void seg_argmax(float& v, int& i, int lg) {
    if (lg >= 1) argmax_step(v, i, __uint_as_float(dpp_xor1(__float_as_uint(v))), static_cast<int>(dpp_xor1(i)));
    if (lg >= 2) argmax_step(v, i, __uint_as_float(dpp_xor2(__float_as_uint(v))), static_cast<int>(dpp_xor2(i)));
    if (lg >= 3) argmax_step(v, i, __uint_as_float(dpp_mirror8(__float_as_uint(v))), static_cast<int>(dpp_mirror8(i)));
    if (lg >= 4) argmax_step(v, i, __uint_as_float(dpp_mirror16(__float_as_uint(v))), static_cast<int>(dpp_mirror16(i)));
    if (lg >= 5) {
        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        const auto y = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(i), static_cast<uint32_t>(i), false, false);
        v = __uint_as_float(x[0]);
        i = static_cast<int>(y[0]);
        argmax_step(v, i, __uint_as_float(x[1]), static_cast<int>(y[1]));
    }
    if (lg >= 6) {
        const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        const auto y = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(i), static_cast<uint32_t>(i), false, false);
        v = __uint_as_float(x[0]);
        i = static_cast<int>(y[0]);
        argmax_step(v, i, __uint_as_float(x[1]), static_cast<int>(y[1]));
    }
}

// p_v(x) as the residual and sampling passes evaluate it (fp32): the
// weight 2^((l - M) * c2) / S, c2 = log2(e) / T.
__device__ __forceinline__ float target_prob(float l, float M, float c2, float invS) {
    return __builtin_amdgcn_exp2f((l - M) * c2) * invS;
}

// Element e of this thread's share of a chunk starting at x0: strided by
// the block (coalesced), in runs of four with 16-byte loads.  Its token id is
// x0 + 4 * threadIdx.x + elem_off(e) with 16-byte loads, else
// x0 + threadIdx.x + elem_off(e); offsets ascend with e.
__device__ __forceinline__ int elem_off(int e, bool vec4) {
    return vec4 ? 4 * kThreads * (e >> 2) + (e & 3) : kThreads * e;
}

template <int EPT>
struct Vals {
    float v[EPT];
};

// The loads are unconditional (from a clamped address inside the chunk) and
// the fill is selected afterwards, so every load of the thread is in flight
// at once; a load under a branch would make the compiler wait for it before
// the next.  With 16-byte rows x1 is a multiple of 4, like every x here, so
// a run of four is either wholly inside the chunk or wholly outside.
template <int EPT, bool NT = false>
__device__ __forceinline__ Vals<EPT> load_chunk(const float* row, int x0, int x1, bool vec4, float fill) {
    Vals<EPT> r;
    if (vec4) {
#pragma unroll
        for (int j = 0; j < EPT / 4; ++j) {
            const int x = x0 + 4 * (static_cast<int>(threadIdx.x) + kThreads * j);
            const float* src = row + static_cast<unsigned>(min(x, x1 - 4));
            const float4 v = NT ? ld_stream_f4(src) : *reinterpret_cast<const float4*>(src);
            const bool in = x < x1;
            r.v[4 * j] = in ? v.x : fill;
            r.v[4 * j + 1] = in ? v.y : fill;
            r.v[4 * j + 2] = in ? v.z : fill;
            r.v[4 * j + 3] = in ? v.w : fill;
        }
    } else {
        // Element e sits kThreads * e past this thread's first element; lim
        // is the last in-range offset (negative: the thread has none), and
        // out-of-range loads read the chunk's first element instead.
        const int tid = static_cast<int>(threadIdx.x);
        const float* p = row + x0 + tid;
        const int lim = x1 - x0 - tid - 1;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const bool in = kThreads * e <= lim;
            const float v = p[in ? kThreads * e : -tid];
            r.v[e] = in ? v : fill;
        }
    }
    return r;
}

// The same chunk of two rows, every load of both issued before the first
// select (one branch on the layout for the pair).
template <int EPT>
__device__ __forceinline__ void load_chunk2(const float* row, const float* qrow, int x0, int x1, bool vec4, Vals<EPT>& l,
                                            Vals<EPT>& q) {
    if (vec4) {
        float4 lv[EPT / 4], qv[EPT / 4];
#pragma unroll
        for (int j = 0; j < EPT / 4; ++j) {
            const unsigned x = static_cast<unsigned>(min(x0 + 4 * (static_cast<int>(threadIdx.x) + kThreads * j), x1 - 4));
            lv[j] = *reinterpret_cast<const float4*>(row + x);
            qv[j] = *reinterpret_cast<const float4*>(qrow + x);
        }
#pragma unroll
        for (int j = 0; j < EPT / 4; ++j) {
            const bool in = x0 + 4 * (static_cast<int>(threadIdx.x) + kThreads * j) < x1;
            l.v[4 * j] = in ? lv[j].x : -INFINITY;
            l.v[4 * j + 1] = in ? lv[j].y : -INFINITY;
            l.v[4 * j + 2] = in ? lv[j].z : -INFINITY;
            l.v[4 * j + 3] = in ? lv[j].w : -INFINITY;
            q.v[4 * j] = in ? qv[j].x : 0.f;
            q.v[4 * j + 1] = in ? qv[j].y : 0.f;
            q.v[4 * j + 2] = in ? qv[j].z : 0.f;
            q.v[4 * j + 3] = in ? qv[j].w : 0.f;
        }
    } else {
        const int tid = static_cast<int>(threadIdx.x);
        const int lim = x1 - x0 - tid - 1;
        float lv[EPT], qv[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int off = x0 + tid + (kThreads * e <= lim ? kThreads * e : -tid);
            lv[e] = row[off];
            qv[e] = qrow[off];
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const bool in = kThreads * e <= lim;
            l.v[e] = in ? lv[e] : -INFINITY;
            q.v[e] = in ? qv[e] : 0.f;
        }
    }
}

// In-place pairwise (tree) sum of n floats; the total lands in v[0].
template <int n>
__device__ __forceinline__ void pairwise_sum(float (&v)[n]) {
#pragma unroll
    for (int w = n / 2; w >= 1; w /= 2)
#pragma unroll
        for (int e = 0; e < w; ++e) v[e] += v[e + w];
}

// Per-wave partial results of a chunk reduction.
struct WaveRed {
    float m[4];
    int i[4];
    double s[4], a[4];
};

// Chunk statistics of one target row: max logit with its lowest index and,
// for T > 0, S = sum 2^t2 and A2 = sum t2 * 2^t2 with t2 = (l - max) * c2
// (so sum exp(t) = S and sum t * exp(t) = ln2 * A2 for t = (l - max) / T).
// Branch-free per element: the thread's elements ascend in token id, so the
// lowest index of the max is the first element equal to it.  Each wave
// reduces relative to its own max; one barrier, then wave 0 merges the four
// waves (the results are valid in wave 0 only).
// ARG = false skips the lowest argmax (arg is left at 0x7fffffff) and ENT =
// false the entropy sum (A2 stays 0): the rejection rule at T > 0 uses
// neither, and both cost VALU work per element in a VALU-heavy pass.
template <int EPT, bool FILT = false, bool ARG = true, bool ENT = true>
__device__ __forceinline__ void chunk_reduce(const Vals<EPT>& vals, int x0, int x1, bool vec4, float T, float& M,
                                             int& arg, double& S, double& A2, WaveRed* s, uint32_t tau = 0u) {
    const int tid = static_cast<int>(threadIdx.x);
    // Element e has token id first + off(e); it is in range iff off(e) < lim
    // (with 16-byte rows a run of four is wholly in or out).
    const int first = x0 + (vec4 ? 4 * tid : tid), lim = x1 - first;
    auto off = [vec4](int e) { return elem_off(e, vec4); };
    float best = -INFINITY;
#pragma unroll
    for (int e = 0; e < EPT; ++e) best = fmaxf(best, vals.v[e]);
    int bi = 0x7fffffff;
    if constexpr (ARG) {
#pragma unroll
        for (int e = EPT - 1; e >= 0; --e) bi = vals.v[e] == best && off(e) < lim ? first + off(e) : bi;
        wave_argmax(best, bi);
    } else {
        best = wave_max(best);
    }
    double sw = 0.0, aw = 0.0;
    if (T > 0.f && best > -INFINITY) {
        // The thread's terms are summed pairwise in fp32 (same-sign terms:
        // relative error below log2(EPT) * 2^-24), the threads' sums in fp64.
        const float c2 = 1.4426950408889634f / T;
        float ex[EPT], ax[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const float t2 = (vals.v[e] - best) * c2;
            // (truncated rows: only kept tokens carry mass; the max stays
            // the chunk's, which is kept whenever any token of it is)
            const bool in = off(e) < lim && (!FILT || logit_key(vals.v[e]) >= tau);
            ex[e] = in ? __builtin_amdgcn_exp2f(t2) : 0.f;
            ax[e] = ENT && in ? t2 * ex[e] : 0.f;
        }
        pairwise_sum<EPT>(ex);
        sw = wave_sum(static_cast<double>(ex[0]));
        if constexpr (ENT) {
            pairwise_sum<EPT>(ax);
            aw = wave_sum(static_cast<double>(ax[0]));
        }
    }
    const int lane = tid & 63, wv = tid >> 6;
    if (lane == 0) {
        s->m[wv] = best;
        s->i[wv] = bi;
        s->s[wv] = sw;
        s->a[wv] = aw;
    }
    __syncthreads();
    M = -INFINITY;
    arg = 0x7fffffff;
    S = 0.0;
    A2 = 0.0;
    if (wv != 0) return;
    M = s->m[0];
    arg = s->i[0];
#pragma unroll
    for (int k = 1; k < 4; ++k)
        if (s->m[k] > M || (s->m[k] == M && s->i[k] < arg)) {
            M = s->m[k];
            arg = s->i[k];
        }
    if (T > 0.f) {
        const double c2 = 1.4426950408889634 / static_cast<double>(T);
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (s->m[k] > -INFINITY) {
                const double dl = (static_cast<double>(s->m[k]) - M) * c2;
                const double w = exp2(dl);
                S += w * s->s[k];
                A2 += w * (s->a[k] + dl * s->s[k]);
            }
    }
}

template <int EPT, bool FILT = false, bool ARG = true, bool ENT = true, bool NT = false>
__device__ __forceinline__ void chunk_stats(const float* row, int x0, int x1, bool vec4, float T, float& M, int& arg,
                                            double& S, double& A2, WaveRed* s, uint32_t tau = 0u) {
    const Vals<EPT> vals = load_chunk<EPT, NT>(row, x0, x1, vec4, -INFINITY);
    chunk_reduce<EPT, FILT, ARG, ENT>(vals, x0, x1, vec4, T, M, arg, S, A2, s, tau);
}

// Does node u of request b have a child?  (Wave-uniform; chains need no load.)
__device__ __forceinline__ bool row_has_children(const AcceptArgs& a, int b, int u) {
    if (!a.parent) return u < a.N - 1;
    const int i = (threadIdx.x & 63) + 1;
    const int p = i < a.N ? tree_parent(a.parent, a.N, b, i) : -1;
    return __ballot(p == u) != 0ull;
}

// NT: non-temporal row loads (rows that would only evict other data from
// the caches); small batches keep them cached for the sampling pass, which
// reads the stop row again.
template <int EPT, bool ARG, bool ENT, bool NT>
__global__ __launch_bounds__(kThreads) void accept_rowstats(AcceptArgs a) {
    const int c = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
    __shared__ WaveRed s_red;
    if (!row_has_children(a, b, u)) return;  // leaves need no statistics
    const float* row = a.logits + (static_cast<size_t>(b) * a.N + u) * a.V;
    const int x0 = c * a.chunk, x1 = min(x0 + a.chunk, a.V);
    float M;
    int arg;
    double S, A2;
    chunk_stats<EPT, false, ARG, ENT, NT>(row, x0, x1, a.vec4 != 0, a.T, M, arg, S, A2, &s_red);
    if (threadIdx.x == 0) {
        RowStat rs;
        rs.S = S;
        rs.A = A2;
        rs.M = M;
        rs.arg = arg;
        a.rowstat[(static_cast<size_t>(b) * a.N + u) * a.nchunk + c] = rs;
    }
}

// Decision of request b from the chunk statistics.  Every accept_sample
// workgroup of the request computes it (same inputs, same code, same result);
// only the writer stores path, accepted tokens, accept_len and the record.
// Every load that depends on nothing else is issued first: the tree, the
// drafted tokens and uniforms, and the chunk records of every row (a leaf's
// records are stale and never used).
// FILT: the target rows are truncated (top-k / nucleus); their statistics
// come whole from the per-row records, for every row (the stop row may be a
// leaf).
// LDS state of one request's decision: per node row, the row max M, its
// lowest argmax, S = sum exp((l - M)/T) and the entropy H (natural log) of
// p = softmax(l/T); the accepted path, the drafted tokens and the record.
struct DecLds {
    float M[kMaxNodes];
    int arg[kMaxNodes];
    double S[kMaxNodes], H[kMaxNodes];
    int path[kMaxNodes];
    uint32_t tau[kMaxNodes];
    int tok[kMaxNodes];
    Decision dec;
};

// The decision of request b, by wave 0 alone, from the row statistics in L
// (rows with children; every row when truncated) and lane i's node inputs:
// parent pi (-1 root, -2 unreachable), token xi (clamped), accept uniform
// ui, the logit of the parent row at the token glf and the draft
// probability gq.  Node tests in fp64; a node is accepted when every node
// on its root path passed; the stop node v is the deepest accepted node,
// the lowest index among equals.  Lane 0 writes L.dec, the lanes on the
// path L.path.
template <bool FILT>
__device__ __forceinline__ void decide_core(const AcceptArgs& a, int b, int pi, int xi, float ui, float usi, float glf,
                                            double gq, DecLds& L) {
    const int N = a.N, lane = threadIdx.x & 63;
    const double T = a.T;
    const double gl = glf;
    // Node tests in fp64 from the gathered values.
    bool ok = false;
    if (lane >= 1 && lane < N && pi >= 0) {
        double pu;
        if (T > 0.0)
            pu = FILT && logit_key(glf) < L.tau[pi] ? 0.0 : exp((gl - static_cast<double>(L.M[pi])) / T) / L.S[pi];
        else
            pu = xi == L.arg[pi] ? 1.0 : 0.0;
        if (a.rule == 0) {
            ok = static_cast<double>(ui) * gq < pu;
        } else {
            const double thr = fmin(static_cast<double>(a.eps), static_cast<double>(a.delta) * exp(-L.H[pi]));
            ok = pu > thr;
        }
    }
    const uint64_t okm = __ballot(ok) | 1ull;  // the root is always accepted
    // Root paths by pointer doubling: after round k a lane holds its
    // first 2^k path nodes and its 2^k-th ancestor.
    const int me = lane < N ? lane : 0;
    uint64_t anc;
    if (!a.parent) {  // chain: nodes 0..me
        anc = me == 63 ? ~0ull : (2ull << me) - 1ull;
    } else {
        int up = lane < N ? pi : -1;
        anc = 1ull << me;
#pragma unroll
        for (int r = 0; r < 6; ++r) {
            const int src = up >= 0 ? up : 0;
            const uint32_t lo = __shfl(static_cast<uint32_t>(anc), src),
                           hi = __shfl(static_cast<uint32_t>(anc >> 32), src);
            const int upup = __shfl(up, src);
            if (up >= 0) {
                anc |= static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
                up = upup;
            }
        }
    }
    // Accepted: every node on the root path passed.  The stop node is the
    // deepest accepted node, the lowest index among equals.
    const bool accepted = lane < N && (anc & ~okm) == 0ull;
    const int depth = __popcll(anc) - 1;
    // deepest accepted node, lowest index among equals: one integer max
    int key = accepted ? (depth << 6) | (63 - lane) : -1, unused = 0;
    wave_min_max_i(unused, key);
    const int v = 63 - (key & 63);
    const int dv = key >> 6;
    const uint32_t vlo = __shfl(static_cast<uint32_t>(anc), v), vhi = __shfl(static_cast<uint32_t>(anc >> 32), v);
    const uint64_t anc_v = static_cast<uint64_t>(vlo) | (static_cast<uint64_t>(vhi) << 32);
    if (lane < N && ((anc_v >> lane) & 1ull)) L.path[depth] = lane;
    const uint64_t kids = __ballot(lane >= 1 && lane < N && pi == v);
    const bool v_has = kids != 0ull;
    const float uv = __shfl(usi, v);  // the stop node's sample uniform, loaded with the node inputs
    if (lane == 0) {
        Decision d;
        d.v = v;
        d.c = v_has ? __ffsll(static_cast<long long>(kids)) - 1 : -1;
        d.a = dv;
        d.u = uv;
        d.M = v_has || FILT ? L.M[v] : 0.f;
        d.S = v_has || FILT ? L.S[v] : 0.0;
        d.tau = FILT ? L.tau[v] : 0u;
        if (a.rule == 1 || !(T > 0.0))
            d.mode = v_has ? MODE_DONE : MODE_ARGMAX;
        else
            d.mode = v_has ? MODE_RESID : MODE_BONUS;
        L.dec = d;
    }
}

// path, accepted tokens (and the last token when the decision fixes it)
// and accept_len of request b, by threads 0..N-1.
__device__ __forceinline__ void write_decision(const AcceptArgs& a, int b, const Decision& d, const DecLds& L) {
    const int tid = threadIdx.x, N = a.N;
    if (tid < N) {
        const size_t o = static_cast<size_t>(b) * N + tid;
        a.path[o] = tid <= d.a ? L.path[tid] : -1;
        int tok = tid < d.a ? L.tok[L.path[tid + 1]] : -1;  // from LDS: no dependent load after the decision
        if (tid == d.a && d.mode == MODE_DONE) tok = L.arg[d.v];
        a.out_tokens[o] = tok;
    }
    if (tid == 0) a.accept_len[b] = d.a;
}

template <int RPW, bool FILT = false>  // combining passes per wave (rows <= 4 * RPW * 64 / L)
__device__ __forceinline__ Decision decide_request(const AcceptArgs& a, int b, bool writer) {
    const int N = a.N, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ DecLds L;
    float* s_M = L.M;
    int* s_arg = L.arg;
    double* s_S = L.S;
    double* s_H = L.H;
    uint32_t* s_tau = L.tau;

    // The node's parent entry, token and uniform: three independent loads
    // with no branch between them (a chain's absent parent array and an
    // absent uniform array read the tokens instead, selected away later).
    // Their uses wait until the chunk records are in flight as well.
    // Every thread loads (lanes past N read node N - 1's entries): a load
    // under a branch would pull the uses into the branch, ahead of the chunk
    // records' loads.
    int praw, xraw;
    float uraw, usraw;
    {
        const size_t o = static_cast<size_t>(b) * N + min(lane, N - 1);
        const int32_t* psrc = a.parent ? a.parent : a.tokens;
        const float* usrc = a.rule == 0 && a.u_acc ? a.u_acc : reinterpret_cast<const float*>(a.tokens);
        praw = psrc[o];
        xraw = a.tokens[o];
        uraw = usrc[o];
        usraw = a.u_smp ? a.u_smp[o] : 0.f;
    }
    int pi = -1, xi = 0;
    float ui = 0.f;
    auto node_inputs = [&]() {  // same as tree_parent(), the token clamped into the vocabulary
        // (selects rather than a branch, so the compiler keeps the uses here,
        // behind the chunk records' loads)
        // (integer masks: a select on a uniform flag becomes a branch, and
        // the compiler then sinks the loads into it)
        const int mine = -static_cast<int>(wave == 0 && lane < N);
        const int tree = -static_cast<int>(a.parent != nullptr);
        const int ptree = (praw >= 0 && praw < lane) ? praw : -2;
        const int p = (ptree & tree) | ((lane - 1) & ~tree);
        pi = (p & mine) | (-1 & ~mine);
        xi = min(max(xraw, 0), a.V - 1) & mine;
        const int uon = mine & -static_cast<int>(a.rule == 0 && a.u_acc != nullptr);
        ui = __int_as_float(__float_as_int(uraw) & uon);
    };
    // The tested values, gathered at the drafted tokens as soon as they land
    // (issued after the loads that depend on nothing).
    float glf = 0.f;
    double gq = 0.0;
    auto gather = [&]() {
        node_inputs();
        if (wave == 0 && lane >= 1 && lane < N && pi >= 0) {
            glf = a.logits[(static_cast<size_t>(b) * N + pi) * a.V + xi];
            if (a.rule == 0) gq = a.draft[(static_cast<size_t>(b) * N + lane) * a.V + xi];
        }
    };
    const double T = a.T;
    if constexpr (FILT) {
        RowRec r{};
        if (tid < N) r = a.rowrec[static_cast<size_t>(b) * N + tid];
        gather();
        if (tid < N) {
            s_M[tid] = r.M;
            s_arg[tid] = r.arg;
            s_S[tid] = r.S;
            s_H[tid] = 0.0;
            s_tau[tid] = r.tau;
        }
    } else {
    // Whole-row statistics, several rows per pass: the chunks of a row sit
    // on an aligned segment of L = 2^lg_seg lanes (L >= chunks, at most 64),
    // so a wave combines 64 / L rows at once.  Wave w owns rows w, w + 4, ...,
    // taken 64 / L to a pass; vocabularies of more than 64 chunks loop over
    // the extra chunks on all 64 lanes (one row per pass).
    const double c2 = T > 0.0 ? 1.4426950408889634 / T : 0.0;
    const int nrows = N - 1 + (a.parent != nullptr);
    const int lg = a.lg_seg, R = 64 >> lg, sr = lane >> lg, cc = lane & ((1 << lg) - 1);
    const int mine = nrows > wave ? (nrows - wave + 3) / 4 : 0;
    const int passes = (mine + R - 1) / R;
    // Loads from clamped (always valid) indexes, selected afterwards: no
    // load under a branch, so all of them are in flight at once.  Entries
    // of rows that are not combined are read and dropped.
    RowStat rr[RPW];
    {
        const int cl = min(cc, a.nchunk - 1);
#pragma unroll
        for (int t = 0; t < RPW; ++t)
            rr[t] = a.rowstat[(static_cast<size_t>(b) * N + min(wave + 4 * (t * R + sr), N - 1)) * a.nchunk + cl];
    }
    gather();
    // Below 16 passes every pass runs (passes past the last row combine
    // nothing and store nothing), so the compiler can interleave them.
#pragma unroll
    for (int t = 0; t < RPW; ++t) {
        if (RPW < kRowsPerWave || t < passes) {  // wave-uniform
            const int u = wave + 4 * (t * R + sr);
            const bool row_in = u < nrows, in = row_in && cc < a.nchunk;
            float m = in ? rr[t].M : -INFINITY;
            int ar = in ? rr[t].arg : 0x7fffffff;
            const size_t rbase = (static_cast<size_t>(b) * N + min(u, N - 1)) * a.nchunk;
            if (row_in)
                for (int c = lane + 64; c < a.nchunk; c += 64) {
                    const RowStat& r = a.rowstat[rbase + c];
                    if (r.M > m || (r.M == m && r.arg < ar)) {
                        m = r.M;
                        ar = r.arg;
                    }
                }
            seg_argmax(m, ar, lg);
            double S = 0.0, A2 = 0.0;
            if (T > 0.0) {
                if (in) {
                    const double dl = (static_cast<double>(rr[t].M) - m) * c2;
                    const double w = exp2(dl);
                    S = w * rr[t].S;
                    A2 = w * (rr[t].A + dl * rr[t].S);
                }
                if (row_in)
                    for (int c = lane + 64; c < a.nchunk; c += 64) {
                        const RowStat r = a.rowstat[rbase + c];
                        const double dl = (static_cast<double>(r.M) - m) * c2;
                        const double w = exp2(dl);
                        S += w * r.S;
                        A2 += w * (r.A + dl * r.S);
                    }
                S = seg_sum(S, lg);
                A2 = seg_sum(A2, lg);
            }
            // the entropy only for the typical rule
            const double H = T > 0.0 && a.rule == 1 ? log(S) - 0.6931471805599453 * A2 / S : 0.0;
            if (cc == 0 && row_in) {
                s_M[u] = m;
                s_arg[u] = ar;
                s_S[u] = S;
                s_H[u] = H;
            }
        }
    }
    }  // row statistics
    if (wave == 0 && lane < N) L.tok[lane] = xraw;
    __syncthreads();
    if (wave == 0) decide_core<FILT>(a, b, pi, xi, ui, usraw, glf, gq, L);
    __syncthreads();
    const Decision d = L.dec;
    if (writer) {
        write_decision(a, b, d, L);
        if (tid == 0) a.dec[b] = d;
    }
    return d;
}

// Chunk c of the stop row of request b, as decision d requires (valid in
// thread 0): the residual mass sum max(0, p_v - q_c) and the plain mass
// sum p_v (MODE_RESID), or the chunk max with its lowest index and
// sum 2^((l - max) * log2(e) / T) (MODE_BONUS), or only the max (MODE_ARGMAX).
template <int EPT, bool FILT = false>
__device__ __forceinline__ ChunkStat chunk_work(const AcceptArgs& a, int b, const Decision& d, int c, WaveRed* s_red,
                                                double* s_sl) {
    constexpr int NS = EPT / 4;  // 1024-token slices of the chunk
    static_assert(NS >= 1 && NS <= kSubMax, "slices per chunk");
    const float* row = a.logits + (static_cast<size_t>(b) * a.N + d.v) * a.V;
    const int x0 = c * a.chunk, x1 = min(x0 + a.chunk, a.V);
    ChunkStat cs;
    cs.m1 = cs.m2 = 0.0;
    cs.M = 0.f;
    cs.arg = 0;
    const bool vec4 = a.vec4 != 0;
    const int lim = x1 - (x0 + (vec4 ? 4 * static_cast<int>(threadIdx.x) : static_cast<int>(threadIdx.x)));
    // Per slice (entries 4j .. 4j + 3 of every thread): fp32 pairwise per
    // thread, fp64 across threads; the chunk's mass is the slices' sum.  The
    // plain target mass (the residual's rare fallback) is kept per chunk only.
    double sa[NS], sb = 0.0;
    if (d.mode == MODE_RESID) {
        const float* qrow = a.draft + (static_cast<size_t>(b) * a.N + d.c) * a.V;
        const float invS = static_cast<float>(1.0 / d.S);
        const float c2 = 1.4426950408889634f / a.T;
        Vals<EPT> lvals, qvals;
        load_chunk2<EPT>(row, qrow, x0, x1, vec4, lvals, qvals);
        float rv[EPT], pvv[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const bool in = elem_off(e, vec4) < lim && (!FILT || logit_key(lvals.v[e]) >= d.tau);
            const float pv = in ? target_prob(lvals.v[e], d.M, c2, invS) : 0.f;
            pvv[e] = pv;
            rv[e] = in ? fmaxf(pv - qvals.v[e], 0.f) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < NS; ++j) sa[j] = (rv[4 * j] + rv[4 * j + 1]) + (rv[4 * j + 2] + rv[4 * j + 3]);
        pairwise_sum<EPT>(pvv);
        sb = pvv[0];
        block_sum_slices<NS, true>(sa, sb, s_sl);
    } else if (d.mode == MODE_BONUS) {
        // 2^((l - M) * log2(e) / T) relative to the chunk max M (the truncated
        // rule keeps only tokens at or above tau; the max stays the chunk's)
        const Vals<EPT> v = load_chunk<EPT>(row, x0, x1, vec4, -INFINITY);
        float bm = -INFINITY;
#pragma unroll
        for (int e = 0; e < EPT; ++e) bm = fmaxf(bm, v.v[e]);
        bm = wave_max(bm);
        if ((threadIdx.x & 63) == 0) s_red->m[threadIdx.x >> 6] = bm;
        __syncthreads();
        const float M = fmaxf(fmaxf(s_red->m[0], s_red->m[1]), fmaxf(s_red->m[2], s_red->m[3]));
        const float c2 = 1.4426950408889634f / a.T;
        float ex[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const bool in = elem_off(e, vec4) < lim && (!FILT || logit_key(v.v[e]) >= d.tau);
            ex[e] = in ? __builtin_amdgcn_exp2f((v.v[e] - M) * c2) : 0.f;
        }
#pragma unroll
        for (int j = 0; j < NS; ++j) sa[j] = (ex[4 * j] + ex[4 * j + 1]) + (ex[4 * j + 2] + ex[4 * j + 3]);
        block_sum_slices<NS, false>(sa, sb, s_sl);
        cs.M = M;
    } else {  // MODE_ARGMAX
        float M;
        int arg;
        double S, A2;
        chunk_stats<EPT, FILT>(row, x0, x1, vec4, 0.f, M, arg, S, A2, s_red, d.tau);
        cs.M = M;
        cs.arg = arg;
        return cs;
    }
    double m1 = 0.0;
#pragma unroll
    for (int j = 0; j < NS; ++j) m1 += sa[j];
    cs.m1 = m1;
    cs.m2 = sb;
    if (NS >= 4 && threadIdx.x < NS) {  // the slices, for the token search of chunks of four or more
        const int j = threadIdx.x;
        double val = 0.0;
#pragma unroll
        for (int i = 0; i < NS; ++i)
            if (i == j) val = sa[i];
        a.cslice[(static_cast<size_t>(b) * a.nchunk + c) * kSubMax + j] = val;
    }
    return cs;
}

template <int EPT, int RPW, bool FILT = false>
__global__ __launch_bounds__(kThreads) void accept_sample(AcceptArgs a) {
    const int c = blockIdx.x, b = blockIdx.y;
    __shared__ WaveRed s_red;
    __shared__ double s_sl[4 * (EPT / 4 + 1)];
    const Decision d = decide_request<RPW, FILT>(a, b, c == 0);
    if (d.mode == MODE_DONE) return;
    const ChunkStat cs = chunk_work<EPT, FILT>(a, b, d, c, &s_red, s_sl);
    if (threadIdx.x == 0) a.cstat[static_cast<size_t>(b) * a.nchunk + c] = cs;
}

// ---------------------------------------------------------------------------
// 64-bit DPP move of a double (both halves with the same control); lanes
// without a source read 0.
// This thread's run of EPT consecutive tokens first .. first + EPT - 1 of a
// chunk ending at x1, from two rows (16-byte loads when the rows allow):
// the layout of the token search, which walks each run in token order.
// Loads from clamped addresses, selected afterwards (all in flight at once).
template <int EPT>
__device__ __forceinline__ void load_run2(const float* row, const float* qrow, int first, int x1, bool vec4,
                                          Vals<EPT>& l, Vals<EPT>& q) {
    if (vec4) {
        float4 lv[EPT / 4], qv[EPT / 4];
#pragma unroll
        for (int j = 0; j < EPT / 4; ++j) {
            const unsigned x = static_cast<unsigned>(min(first + 4 * j, x1 - 4));
            lv[j] = *reinterpret_cast<const float4*>(row + x);
            qv[j] = *reinterpret_cast<const float4*>(qrow + x);
        }
#pragma unroll
        for (int j = 0; j < EPT / 4; ++j) {
            const bool in = first + 4 * j < x1;
            l.v[4 * j] = in ? lv[j].x : -INFINITY;
            l.v[4 * j + 1] = in ? lv[j].y : -INFINITY;
            l.v[4 * j + 2] = in ? lv[j].z : -INFINITY;
            l.v[4 * j + 3] = in ? lv[j].w : -INFINITY;
            q.v[4 * j] = in ? qv[j].x : 0.f;
            q.v[4 * j + 1] = in ? qv[j].y : 0.f;
            q.v[4 * j + 2] = in ? qv[j].z : 0.f;
            q.v[4 * j + 3] = in ? qv[j].w : 0.f;
        }
    } else {
        float lv[EPT], qv[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const unsigned x = static_cast<unsigned>(min(first + e, x1 - 1));
            lv[e] = row[x];
            qv[e] = qrow[x];
        }
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const bool in = first + e < x1;
            l.v[e] = in ? lv[e] : -INFINITY;
            q.v[e] = in ? qv[e] : 0.f;
        }
    }
}

// The token search over [xs0, xs1): thread tid owns tokens xs0 + RL*tid ..
// + RL - 1 (weights past xs1 are 0); base is the mass before xs0 (-inf:
// take the last token with weight).
template <int RL, bool FILT>
__device__ __forceinline__ void search_run(const AcceptArgs& a, const Decision& d, const float* row,
                                           const float* qrow, int xs0, int xs1, bool vec4, double base, bool usep,
                                           float Mc, double scale, float invS, float c2, double t, int x0, int32_t* out,
                                           double* s_wtot, int* s_mn, int* s_mx) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int first = xs0 + tid * RL;
    Vals<RL> lvals, qvals;
    load_run2<RL>(row, qrow, first, xs1, vec4, lvals, qvals);
    double wv[RL];
    if (d.mode == MODE_RESID) {
#pragma unroll
        for (int e = 0; e < RL; ++e) {
            const float pv = target_prob(lvals.v[e], d.M, c2, invS);
            const float wgt = usep ? pv : fmaxf(pv - qvals.v[e], 0.f);
            const bool in = first + e < xs1 && (!FILT || logit_key(lvals.v[e]) >= d.tau);
            wv[e] = in ? static_cast<double>(wgt) : 0.0;
        }
    } else {
#pragma unroll
        for (int e = 0; e < RL; ++e) {
            const float wgt = __builtin_amdgcn_exp2f((lvals.v[e] - Mc) * c2);
            const bool in = first + e < xs1 && (!FILT || logit_key(lvals.v[e]) >= d.tau);
            wv[e] = in ? static_cast<double>(wgt) * scale : 0.0;
        }
    }
    // Mass before this thread's run: block exclusive scan of the run totals.
    double mine = 0.0;
#pragma unroll
    for (int e = 0; e < RL; ++e) mine += wv[e];
    const double incl_r = wave_incl_scan(mine);
    if (lane == 63) s_wtot[4 + wave] = incl_r;  // slots 4..7: the chunk scan's 0..3 may still be read
    __syncthreads();
    double c = base + (incl_r - mine);
    for (int k = 0; k < wave; ++k) c += s_wtot[4 + k];
    // Walk the run in token order: the first token whose cumulative mass
    // exceeds t, and the last token with weight (the fallback when rounding
    // leaves the slice's recomputed mass short of t).
    int xhit = 0x7fffffff, lastnz = -1;
#pragma unroll
    for (int e = 0; e < RL; ++e) {
        const bool nz = wv[e] > 0.0;
        c += wv[e];
        lastnz = nz ? first + e : lastnz;
        xhit = nz && xhit == 0x7fffffff && c > t ? first + e : xhit;
    }
    int ix = xhit, iz = lastnz;
    block_min_max_i(ix, iz, s_mn, s_mx);
    if (tid == 0) {
        int final = ix != 0x7fffffff ? ix : iz;
        if (final < 0) final = x0;
        *out = final;
    }
}

// Sampling by inverse CDF over the stop row in ascending token order: the
// chunk totals locate the chunk that holds u * total, then the chunk's
// weights (recomputed from the same fp32 terms accept_sample summed) locate
// the token.  Zero-weight tokens are never drawn; if rounding leaves u*total
// past the end, the last token with weight is taken.
// load_cs(i) gives chunk record i of the request (i < a.nchunk).
template <int EPT, bool FILT, class LoadCS>
__device__ __forceinline__ void select_token(const AcceptArgs& a, int b, const Decision& d, LoadCS load_cs) {
    constexpr int CPT = kMaxChunks / kThreads;  // chunk records per thread
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    __shared__ double s_red[8];
    __shared__ double s_wtot[8];
    __shared__ int s_pick;
    __shared__ double s_base;
    __shared__ int s_mn[4], s_mx[4];

    // This thread's run of chunk records.
    ChunkStat cs[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) cs[k] = load_cs(min(tid * CPT + k, a.nchunk - 1));  // clamped: no load under a branch
#pragma unroll
    for (int k = 0; k < CPT; ++k)
        if (tid * CPT + k >= a.nchunk) {
            cs[k].m1 = cs[k].m2 = 0.0;
            cs[k].M = -INFINITY;
            cs[k].arg = 0x7fffffff;
        }
    if (d.mode == MODE_DONE) return;
    int32_t* out = a.out_tokens + static_cast<size_t>(b) * a.N + d.a;

    if (d.mode == MODE_ARGMAX) {
        float best = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int k = 0; k < CPT; ++k)
            if (cs[k].M > best || (cs[k].M == best && cs[k].arg < bi)) {
                best = cs[k].M;
                bi = cs[k].arg;
            }
        block_argmax(best, bi, s_v, s_i);
        if (tid == 0) *out = bi;
        return;
    }

    // Chunk weights in token order (thread t owns chunks t*CPT .. t*CPT+CPT-1).
    const double T = a.T;
    const double c2d = 1.4426950408889634 / T;
    double Mg = -INFINITY;
    if (d.mode == MODE_BONUS) {
        float mloc = -INFINITY;
        int dummy = 0;
#pragma unroll
        for (int k = 0; k < CPT; ++k) mloc = fmaxf(mloc, cs[k].M);
        block_argmax(mloc, dummy, s_v, s_i);
        Mg = mloc;
    }
    // Chunk weights, then the exclusive prefix of this thread's run (wave
    // scan + wave totals).  A residual of zero total mass falls back to p_v:
    // its masses are scanned instead (rare).
    bool usep = false;
    double w[CPT], run, incl, total;
    for (int pass = 0; pass < 2; ++pass) {
        run = 0.0;
#pragma unroll
        for (int k = 0; k < CPT; ++k) {
            w[k] = tid * CPT + k >= a.nchunk ? 0.0
                   : d.mode == MODE_BONUS    ? cs[k].m1 * exp2((static_cast<double>(cs[k].M) - Mg) * c2d)
                   : usep                    ? cs[k].m2
                                             : cs[k].m1;
            run += w[k];
        }
        incl = wave_incl_scan(run);
        if (pass) __syncthreads();  // the first pass's totals are read before they are replaced
        if (lane == 63) s_wtot[wave] = incl;
        __syncthreads();
        total = s_wtot[0] + s_wtot[1] + s_wtot[2] + s_wtot[3];
        if (d.mode != MODE_RESID || total > 0.0 || usep) break;
        usep = true;
    }
    double before = incl - run;
    for (int k = 0; k < wave; ++k) before += s_wtot[k];
    const double t = static_cast<double>(d.u) * total;
    int hit = 0x7fffffff, lastc = -1;
    double hit_base = 0.0, cum = before;
#pragma unroll
    for (int k = 0; k < CPT; ++k) {
        if (w[k] > 0.0) {
            lastc = tid * CPT + k;
            if (hit == 0x7fffffff && cum + w[k] > t) {
                hit = tid * CPT + k;
                hit_base = cum;
            }
        }
        cum += w[k];
    }
    // smallest chunk with a hit, else the last chunk with weight
    int ih = hit, il = lastc;
    block_min_max_i(ih, il, s_mn, s_mx);
    if (tid == 0) {
        s_pick = ih != 0x7fffffff ? ih : max(il, 0);
        s_base = ih != 0x7fffffff ? 0.0 : -INFINITY;  // -inf: take the last token with weight
    }
    __syncthreads();
    if (ih != 0x7fffffff && hit == ih) s_base = hit_base;
    __syncthreads();

    // The chunk's slice that holds t, from the slice masses the sampling
    // pass stored (the same fp32 terms, in the units of the chunk scan),
    // then the token inside that slice.
    const int pc = s_pick;
    const double base = s_base;
    const int x0 = pc * a.chunk, x1 = min(x0 + a.chunk, a.V);
    const bool vec4 = a.vec4 != 0;
    const float* row = a.logits + (static_cast<size_t>(b) * a.N + d.v) * a.V;
    // Outside the residual mode the second row is the stop row again (read,
    // never used), so the pair's loads need no branch.
    const float* qrow = d.mode == MODE_RESID ? a.draft + (static_cast<size_t>(b) * a.N + d.c) * a.V : row;
    const float invS = d.mode == MODE_RESID ? static_cast<float>(1.0 / d.S) : 0.f;
    const float c2 = 1.4426950408889634f / a.T;
#pragma unroll
    for (int k = 0; k < CPT; ++k)
        if (tid * CPT + k == pc) s_v[0] = cs[k].M;
    __shared__ int s_js;
    __shared__ double s_sbase;
    // Chunks of two slices (8 entries a thread) are searched whole: there
    // the slice masses' extra round trip costs more than the reload saves.
    // The residual's rare fallback to the plain mass searches the chunk whole
    // too (only the residual or bonus mass is kept per slice).
    constexpr int NS = EPT / 4;
    constexpr bool kSliced = NS >= 4;
    const bool sliced = kSliced && !usep;
    // (every wave loads, from clamped slots: no load under a branch)
    const size_t so = (static_cast<size_t>(b) * a.nchunk + pc) * kSubMax;
    const double raw = kSliced ? a.cslice[so + min(lane, NS - 1)] : 0.0;
    __syncthreads();  // s_v[0]
    if (sliced && wave == 0) {  // (workgroup-uniform)
        const double scl = d.mode == MODE_BONUS ? exp2((static_cast<double>(s_v[0]) - Mg) * c2d) : 1.0;
        const double w = lane < NS ? raw * scl : 0.0;
        const double incl = wave_incl_scan(w);
        const uint64_t hm = __ballot(w > 0.0 && base + incl > t), nz = __ballot(w > 0.0);
        const int jh = hm ? __ffsll(static_cast<long long>(hm)) - 1 : -1;
        const int jl = nz ? 63 - __clzll(static_cast<long long>(nz)) : 0;
        const double bef = __shfl(incl - w, jh >= 0 ? jh : 0);
        if (lane == 0) {
            // the first slice whose mass reaches past t, else the last slice
            // with mass and its last token with weight
            s_js = jh >= 0 ? jh : jl;
            s_sbase = jh >= 0 ? base + bef : -INFINITY;
        }
    }
    __syncthreads();
    const float Mc = s_v[0];
    const double scale = d.mode == MODE_BONUS ? exp2((static_cast<double>(Mc) - Mg) * c2d) : 1.0;
    // Thread tid owns tokens first .. first + RL - 1 of the slice (or of the
    // chunk); weights of tokens past its end are 0.
    if (sliced)
        search_run<4, FILT>(a, d, row, qrow, x0 + s_js * kSubTokens, min(x0 + (s_js + 1) * kSubTokens, x1), vec4,
                            s_sbase, usep, Mc, scale, invS, c2, t, x0, out, s_wtot, s_mn, s_mx);
    else
        search_run<EPT, FILT>(a, d, row, qrow, x0, x1, vec4, base, usep, Mc, scale, invS, c2, t, x0, out, s_wtot,
                              s_mn, s_mx);
}

template <int EPT, bool FILT = false>
__global__ __launch_bounds__(kThreads) void accept_select(AcceptArgs a) {
    const int b = blockIdx.x;
    // The decision and the chunk records, loaded together.
    const Decision d = a.dec[b];
    const ChunkStat* csb = a.cstat + static_cast<size_t>(b) * a.nchunk;
    select_token<EPT, FILT>(a, b, d, [&](int i) { return csb[i]; });
}

// ---------------------------------------------------------------------------
// Entries per thread and chunk: 8, raised to 16 or 32 for large batches so
// the statistics kernel launches at most ~2k workgroups of useful size (on
// 8 requests of 46-node trees over 32000 tokens, ~5.9k short-lived
// workgroups ran in about three rounds: the acceptance took 22.1 us against
// 20.8 at a ~4k bound and 19.0 at ~2k), and for rows of more than 32 chunks
// (the decision then combines two or more rows per wave pass, and the
// truncation's finish gathers fewer chunk records).
static int accept_ept(int B, int N, int V) {
    int ept = 8;
    auto nchunk = [&](int e) { return (V + e * kThreads - 1) / (e * kThreads); };
    while (ept < 32 && (static_cast<long>(B) * N * nchunk(ept) > 2048 || nchunk(ept) > 32)) ept *= 2;
    return ept;
}

// ---------------------------------------------------------------------------
// Truncated target rows (top-k, then nucleus on the renormalised top-k
// distribution), one workgroup per (request, node row): the row max with its
// lowest index, the key threshold tau of the kept set and the kept mass.
// The thresholds come from radix selection on the order-preserving logit
// keys (11 + 11 + 10 bits) over LDS histograms: counts for top-k (the k-th
// largest key, so ties with it are kept); for the nucleus, masses
// 2^((l - M) * log2(e) / T) in 2^-44 fixed point (integer sums, independent
// of the order of the atomics), the key at which the mass from the top first
// reaches top_p of the top-k mass.  Every histogram also sums the
// fixed-point masses, so the kept mass comes out of the selection itself.
constexpr int kFThreads = 1024;
constexpr int kFWaves = kFThreads / 64;
constexpr int kFSplitThreads = 256;
constexpr int kFUnroll = 8;
constexpr float kFixedOne = 17592186044416.0f;  // 2^44

// f(x, l) for every element of the row, this thread's elements in ascending
// order; kFUnroll loads are issued before the first f.
template <int NT, class F>
__device__ __forceinline__ void for_row(const float* row, int V, bool vec4, F f) {
    const int tid = threadIdx.x;
    if (vec4) {
        for (int base = 4 * tid; base < V; base += 4 * NT * kFUnroll) {
            float4 v[kFUnroll];
#pragma unroll
            for (int u = 0; u < kFUnroll; ++u)
                v[u] = *reinterpret_cast<const float4*>(row + min(base + 4 * NT * u, V - 4));
#pragma unroll
            for (int u = 0; u < kFUnroll; ++u) {
                const int x = base + 4 * NT * u;
                if (x < V) {
                    f(x, v[u].x);
                    f(x + 1, v[u].y);
                    f(x + 2, v[u].z);
                    f(x + 3, v[u].w);
                }
            }
        }
    } else {
        for (int base = tid; base < V; base += NT * kFUnroll) {
            float v[kFUnroll];
#pragma unroll
            for (int u = 0; u < kFUnroll; ++u) v[u] = row[min(base + NT * u, V - 1)];
#pragma unroll
            for (int u = 0; u < kFUnroll; ++u)
                if (base + NT * u < V) f(base + NT * u, v[u]);
        }
    }
}

template <int NT>
__device__ __forceinline__ unsigned long long block_incl_scan_u64(unsigned long long v, unsigned long long* s_w,
                                                                  unsigned long long& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    __syncthreads();
    if (lane == 63) s_w[wave] = v;
    __syncthreads();
    total = 0;
    for (int k = 0; k < NT / 64; ++k) {
        if (k < wave) v += s_w[k];
        total += s_w[k];
    }
    return v;
}

// One radix step: h[0, nb) are the counts (or masses) of the candidate keys
// by digit.  Scanning digits from the top, finds the digit d at which the
// running total first reaches need; *above is the total of the digits above
// d.  need_frac > 0: need = ceil(need_frac * total of the bins) (nucleus
// first step).
template <int NT>
__device__ __forceinline__ void radix_step(const unsigned long long* h, int nb, unsigned long long& need,
                                           double need_frac, int& d, unsigned long long& above,
                                           unsigned long long* s_w, int* s_d, unsigned long long* s_above) {
    const int tid = threadIdx.x, per = nb / NT;
    unsigned long long loc = 0;
    for (int j = 0; j < per; ++j) loc += h[nb - 1 - per * tid - j];
    unsigned long long total;
    const unsigned long long incl = block_incl_scan_u64<NT>(loc, s_w, total);
    if (need_frac > 0.0) {
        const double want = ceil(need_frac * static_cast<double>(total));
        need = want < 1.0 ? 1ull : (want > static_cast<double>(total) ? total : static_cast<unsigned long long>(want));
    }
    if (tid == 0) {
        *s_d = 0;
        *s_above = 0;
    }
    __syncthreads();
    const unsigned long long excl = incl - loc;
    if (excl < need && need <= incl) {  // the crossing lies in this thread's digits
        unsigned long long run = excl;
        for (int j = 0; j < per; ++j) {
            const int bin = nb - 1 - per * tid - j;
            if (run + h[bin] >= need) {
                *s_d = bin;
                *s_above = run;
                break;
            }
            run += h[bin];
        }
    }
    __syncthreads();
    d = *s_d;
    above = *s_above;
}

// Inverse of logit_key.
__device__ __forceinline__ float key_logit(uint32_t key) {
    return __uint_as_float(key ^ ((key >> 31) ? 0x80000000u : 0xFFFFFFFFu));
}

// Appends key to cand when match holds (wave-aggregated: one LDS atomic per
// wave); positions past cap are counted but not stored.
__device__ __forceinline__ void append_key(bool match, uint32_t key, uint32_t* cand, int* s_n, int cap) {
    const uint64_t m = __ballot(match);
    if (m == 0ull) return;
    const int lane = threadIdx.x & 63, leader = __ffsll(static_cast<long long>(m)) - 1;
    int base = 0;
    if (lane == leader) base = atomicAdd(s_n, __popcll(m));
    base = __shfl(base, leader);
    const int off = __popcll(m & ((1ull << lane) - 1ull));
    if (match && base + off < cap) cand[base + off] = key;
}

constexpr int kFCand = 16384;  // LDS candidate keys (64 KB)

// The truncation of row rid = request * N + node by one 1024-thread
// workgroup.  split: the chunk passes have left the row max, the first digit
// and the keys at or above it in the workspace; when those keys fit
// (kFCandRow) the selection starts from them, else from the row.
template <int NT>
__device__ __forceinline__ void filter_row(const AcceptArgs& a, int rid, bool split) {
    // LDS candidate keys: the whole-row workgroup keeps up to kFCand; the
    // split finish needs at most kFCandRow (more go back to the row).
    constexpr int CAP = NT == kFThreads ? kFCand : kFCandRow;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* row = a.logits + static_cast<size_t>(rid) * a.V;
    const bool vec4 = a.vec4 != 0;
    __shared__ unsigned long long s_cnt[2048], s_mass[2048];
    __shared__ uint32_t s_cand[CAP];
    __shared__ unsigned long long s_w[NT / 64];
    __shared__ float s_m[NT / 64];
    __shared__ int s_i[NT / 64];
    __shared__ int s_d, s_n;
    __shared__ unsigned long long s_above;
    const bool use_k = a.top_k > 0 && a.top_k < a.V, use_p = a.top_p < 1.f;
    constexpr int kShift[3] = {21, 10, 0};
    constexpr int kBits[3] = {11, 11, 10};
    auto clear = [&](int nb) {
        for (int i = tid; i < nb; i += NT) {
            s_cnt[i] = 0ull;
            s_mass[i] = 0ull;
        }
    };

    // Split: the chunk records give the row max, their top digits' counts
    // give the first digit d0 of the k-th largest key, and their keys of
    // digit >= d0 are the candidates (every such key: d0 is at or above each
    // chunk's own top-k digit, since the row's k-th largest key is at least
    // any chunk's).
    bool have = false;
    int d0s = 0, n_split = 0;
    unsigned long long need_s = 0ull;
    float Ms = -INFINITY;
    int args = 0x7fffffff;
    if (split && use_k) {
        __shared__ int s_ovf;
        __shared__ int s_nb[kMaxChunks], s_nk[kMaxChunks];
        const int nch = a.nchunk;
        const ChunkRec* rec = a.frec + static_cast<size_t>(rid) * nch;
        clear(2048);
        if (tid == 0) {
            s_ovf = 0;
            s_n = 0;
        }
        for (int c = tid; c < nch; c += NT) {  // the row max (its argmax is not needed at T > 0)
            const ChunkRec r = rec[c];
            if (r.M > Ms) {
                Ms = r.M;
                args = r.arg;
            }
            s_nb[c] = min(r.nbins, kFBinCap);
            s_nk[c] = min(r.nkeys, kFKeyCap);
            if (r.nbins > kFBinCap || r.nkeys > kFKeyCap) s_ovf = 1;
        }
        wave_argmax(Ms, args);
        if (lane == 0) {
            s_m[wave] = Ms;
            s_i[wave] = args;
        }
        __syncthreads();
        Ms = s_m[0];
        args = s_i[0];
        for (int k = 1; k < NT / 64; ++k)
            if (s_m[k] > Ms || (s_m[k] == Ms && s_i[k] < args)) {
                Ms = s_m[k];
                args = s_i[k];
            }
        if (!s_ovf) {  // workgroup-uniform
            // Wave w takes chunks w, w + NT/64, ... in groups of eight, lane
            // j entry j (then j + 64, ...) of each: eight loads in flight per
            // lane from clamped slots, the unused ones dropped.
            constexpr int NW = NT / 64;
            const uint32_t* bins = a.fbins + static_cast<size_t>(rid) * nch * kFBinCap;
            for (int g0 = wave; g0 < nch; g0 += 8 * NW) {
                uint32_t w[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int c = min(g0 + u * NW, nch - 1);
                    w[u] = bins[c * kFBinCap + lane];  // (kFBinCap == 64: one entry a lane)
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int c = g0 + u * NW;
                    if (c < nch && lane < s_nb[c])
                        atomicAdd(&s_cnt[w[u] >> 20], static_cast<unsigned long long>(w[u] & 0xFFFFFu));
                }
            }
            __syncthreads();
            unsigned long long above;
            need_s = static_cast<unsigned long long>(a.top_k);
            radix_step<NT>(s_cnt, 2048, need_s, 0.0, d0s, above, s_w, &s_d, &s_above);
            need_s -= above;
            // the candidates: every chunk key of digit >= d0
            const uint32_t* keys = a.fkeys + static_cast<size_t>(rid) * nch * kFKeyCap;
            for (int g0 = wave; g0 < nch; g0 += 8 * NW) {
                int most = 0;  // the group's largest key count (wave-uniform)
#pragma unroll
                for (int u = 0; u < 8; ++u) most = max(most, g0 + u * NW < nch ? s_nk[g0 + u * NW] : 0);
                for (int j0 = 0; j0 < most; j0 += 64) {
                    uint32_t kv[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int c = min(g0 + u * NW, nch - 1);
                        kv[u] = keys[c * kFKeyCap + j0 + lane];
                    }
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const int c = g0 + u * NW;
                        append_key(c < nch && j0 + lane < s_nk[c] && static_cast<int>(kv[u] >> kShift[0]) >= d0s, kv[u],
                                   s_cand, &s_n, CAP);
                    }
                }
            }
            __syncthreads();
            n_split = s_n;
            have = n_split <= CAP;
        }
        __syncthreads();  // (every thread has read s_ovf and s_n before either is reused)
    }
    float M, best = -INFINITY;
    int arg, bi = 0x7fffffff;
    if (have) {
        M = Ms;
        arg = args;
    } else {
    // Pass 1: the row max with its lowest index and, for top-k, the first
    // digit's count histogram (counts need no max).
    clear(2048);
    if (tid == 0) s_n = 0;
    __syncthreads();
    for_row<NT>(row, a.V, vec4, [&](int x, float l) {
        if (l > best) {
            best = l;
            bi = x;
        }
        if (use_k) atomicAdd(&s_cnt[logit_key(l) >> kShift[0]], 1ull);
    });
    wave_argmax(best, bi);
    if (lane == 0) {
        s_m[wave] = best;
        s_i[wave] = bi;
    }
    __syncthreads();
    M = s_m[0];
    arg = s_i[0];
    for (int k = 1; k < NT / 64; ++k)
        if (s_m[k] > M || (s_m[k] == M && s_i[k] < arg)) {
            M = s_m[k];
            arg = s_i[k];
        }
    }
    const float c2 = 1.4426950408889634f / a.T;
    auto mass_of = [&](float l) { return __float2ull_rn(__builtin_amdgcn_exp2f((l - M) * c2) * kFixedOne); };

    // The remaining digits of a selection, from round r0 on, over the keys
    // matching (prefix, pmask) and >= floor_key: from the LDS candidates when
    // they all fit (n <= CAP), else from the row.  by_mass selects where the
    // mass from the top reaches need, else where the count does.  Adds to kept
    // the mass of the candidates >= the selected key.
    auto finish = [&](int r0, uint32_t prefix, uint32_t pmask, bool by_mass, uint32_t floor_key,
                      unsigned long long need, int n, unsigned long long& kept, double need_frac) {
        const bool lds = n <= CAP;
        for (int r = r0; r < 3; ++r) {
            const int nb = 1 << kBits[r];
            clear(nb);
            __syncthreads();
            auto add = [&](uint32_t key, float l) {
                if ((key & pmask) == prefix && key >= floor_key) {
                    const int bin = (key >> kShift[r]) & (nb - 1);
                    atomicAdd(&s_mass[bin], mass_of(l));
                    if (!by_mass) atomicAdd(&s_cnt[bin], 1ull);
                }
            };
            if (lds) {
                for (int i = tid; i < n; i += NT) add(s_cand[i], key_logit(s_cand[i]));
            } else {
                for_row<NT>(row, a.V, vec4, [&](int, float l) { add(logit_key(l), l); });
            }
            __syncthreads();
            int d;
            unsigned long long above;
            radix_step<NT>(by_mass ? s_mass : s_cnt, nb, need, r == 0 ? need_frac : 0.0, d, above, s_w, &s_d, &s_above);
            need -= above;
            if (by_mass) {
                kept += above;
            } else {
                unsigned long long mine = 0ull, tot;
                for (int i = tid; i < nb; i += NT)
                    if (i > d) mine += s_mass[i];
                (void)block_incl_scan_u64<NT>(mine, s_w, tot);
                kept += tot;
            }
            if (r == 2) kept += s_mass[d];
            prefix |= static_cast<uint32_t>(d) << kShift[r];
            pmask |= static_cast<uint32_t>(nb - 1) << kShift[r];
            __syncthreads();
        }
        return prefix;
    };
    // Pass over the row collecting the keys of first digit d0 (>= floor_key;
    // with also_above every digit >= d0) into LDS and summing the mass of the
    // keys above digit d0.
    auto collect = [&](int d0, uint32_t floor_key, bool also_above, unsigned long long& mass_above) {
        if (tid == 0) s_n = 0;
        __syncthreads();
        unsigned long long mine = 0ull;
        for_row<NT>(row, a.V, vec4, [&](int, float l) {
            const uint32_t key = logit_key(l);
            const int dig = static_cast<int>(key >> kShift[0]);
            if (dig > d0 && key >= floor_key) mine += mass_of(l);
            append_key((also_above ? dig >= d0 : dig == d0) && key >= floor_key, key, s_cand, &s_n, CAP);
        });
        unsigned long long tot;
        (void)block_incl_scan_u64<NT>(mine, s_w, tot);  // (its barriers also publish s_n)
        mass_above = tot;
        return s_n;
    };

    uint32_t tau = 0u;
    unsigned long long kept = 0ull;
    int n_k = CAP + 1;  // keys >= the top-k threshold held in LDS (when <= CAP)
    if (use_k) {
        // first digit from the pass-1 counts, then the rest from its keys;
        // with a nucleus to follow, the keys above the digit (fewer than k)
        // are collected too, so that the nucleus needs no further pass
        unsigned long long need = static_cast<unsigned long long>(a.top_k);
        int d0;
        unsigned long long mass_above;
        int n;
        if (have) {
            // the chunks' candidates (in LDS): every key of digit >= d0
            d0 = d0s;
            need = need_s;
            n = n_split;
            unsigned long long mine = 0ull;
            for (int i = tid; i < n; i += NT) {
                const uint32_t key = s_cand[i];
                if (static_cast<int>(key >> kShift[0]) > d0) mine += mass_of(key_logit(key));
            }
            unsigned long long tot;
            (void)block_incl_scan_u64<NT>(mine, s_w, tot);
            mass_above = tot;
        } else {
            unsigned long long above;
            radix_step<NT>(s_cnt, 2048, need, 0.0, d0, above, s_w, &s_d, &s_above);
            need -= above;
            n = collect(d0, 0u, use_p, mass_above);
        }
        kept = mass_above;
        tau = finish(1, static_cast<uint32_t>(d0) << kShift[0], 0x7FFu << kShift[0], false, 0u, need, n, kept, 0.0);
        if (use_p) n_k = n;
    }
    if (use_p && n_k <= CAP) {
        // the nucleus over the top-k-kept keys, all in LDS
        kept = 0ull;
        tau = finish(0, 0u, 0u, true, tau, 0ull, n_k, kept, static_cast<double>(a.top_p));
    } else if (use_p) {
        // first digit from a mass histogram of the top-k-kept keys
        clear(2048);
        __syncthreads();
        const uint32_t floor_key = tau;
        for_row<NT>(row, a.V, vec4, [&](int, float l) {
            const uint32_t key = logit_key(l);
            if (key >= floor_key) atomicAdd(&s_mass[key >> kShift[0]], mass_of(l));
        });
        __syncthreads();
        unsigned long long need = 0ull;
        int d0;
        unsigned long long above;
        radix_step<NT>(s_mass, 2048, need, static_cast<double>(a.top_p), d0, above, s_w, &s_d, &s_above);
        need -= above;
        unsigned long long mass_above;
        const int n = collect(d0, floor_key, false, mass_above);
        kept = mass_above;
        tau = finish(1, static_cast<uint32_t>(d0) << kShift[0], 0x7FFu << kShift[0], true, floor_key, need, n, kept,
                     0.0);
    }

    if (tid == 0) {
        RowRec rr;
        rr.S = static_cast<double>(kept) * (1.0 / 17592186044416.0);  // 2^-44
        rr.M = M;
        rr.tau = tau;
        rr.arg = arg;
        rr.pad = 0;
        a.rowrec[rid] = rr;
    }
}

__global__ __launch_bounds__(kFThreads) void accept_filter(AcceptArgs a) { filter_row<kFThreads>(a, blockIdx.x, false); }

// Split truncation (top-k, then the nucleus), two launches:
//   filt_chunk   grid (chunk, row): the chunk's max with its lowest index,
//                its first-digit counts (LDS), the digit d_c where its own
//                count from the top reaches top_k, and the non-empty digits
//                at or above d_c with their counts and keys, into the
//                chunk's slots of the workspace (no atomics outside LDS);
//   accept_filter_split  grid row: sums the chunks' digit counts, finds the
//                row's first digit d0 and gathers the chunks' keys of digit
//                >= d0, then selects as one workgroup does over a whole row.
// The counts, the digit, the candidate set and the fixed-point masses are
// the same integers as in one workgroup's passes, so the records are
// identical.
// FULL: a whole chunk of a 16-byte-aligned row, so no element needs a
// range test (every chunk of a row but its last).
template <int EPT, bool NT, bool FULL>
__device__ __forceinline__ void filt_chunk_body(const AcceptArgs& a) {
    const int c = blockIdx.x, rid = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    __shared__ uint32_t s_h[2048];
    __shared__ WaveRed s_red;
    __shared__ uint32_t s_wt[kThreads / 64];
    __shared__ int s_dc, s_nb, s_nk;
    const float* row = a.logits + static_cast<size_t>(rid) * a.V;
    const int x0 = c * a.chunk, x1 = min(x0 + a.chunk, a.V);
    const bool vec4 = FULL || a.vec4 != 0;
    Vals<EPT> v;
    if constexpr (FULL) {
#pragma unroll
        for (int j = 0; j < EPT / 4; ++j) {
            const float* src = row + x0 + 4 * (tid + kThreads * j);
            const float4 f = NT ? ld_stream_f4(src) : *reinterpret_cast<const float4*>(src);
            v.v[4 * j] = f.x;
            v.v[4 * j + 1] = f.y;
            v.v[4 * j + 2] = f.z;
            v.v[4 * j + 3] = f.w;
        }
    } else {
        v = load_chunk<EPT, NT>(row, x0, x1, vec4, -INFINITY);
    }
    for (int i = tid; i < 2048; i += kThreads) s_h[i] = 0u;
    if (tid == 0) {
        s_dc = 0;
        s_nb = 0;
        s_nk = 0;
    }
    float M;
    int arg;
    double S, A2;
    // (no argmax: the truncated rule runs at T > 0, where the row's argmax is unused)
    chunk_reduce<EPT, false, false, false>(v, x0, x1, vec4, 0.f, M, arg, S, A2, &s_red);  // (its barrier orders the clear)
    const int lim = x1 - (x0 + (vec4 ? 4 * tid : tid));
    // Keys once, out-of-range elements as 0 (below every digit a chunk of
    // in-range keys selects: d_c is found over the counted keys only).
    uint32_t kk[EPT];
    uint32_t inr = 0u;  // bit e: element e in range
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const bool in = FULL || elem_off(e, vec4) < lim;
        if constexpr (!FULL) inr |= static_cast<uint32_t>(in) << e;
        kk[e] = logit_key(v.v[e]);
        if (in) atomicAdd(&s_h[kk[e] >> 21], 1u);
    }
    __syncthreads();
    // d_c: thread t sums the eight digits 2047 - 8t - 7 .. 2047 - 8t; a
    // block scan from the top finds where the chunk's count reaches k (a
    // chunk of fewer than k keys keeps d_c = 0: all of its digits).
    constexpr int kPer = 2048 / kThreads;
    uint32_t mine = 0u;
#pragma unroll
    for (int j = 0; j < kPer; ++j) mine += s_h[2047 - kPer * tid - j];
    uint32_t incl = mine;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    if (lane == 63) s_wt[wv] = incl;
    __syncthreads();
    for (int w = 0; w < wv; ++w) incl += s_wt[w];
    const uint32_t k = static_cast<uint32_t>(a.top_k), excl = incl - mine;
    if (excl < k && k <= incl) {  // the crossing lies in this thread's digits
        uint32_t run = excl;
        for (int j = 0; j < kPer; ++j) {
            const int bin = 2047 - kPer * tid - j;
            run += s_h[bin];
            if (run >= k) {
                s_dc = bin;
                break;
            }
        }
    }
    __syncthreads();
    const int dc = s_dc;
    const size_t slot = static_cast<size_t>(rid) * a.nchunk + c;
    uint32_t* bins = a.fbins + slot * kFBinCap;
    for (int i = tid; i < 2048; i += kThreads) {
        const uint32_t n = s_h[i];
        if (n && i >= dc) {
            const int at = atomicAdd(&s_nb, 1);
            if (at < kFBinCap) bins[at] = (static_cast<uint32_t>(i) << 20) | n;
        }
    }
    // The keys of those digits: every element's ballot first, one LDS
    // atomic for the wave's total, then each key at its place.
    uint32_t* keys = a.fkeys + slot * kFKeyCap;
    uint64_t m[EPT];
    int total = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        m[e] = __ballot((FULL || ((inr >> e) & 1u)) && static_cast<int>(kk[e] >> 21) >= dc);
        total += __popcll(m[e]);
    }
    if (total > 0) {  // wave-uniform
        int base = 0;
        if (lane == 0) base = atomicAdd(&s_nk, total);
        base = __shfl(base, 0);
        const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            if (m[e] == 0ull) continue;  // wave-uniform: most elements have no match in the wave
            const int at = base + __popcll(m[e] & below);
            if (((m[e] >> lane) & 1ull) && at < kFKeyCap) keys[at] = kk[e];
            base += __popcll(m[e]);
        }
    }
    __syncthreads();
    if (tid == 0) a.frec[slot] = ChunkRec{M, arg, min(s_nb, kFBinCap + 1), min(s_nk, kFKeyCap + 1)};
}

template <int EPT, bool NT>
__global__ __launch_bounds__(kThreads) void filt_chunk(AcceptArgs a) {
    if (a.vec4 != 0 && (static_cast<int>(blockIdx.x) + 1) * a.chunk <= a.V)  // workgroup-uniform
        filt_chunk_body<EPT, NT, true>(a);
    else
        filt_chunk_body<EPT, NT, false>(a);
}

// (from at most kFCandRow candidates: four waves keep the selection's
// many barriers cheap)
__global__ __launch_bounds__(kFSplitThreads) void accept_filter_split(AcceptArgs a) {
    filter_row<kFSplitThreads>(a, blockIdx.x, true);
}

// ---------------------------------------------------------------------------
AcceptPlan plan_accept(int B, int N, int V) {
    AcceptPlan p{};
    p.chunk = accept_ept(B, N, V) * kThreads;
    p.nchunk = (V + p.chunk - 1) / p.chunk;
    size_t off = 0;
    p.off_rowstat = off;
    off = align_up(off + static_cast<size_t>(B) * N * p.nchunk * sizeof(RowStat), 256);
    p.off_dec = off;
    off = align_up(off + static_cast<size_t>(B) * sizeof(Decision), 256);
    p.off_cstat = off;
    off = align_up(off + static_cast<size_t>(B) * p.nchunk * sizeof(ChunkStat), 256);
    p.off_cslice = off;
    off = align_up(off + static_cast<size_t>(B) * p.nchunk * kSubMax * sizeof(double), 256);
    p.ws_bytes = off;
    const size_t slots = static_cast<size_t>(B) * N * p.nchunk;
    p.off_frec = off;
    off = align_up(off + slots * sizeof(ChunkRec), 256);
    p.off_fbins = off;
    off = align_up(off + slots * kFBinCap * sizeof(uint32_t), 256);
    p.off_fkeys = off;
    off = align_up(off + slots * kFKeyCap * sizeof(uint32_t), 256);
    p.ws_filt_bytes = off;
    return p;
}

int max_accept_vocab() { return kMaxChunks * 32 * kThreads; }

template <int EPT, bool FILT>
static int launch_accept_ept(const AcceptArgs& a, const AcceptPlan& p, hipStream_t stream) {
    if (FILT && a.frec) {  // every row's truncation, each row over its chunks
        // (non-temporal row loads above 16 MB of rows, as for the statistics)
        if (static_cast<size_t>(a.B) * a.N * a.V * sizeof(float) > (16u << 20))
            hipLaunchKernelGGL((filt_chunk<EPT, true>), dim3(p.nchunk, a.B * a.N), dim3(kThreads), 0, stream, a);
        else
            hipLaunchKernelGGL((filt_chunk<EPT, false>), dim3(p.nchunk, a.B * a.N), dim3(kThreads), 0, stream, a);
        hipLaunchKernelGGL(accept_filter_split, dim3(a.B * a.N), dim3(kFSplitThreads), 0, stream, a);
        if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    } else if (FILT) {  // every row's truncation (the stop row may be a leaf)
        hipLaunchKernelGGL(accept_filter, dim3(a.B * a.N), dim3(kFThreads), 0, stream, a);
        if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    } else if (a.N > 1) {
        // The rejection rule at T > 0 needs neither the argmax (one-hot at
        // T = 0, greedy final token of the typical rule) nor the entropy.
        // Rows of at most 16 MB in all stay cached (a B = 1 chain: 0.65 us
        // less per call; non-temporal loads for larger batches: 2-3 us less).
        const dim3 grid(p.nchunk, a.N, a.B);
        const bool nt = static_cast<size_t>(a.B) * a.N * a.V * sizeof(float) > (16u << 20);
        if (a.rule == 0 && a.T > 0.f) {
            if (nt) hipLaunchKernelGGL((accept_rowstats<EPT, false, false, true>), grid, dim3(kThreads), 0, stream, a);
            else hipLaunchKernelGGL((accept_rowstats<EPT, false, false, false>), grid, dim3(kThreads), 0, stream, a);
        } else {
            if (nt) hipLaunchKernelGGL((accept_rowstats<EPT, true, true, true>), grid, dim3(kThreads), 0, stream, a);
            else hipLaunchKernelGGL((accept_rowstats<EPT, true, true, false>), grid, dim3(kThreads), 0, stream, a);
        }
        if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    }
    // The decision loads one chunk record per lane and combining pass; a wave
    // owns a quarter of the rows and combines 64 / L of them per pass (L the
    // lanes of a row's chunk segment).  Fewer passes need fewer registers and
    // loads: more workgroups per CU.  The truncated rule reads row records.
    const int nrows = a.N - 1 + (a.parent != nullptr);
    const int passes = FILT ? 1 : (((nrows + 3) / 4) + (64 >> a.lg_seg) - 1) / (64 >> a.lg_seg);
    const dim3 sgrid(p.nchunk, a.B);
    if (passes <= 1)
        hipLaunchKernelGGL((accept_sample<EPT, 1, FILT>), sgrid, dim3(kThreads), 0, stream, a);
    else if (passes <= 2)
        hipLaunchKernelGGL((accept_sample<EPT, 2, FILT>), sgrid, dim3(kThreads), 0, stream, a);
    else if (passes <= 4)
        hipLaunchKernelGGL((accept_sample<EPT, 4, FILT>), sgrid, dim3(kThreads), 0, stream, a);
    else
        hipLaunchKernelGGL((accept_sample<EPT, kRowsPerWave, FILT>), sgrid, dim3(kThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    hipLaunchKernelGGL((accept_select<EPT, FILT>), dim3(a.B), dim3(kThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
}

int launch_accept(int rule, int B, int N, int V, const float* logits, const float* draft,
                  const int32_t* tokens, const int32_t* parent, const float* u_accept,
                  const float* u_sample, float temperature, float epsilon, float delta,
                  int32_t* accept_len, int32_t* path, int32_t* out_tokens, void* workspace,
                  const AcceptPlan& p, hipStream_t stream, int top_k, float top_p, bool split_filter) {
    AcceptArgs a;
    a.logits = logits;
    a.draft = draft;
    a.tokens = tokens;
    a.parent = parent;
    a.u_acc = u_accept;
    a.u_smp = u_sample;
    a.accept_len = accept_len;
    a.path = path;
    a.out_tokens = out_tokens;
    char* ws = static_cast<char*>(workspace);
    a.rowstat = reinterpret_cast<RowStat*>(ws + p.off_rowstat);
    a.rowrec = reinterpret_cast<RowRec*>(ws + p.off_rowstat);  // B*N records fit in B*N*nchunk RowStats
    a.dec = reinterpret_cast<Decision*>(ws + p.off_dec);
    a.cstat = reinterpret_cast<ChunkStat*>(ws + p.off_cstat);
    a.cslice = reinterpret_cast<double*>(ws + p.off_cslice);
    a.B = B;
    a.N = N;
    a.V = V;
    a.chunk = p.chunk;
    a.nchunk = p.nchunk;
    a.rule = rule;
    a.lg_seg = 0;
    while ((1 << a.lg_seg) < std::min(p.nchunk, 64)) ++a.lg_seg;
    a.vec4 = (V % 4 == 0) && (reinterpret_cast<uintptr_t>(logits) % 16 == 0) &&
             (draft == nullptr || reinterpret_cast<uintptr_t>(draft) % 16 == 0);
    a.T = temperature;
    a.eps = epsilon;
    a.delta = delta;
    a.top_k = top_k > 0 && top_k < V ? top_k : 0;
    a.top_p = top_p < 1.f ? top_p : 1.f;
    // Truncation applies to the rejection rule at T > 0 (at T = 0 the target
    // is the argmax, which every truncation keeps).
    const bool filt = rule == 0 && temperature > 0.f && (a.top_k > 0 || a.top_p < 1.f);
    // The chunk passes find the top-k digit; a nucleus alone stays whole-row.
    const bool split = filt && split_filter && a.top_k > 0 && static_cast<long>(B) * N * p.nchunk <= kFMaxSlots;
    a.frec = split ? reinterpret_cast<ChunkRec*>(ws + p.off_frec) : nullptr;
    a.fbins = split ? reinterpret_cast<uint32_t*>(ws + p.off_fbins) : nullptr;
    a.fkeys = split ? reinterpret_cast<uint32_t*>(ws + p.off_fkeys) : nullptr;
    static_assert(sizeof(RowRec) <= sizeof(RowStat), "row records reuse the row-statistics space");
    switch (p.chunk / kThreads) {
        case 8: return filt ? launch_accept_ept<8, true>(a, p, stream) : launch_accept_ept<8, false>(a, p, stream);
        case 16: return filt ? launch_accept_ept<16, true>(a, p, stream) : launch_accept_ept<16, false>(a, p, stream);
        default: return filt ? launch_accept_ept<32, true>(a, p, stream) : launch_accept_ept<32, false>(a, p, stream);
    }
}

}  // namespace specv
