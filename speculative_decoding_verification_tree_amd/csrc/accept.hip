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
//                   chunk that holds u * total and the token inside it (block
//                   scan, ascending token ids).
#include "spec_common.h"
#include "spec_internal.h"

namespace specv {

struct RowStat {  // per (request, node row, chunk)
    double S;     // sum exp((l - M)/T) over the chunk
    double A;     // sum t * exp(t), t = (l - M)/T
    float M;      // chunk max logit
    int arg;      // lowest index of the chunk max
};

enum { MODE_DONE = 0, MODE_RESID = 1, MODE_BONUS = 2, MODE_ARGMAX = 3 };

struct Decision {  // per request
    double S;      // stop row: sum exp((l - M)/T) over the whole row
    float M;       // stop row: max logit
    float u;       // u_sample at the stop node
    int mode, v, c, a;
};

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
    Decision* dec;
    ChunkStat* cstat;
    int B, N, V, chunk, nchunk, rule;  // rule 0 = rejection, 1 = typical
    int vec4;                          // rows are 16-byte aligned: 16-byte loads
    float T, eps, delta;
};

constexpr int kThreads = 256;

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

__device__ __forceinline__ void block_sum2_d(double& a, double& b, double* s_red) {
    a = wave_sum(a);
    b = wave_sum(b);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) {
        s_red[wv] = a;
        s_red[4 + wv] = b;
    }
    __syncthreads();
    a = s_red[0] + s_red[1] + s_red[2] + s_red[3];
    b = s_red[4] + s_red[5] + s_red[6] + s_red[7];
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

// p_v(x) as the residual and sampling passes evaluate it (fp32).
__device__ __forceinline__ float target_prob(float l, float M, float T, float invS) {
    return expf((l - M) / T) * invS;
}

// Element e of this thread's share of a chunk starting at x0: strided by
// the block (coalesced), in runs of four with 16-byte loads.
__device__ __forceinline__ int elem_index(int x0, int e, bool vec4) {
    return vec4 ? x0 + 4 * (static_cast<int>(threadIdx.x) + kThreads * (e >> 2)) + (e & 3)
                : x0 + static_cast<int>(threadIdx.x) + kThreads * e;
}

template <int EPT>
struct Vals {
    float v[EPT];
};

template <int EPT>
__device__ __forceinline__ Vals<EPT> load_chunk(const float* row, int x0, int x1, bool vec4, float fill) {
    Vals<EPT> r;
    if (vec4) {
#pragma unroll
        for (int j = 0; j < EPT / 4; ++j) {
            const int x = x0 + 4 * (static_cast<int>(threadIdx.x) + kThreads * j);
            if (x + 3 < x1) {
                const float4 v = *reinterpret_cast<const float4*>(row + x);
                r.v[4 * j] = v.x;
                r.v[4 * j + 1] = v.y;
                r.v[4 * j + 2] = v.z;
                r.v[4 * j + 3] = v.w;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) r.v[4 * j + k] = x + k < x1 ? row[x + k] : fill;
            }
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int x = x0 + static_cast<int>(threadIdx.x) + kThreads * e;
            r.v[e] = x < x1 ? row[x] : fill;
        }
    }
    return r;
}

// Chunk statistics of one target row: lowest-index argmax, then (T > 0) the
// exp sums relative to the chunk max.
template <int EPT>
__device__ __forceinline__ void row_chunk_stats(const float* row, int x0, int x1, bool vec4, float T, float& best, int& bi,
                                double& S, double& A, float* s_v, int* s_i, double* s_red) {
    const Vals<EPT> vals = load_chunk<EPT>(row, x0, x1, vec4, -INFINITY);
    const float* val = vals.v;
    best = -INFINITY;
    bi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int x = elem_index(x0, e, vec4);
        if (x < x1 && (val[e] > best || (val[e] == best && x < bi))) {
            best = val[e];
            bi = x;
        }
    }
    block_argmax(best, bi, s_v, s_i);
    S = 0.0;
    A = 0.0;
    if (T > 0.f) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            if (elem_index(x0, e, vec4) < x1) {
                const float t = (val[e] - best) / T;
                const float ex = expf(t);
                S += static_cast<double>(ex);
                A += static_cast<double>(t) * static_cast<double>(ex);
            }
        }
        block_sum2_d(S, A, s_red);
    }
}

// ---------------------------------------------------------------------------
// Parent array of request b in LDS, and which nodes have children.
__device__ __forceinline__ void load_tree(const AcceptArgs& a, int b, int* s_par, int* s_has) {
    const int tid = threadIdx.x;
    if (tid < kMaxNodes) s_has[tid] = 0;
    if (tid < a.N) s_par[tid] = tree_parent(a.parent, a.N, b, tid);
    __syncthreads();
    if (tid > 0 && tid < a.N && s_par[tid] >= 0) s_has[s_par[tid]] = 1;
    __syncthreads();
}

// Decision of request b from the chunk statistics.  Every accept_sample
// workgroup of the request computes it (same inputs, same code, same result);
// only the writer stores path, accepted tokens, accept_len and the record.
// (Templated on the caller's chunk width only so that each kernel owns its
// copy of the LDS arrays below.)
template <int EPT>
__device__ __forceinline__ void decide_request(const AcceptArgs& a, int b, bool writer, const int* s_par, const int* s_has,
                               Decision* s_dec) {
    const int N = a.N, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ float s_M[kMaxNodes];
    __shared__ int s_arg[kMaxNodes];
    __shared__ double s_S[kMaxNodes], s_H[kMaxNodes];
    __shared__ int s_path[kMaxNodes], s_depth[kMaxNodes];

    // Whole-row statistics: wave w owns rows w, w+4, ...  Lane c first loads
    // chunk c of every row it serves in one round of independent loads; only
    // vocabularies of more than 64 chunks take the extra loops.
    const double T = a.T;
    float mc[kRowsPerWave], m[kRowsPerWave];
    int ac[kRowsPerWave], ar[kRowsPerWave];
    double sc[kRowsPerWave], scA[kRowsPerWave];
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
        const int u = wave + 4 * k;
        mc[k] = -INFINITY;
        ac[k] = 0x7fffffff;
        sc[k] = 0.0;
        scA[k] = 0.0;
        if (u < N && s_has[u] && lane < a.nchunk) {
            const RowStat r = a.rowstat[(static_cast<size_t>(b) * N + u) * a.nchunk + lane];
            mc[k] = r.M;
            ac[k] = r.arg;
            sc[k] = r.S;
            scA[k] = r.A;
        }
    }
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
        m[k] = mc[k];
        ar[k] = ac[k];
        const int u = wave + 4 * k;
        if (u < N && s_has[u]) {  // wave-uniform
            for (int c = lane + 64; c < a.nchunk; c += 64) {
                const RowStat& r = a.rowstat[(static_cast<size_t>(b) * N + u) * a.nchunk + c];
                if (r.M > m[k] || (r.M == m[k] && r.arg < ar[k])) {
                    m[k] = r.M;
                    ar[k] = r.arg;
                }
            }
            wave_argmax(m[k], ar[k]);
        }
    }
    if (T > 0.0) {
#pragma unroll
        for (int k = 0; k < kRowsPerWave; ++k) {
            const int u = wave + 4 * k;
            double S = 0.0, A = 0.0;
            if (u < N && s_has[u]) {
                if (lane < a.nchunk) {
                    const double dl = (static_cast<double>(mc[k]) - m[k]) / T;
                    const double wgt = exp(dl);
                    S = wgt * sc[k];
                    A = wgt * (scA[k] + dl * sc[k]);
                }
                for (int c = lane + 64; c < a.nchunk; c += 64) {
                    const RowStat r = a.rowstat[(static_cast<size_t>(b) * N + u) * a.nchunk + c];
                    const double dl = (static_cast<double>(r.M) - m[k]) / T;
                    const double wgt = exp(dl);
                    S += wgt * r.S;
                    A += wgt * (r.A + dl * r.S);
                }
            }
            if (u < N && s_has[u]) {  // wave-uniform
                S = wave_sum(S);
                A = wave_sum(A);
                if (lane == 0) {
                    s_S[u] = S;
                    s_H[u] = log(S) - A / S;
                }
            }
        }
    }
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
        const int u = wave + 4 * k;
        if (lane == 0 && u < N && s_has[u]) {
            s_M[u] = m[k];
            s_arg[u] = ar[k];
            if (!(T > 0.0)) {
                s_S[u] = 0.0;
                s_H[u] = 0.0;
            }
        }
    }
    __syncthreads();

    if (wave == 0) {
        // Per-node tests in fp64 from the gathered values (nodes live in wave 0).
        bool ok = false;
        if (lane >= 1 && lane < N) {
            const int u = s_par[lane];
            if (u >= 0) {
                int x = a.tokens[static_cast<size_t>(b) * N + lane];
                x = min(max(x, 0), a.V - 1);
                double pu;
                if (T > 0.0) {
                    const double l = a.logits[(static_cast<size_t>(b) * N + u) * a.V + x];
                    pu = exp((l - static_cast<double>(s_M[u])) / T) / s_S[u];
                } else {
                    pu = x == s_arg[u] ? 1.0 : 0.0;
                }
                if (a.rule == 0) {
                    const double qx = a.draft[(static_cast<size_t>(b) * N + lane) * a.V + x];
                    ok = static_cast<double>(a.u_acc[static_cast<size_t>(b) * N + lane]) * qx < pu;
                } else {
                    const double thr =
                        fmin(static_cast<double>(a.eps), static_cast<double>(a.delta) * exp(-s_H[u]));
                    ok = pu > thr;
                }
            }
        }
        const unsigned long long okm = __ballot(ok);
        if (lane == 0) {
            uint64_t acc = 1ull;  // the root is always accepted
            s_depth[0] = 0;
            int v = 0, dv = 0;
            for (int i = 1; i < N; ++i) {
                const int u = s_par[i];
                const int di = u >= 0 ? s_depth[u] + 1 : 0;
                s_depth[i] = di;
                if (u >= 0 && ((okm >> i) & 1ull) && ((acc >> u) & 1ull)) {
                    acc |= 1ull << i;
                    if (di > dv) {
                        v = i;
                        dv = di;
                    }
                }
            }
            for (int n = v, d = dv; d >= 0; n = s_par[n], --d) s_path[d] = n;
            int c = -1;
            for (int i = v + 1; i < N && c < 0; ++i)
                if (s_par[i] == v) c = i;
            Decision d;
            d.v = v;
            d.c = c;
            d.a = dv;
            d.u = a.u_smp ? a.u_smp[static_cast<size_t>(b) * N + v] : 0.f;
            d.M = s_has[v] ? s_M[v] : 0.f;
            d.S = s_has[v] ? s_S[v] : 0.0;
            if (a.rule == 1 || !(T > 0.0))
                d.mode = s_has[v] ? MODE_DONE : MODE_ARGMAX;
            else
                d.mode = s_has[v] ? MODE_RESID : MODE_BONUS;
            *s_dec = d;
        }
    }
    __syncthreads();
    if (writer) {
        const Decision d = *s_dec;
        if (tid < N) {
            const size_t o = static_cast<size_t>(b) * N + tid;
            a.path[o] = tid <= d.a ? s_path[tid] : -1;
            int tok = tid < d.a ? a.tokens[static_cast<size_t>(b) * N + s_path[tid + 1]] : -1;
            if (tid == d.a && d.mode == MODE_DONE) tok = s_arg[d.v];
            a.out_tokens[o] = tok;
        }
        if (tid == 0) {
            a.accept_len[b] = d.a;
            a.dec[b] = d;
        }
    }
}

template <int EPT>
__global__ __launch_bounds__(kThreads) void accept_rowstats(AcceptArgs a) {
    const int c = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
    __shared__ int s_par[kMaxNodes], s_has[kMaxNodes];
    __shared__ double s_red[8];
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    load_tree(a, b, s_par, s_has);
    if (!s_has[u]) return;  // leaves need no statistics
    const float* row = a.logits + (static_cast<size_t>(b) * a.N + u) * a.V;
    const int x0 = c * a.chunk, x1 = min(x0 + a.chunk, a.V);
    float best;
    int bi;
    double S, A;
    row_chunk_stats<EPT>(row, x0, x1, a.vec4 != 0, a.T, best, bi, S, A, s_v, s_i, s_red);
    if (threadIdx.x == 0) {
        RowStat rs;
        rs.S = S;
        rs.A = A;
        rs.M = best;
        rs.arg = bi;
        a.rowstat[(static_cast<size_t>(b) * a.N + u) * a.nchunk + c] = rs;
    }
}

template <int EPT>
__global__ __launch_bounds__(kThreads) void accept_sample(AcceptArgs a) {
    const int c = blockIdx.x, b = blockIdx.y;
    __shared__ int s_par[kMaxNodes], s_has[kMaxNodes];
    __shared__ Decision s_dec;
    __shared__ double s_red[8];
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    load_tree(a, b, s_par, s_has);
    decide_request<EPT>(a, b, c == 0, s_par, s_has, &s_dec);
    const Decision d = s_dec;
    if (d.mode == MODE_DONE) return;
    const float* row = a.logits + (static_cast<size_t>(b) * a.N + d.v) * a.V;
    const int x0 = c * a.chunk, x1 = min(x0 + a.chunk, a.V);
    ChunkStat cs;
    cs.m1 = cs.m2 = 0.0;
    cs.M = 0.f;
    cs.arg = 0;
    const bool vec4 = a.vec4 != 0;
    if (d.mode == MODE_RESID) {
        const float* qrow = a.draft + (static_cast<size_t>(b) * a.N + d.c) * a.V;
        const float invS = static_cast<float>(1.0 / d.S);
        const Vals<EPT> lvals = load_chunk<EPT>(row, x0, x1, vec4, -INFINITY);
        const Vals<EPT> qvals = load_chunk<EPT>(qrow, x0, x1, vec4, 0.f);
        const float* lv = lvals.v;
        const float* qv = qvals.v;
        double r = 0.0, p = 0.0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            if (elem_index(x0, e, vec4) < x1) {
                const float pv = target_prob(lv[e], d.M, a.T, invS);
                r += static_cast<double>(fmaxf(pv - qv[e], 0.f));
                p += static_cast<double>(pv);
            }
        }
        block_sum2_d(r, p, s_red);
        cs.m1 = r;
        cs.m2 = p;
    } else {
        float best;
        int bi;
        double S, A;
        row_chunk_stats<EPT>(row, x0, x1, vec4, d.mode == MODE_BONUS ? a.T : 0.f, best, bi, S, A, s_v, s_i, s_red);
        cs.M = best;
        cs.arg = bi;
        cs.m1 = S;
    }
    if (threadIdx.x == 0) a.cstat[static_cast<size_t>(b) * a.nchunk + c] = cs;
}

// ---------------------------------------------------------------------------
template <int EPT>
__global__ __launch_bounds__(kThreads) void accept_select(AcceptArgs a) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    __shared__ Decision s_d;
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    __shared__ double s_red[8];
    __shared__ double s_w[kMaxChunks];
    __shared__ double s_scan[kThreads];
    __shared__ float s_wt[EPT * kThreads];
    __shared__ int s_pick;
    __shared__ double s_base;
    if (tid == 0) s_d = a.dec[b];
    __syncthreads();
    const Decision d = s_d;
    if (d.mode == MODE_DONE) return;
    const ChunkStat* cs = a.cstat + static_cast<size_t>(b) * a.nchunk;
    int32_t* out = a.out_tokens + static_cast<size_t>(b) * a.N + d.a;

    if (d.mode == MODE_ARGMAX) {
        float best = -INFINITY;
        int bi = 0x7fffffff;
        for (int c = tid; c < a.nchunk; c += kThreads)
            if (cs[c].M > best || (cs[c].M == best && cs[c].arg < bi)) {
                best = cs[c].M;
                bi = cs[c].arg;
            }
        block_argmax(best, bi, s_v, s_i);
        if (tid == 0) *out = bi;
        return;
    }

    // Chunk weights in token order.
    const double T = a.T;
    double Mg = -INFINITY, tot1 = 0.0;
    if (d.mode == MODE_BONUS) {
        float mloc = -INFINITY;
        int dummy = 0;
        for (int c = tid; c < a.nchunk; c += kThreads) mloc = fmaxf(mloc, cs[c].M);
        block_argmax(mloc, dummy, s_v, s_i);
        Mg = mloc;
    } else {
        double t1 = 0.0;
        for (int c = tid; c < a.nchunk; c += kThreads) t1 += cs[c].m1;
        tot1 = block_sum_d(t1, s_red);
    }
    const bool usep = d.mode == MODE_RESID && !(tot1 > 0.0);  // all-zero residual: fall back to p_v
    for (int c = tid; c < a.nchunk; c += kThreads)
        s_w[c] = d.mode == MODE_BONUS ? cs[c].m1 * exp((static_cast<double>(cs[c].M) - Mg) / T)
                                      : (usep ? cs[c].m2 : cs[c].m1);
    __syncthreads();
    // Inclusive scan of the chunk weights: each thread owns a run of chunks.
    const int per = (a.nchunk + kThreads - 1) / kThreads;
    const int c0 = tid * per, c1 = min(c0 + per, a.nchunk);
    double run = 0.0;
    for (int c = c0; c < c1; ++c) run += s_w[c];
    s_scan[tid] = run;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const double add = tid >= off ? s_scan[tid - off] : 0.0;
        __syncthreads();
        s_scan[tid] += add;
        __syncthreads();
    }
    const double total = s_scan[kThreads - 1];
    const double t = static_cast<double>(d.u) * total;
    double cum = s_scan[tid] - run;
    int hit = 0x7fffffff, lastc = -1;
    double hit_base = 0.0;
    for (int c = c0; c < c1; ++c) {
        if (s_w[c] > 0.0) {
            lastc = c;
            if (hit == 0x7fffffff && cum + s_w[c] > t) {
                hit = c;
                hit_base = cum;
            }
        }
        cum += s_w[c];
    }
    // smallest chunk with a hit, else the last chunk with weight
    float fh = hit == 0x7fffffff ? -INFINITY : -static_cast<float>(hit);
    int ih = hit;
    block_argmax(fh, ih, s_v, s_i);
    float fl = static_cast<float>(lastc);
    int il = -lastc;
    block_argmax(fl, il, s_v, s_i);
    if (tid == 0) {
        s_pick = ih != 0x7fffffff ? ih : max(-il, 0);
        s_base = ih != 0x7fffffff ? 0.0 : -INFINITY;  // -inf: take the last token with weight
    }
    __syncthreads();
    if (ih != 0x7fffffff && hit == ih) s_base = hit_base;
    __syncthreads();

    // Token inside the chosen chunk.  Weights are computed from coalesced
    // loads and staged in LDS (fp32, the same values accept_sample summed);
    // each thread then scans a contiguous run in ascending token order.
    const int pc = s_pick;
    const int x0 = pc * a.chunk, x1 = min(x0 + a.chunk, a.V);
    const bool vec4 = a.vec4 != 0;
    const float* row = a.logits + (static_cast<size_t>(b) * a.N + d.v) * a.V;
    const float* qrow = d.mode == MODE_RESID ? a.draft + (static_cast<size_t>(b) * a.N + d.c) * a.V : nullptr;
    const float invS = d.mode == MODE_RESID ? static_cast<float>(1.0 / d.S) : 0.f;
    const float Mc = cs[pc].M;
    const double scale = d.mode == MODE_BONUS ? exp((static_cast<double>(Mc) - Mg) / T) : 1.0;
    {
        const Vals<EPT> lvals = load_chunk<EPT>(row, x0, x1, vec4, -INFINITY);
        const Vals<EPT> qvals = d.mode == MODE_RESID ? load_chunk<EPT>(qrow, x0, x1, vec4, 0.f) : Vals<EPT>{};
        const float* lv = lvals.v;
        const float* qv = qvals.v;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int x = elem_index(x0, e, vec4);
            float wgt = 0.f;
            if (x < x1) {
                if (d.mode == MODE_RESID) {
                    const float pv = target_prob(lv[e], d.M, a.T, invS);
                    wgt = usep ? pv : fmaxf(pv - qv[e], 0.f);
                } else {
                    wgt = expf((lv[e] - Mc) / a.T);
                }
            }
            if (x - x0 < EPT * kThreads) s_wt[x - x0] = wgt;
        }
    }
    __syncthreads();
    const int xs = x0 + tid * EPT;
    double wv[EPT];
    run = 0.0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        wv[e] = static_cast<double>(s_wt[tid * EPT + e]) * scale;
        run += wv[e];
    }
    __syncthreads();
    s_scan[tid] = run;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const double add = tid >= off ? s_scan[tid - off] : 0.0;
        __syncthreads();
        s_scan[tid] += add;
        __syncthreads();
    }
    cum = s_base + (s_scan[tid] - run);
    int xhit = 0x7fffffff, lastnz = -1;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int x = xs + e;
        if (wv[e] > 0.0) {
            lastnz = x;
            cum += wv[e];
            if (xhit == 0x7fffffff && cum > t) xhit = x;
        }
    }
    float fx = xhit == 0x7fffffff ? -INFINITY : -static_cast<float>(xhit);
    int ix = xhit;
    block_argmax(fx, ix, s_v, s_i);
    float fz = static_cast<float>(lastnz);
    int iz = -lastnz;
    block_argmax(fz, iz, s_v, s_i);
    if (tid == 0) {
        int final = ix != 0x7fffffff ? ix : -iz;
        if (final < 0) final = x0;
        *out = final;
    }
}

// ---------------------------------------------------------------------------
// Entries per thread and chunk: 8, raised to 16 or 32 for large batches so
// the statistics kernel launches at most ~8k workgroups of useful size.
static int accept_ept(int B, int N, int V) {
    int ept = 8;
    auto nchunk = [&](int e) { return (V + e * kThreads - 1) / (e * kThreads); };
    while (ept < 32 && (static_cast<long>(B) * N * nchunk(ept) > 8192 || nchunk(ept) > kMaxChunks)) ept *= 2;
    return ept;
}

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
    p.ws_bytes = off;
    return p;
}

int max_accept_vocab() { return kMaxChunks * 32 * kThreads; }

template <int EPT>
static int launch_accept_ept(const AcceptArgs& a, const AcceptPlan& p, hipStream_t stream) {
    if (a.N > 1) {
        hipLaunchKernelGGL((accept_rowstats<EPT>), dim3(p.nchunk, a.N, a.B), dim3(kThreads), 0, stream, a);
        if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    }
    hipLaunchKernelGGL((accept_sample<EPT>), dim3(p.nchunk, a.B), dim3(kThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    hipLaunchKernelGGL((accept_select<EPT>), dim3(a.B), dim3(kThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
}

int launch_accept(int rule, int B, int N, int V, const float* logits, const float* draft,
                  const int32_t* tokens, const int32_t* parent, const float* u_accept,
                  const float* u_sample, float temperature, float epsilon, float delta,
                  int32_t* accept_len, int32_t* path, int32_t* out_tokens, void* workspace,
                  const AcceptPlan& p, hipStream_t stream) {
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
    a.dec = reinterpret_cast<Decision*>(ws + p.off_dec);
    a.cstat = reinterpret_cast<ChunkStat*>(ws + p.off_cstat);
    a.B = B;
    a.N = N;
    a.V = V;
    a.chunk = p.chunk;
    a.nchunk = p.nchunk;
    a.rule = rule;
    a.vec4 = (V % 4 == 0) && (reinterpret_cast<uintptr_t>(logits) % 16 == 0) &&
             (draft == nullptr || reinterpret_cast<uintptr_t>(draft) % 16 == 0);
    a.T = temperature;
    a.eps = epsilon;
    a.delta = delta;
    switch (p.chunk / kThreads) {
        case 8: return launch_accept_ept<8>(a, p, stream);
        case 16: return launch_accept_ept<16>(a, p, stream);
        default: return launch_accept_ept<32>(a, p, stream);
    }
}

}  // namespace specv
