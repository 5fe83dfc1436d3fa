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
// Kernels, in stream order:
//   accept_rowstats  grid (chunks, N, B): for every node row that has
//                    children, per vocabulary chunk: max logit (+ lowest
//                    argmax), sum exp((l - max)/T) and sum t*exp(t) (entropy)
//   accept_decide    grid B, one wavefront: combine the chunk statistics,
//                    run every node's test in fp64 from the gathered logit and
//                    draft probability, pick the stop node and write path /
//                    accepted tokens; decide what the last token needs
//   accept_chunks    grid (chunks, B): per chunk of the stop row, the residual
//                    mass, the bonus mass or the argmax
//   accept_select    grid B: pick the chunk holding u * total by an ordered
//                    scan of the chunk masses, then the token by a block scan
//                    inside that chunk (ascending token ids)
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
    double m1;      // residual mass | bonus mass relative to M
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
    float T, eps, delta;
};

constexpr int kThreads = 256;

// Block-wide reductions (256 threads = 4 waves).
__device__ double block_sum_d(double v, double* s_red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) s_red[wv] = v;
    __syncthreads();
    return s_red[0] + s_red[1] + s_red[2] + s_red[3];
}

__device__ void block_argmax(float& v, int& i, float* s_v, int* s_i) {
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

// p_v(x) as the stop-row residual and sampling kernels evaluate it (fp32).
__device__ __forceinline__ float target_prob(float l, float M, float T, float invS) {
    return expf((l - M) / T) * invS;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void accept_rowstats(AcceptArgs a) {
    const int c = blockIdx.x, u = blockIdx.y, b = blockIdx.z;
    __shared__ int s_has;
    __shared__ double s_red[4];
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    if (threadIdx.x == 0) s_has = 0;
    __syncthreads();
    for (int i = 1 + threadIdx.x; i < a.N; i += kThreads)
        if (tree_parent(a.parent, a.N, b, i) == u) s_has = 1;
    __syncthreads();
    if (!s_has) return;

    const float* row = a.logits + (static_cast<size_t>(b) * a.N + u) * a.V;
    const int x0 = c * a.chunk, x1 = min(x0 + a.chunk, a.V);
    constexpr int EPT = 8;  // chunk == 8 * kThreads
    float val[EPT];
    float best = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int x = x0 + threadIdx.x + e * kThreads;
        val[e] = x < x1 ? row[x] : -INFINITY;
        if (x < x1 && (val[e] > best || (val[e] == best && x < bi))) {
            best = val[e];
            bi = x;
        }
    }
    block_argmax(best, bi, s_v, s_i);
    double S = 0.0, A = 0.0;
    if (a.T > 0.f) {
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int x = x0 + threadIdx.x + e * kThreads;
            if (x < x1) {
                const float t = (val[e] - best) / a.T;
                const float ex = expf(t);
                S += static_cast<double>(ex);
                A += static_cast<double>(t) * static_cast<double>(ex);
            }
        }
        S = block_sum_d(S, s_red);
        A = block_sum_d(A, s_red);
    }
    if (threadIdx.x == 0) {
        RowStat rs;
        rs.S = S;
        rs.A = A;
        rs.M = best;
        rs.arg = bi;
        a.rowstat[(static_cast<size_t>(b) * a.N + u) * a.nchunk + c] = rs;
    }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void accept_decide(AcceptArgs a) {
    const int b = blockIdx.x, lane = threadIdx.x;
    const int N = a.N;
    __shared__ int s_par[kMaxNodes], s_has[kMaxNodes], s_arg[kMaxNodes], s_path[kMaxNodes];
    __shared__ float s_M[kMaxNodes];
    __shared__ double s_S[kMaxNodes], s_H[kMaxNodes];
    __shared__ int s_v, s_a, s_c;
    if (lane < N) {
        s_par[lane] = tree_parent(a.parent, N, b, lane);
        s_has[lane] = 0;
    }
    __syncthreads();
    if (lane > 0 && lane < N && s_par[lane] >= 0) s_has[s_par[lane]] = 1;
    __syncthreads();

    // Whole-row statistics of every node row with children.
    for (int u = 0; u < N; ++u) {
        if (!s_has[u]) continue;
        const RowStat* rs = a.rowstat + (static_cast<size_t>(b) * N + u) * a.nchunk;
        float M = -INFINITY;
        int arg = 0x7fffffff;
        for (int c = lane; c < a.nchunk; c += 64) {
            const float m = rs[c].M;
            const int i = rs[c].arg;
            if (m > M || (m == M && i < arg)) {
                M = m;
                arg = i;
            }
        }
        wave_argmax(M, arg);
        double S = 0.0, A = 0.0;
        if (a.T > 0.f) {
            const double T = a.T;
            for (int c = lane; c < a.nchunk; c += 64) {
                const double dl = (static_cast<double>(rs[c].M) - M) / T;
                const double wgt = exp(dl);
                S += wgt * rs[c].S;
                A += wgt * (rs[c].A + dl * rs[c].S);
            }
            S = wave_sum(S);
            A = wave_sum(A);
        }
        if (lane == 0) {
            s_M[u] = M;
            s_arg[u] = arg;
            s_S[u] = S;
            s_H[u] = a.T > 0.f ? log(S) - A / S : 0.0;
        }
    }
    __syncthreads();

    // Per-node tests, evaluated in fp64 from the gathered values.
    bool ok = false;
    if (lane >= 1 && lane < N) {
        const int u = s_par[lane];
        if (u >= 0) {
            int x = a.tokens[static_cast<size_t>(b) * N + lane];
            x = min(max(x, 0), a.V - 1);
            double pu;
            if (a.T > 0.f) {
                const double l = a.logits[(static_cast<size_t>(b) * N + u) * a.V + x];
                pu = exp((l - static_cast<double>(s_M[u])) / static_cast<double>(a.T)) / s_S[u];
            } else {
                pu = x == s_arg[u] ? 1.0 : 0.0;
            }
            if (a.rule == 0) {
                const double qx = a.draft[(static_cast<size_t>(b) * N + lane) * a.V + x];
                ok = static_cast<double>(a.u_acc[static_cast<size_t>(b) * N + lane]) * qx < pu;
            } else {
                const double thr = fmin(static_cast<double>(a.eps), static_cast<double>(a.delta) * exp(-s_H[u]));
                ok = pu > thr;
            }
        }
    }
    const unsigned long long okm = __ballot(ok);

    if (lane == 0) {
        uint64_t acc = 1ull;  // root
        int depth[kMaxNodes];
        depth[0] = 0;
        int v = 0;
        for (int i = 1; i < N; ++i) {
            const int u = s_par[i];
            depth[i] = u >= 0 ? depth[u] + 1 : 0;
            if (u >= 0 && ((okm >> i) & 1ull) && ((acc >> u) & 1ull)) {
                acc |= 1ull << i;
                if (depth[i] > depth[v]) v = i;
            }
        }
        const int av = depth[v];
        for (int n = v, d = av; d >= 0; n = s_par[n], --d) s_path[d] = n;
        int c = -1;
        for (int i = v + 1; i < N && c < 0; ++i)
            if (s_par[i] == v) c = i;
        s_v = v;
        s_a = av;
        s_c = c;
    }
    __syncthreads();
    const int v = s_v, av = s_a, c = s_c;
    if (lane < N) {
        const size_t o = static_cast<size_t>(b) * N + lane;
        a.path[o] = lane <= av ? s_path[lane] : -1;
        a.out_tokens[o] = lane < av ? a.tokens[static_cast<size_t>(b) * N + s_path[lane + 1]] : -1;
    }
    if (lane == 0) {
        a.accept_len[b] = av;
        Decision d;
        d.v = v;
        d.c = c;
        d.a = av;
        d.u = a.u_smp ? a.u_smp[static_cast<size_t>(b) * N + v] : 0.f;
        d.M = s_has[v] ? s_M[v] : 0.f;
        d.S = s_has[v] ? s_S[v] : 0.0;
        if (a.rule == 1 || a.T == 0.f) {
            if (s_has[v]) {
                d.mode = MODE_DONE;
                a.out_tokens[static_cast<size_t>(b) * N + av] = s_arg[v];
            } else {
                d.mode = MODE_ARGMAX;
            }
        } else {
            d.mode = s_has[v] ? MODE_RESID : MODE_BONUS;
        }
        a.dec[b] = d;
    }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void accept_chunks(AcceptArgs a) {
    const int c = blockIdx.x, b = blockIdx.y;
    const Decision d = a.dec[b];
    if (d.mode == MODE_DONE) return;
    __shared__ double s_red[4];
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    const float* row = a.logits + (static_cast<size_t>(b) * a.N + d.v) * a.V;
    const int x0 = c * a.chunk, x1 = min(x0 + a.chunk, a.V);
    constexpr int EPT = 8;
    ChunkStat cs;
    cs.m1 = cs.m2 = 0.0;
    cs.M = 0.f;
    cs.arg = 0;
    if (d.mode == MODE_RESID) {
        const float* qrow = a.draft + (static_cast<size_t>(b) * a.N + d.c) * a.V;
        const float invS = static_cast<float>(1.0 / d.S);
        double r = 0.0, p = 0.0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int x = x0 + threadIdx.x + e * kThreads;
            if (x < x1) {
                const float pv = target_prob(row[x], d.M, a.T, invS);
                r += static_cast<double>(fmaxf(pv - qrow[x], 0.f));
                p += static_cast<double>(pv);
            }
        }
        cs.m1 = block_sum_d(r, s_red);
        cs.m2 = block_sum_d(p, s_red);
    } else {
        float val[EPT];
        float best = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int x = x0 + threadIdx.x + e * kThreads;
            val[e] = x < x1 ? row[x] : -INFINITY;
            if (x < x1 && (val[e] > best || (val[e] == best && x < bi))) {
                best = val[e];
                bi = x;
            }
        }
        block_argmax(best, bi, s_v, s_i);
        cs.M = best;
        cs.arg = bi;
        if (d.mode == MODE_BONUS) {
            double S = 0.0;
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const int x = x0 + threadIdx.x + e * kThreads;
                if (x < x1) S += static_cast<double>(expf((val[e] - best) / a.T));
            }
            cs.m1 = block_sum_d(S, s_red);
        }
    }
    if (threadIdx.x == 0) a.cstat[static_cast<size_t>(b) * a.nchunk + c] = cs;
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void accept_select(AcceptArgs a) {
    const int b = blockIdx.x;
    const Decision d = a.dec[b];
    if (d.mode == MODE_DONE) return;
    const int tid = threadIdx.x;
    const ChunkStat* cs = a.cstat + static_cast<size_t>(b) * a.nchunk;
    int32_t* out = a.out_tokens + static_cast<size_t>(b) * a.N + d.a;
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    __shared__ double s_scan[kThreads];
    __shared__ int s_chunk, s_usep;
    __shared__ double s_base, s_t, s_scale;
    __shared__ float s_Mc;

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

    // Ordered scan of the chunk masses (one thread, at most a few hundred chunks).
    if (tid == 0) {
        const double T = a.T;
        double Mg = -INFINITY;
        if (d.mode == MODE_BONUS)
            for (int c = 0; c < a.nchunk; ++c) Mg = fmax(Mg, static_cast<double>(cs[c].M));
        int usep = 0;
        double total = 0.0;
        for (int c = 0; c < a.nchunk; ++c) total += d.mode == MODE_RESID ? cs[c].m1 : cs[c].m1 * exp((cs[c].M - Mg) / T);
        if (d.mode == MODE_RESID && !(total > 0.0)) {
            usep = 1;
            total = 0.0;
            for (int c = 0; c < a.nchunk; ++c) total += cs[c].m2;
        }
        const double t = static_cast<double>(d.u) * total;
        double cum = 0.0, base = 0.0;
        int pick = -1, last = -1;
        for (int c = 0; c < a.nchunk; ++c) {
            const double wgt = d.mode == MODE_RESID ? (usep ? cs[c].m2 : cs[c].m1) : cs[c].m1 * exp((cs[c].M - Mg) / T);
            if (wgt > 0.0) last = c;
            if (pick < 0 && wgt > 0.0 && cum + wgt > t) {
                pick = c;
                base = cum;
            }
            cum += wgt;
        }
        if (pick < 0) {  // rounding: fall back to the last chunk with mass
            pick = last < 0 ? 0 : last;
            base = -INFINITY;
        }
        s_chunk = pick;
        s_usep = usep;
        s_base = base;
        s_t = t;
        s_Mc = cs[pick].M;
        s_scale = d.mode == MODE_BONUS ? exp((cs[pick].M - Mg) / T) : 1.0;
    }
    __syncthreads();
    const int c = s_chunk;
    const int x0 = c * a.chunk, x1 = min(x0 + a.chunk, a.V);
    constexpr int EPT = 8;
    const int xs = x0 + tid * EPT;  // contiguous run per thread: ascending order
    const float* row = a.logits + (static_cast<size_t>(b) * a.N + d.v) * a.V;
    const float* qrow = d.mode == MODE_RESID ? a.draft + (static_cast<size_t>(b) * a.N + d.c) * a.V : nullptr;
    const float invS = d.mode == MODE_RESID ? static_cast<float>(1.0 / d.S) : 0.f;
    double wv[EPT];
    double run = 0.0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int x = xs + e;
        double wgt = 0.0;
        if (x < x1) {
            if (d.mode == MODE_RESID) {
                const float pv = target_prob(row[x], d.M, a.T, invS);
                wgt = s_usep ? static_cast<double>(pv) : static_cast<double>(fmaxf(pv - qrow[x], 0.f));
            } else {
                wgt = static_cast<double>(expf((row[x] - s_Mc) / a.T)) * s_scale;
            }
        }
        wv[e] = wgt;
        run += wgt;
    }
    // exclusive scan of the per-thread totals (ascending thread order)
    s_scan[tid] = run;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
        const double add = tid >= off ? s_scan[tid - off] : 0.0;
        __syncthreads();
        s_scan[tid] += add;
        __syncthreads();
    }
    double cum = s_base + (s_scan[tid] - run);
    int hit = 0x7fffffff, lastnz = -1;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int x = xs + e;
        if (wv[e] > 0.0) {
            lastnz = x;
            cum += wv[e];
            if (hit == 0x7fffffff && cum > s_t) hit = x;
        }
    }
    // first hit (smallest token id), else the last token with weight
    float fh = hit == 0x7fffffff ? -INFINITY : -static_cast<float>(hit);
    int ih = hit;
    block_argmax(fh, ih, s_v, s_i);
    float fl = static_cast<float>(lastnz);
    int il = -lastnz;
    block_argmax(fl, il, s_v, s_i);
    if (tid == 0) {
        int final = ih != 0x7fffffff && fh != -INFINITY ? ih : -il;
        if (final < 0) final = x0;
        *out = final;
    }
}

// ---------------------------------------------------------------------------
AcceptPlan plan_accept(int B, int N, int V) {
    AcceptPlan p{};
    p.chunk = 8 * kThreads;
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
    a.T = temperature;
    a.eps = epsilon;
    a.delta = delta;
    if (N > 1) {
        hipLaunchKernelGGL(accept_rowstats, dim3(p.nchunk, N, B), dim3(kThreads), 0, stream, a);
        if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    }
    hipLaunchKernelGGL(accept_decide, dim3(B), dim3(64), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    hipLaunchKernelGGL(accept_chunks, dim3(p.nchunk, B), dim3(kThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    hipLaunchKernelGGL(accept_select, dim3(B), dim3(kThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    return SPEC_OK;
}

}  // namespace specv
