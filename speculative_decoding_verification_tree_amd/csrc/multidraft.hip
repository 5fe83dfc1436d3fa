// Multi-draft tree rejection by recursive residuals on gfx950, several
// workgroups per request.
//
// The rule (a reading of the "Speculative Sampling" and MEDUSA sections of
// the blog page "Fast Inference from Transformers via Speculative
// Decoding"): starting at the root v with r = p_v, the children c of v are
// tested in ascending index, c with token x passing when
// u_accept[c] * q_c(x) < r(x); a rejected child replaces r by
// norm(max(0, r - q_c)) (kept when that is all zero); the first passing child
// becomes v.  When every child of v is rejected the last token is drawn from
// r, at a leaf from p_v (inverse CDF in ascending token order).
//
// The walk is sequential, but each of its vocabulary passes is not: request
// b gets P workgroups, part p owning the tokens [p*cw, (p+1)*cw).  A part
// keeps its slice of the residual rows to itself; only scalars cross parts:
// after each pass every part publishes one record (its share of a max, a
// sum) and waits until the request's P records of that round are in, then
// reduces them in part order -- the same inputs and code in every part, so
// all parts take the same decisions without further exchange.  A test at
// token x needs r(x): every part recomputes it from the target row, the
// rejected children's draft rows at x and the history of totals, with the
// very arithmetic of the passes.  The grid is sized to be co-resident (the
// waits need every part running); the waits are bounded, so a grid that is
// not co-resident ends with accept_len = -1 instead of hanging.
#include <atomic>

#include "spec_common.h"
#include "spec_internal.h"

namespace specv {

constexpr int kMdThreads = 256;
constexpr int kMdWaves = kMdThreads / 64;
constexpr int kMdMaxParts = 64;
constexpr uint32_t kMdSpinLimit = 1u << 22;  // polls of a wait before it gives up (well over a second)

struct MdRec {  // one part's share of a round
    double s;   // a sum (row statistics: relative to m)
    float m;    // a max logit
    int arg;    // its lowest index
};

struct MdArgs {
    const float* logits;
    const float* draft;
    const int32_t* tokens;
    const int32_t* parent;
    const float* u_acc;
    const float* u_smp;
    int32_t* accept_len;
    int32_t* path;
    int32_t* out_tokens;
    float* resid;    // [B][2][V]: the part's slices of the two residual rows
    MdRec* recs;     // [B][2][kMdMaxParts]: the records of the last two rounds (tags cleared before the launch)
    int B, N, V;
    int P, cw;       // parts per request, tokens per part (a multiple of 4)
    float T;
    int vec4;
};


// One residual element: max(0, r * inv - q) rounded to fp32, r the previous
// residual (or the unnormalised target weight) and inv the reciprocal of its
// total.  Shared by the passes and the point evaluation, and never
// contracted into an fma, so both round identically.
__device__ __forceinline__ float md_resid(double r, double inv, float q) {
#pragma clang fp contract(off)
    const double ry = r * inv;
    return static_cast<float>(fmax(ry - static_cast<double>(q), 0.0));
}

// Lane `src`'s value (wave-uniform src).
__device__ __forceinline__ double md_readlane(double v, int src) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(u)), src));
    const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(u >> 32), src));
    return __builtin_bit_cast(double, static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}

__device__ __forceinline__ double md_block_sum(double v, double* s_red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) s_red[wv] = v;
    __syncthreads();
    double t = 0.0;
    for (int k = 0; k < kMdWaves; ++k) t += s_red[k];
    return t;
}

// f(x, value) over the part's tokens [x0, x1) of one row, 16-byte loads when
// the rows allow (x0 and x1 are then multiples of 4).
template <class F>
__device__ __forceinline__ void md_for(const float* row, int x0, int x1, bool vec4, F f) {
    if (vec4) {
        for (int x = x0 + 4 * threadIdx.x; x < x1; x += 4 * kMdThreads) {
            const float4 v = *reinterpret_cast<const float4*>(row + x);
            f(x, v.x);
            f(x + 1, v.y);
            f(x + 2, v.z);
            f(x + 3, v.w);
        }
    } else {
        for (int x = x0 + threadIdx.x; x < x1; x += kMdThreads) f(x, row[x]);
    }
}

template <class F>
__device__ __forceinline__ void md_for2(const float* ra, const float* rb, int x0, int x1, bool vec4, F f) {
    if (vec4) {
        for (int x = x0 + 4 * threadIdx.x; x < x1; x += 4 * kMdThreads) {
            const float4 va = *reinterpret_cast<const float4*>(ra + x);
            const float4 vb = *reinterpret_cast<const float4*>(rb + x);
            f(x, va.x, vb.x);
            f(x + 1, va.y, vb.y);
            f(x + 2, va.z, vb.z);
            f(x + 3, va.w, vb.w);
        }
    } else {
        for (int x = x0 + threadIdx.x; x < x1; x += kMdThreads) f(x, ra[x], rb[x]);
    }
}

// A record in memory: word 0 the sum, word 1 the max's bits, then its index
// (24 bits, 0xFFFFFF: none) and the round's tag (8 bits) in the high half.
// The tag tells a reader that the record is the round's: the writer stores
// word 0, waits for it, then stores word 1.  Rounds stay below 255 (at most
// two per node and one for the draw); cleared records carry tag 0xFF.
constexpr uint32_t kMdNoArg = 0xFFFFFFu;
__device__ __forceinline__ uint64_t md_word1(float m, int arg, uint32_t round) {
    const uint32_t a24 = arg < 0 || arg >= static_cast<int>(kMdNoArg) ? kMdNoArg : static_cast<uint32_t>(arg);
    return static_cast<uint64_t>(__float_as_uint(m)) | (static_cast<uint64_t>(a24 | ((round & 0xFFu) << 24)) << 32);
}

__global__ void md_clear(uint64_t* recs, size_t nwords) {
    const size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i < nwords) recs[i] = ~0ull;  // (word 1 of every record: tag 0xFF)
}

__global__ __launch_bounds__(kMdThreads) void accept_md(MdArgs a) {
    const int p = blockIdx.x, b = blockIdx.y, N = a.N, V = a.V, P = a.P;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int x0 = min(p * a.cw, V), x1 = min(x0 + a.cw, V);
    const bool vec4 = a.vec4 != 0;
    __shared__ int s_par[kMaxNodes], s_tok[kMaxNodes], s_path[kMaxNodes];
    __shared__ int s_hc[kMaxNodes];     // effective rejections at the current node: child
    __shared__ double s_hz[kMaxNodes];  // and the residual total after it
    __shared__ MdRec s_rec[kMdMaxParts];
    __shared__ double s_tot[kMdMaxParts];  // per-part masses of the weights a last token is drawn from
    __shared__ double s_red[kMdWaves];
    __shared__ float s_v[kMdWaves];
    __shared__ int s_i[kMdWaves], s_j[kMdWaves];
    __shared__ double s_rx;
    __shared__ int s_fail;
    if (tid < N) {
        s_par[tid] = tree_parent(a.parent, N, b, tid);
        s_tok[tid] = min(max(a.tokens[static_cast<size_t>(b) * N + tid], 0), V - 1);
    }
    if (tid == 0) {
        s_path[0] = 0;
        s_fail = 0;
    }
    float* R[2] = {a.resid + static_cast<size_t>(2 * b) * V, a.resid + static_cast<size_t>(2 * b + 1) * V};
    const bool greedy = !(a.T > 0.f);
    const float c2 = greedy ? 0.f : 1.4426950408889634f / a.T;
    const double c2d = c2;
    uint32_t round = 0;
    __syncthreads();

    // Publish this part's record of the round and gather the request's P
    // records into s_rec (part order).
    auto exchange = [&](MdRec mine) {
        if (P > 1) {
            MdRec* slots = a.recs + (static_cast<size_t>(b) * 2 + (round & 1u)) * kMdMaxParts;
            if (tid == 0) {
                agent_st64(&slots[p].s, __builtin_bit_cast(uint64_t, mine.s));
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the sum is stored before the tagged word
                agent_st64(&slots[p].m, md_word1(mine.m, mine.arg, round));
            }
            if (wave == 0) {
                // Lane k waits for part k's tagged word (a bounded poll), then
                // reads the sum, which was stored before it.
                const int k = min(lane, P - 1);
                uint64_t w = 0ull;
                uint32_t polls = 0;
                for (;;) {
                    w = agent_ld64(&slots[k].m);
                    const bool here = ((w >> 56) & 0xFFu) == (round & 0xFFu);
                    if (__ballot(!here) == 0ull) break;  // (wave-uniform exit)
                    __builtin_amdgcn_s_sleep(2);
                    if (++polls > kMdSpinLimit) {
                        if (lane == 0) s_fail = 1;
                        break;
                    }
                }
                if (lane < P) {
                    MdRec r;
                    r.s = __builtin_bit_cast(double, agent_ld64(&slots[k].s));
                    r.m = __uint_as_float(static_cast<uint32_t>(w));
                    const uint32_t a24 = static_cast<uint32_t>(w >> 32) & kMdNoArg;
                    r.arg = a24 == kMdNoArg ? 0x7fffffff : static_cast<int>(a24);
                    s_rec[lane] = r;
                }
            }
        } else if (tid == 0) {
            s_rec[0] = mine;
        }
        __syncthreads();
        ++round;
    };

    int v = 0, depth = 0, final = 0, writer = 0;
    for (;;) {
        const float* row = a.logits + (static_cast<size_t>(b) * N + v) * V;
        // Row statistics: the part's max (lowest index) and, at T > 0, its
        // sum of 2^((l - m) c2); then the row's M, argmax and S.
        // (one pass: each thread's running max and its sum relative to it,
        // rescaled when the max moves)
        float best = -INFINITY;
        int bi = 0x7fffffff;
        double ts = 0.0;
        md_for(row, x0, x1, vec4, [&](int x, float l) {
            if (l > best) {
                if (!greedy) ts = best > -INFINITY ? ts * __builtin_amdgcn_exp2f((best - l) * c2) + 1.0 : 1.0;
                best = l;
                bi = x;
            } else if (!greedy) {
                ts += __builtin_amdgcn_exp2f((l - best) * c2);
            }
        });
        const float tbest = best;
        wave_argmax(best, bi);
        __syncthreads();
        if (lane == 0) {
            s_v[wave] = best;
            s_i[wave] = bi;
        }
        __syncthreads();
        float m = s_v[0];
        int marg = s_i[0];
        for (int k = 1; k < kMdWaves; ++k)
            if (s_v[k] > m || (s_v[k] == m && s_i[k] < marg)) {
                m = s_v[k];
                marg = s_i[k];
            }
        double s = 0.0;
        if (!greedy) {
            const double mine = tbest > -INFINITY ? ts * __builtin_amdgcn_exp2f((tbest - m) * c2) : 0.0;
            s = md_block_sum(mine, s_red);
        }
        exchange(MdRec{s, m, marg});
        // The records reduced across the lanes (lane k: part k), the same in
        // every wave and every part.
        const MdRec rk = lane < P ? s_rec[lane] : MdRec{0.0, -INFINITY, 0x7fffffff};
        float M = rk.m;
        int arg = rk.arg;
        wave_argmax(M, arg);
        double S = 1.0;
        if (!greedy) {
            const double t = rk.m > -INFINITY ? rk.s * exp2((static_cast<double>(rk.m) - M) * c2d) : 0.0;
            if (tid < kMdMaxParts) s_tot[tid] = t;
            S = wave_sum(t);
            __syncthreads();  // s_tot before any read
        }
        // Children in ascending index against the current residual.
        int cur = -1;  // residual row holding r (unnormalised, total Z); -1: r = p_v
        double Z = 1.0;
        int nh = 0, next = -1;
        for (int c = 1; c < N; ++c) {
            if (s_par[c] != v) continue;  // uniform: LDS values
            const int x = s_tok[c];
            if (wave == 0) {
                // Every load of the test at once (lane j: the j-th rejected
                // sibling's draft probability at x), then r(x) through the
                // effective rejections, as the passes computed it.
                const float qh = lane < nh ? a.draft[(static_cast<size_t>(b) * N + s_hc[lane]) * V + x] : 0.f;
                const float lx = row[x];
                const double qx = a.draft[(static_cast<size_t>(b) * N + c) * V + x];
                const double ua = a.u_acc[static_cast<size_t>(b) * N + c];
                double rx;
                if (greedy) {
                    rx = x == arg ? 1.0 : 0.0;
                } else {
                    float e = __builtin_amdgcn_exp2f((lx - M) * c2);
                    double tot = S;
                    for (int j = 0; j < nh; ++j) {
                        e = md_resid(static_cast<double>(e), 1.0 / tot, __shfl(qh, j));
                        tot = s_hz[j];
                    }
                    rx = static_cast<double>(e) / tot;
                }
                if (lane == 0) s_rx = ua * qx < rx ? 1.0 : 0.0;
            }
            __syncthreads();
            const bool acc = s_rx != 0.0;
            __syncthreads();
            if (acc) {
                next = c;
                break;
            }
            if (greedy) continue;  // r stays the one-hot argmax
            // r <- max(0, r - q_c) over the part's tokens, into the other row
            const int dst = cur == 0 ? 1 : 0;
            float* out = R[dst];
            const float* qrow = a.draft + (static_cast<size_t>(b) * N + c) * V;
            const double inv = cur >= 0 ? 1.0 / Z : 1.0 / S;
            double zs = 0.0;
            md_for2(cur >= 0 ? R[cur] : row, qrow, x0, x1, vec4, [&](int y, float src, float qy) {
                const double r = cur >= 0 ? static_cast<double>(src)
                                          : static_cast<double>(__builtin_amdgcn_exp2f((src - M) * c2));
                const float e = md_resid(r, inv, qy);
                out[y] = e;
                zs += e;
            });
            zs = md_block_sum(zs, s_red);
            exchange(MdRec{zs, 0.f, 0});
            const double zk = lane < P ? s_rec[lane].s : 0.0;
            const double Zn = wave_sum(zk);
            if (Zn > 0.0) {
                cur = dst;
                Z = Zn;
                if (tid == 0) {
                    s_hc[nh] = c;
                    s_hz[nh] = Zn;
                }
                if (tid < kMdMaxParts) s_tot[tid] = zk;
                ++nh;
                __syncthreads();
            }
        }
        if (next >= 0) {
            v = next;
            ++depth;
            if (tid == 0) s_path[depth] = v;
            __syncthreads();
            continue;
        }
        if (greedy) {
            final = arg;
            writer = 0;
            break;
        }
        // Last token, drawn from r (v had children) or p_v (a leaf): the
        // part whose mass holds u * total draws it from its tokens.
        const double u = a.u_smp ? static_cast<double>(a.u_smp[static_cast<size_t>(b) * N + v]) : 0.0;
        // Part masses in part order (lane k: part k): their running sums by
        // one wave scan, the first part whose running sum passes u * total.
        const double mk = lane < P ? s_tot[lane] : 0.0;
        const double pincl = wave_incl_scan(mk);
        const double total = md_readlane(pincl, 63);
        const double t = u * total;
        const uint64_t hits = __ballot(mk > 0.0 && pincl > t), nz = __ballot(mk > 0.0);
        int h;
        double hbase;
        if (hits) {
            h = __builtin_ctzll(hits);
            hbase = md_readlane(pincl - mk, h);  // part h's exclusive running sum
        } else {  // rounding left u * total past the end: the last part with mass
            h = nz ? 63 - __builtin_clzll(nz) : 0;
            hbase = -INFINITY;  // take its last token with weight
        }
        writer = h;
        if (p != h) break;
        const int len = x1 - x0, run = (len + kMdThreads - 1) / kMdThreads;
        const int r0 = min(x0 + tid * run, x1), r1 = min(r0 + run, x1);
        auto weight = [&](int y) {
            return cur >= 0 ? static_cast<double>(R[cur][y])
                            : static_cast<double>(__builtin_amdgcn_exp2f((row[y] - M) * c2));
        };
        double mine = 0.0;
        for (int y = r0; y < r1; ++y) mine += weight(y);
        const double incl = wave_incl_scan(mine);
        __syncthreads();
        if (lane == 63) s_red[wave] = incl;
        __syncthreads();
        double cum = hbase + (incl - mine);
        for (int k = 0; k < wave; ++k) cum += s_red[k];
        int hit = 0x7fffffff, lastnz = -1;
        for (int y = r0; y < r1; ++y) {
            const double w = weight(y);
            if (w > 0.0) {
                lastnz = y;
                cum += w;
                if (hit == 0x7fffffff && cum > t) hit = y;
            }
        }
        int ih = hit, il = lastnz;
        wave_min_max_i(ih, il);
        __syncthreads();
        if (lane == 0) {
            s_i[wave] = ih;
            s_j[wave] = il;
        }
        __syncthreads();
        int hh = 0x7fffffff, ll = -1;
        for (int k = 0; k < kMdWaves; ++k) {
            hh = min(hh, s_i[k]);
            ll = max(ll, s_j[k]);
        }
        final = hh != 0x7fffffff ? hh : (ll >= 0 ? ll : x0);
        break;
    }
    if (p != writer) {
        if (s_fail && tid == 0) a.accept_len[b] = -1;
        return;
    }
    // Outputs, from one part.
    if (tid < N) {
        const size_t o = static_cast<size_t>(b) * N + tid;
        a.path[o] = tid <= depth ? s_path[tid] : -1;
        a.out_tokens[o] = tid < depth ? s_tok[s_path[tid + 1]] : (tid == depth ? final : -1);
    }
    if (tid == 0) a.accept_len[b] = s_fail ? -1 : depth;
}

static size_t md_resid_bytes(int B, int V) { return align_up(static_cast<size_t>(B) * 2 * V * sizeof(float), 256); }
static size_t md_rec_bytes(int B) { return align_up(static_cast<size_t>(B) * 2 * kMdMaxParts * sizeof(MdRec), 256); }

size_t multidraft_workspace_bytes(int B, int V) {
    return md_resid_bytes(B, V) + md_rec_bytes(B);
}

// Parts per request: as many as the device holds at once for the batch
// (every part of a request must run concurrently), at most kMdMaxParts and
// about a thousand tokens each at least.
static int md_parts(int B, int V) {
    static std::atomic<int> resident[64];  // per device, cached (host threads may race to fill it)
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 1;
    int res = resident[dev].load(std::memory_order_relaxed);
    if (res == 0) {
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, accept_md, kMdThreads, 0) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
        res = per_cu * cus;
        resident[dev].store(res, std::memory_order_relaxed);
    }
    long P = res / std::max(B, 1);
    P = std::min<long>(P, kMdMaxParts);
    P = std::min<long>(P, (V + 1023) / 1024);
    return static_cast<int>(std::max<long>(P, 1));
}

int launch_accept_multidraft(int B, int N, int V, const float* logits, const float* draft, const int32_t* tokens,
                             const int32_t* parent, const float* u_accept, const float* u_sample, float temperature,
                             int32_t* accept_len, int32_t* path, int32_t* out_tokens, void* workspace,
                             hipStream_t stream) {
    MdArgs a{};
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
    a.resid = reinterpret_cast<float*>(ws);
    a.recs = reinterpret_cast<MdRec*>(ws + md_resid_bytes(B, V));
    a.B = B;
    a.N = N;
    a.V = V;
    a.T = temperature;
    a.vec4 = (V % 4 == 0) && (reinterpret_cast<uintptr_t>(logits) % 16 == 0) &&
             (draft == nullptr || reinterpret_cast<uintptr_t>(draft) % 16 == 0) &&
             (reinterpret_cast<uintptr_t>(workspace) % 16 == 0);
    const int P0 = md_parts(B, V);
    a.cw = ((V + P0 - 1) / P0 + 3) / 4 * 4;
    a.P = (V + a.cw - 1) / a.cw;  // no empty part
    const size_t nwords = static_cast<size_t>(B) * 2 * kMdMaxParts * sizeof(MdRec) / sizeof(uint64_t);
    hipLaunchKernelGGL(md_clear, dim3(static_cast<unsigned>((nwords + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<uint64_t*>(a.recs), nwords);
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    hipLaunchKernelGGL(accept_md, dim3(a.P, B), dim3(kMdThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_EHIP;
}

}  // namespace specv
