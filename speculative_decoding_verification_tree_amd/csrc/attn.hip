// Tree-verify attention for gfx950.
//
// Computes, for every request b, kv head g and query row r = node * G + j
// (q head g*G + j), softmax(scale * q k^T) v over the verified prefix rows
// [0, L_b) plus the tree rows L_b + n for every n on the root path of the
// row's node (MEDUSA section of the blog page "Fast Inference from
// Transformers via Speculative Decoding", tree-attention paragraph; the
// parallel scoring of all draft positions is the "Speculative Sampling"
// section of the same page).
//
// Work decomposition: the key axis of one (b, g) is shared by S splits
// (split-KV, S = ceil(keys / chunk)); split s and its waves take the 32-key
// blocks s*WK + wave + t*S*WK, so the splits of a slab sweep it front to back
// together.  A workgroup holds every query row of its row group, so each KV
// element is read from HBM once and shared by all N * G rows.  The waves merge
// their (max, sum, O) at the end through LDS; splits merge in attn_combine
// with an exact log-sum-exp rescale.
//
// bf16 MFMA path (v_mfma_f32_16x16x32_bf16):
//   S^T = K * Q^T : A = 16 keys x 32 dims of K straight from HBM (16-byte
//                   loads), B = Q^T held in registers for the whole chunk.
//   The two 16-key halves of a block use the key order
//     row m of half h  <->  key 8*(m/4) + 4*h + m%4
//   so that lane (n, q) ends up holding row n's scores for keys 8q..8q+7:
//   exactly the A operand of the PV product, with no register shuffle.
//   O += P * V    : B = V^T slice read from a per-wave transposed LDS copy
//                   (16-byte reads, XOR-swizzled 16-byte columns).
// fp32 (and any dtype) VALU path: 32 rows x 32 keys tiles through LDS.
#include <stdlib.h>

#include "spec_common.h"
#include "spec_internal.h"

namespace specv {

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* ws_o;    // [B][Hkv][S][R][D]  unnormalised partial O per split
    float2* ws_ml;  // [B][Hkv][S][R]     (max in log2 units, sum)
    const int32_t* prefix_len;
    const int32_t* parent;
    int B, N, Hq, Hkv, G, cap, R, nrg, chunk, nsplit_max;
    int max_keys;      // host bound on L_b + N (sizes the split workspace)
    float scale_log2;  // softmax scale * log2(e)
};

// Ancestor-or-self bit masks of every node, built from the parent array.
__device__ __forceinline__ void build_anc(const AttnArgs& a, int b, uint64_t* s_anc) {
    const int tid = threadIdx.x;
    if (tid < a.N) {
        uint64_t m = 0;
        int n = tid;
        for (int s = 0; s < kMaxNodes && n >= 0; ++s) {
            m |= 1ull << n;
            n = tree_parent(a.parent, a.N, b, n);
        }
        s_anc[tid] = m;
    }
}

// Workgroup -> (request, kv head, split, row group).  The row groups of one
// chunk get consecutive dispatch slots on one XCD (block i runs on XCD i % 8),
// so they share the chunk through that XCD's L2.
struct Work {
    int b, g, s, rg;
    bool live;
};

__device__ __forceinline__ Work decode_block(const AttnArgs& a) {
    const int i = blockIdx.x;
    const int xcd = i & 7, j = i >> 3;
    const int unit = (j / a.nrg) * 8 + xcd;
    Work w;
    w.rg = j % a.nrg;
    w.s = unit % a.nsplit_max;
    const int bg = unit / a.nsplit_max;
    w.live = bg < a.B * a.Hkv;
    w.b = w.live ? bg / a.Hkv : 0;
    w.g = w.live ? bg % a.Hkv : 0;
    return w;
}

__device__ __forceinline__ void store_out(void* out, bool bf16, size_t idx, float val) {
    if (bf16)
        static_cast<uint16_t*>(out)[idx] = static_cast<uint16_t>(f32_to_bf16_bits(val));
    else
        static_cast<float*>(out)[idx] = val;
}

// XOR swizzle of the four 16-byte key columns of a transposed-V row.
__device__ __forceinline__ int vt_swz(int d) { return ((d >> 1) ^ (d >> 3)) & 3; }

// ----------------------------------------------------------------------------
// MFMA path (bf16).  D in {64, 128}; RT 16-row tiles per wave; WK waves.
// ----------------------------------------------------------------------------
// K fragments (A operand, paired-half key order) and V rows of one 32-key
// block, held in registers between the load and its use.
template <int D>
struct KVBlock {
    static constexpr int NC32 = D / 32;
    static constexpr int KPL = 32 / (64 / (D / 8));
    u32x4 kf[2][NC32];
    u32x4 vr[KPL];
};

// Issue the loads of the block starting at key kb; rows are clamped to
// row_max so every address is inside the cache.
template <int D>
__device__ __forceinline__ void load_kv_block(KVBlock<D>& blk, const uint16_t* kbase, const uint16_t* vbase, int kb,
                                              int row_max, int n16, int q4, int vch, int vkg) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = min(kb + 8 * (n16 >> 2) + 4 * h + (n16 & 3), row_max);
#pragma unroll
        for (int c = 0; c < KVBlock<D>::NC32; ++c)
            blk.kf[h][c] = *reinterpret_cast<const u32x4*>(kbase + static_cast<size_t>(row) * D + 32 * c + 8 * q4);
    }
#pragma unroll
    for (int jj = 0; jj < KVBlock<D>::KPL; ++jj) {
        const int row = min(kb + vkg * KVBlock<D>::KPL + jj, row_max);
        blk.vr[jj] = *reinterpret_cast<const u32x4*>(vbase + static_cast<size_t>(row) * D + 8 * vch);
    }
}

template <int D, int RT, int WK>
__global__ __launch_bounds__(64 * WK) void attn_mfma(AttnArgs a) {
    constexpr int NC32 = D / 32;  // k-steps of the QK product
    constexpr int NC16 = D / 16;  // n-tiles of the PV product
    constexpr int CPR = D / 8;    // 16-byte chunks per cache row
    constexpr int KPL = KVBlock<D>::KPL;  // keys per lane in the V load (8 or 4)
    constexpr int VT_BYTES = D * 64;
    constexpr int MERGE_BYTES = WK * 16 * RT * D * 4;
    constexpr int LDS_BYTES = (WK * VT_BYTES > MERGE_BYTES) ? WK * VT_BYTES : MERGE_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char s_buf[LDS_BYTES];
    __shared__ uint64_t s_anc[kMaxNodes];
    __shared__ float s_m[WK][16 * RT];
    __shared__ float s_l[WK][16 * RT];
    __shared__ float2 s_row[16 * RT];

    const Work w = decode_block(a);
    if (!w.live) return;
    const int b = w.b, g = w.g;
    const int k0 = w.s * a.chunk;
    if (k0 >= a.max_keys) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, q4 = lane >> 4;
    const int vch = lane % CPR, vkg = lane / CPR;
    const size_t head = (static_cast<size_t>(b) * a.Hkv + g) * a.cap;
    const uint16_t* kbase = static_cast<const uint16_t*>(a.k) + head * D;
    const uint16_t* vbase = static_cast<const uint16_t*>(a.v) + head * D;

    // Everything that does not depend on the prefix length goes out first:
    // the prefix length itself, the first KV block (rows clamped to the cache,
    // out-of-range values masked once L is known), the tree and the queries.
    const int L = a.prefix_len[b];
    // Split s of a (request, kv head) takes the interleaved 32-key blocks
    // s*WK + wave + t*S*WK, S = the request's split count: the splits of one
    // slab sweep it together, front to back, like one streaming read.
    const int first_blk = w.s * WK + wave;
    int kb = first_blk * 32;
    KVBlock<D> cur;
    load_kv_block<D>(cur, kbase, vbase, kb, a.cap - 1, n16, q4, vch, vkg);
    build_anc(a, b, s_anc);
    bf16x8 qf[RT][NC32];
    int rnode[RT];
    const uint16_t* qb = static_cast<const uint16_t*>(a.q);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int r = (w.rg * RT + t) * 16 + n16;
        const bool valid = r < a.R;
        rnode[t] = valid ? r / a.G : -1;
        const int hq = g * a.G + (valid ? r % a.G : 0);
        const uint16_t* qrow = qb + ((static_cast<size_t>(b) * a.N + (valid ? rnode[t] : 0)) * a.Hq + hq) * D;
#pragma unroll
        for (int c = 0; c < NC32; ++c) {
            u32x4 u = {0u, 0u, 0u, 0u};
            if (valid) u = *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * q4);
            qf[t][c] = __builtin_bit_cast(bf16x8, u);
        }
    }
    __syncthreads();

    const int Tk = L + a.N;
    if (L < 0 || Tk > a.cap || Tk > a.max_keys) return;  // outside the contract: leave out unwritten
    if (k0 >= Tk) return;
    const int nsplit = (Tk + a.chunk - 1) / a.chunk;
    const int k1 = Tk;                  // keys past the request's end are masked
    const int kstep = 32 * WK * nsplit;  // interleave stride of this request
    uint64_t anc[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) anc[t] = rnode[t] >= 0 ? s_anc[rnode[t]] : ~0ull;

    float m_run[RT], l_run[RT];
    f32x4 o[RT][NC16];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        m_run[t] = -INFINITY;
        l_run[t] = 0.f;
#pragma unroll
        for (int c = 0; c < NC16; ++c) o[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    unsigned char* vt = s_buf + wave * VT_BYTES;

    for (; kb < k1; kb += kstep) {
        // Prefetch the wave's next block while this one is processed.  The
        // loads are unconditional (past the end they re-read this block:
        // cache hits) so the wait before using this block counts only the
        // older loads and never drains the prefetch.
        KVBlock<D> nxt;
        const int kn = kb + kstep;
        load_kv_block<D>(nxt, kbase, vbase, kn < k1 ? kn : kb, Tk - 1, n16, q4, vch, vkg);

        // Transpose V into LDS (row d holds the block's 32 keys); keys at or
        // past the split end are zeroed so no stale value reaches P*V.
#pragma unroll
        for (int jj = 0; jj < KPL; ++jj)
            if (kb + vkg * KPL + jj >= k1) cur.vr[jj] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int d = 8 * vch + t;
            const int key0 = vkg * KPL;
            const int pch = (key0 >> 3) ^ vt_swz(d);
            unsigned char* dst = vt + d * 64 + pch * 16 + (key0 & 7) * 2;
            // element t of two keys' rows -> one dword (byte select: low or high half)
            const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
            if constexpr (KPL == 8) {
                u32x4 wv;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    wv[e] = __builtin_amdgcn_perm(cur.vr[2 * e + 1][t >> 1], cur.vr[2 * e][t >> 1], sel);
                *reinterpret_cast<u32x4*>(dst) = wv;
            } else {
                uint2 wv;
                wv.x = __builtin_amdgcn_perm(cur.vr[1][t >> 1], cur.vr[0][t >> 1], sel);
                wv.y = __builtin_amdgcn_perm(cur.vr[3][t >> 1], cur.vr[2][t >> 1], sel);
                *reinterpret_cast<uint2*>(dst) = wv;
            }
        }
        wave_lds_sync();

        // Blocks wholly inside the prefix and the split need no key mask.
        const bool interior = kb + 32 <= L && kb + 32 <= k1;
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            f32x4 st[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < NC32; ++c)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cur.kf[h][c]), qf[t][c],
                                                                  acc, 0, 0, 0);
                st[h] = acc;
            }
            // This lane's keys are kb + 8*q4 + e, e = 0..7 (e = 4h + ii).
            // Bit e of the mask: key below the split end and either a prefix
            // key or a tree key on the row's root path.
            uint32_t kmask = 0xFFu;
            if (!interior) {
                const int base = kb + 8 * q4;
                const int nend = min(max(k1 - base, 0), 8);
                const int npre = min(max(L - base, 0), 8);
                const int sh = base - L;  // tree offset of key e is sh + e
                const uint32_t tree = sh >= 0 ? static_cast<uint32_t>(anc[t] >> min(sh, 63))
                                              : static_cast<uint32_t>(anc[t] << min(-sh, 63));
                const uint32_t pre = (1u << npre) - 1u;
                kmask = ((tree & 0xFFu) | pre) & ((1u << nend) - 1u);
            }
            float s[8];
            float bm = -INFINITY;
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) {
                    const int e = 4 * h + ii;
                    const float x = ((kmask >> e) & 1u) ? st[h][ii] * a.scale_log2 : -INFINITY;
                    s[e] = x;
                    bm = fmaxf(bm, x);
                }
            bm = max_across_rows(bm);
            // Lazy rescale: keep the running max unless a row's block max
            // exceeds it by more than 8 (probabilities stay <= 2^8, exact in
            // fp32 and as precise in bf16); the decision is wave-uniform.
            if (__builtin_amdgcn_ballot_w64(bm > m_run[t] + 8.f) != 0ull) {
                const float mn = fmaxf(m_run[t], bm);
                const float alpha = m_run[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[t] - mn);
                l_run[t] *= alpha;
#pragma unroll
                for (int c = 0; c < NC16; ++c) o[t][c] *= alpha;  // o holds row n16 of this lane
                m_run[t] = mn;
            }
            const float mu = m_run[t] == -INFINITY ? 0.f : m_run[t];
            float rs = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                s[e] = __builtin_amdgcn_exp2f(s[e] - mu);
                rs += s[e];
            }
            l_run[t] += sum_across_rows(rs);
            u32x4 pp;
            pp[0] = pack_bf16x2(s[0], s[1]);
            pp[1] = pack_bf16x2(s[2], s[3]);
            pp[2] = pack_bf16x2(s[4], s[5]);
            pp[3] = pack_bf16x2(s[6], s[7]);
            const bf16x8 pa = __builtin_bit_cast(bf16x8, pp);
#pragma unroll
            for (int c = 0; c < NC16; ++c) {
                // O^T = V^T P^T: A = V^T (lane: keys 8q..8q+7 of dim 16c + n,
                // straight from LDS), B = P^T; the result lands as
                // O[row n][dims 16c + 4q .. 16c + 4q + 3] in this lane.
                const int d = 16 * c + n16;
                const u32x4 vf = *reinterpret_cast<const u32x4*>(vt + d * 64 + ((q4 ^ vt_swz(d)) * 16));
                o[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, vf), pa, o[t][c], 0, 0, 0);
            }
        }
        wave_lds_sync();
        cur = nxt;
    }

    // ---- merge the waves of this workgroup --------------------------------
    __syncthreads();
    if (q4 == 0) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            s_m[wave][t * 16 + n16] = m_run[t];
            s_l[wave][t * 16 + n16] = l_run[t];
        }
    }
    __syncthreads();
    if (tid < 16 * RT) {  // per-row (max, sum) of the workgroup
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < WK; ++x) M = fmaxf(M, s_m[x][tid]);
        const float Mu = M == -INFINITY ? 0.f : M;
        float lsum = 0.f;
#pragma unroll
        for (int x = 0; x < WK; ++x) lsum += s_l[x][tid] * exp2f(s_m[x][tid] - Mu);
        s_row[tid] = make_float2(M, lsum);
    }
    float* reg = reinterpret_cast<float*>(s_buf);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int row = t * 16 + n16;
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < WK; ++x) M = fmaxf(M, s_m[x][row]);
        const float sc = exp2f(m_run[t] - (M == -INFINITY ? 0.f : M));
#pragma unroll
        for (int c = 0; c < NC16; ++c)
            *reinterpret_cast<f32x4*>(reg + (wave * 16 * RT + row) * D + 16 * c + 4 * q4) = o[t][c] * sc;
    }
    __syncthreads();

    const int rbase = w.rg * RT * 16;
    const int rows = min(16 * RT, a.R - rbase);
    const size_t pbase = (static_cast<size_t>(b) * a.Hkv + g) * a.nsplit_max;
    for (int e = tid; e < rows * D; e += 64 * WK) {
        const int row = e / D, d = e % D;
        float osum = 0.f;
#pragma unroll
        for (int x = 0; x < WK; ++x) osum += reg[(x * 16 * RT + row) * D + d];
        const int r = rbase + row;
        if (nsplit == 1) {
            const int node = r / a.G, hq = g * a.G + r % a.G;
            const float lsum = s_row[row].y;
            const size_t oi = ((static_cast<size_t>(b) * a.N + node) * a.Hq + hq) * D + d;
            store_out(a.out, true, oi, lsum > 0.f ? osum / lsum : 0.f);
        } else {
            a.ws_o[((pbase + w.s) * a.R + r) * D + d] = osum;
            if (d == 0) a.ws_ml[(pbase + w.s) * a.R + r] = s_row[row];
        }
    }
}

// ----------------------------------------------------------------------------
// VALU path: 32 query rows x 32-key tiles staged in LDS, fp32 arithmetic.
// ----------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float load_elem(const T* p, size_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float* p, size_t i) {
    return p[i];
}
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t* p, size_t i) {
    return bf16_bits_to_f32(p[i]);
}

template <typename T, int D>
__global__ __launch_bounds__(256) void attn_valu(AttnArgs a) {
    constexpr int DP = D + 1;
    __shared__ float s_q[32][DP];
    __shared__ float s_k[32][DP];
    __shared__ float s_v[32][DP];
    __shared__ float s_p[32][33];
    __shared__ uint64_t s_anc[kMaxNodes];

    const Work w = decode_block(a);
    if (!w.live) return;
    const int b = w.b, g = w.g;
    const int L = a.prefix_len[b];
    const int Tk = L + a.N;
    if (L < 0 || Tk > a.cap || Tk > a.max_keys) return;  // outside the contract: leave out unwritten
    const int k0 = w.s * a.chunk;
    if (k0 >= Tk) return;
    const int k1 = min(k0 + a.chunk, Tk);
    const int nsplit = (Tk + a.chunk - 1) / a.chunk;

    build_anc(a, b, s_anc);
    const int tid = threadIdx.x;
    const T* qp = static_cast<const T*>(a.q);
    for (int e = tid; e < 32 * D; e += 256) {
        const int lr = e / D, d = e % D;
        const int r = w.rg * 32 + lr;
        float x = 0.f;
        if (r < a.R) {
            const int node = r / a.G, hq = g * a.G + r % a.G;
            x = load_elem(qp, ((static_cast<size_t>(b) * a.N + node) * a.Hq + hq) * D + d);
        }
        s_q[lr][d] = x;
    }
    __syncthreads();

    const int sr = tid >> 3, sk = tid & 7;
    const int r = w.rg * 32 + sr;
    const bool rvalid = r < a.R;
    const uint64_t anc = rvalid ? s_anc[r / a.G] : ~0ull;
    float m_run = -INFINITY, l_run = 0.f;
    float o[D / 8];
#pragma unroll
    for (int j = 0; j < D / 8; ++j) o[j] = 0.f;

    const size_t head = (static_cast<size_t>(b) * a.Hkv + g) * a.cap;
    const T* kp = static_cast<const T*>(a.k) + head * D;
    const T* vp = static_cast<const T*>(a.v) + head * D;

    for (int kb = k0; kb < k1; kb += 32) {
        __syncthreads();
        for (int e = tid; e < 32 * D; e += 256) {
            const int kk = e / D, d = e % D;
            const size_t row = static_cast<size_t>(min(kb + kk, Tk - 1));
            s_k[kk][d] = load_elem(kp, row * D + d);
            s_v[kk][d] = load_elem(vp, row * D + d);
        }
        __syncthreads();
        float s[4];
        float bm = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int kk = sk + 8 * jj;
            const int key = kb + kk;
            float dot = 0.f;
#pragma unroll 8
            for (int d = 0; d < D; ++d) dot = fmaf(s_q[sr][d], s_k[kk][d], dot);
            const bool ok = key < k1 && (key < L || ((anc >> (key - L)) & 1ull));
            s[jj] = ok ? dot * a.scale_log2 : -INFINITY;
            bm = fmaxf(bm, s[jj]);
        }
        // reductions over the 8 lanes of a row (xor 1, xor 2, mirror within 8)
        bm = fmaxf(bm, __uint_as_float(dpp_xor1(__float_as_uint(bm))));
        bm = fmaxf(bm, __uint_as_float(dpp_xor2(__float_as_uint(bm))));
        bm = fmaxf(bm, __uint_as_float(dpp_mirror8(__float_as_uint(bm))));
        const float mn = fmaxf(m_run, bm);
        const float mu = mn == -INFINITY ? 0.f : mn;
        const float alpha = exp2f(m_run - mu);
        float rs = 0.f;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const float p = exp2f(s[jj] - mu);
            s_p[sr][sk + 8 * jj] = p;
            rs += p;
        }
        rs += __uint_as_float(dpp_xor1(__float_as_uint(rs)));
        rs += __uint_as_float(dpp_xor2(__float_as_uint(rs)));
        rs += __uint_as_float(dpp_mirror8(__float_as_uint(rs)));
        l_run = l_run * alpha + rs;
        m_run = mn;
#pragma unroll
        for (int j = 0; j < D / 8; ++j) o[j] *= alpha;
        __syncthreads();
        for (int kk = 0; kk < 32; ++kk) {
            const float p = s_p[sr][kk];
#pragma unroll
            for (int j = 0; j < D / 8; ++j) o[j] = fmaf(p, s_v[kk][sk + 8 * j], o[j]);
        }
    }
    if (!rvalid) return;
    const int node = r / a.G, hq = g * a.G + r % a.G;
    const bool bf16_out = sizeof(T) == 2;
    if (nsplit == 1) {
        const size_t ob = ((static_cast<size_t>(b) * a.N + node) * a.Hq + hq) * D;
#pragma unroll
        for (int j = 0; j < D / 8; ++j) store_out(a.out, bf16_out, ob + sk + 8 * j, l_run > 0.f ? o[j] / l_run : 0.f);
    } else {
        const size_t pi = (static_cast<size_t>(b) * a.Hkv + g) * a.nsplit_max + w.s;
#pragma unroll
        for (int j = 0; j < D / 8; ++j) a.ws_o[(pi * a.R + r) * D + sk + 8 * j] = o[j];
        if (sk == 0) a.ws_ml[pi * a.R + r] = make_float2(m_run, l_run);
    }
}

// ----------------------------------------------------------------------------
// Split combine: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// One wavefront per (request, kv head, query row).
// ----------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, int bf16_out) {
    constexpr int DPL = D / 64;  // output elements per lane
    constexpr int SB = 16;       // splits whose loads are in flight together
    const int lane = threadIdx.x & 63;
    const long id = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (id >= static_cast<long>(a.B) * a.Hkv * a.R) return;
    const int r = static_cast<int>(id % a.R);
    const int bg = static_cast<int>(id / a.R);
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int L = a.prefix_len[b];
    const int Tk = L + a.N;
    if (L < 0 || Tk > a.cap || Tk > a.max_keys) return;  // outside the contract: leave out unwritten
    const int nsplit = (Tk + a.chunk - 1) / a.chunk;
    if (nsplit <= 1) return;
    const size_t base = static_cast<size_t>(bg) * a.nsplit_max;
    // Running (max, sum, O) over batches of SB splits, each batch one round of loads.
    float M = -INFINITY, lsum = 0.f;
    float acc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += SB) {
        float2 ml[SB];
        float ov[SB][DPL];
#pragma unroll
        for (int k = 0; k < SB; ++k) {
            const int s = s0 + k;
            ml[k] = make_float2(-INFINITY, 0.f);
#pragma unroll
            for (int j = 0; j < DPL; ++j) ov[k][j] = 0.f;
            if (s < nsplit) {
                ml[k] = a.ws_ml[(base + s) * a.R + r];
#pragma unroll
                for (int j = 0; j < DPL; ++j) ov[k][j] = a.ws_o[((base + s) * a.R + r) * D + lane + 64 * j];
            }
        }
        float Mn = M;
#pragma unroll
        for (int k = 0; k < SB; ++k) Mn = fmaxf(Mn, ml[k].x);
        const float Mu = Mn == -INFINITY ? 0.f : Mn;
        const float sc = exp2f(M - Mu);
        lsum *= sc;
#pragma unroll
        for (int j = 0; j < DPL; ++j) acc[j] *= sc;
#pragma unroll
        for (int k = 0; k < SB; ++k) {
            const float wgt = exp2f(ml[k].x - Mu);
            lsum += wgt * ml[k].y;
#pragma unroll
            for (int j = 0; j < DPL; ++j) acc[j] += wgt * ov[k][j];
        }
        M = Mn;
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int node = r / a.G, hq = g * a.G + r % a.G;
    const size_t ob = ((static_cast<size_t>(b) * a.N + node) * a.Hq + hq) * D;
#pragma unroll
    for (int j = 0; j < DPL; ++j) store_out(a.out, bf16_out != 0, ob + lane + 64 * j, acc[j] * inv);
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
static int env_chunk_override() {
    static int v = -1;
    if (v < 0) {
        const char* s = getenv("SPEC_VERIFY_KV_CHUNK");
        v = s ? atoi(s) : 0;
        if (v < 0) v = 0;
    }
    return v;
}

AttnPlan plan_attn(const spec_attn_desc& d, int max_prefix_len) {
    AttnPlan p{};
    const int G = d.num_q_heads / d.num_kv_heads;
    p.rows = d.num_nodes * G;
    int unit_keys;
    if (d.dtype == SPEC_BF16) {
        p.mfma = true;
        if (p.rows <= 64) {
            p.row_tiles = (p.rows + 15) / 16;
            p.row_groups = 1;
        } else {
            p.row_tiles = 4;
            p.row_groups = (p.rows + 63) / 64;
        }
        p.waves = p.row_tiles <= 2 ? 4 : 2;
        unit_keys = 32 * p.waves;
    } else {
        p.mfma = false;
        p.row_tiles = 0;
        p.row_groups = (p.rows + 31) / 32;
        p.waves = 4;
        unit_keys = 32;
    }
    const long keys_max = static_cast<long>(max_prefix_len) + d.num_nodes;
    const long units = static_cast<long>(d.batch) * d.num_kv_heads * p.row_groups;
    const long want = units >= 1024 ? 1 : (1024 + units - 1) / units;
    long chunk = (keys_max + want - 1) / want;
    const long min_chunk = env_chunk_override() > 0 ? env_chunk_override() : 256;
    if (chunk < min_chunk) chunk = min_chunk;
    chunk = (chunk + unit_keys - 1) / unit_keys * unit_keys;
    p.chunk = static_cast<int>(chunk);
    p.nsplit_max = static_cast<int>((keys_max + chunk - 1) / chunk);
    p.max_keys = static_cast<int>(keys_max);
    if (p.nsplit_max < 1) p.nsplit_max = 1;
    if (p.nsplit_max > 1) {
        const size_t parts = static_cast<size_t>(d.batch) * d.num_kv_heads * p.nsplit_max * p.rows;
        p.ws_bytes = align_up(parts * d.head_dim * sizeof(float), 256) + align_up(parts * sizeof(float2), 256);
    } else {
        p.ws_bytes = 0;
    }
    return p;
}

template <int D>
static void launch_mfma_rt(const AttnPlan& p, const AttnArgs& a, dim3 grid, hipStream_t st) {
    switch (p.row_tiles) {
        case 1: hipLaunchKernelGGL((attn_mfma<D, 1, 4>), grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL((attn_mfma<D, 2, 4>), grid, dim3(256), 0, st, a); break;
        case 3: hipLaunchKernelGGL((attn_mfma<D, 3, 2>), grid, dim3(128), 0, st, a); break;
        default: hipLaunchKernelGGL((attn_mfma<D, 4, 2>), grid, dim3(128), 0, st, a); break;
    }
}

int launch_verify_attn(const spec_attn_desc& d, const AttnPlan& p, const void* q, const void* k,
                       const void* v, const int32_t* prefix_len, const int32_t* parent, void* out,
                       void* workspace, hipStream_t stream) {
    AttnArgs a;
    a.q = q;
    a.k = k;
    a.v = v;
    a.out = out;
    a.prefix_len = prefix_len;
    a.parent = parent;
    a.B = d.batch;
    a.N = d.num_nodes;
    a.Hq = d.num_q_heads;
    a.Hkv = d.num_kv_heads;
    a.G = d.num_q_heads / d.num_kv_heads;
    a.cap = d.kv_capacity;
    a.R = p.rows;
    a.nrg = p.row_groups;
    a.chunk = p.chunk;
    a.nsplit_max = p.nsplit_max;
    a.max_keys = p.max_keys;
    const float scale = d.softmax_scale > 0.f ? d.softmax_scale : 1.0f / sqrtf(static_cast<float>(d.head_dim));
    a.scale_log2 = scale * 1.4426950408889634f;
    if (p.nsplit_max > 1) {
        const size_t parts = static_cast<size_t>(d.batch) * d.num_kv_heads * p.nsplit_max * p.rows;
        char* ws = static_cast<char*>(workspace);
        a.ws_o = reinterpret_cast<float*>(ws);
        ws += align_up(parts * d.head_dim * sizeof(float), 256);
        a.ws_ml = reinterpret_cast<float2*>(ws);
    } else {
        a.ws_o = nullptr;
        a.ws_ml = nullptr;
    }
    const long units = static_cast<long>(d.batch) * d.num_kv_heads * p.nsplit_max;
    const long units_pad = (units + 7) / 8 * 8;
    const dim3 grid(static_cast<unsigned>(units_pad * p.row_groups));
    if (p.mfma) {
        if (d.head_dim == 128)
            launch_mfma_rt<128>(p, a, grid, stream);
        else
            launch_mfma_rt<64>(p, a, grid, stream);
    } else if (d.dtype == SPEC_F32) {
        if (d.head_dim == 128)
            hipLaunchKernelGGL((attn_valu<float, 128>), grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((attn_valu<float, 64>), grid, dim3(256), 0, stream, a);
    } else {
        if (d.head_dim == 128)
            hipLaunchKernelGGL((attn_valu<uint16_t, 128>), grid, dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL((attn_valu<uint16_t, 64>), grid, dim3(256), 0, stream, a);
    }
    if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    if (p.nsplit_max > 1) {
        const long rows = static_cast<long>(d.batch) * d.num_kv_heads * p.rows;
        const dim3 cgrid(static_cast<unsigned>((rows + 3) / 4));
        const int bf16_out = d.dtype == SPEC_BF16;
        if (d.head_dim == 128)
            hipLaunchKernelGGL((attn_combine<128>), cgrid, dim3(256), 0, stream, a, bf16_out);
        else
            hipLaunchKernelGGL((attn_combine<64>), cgrid, dim3(256), 0, stream, a, bf16_out);
        if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    }
    return SPEC_OK;
}

}  // namespace specv
