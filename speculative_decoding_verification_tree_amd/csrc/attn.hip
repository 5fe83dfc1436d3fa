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
// Work decomposition.  The keys of one (b, g) -- a slab -- are cut into
// 32-key blocks.  A workgroup holds every query row of its row group, so each
// KV element is read from HBM once per row group and shared by all its rows;
// it walks one or more segments (a run of consecutive blocks of one slab).
// Two ways to hand out segments:
//   balanced : the blocks of all slabs, concatenated slab after slab, are cut
//              into P equal ranges, one per workgroup, with P about the number
//              of workgroups the chip holds at once.  Ragged prefix lengths
//              then cost nothing in balance, and no second wave of workgroups
//              runs at partial occupancy.  Segment (workgroup p, slab q) has
//              partial index p + q: both grow along the concatenation.
//   fixed    : split s of slab q takes blocks [s*C, (s+1)*C) (large batches,
//              where slabs far outnumber resident workgroups; VALU path).
// A slab covered by one segment is written straight to out; otherwise each
// segment writes its unnormalised partial (O, max, sum) -- O in bf16 from
// the one-row-group kernels, fp32 from the many-row kernel -- and
// attn_combine4 (few partials per slab) or attn_combine (many) merges a
// slab's partials with an exact log-sum-exp
// rescale, from the (first partial, count) table the segments leave in the
// workspace.
//
// The MFMA path runs one wavefront per workgroup: the wave streams its range
// with nothing to wait for but its own loads (no workgroup barrier, no
// cross-wave merge), prefetching one block ahead, across segment ends too.
//
// bf16 MFMA path (v_mfma_f32_16x16x32_bf16):
//   S^T = K * Q^T : A = 16 keys x 32 dims of K, B = Q^T held in registers.
//   The two 16-key halves of a block use the key order
//     row m of half h  <->  key 8*(m/4) + 4*h + m%4
//   so that lane (n, q) ends up holding row n's scores for keys 8q..8q+7:
//   exactly the A operand of the PV product, with no register shuffle.
//   O += P * V    : B = V^T slice read from a per-wave transposed LDS copy
//                   (16-byte reads, XOR-swizzled 16-byte columns).
//   A block is loaded into registers one iteration ahead; at the top of its
//   iteration it is moved to the wave's LDS stage (K as loaded, V
//   transposed) and the same registers take the next block's loads, so only
//   one block per wave occupies registers.
// fp32 (and any dtype) VALU path: 32 rows x 32 keys tiles through LDS.
#include <stdlib.h>

#include <atomic>

#include "spec_common.h"
#include "spec_internal.h"

namespace specv {

struct AttnArgs {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* ws_o;    // [parts][R][D]  unnormalised partial O
    float2* ws_ml;  // [parts][R]     (max in log2 units, sum)
    int2* seg;      // [B*Hkv]        (first partial, partial count) of each slab
    const int32_t* prefix_len;
    const int32_t* parent;
    int B, N, Hq, Hkv, G, cap, R, nrg;
    int balanced;      // 1: balanced ranges; 0: fixed splits
    int nparts;        // balanced: P; fixed: splits per slab
    int split_blocks;  // fixed: 32-key blocks per split
    int max_keys;      // host bound on L_b + N
    float scale_log2;  // softmax scale * log2(e)
    int bf16p;         // MFMA partials stored as bf16 (one-row-group kernels)
    int rope;          // fused depth-position rotary embedding of q and the tree's K rows
    RopeTable rope_tab;
};

// The rotary table into LDS (lanes 0 .. D/2 - 1 of every wave, which all
// write the same values): each takes its entry by selects over the unrolled
// constant indices, so the kernel argument is never indexed per lane.
template <int D>
__device__ __forceinline__ void rope_table_to_lds(const AttnArgs& a, double* s_rev) {
    const int t = threadIdx.x & 63;
    if (t < D / 2) {
        double v = 0.0;
#pragma unroll
        for (int j = 0; j < D / 2; ++j) v = t == j ? a.rope_tab.rev[j] : v;
        s_rev[t] = v;
    }
}

// Depth of every node of request b (lane i: node i) into LDS, from the
// ancestor-or-self masks.
__device__ __forceinline__ void depths_to_lds(const AttnArgs& a, uint64_t node_anc, int* s_depth) {
    const int lane = threadIdx.x & 63;
    if (lane < a.N) s_depth[lane] = __popcll(node_anc) - 1;
}

// q fragments of RT row tiles rotated at their rows' positions L + depth
// (anc[t]: the lane's row's ancestor mask; rows past R hold zeros).
template <int D, int RT>
__device__ __forceinline__ void rope_q_frags(bf16x8 (&qf)[RT][D / 32], const uint64_t (&anc)[RT], int L,
                                             const double* s_rev) {
    constexpr int H = D / 64;  // k-chunks holding the low half of the dims
    const int q4 = (threadIdx.x & 63) >> 4;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int pos = L + __popcll(anc[t]) - 1;
#pragma unroll
        for (int c = 0; c < H; ++c) {
            u32x4 lo = __builtin_bit_cast(u32x4, qf[t][c]), hi = __builtin_bit_cast(u32x4, qf[t][c + H]);
            rope_bf16x8(lo, hi, pos, s_rev, 32 * c + 8 * q4);
            qf[t][c] = __builtin_bit_cast(bf16x8, lo);
            qf[t][c + H] = __builtin_bit_cast(bf16x8, hi);
        }
    }
}

// Largest batch the balanced mode serves (its block-count scan lives in LDS).
constexpr int kMaxBalancedBatch = 480;

// Number of 32-key blocks of request b's slabs; 0 outside the contract
// (L < 0 or L + N beyond the cache or the host bound): such requests are
// skipped and their output is left unwritten.
__device__ __forceinline__ int request_blocks(const AttnArgs& a, int L) {
    const int Tk = L + a.N;
    return (L < 0 || Tk > a.cap || Tk > a.max_keys) ? 0 : (Tk + 31) >> 5;
}

// Workgroup -> (unit, row group).  The row groups of one unit get
// consecutive dispatch slots on one XCD (block i runs on XCD i % 8), so they
// share the unit's KV blocks through that XCD's L2.
__device__ __forceinline__ void decode_unit(const AttnArgs& a, int& unit, int& rg) {
    const int i = blockIdx.x;
    const int xcd = i & 7, j = i >> 3;
    rg = j % a.nrg;
    unit = (j / a.nrg) * 8 + xcd;
}

// s_cum[b] = blocks of requests 0..b-1 (per kv head), b = 0..B, and
// s_len[b] = prefix length of request b, computed by one wavefront.
// Balanced mode only (B <= kMaxBalancedBatch).
__device__ __forceinline__ void scan_request_blocks(const AttnArgs& a, int* s_cum, int* s_len) {
    const int lane = threadIdx.x & 63;
    const int per = (a.B + 63) / 64;
    const int lo = lane * per, hi = min(lo + per, a.B);
    int sum = 0;
    for (int i = lo; i < hi; ++i) {
        const int L = a.prefix_len[i];
        const int nb = request_blocks(a, L);
        s_len[i] = L;
        s_cum[i + 1] = nb;
        sum += nb;
    }
    int incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(incl, o);
        if (lane >= o) incl += t;
    }
    wave_lds_sync();
    int run = incl - sum;
    for (int i = lo; i < hi; ++i) {
        run += s_cum[i + 1];
        s_cum[i + 1] = run;
    }
    if (lane == 0) s_cum[0] = 0;
    wave_lds_sync();
}

// One segment: blocks [blk0, blk1) of slab (b, g); L = prefix length of b.
struct Seg {
    int b, g, blk0, blk1, L;
    int part;    // partial index (unused when direct)
    int direct;  // the segment covers its whole slab: write out
    int table;   // this workgroup records the slab's (first, count)
    int first, count;
};

struct SegIter {
    int x, hi, nb_total;  // balanced: next block, end of range, all blocks
    int P;                // balanced: ranges in use (a.nparts capped by the actual blocks)
    int unit;
    bool done;
};

// floor(num / den) for 0 <= num < 2^52, 0 < den < 2^31: a correctly rounded
// double quotient is off by at most one, fixed with exact integer products
// (a 64-bit integer division is a long software sequence here).
__device__ __forceinline__ int floor_div(long num, int den) {
    int q = static_cast<int>(static_cast<double>(num) / static_cast<double>(den));
    if (static_cast<long>(q) * den > num) --q;
    else if (static_cast<long>(q + 1) * den <= num) ++q;
    return q;
}

// Workgroup of global block x in balanced mode: p with floor(p*NB/P) <= x.
__device__ __forceinline__ int part_of(int x, int nb_total, int P) {
    return floor_div(static_cast<long>(x + 1) * P - 1, nb_total);
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Start the segment walk of this workgroup.  In balanced mode `scan` has one
// wavefront scan the request block counts into s_cum / s_len first;
// without it they must already be there.
__device__ __forceinline__ SegIter begin_segments(const AttnArgs& a, int unit, int* s_cum, int* s_len,
                                                  bool scan = true) {
    SegIter it;
    it.unit = unit;
    it.done = false;
    it.x = it.hi = it.nb_total = 0;
    it.P = 1;
    if (a.balanced) {
        if (scan) scan_request_blocks(a, s_cum, s_len);
        it.nb_total = a.Hkv * s_cum[a.B];
        // The host sized P from its prefix bound; the actual blocks may be
        // fewer (ragged or loose bounds).  Capping P at nb_total / split_blocks
        // keeps every range non-empty (at least split_blocks blocks when there
        // are that many): an empty range inside a slab would leave a partial
        // slot between the slab's first and last partial unwritten.
        it.P = max(1, min(a.nparts, it.nb_total / a.split_blocks));
        if (unit < it.P) {
            it.x = floor_div(static_cast<long>(unit) * it.nb_total, it.P);
            it.hi = floor_div(static_cast<long>(unit + 1) * it.nb_total, it.P);
        }
    }
    return it;
}

__device__ __forceinline__ bool next_segment(const AttnArgs& a, SegIter& it, const int* s_cum, const int* s_len,
                                             Seg& sg) {
    if (a.balanced) {
        if (it.x >= it.hi) return false;
        // request b: s_cum[b] <= x / Hkv < s_cum[b + 1]
        const int y = it.x / a.Hkv;
        int lo = 0, hi = a.B;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (s_cum[mid] <= y) lo = mid; else hi = mid - 1;
        }
        const int b = uniform(lo);
        const int nb = s_cum[b + 1] - s_cum[b];
        const int local = it.x - a.Hkv * s_cum[b];
        const int g = local / nb, off = local - g * nb;
        const int begin = it.x - off, end = begin + nb;
        const int x1 = end < it.hi ? end : it.hi;
        const int q = b * a.Hkv + g;
        const int pf = part_of(begin, it.nb_total, it.P), pl = part_of(end - 1, it.nb_total, it.P);
        sg.b = b;
        sg.L = uniform(s_len[b]);
        sg.g = uniform(g);
        sg.blk0 = uniform(off);
        sg.blk1 = uniform(off + (x1 - it.x));
        sg.part = it.unit + q;
        sg.direct = pf == pl;
        sg.table = off == 0;
        sg.first = pf + q;
        sg.count = pl - pf + 1;
        it.x = x1;
        return true;
    }
    if (it.done) return false;
    it.done = true;
    const int q = it.unit / a.nparts, s = it.unit % a.nparts;
    if (q >= a.B * a.Hkv) return false;
    const int b = q / a.Hkv;
    const int L = a.prefix_len[b];
    const int nb = request_blocks(a, L);
    const int x0 = s * a.split_blocks;
    if (x0 >= nb) return false;
    sg.b = b;
    sg.L = L;
    sg.g = q % a.Hkv;
    sg.blk0 = x0;
    sg.blk1 = min(nb, x0 + a.split_blocks);
    sg.part = q * a.nparts + s;
    sg.count = (nb + a.split_blocks - 1) / a.split_blocks;
    sg.direct = sg.count == 1;
    sg.table = s == 0;
    sg.first = q * a.nparts;
    return true;
}

// Ancestor-or-self bit mask of node `lane` of request b (lanes >= N give
// node 0's), by pointer doubling over the parent array in one wavefront:
// after round k a lane holds its first 2^k path nodes and its 2^k-th
// ancestor.
__device__ __forceinline__ uint64_t anc_mask(const AttnArgs& a, int b) {
    const int lane = threadIdx.x & 63;
    const int i = lane < a.N ? lane : 0;
    if (!a.parent) return i == 63 ? ~0ull : (2ull << i) - 1ull;  // chain: nodes 0..i
    int up = tree_parent(a.parent, a.N, b, i);
    uint64_t m = 1ull << i;
#pragma unroll
    for (int k = 0; k < 6; ++k) {
        const int src = up >= 0 ? up : 0;
        const uint32_t lo = __shfl(static_cast<uint32_t>(m), src), hi = __shfl(static_cast<uint32_t>(m >> 32), src);
        const int upup = __shfl(up, src);
        if (up >= 0) {
            m |= static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
            up = upup;
        }
    }
    return m;
}

__device__ __forceinline__ uint64_t shfl_u64(uint64_t v, int src) {
    const uint32_t lo = __shfl(static_cast<uint32_t>(v), src), hi = __shfl(static_cast<uint32_t>(v >> 32), src);
    return static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
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
// MFMA path (bf16).  D in {64, 128}; RT 16-row tiles; one wavefront.
// ----------------------------------------------------------------------------
// K fragments (A operand, paired-half key order) and V rows of one 32-key
// block, held in registers between the load and the LDS stage.
template <int D>
struct KVBlock {
    static constexpr int NC32 = D / 32;
    static constexpr int KPL = 32 / (64 / (D / 8));
    u32x4 kf[2][NC32];
    u32x4 vr[KPL];
};

// Issue the loads of the block starting at key kb; rows are clamped to
// row_max (the slab's last key) so no row past the tree is read.
template <int D>
__device__ __forceinline__ void load_kv_block(KVBlock<D>& blk, const uint16_t* kbase, const uint16_t* vbase, int kb,
                                              int row_max, int n16, int q4, int vch, int vkg) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = min(kb + 8 * (n16 >> 2) + 4 * h + (n16 & 3), row_max);
#pragma unroll
        for (int c = 0; c < KVBlock<D>::NC32; ++c)
            blk.kf[h][c] = ld_stream(kbase + static_cast<size_t>(row) * D + 32 * c + 8 * q4);
    }
#pragma unroll
    for (int jj = 0; jj < KVBlock<D>::KPL; ++jj) {
        const int row = min(kb + vkg * KVBlock<D>::KPL + jj, row_max);
        blk.vr[jj] = ld_stream(vbase + static_cast<size_t>(row) * D + 8 * vch);
    }
}

// Query fragments (B operand of S^T = K Q^T) and ancestor masks of the 16-row
// tiles starting at row0; rows past R get zero queries and no key mask.
template <int D, int RT>
__device__ __forceinline__ void load_q(const AttnArgs& a, int b, int g, int row0, uint64_t node_anc,
                                       bf16x8 (&qf)[RT][D / 32], uint64_t (&anc)[RT]) {
    const int lane = threadIdx.x & 63, n16 = lane & 15, q4 = lane >> 4;
    const uint16_t* qb = static_cast<const uint16_t*>(a.q);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int r = row0 + t * 16 + n16;
        const bool valid = r < a.R;
        const int node = valid ? r / a.G : 0;
        const uint64_t m = shfl_u64(node_anc, node);
        anc[t] = valid ? m : ~0ull;
        const int hq = g * a.G + (valid ? r % a.G : 0);
        const uint16_t* qrow = qb + ((static_cast<size_t>(b) * a.N + node) * a.Hq + hq) * D;
#pragma unroll
        for (int c = 0; c < D / 32; ++c) {
            u32x4 u = {0u, 0u, 0u, 0u};
            if (valid) u = *reinterpret_cast<const u32x4*>(qrow + 32 * c + 8 * q4);
            qf[t][c] = __builtin_bit_cast(bf16x8, u);
        }
    }
}

// One 32-key block for RT row tiles: S^T = K Q^T (kread(h, c) gives the K
// fragment of half h, k-step c), the key mask, the online softmax, and
// O^T += V^T P^T from the transposed V in vt.
template <int D, int RT, bool PHASED, class KRead>
__device__ __forceinline__ void block_update(const KRead& kread, const unsigned char* vt, const bf16x8 (&qf)[RT][D / 32],
                                             const uint64_t (&anc)[RT], int kb, int L, int Tk, float scale_log2,
                                             float (&m_run)[RT], float (&l_run)[RT], f32x4 (&o)[RT][D / 16]) {
    constexpr int NC32 = D / 32, NC16 = D / 16;
    const int lane = threadIdx.x & 63, n16 = lane & 15, q4 = lane >> 4;
    // Blocks wholly inside the prefix need no key mask.
    const bool interior = kb + 32 <= L;
    // PHASED: the scores of every tile first, each K fragment read once
    // and feeding 2*RT independent accumulator chains (more registers);
    // otherwise tile by tile, re-reading the K fragments.
    f32x4 sc[PHASED ? RT : 1][2];
    if constexpr (PHASED) {
#pragma unroll
        for (int t = 0; t < RT; ++t) sc[t][0] = sc[t][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC32; ++c)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const bf16x8 kf = __builtin_bit_cast(bf16x8, kread(h, c));
#pragma unroll
                for (int t = 0; t < RT; ++t)
                    sc[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[t][c], sc[t][h], 0, 0, 0);
            }
    }
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        if constexpr (!PHASED) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < NC32; ++c)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kread(h, c)), qf[t][c], acc,
                                                                  0, 0, 0);
                sc[0][h] = acc;
            }
        }
        const f32x4* st = sc[PHASED ? t : 0];
        // This lane's keys are kb + 8*q4 + e, e = 0..7 (e = 4h + ii).  Bit e
        // of the mask: key below the slab end and either a prefix key or a
        // tree key on the row's root path.
        uint32_t kmask = 0xFFu;
        if (!interior) {
            const int base = kb + 8 * q4;
            const int nend = min(max(Tk - base, 0), 8);
            const int npre = min(max(L - base, 0), 8);
            const int sh = base - L;  // tree offset of key e is sh + e
            const uint32_t tree = sh >= 0 ? static_cast<uint32_t>(anc[t] >> min(sh, 63))
                                          : static_cast<uint32_t>(anc[t] << min(-sh, 63));
            const uint32_t pre = (1u << npre) - 1u;
            kmask = ((tree & 0xFFu) | pre) & ((1u << nend) - 1u);
        }
        // Raw scores (masked to -inf only in blocks that reach past the
        // prefix: a wave-uniform branch).  The softmax scale (times log2 e,
        // > 0) is applied once to the lane's max -- rounding is monotonic, so
        // max(s) * c == max(s * c) exactly -- and folded into the exponent's
        // fma below, instead of one multiply per score.
        float s[8];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) s[4 * h + ii] = st[h][ii];
        if (!interior) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s[e] = ((kmask >> e) & 1u) ? s[e] : -INFINITY;
        }
        // Lazy rescale: keep the running max (log2 units) unless a row's
        // block max exceeds it by more than 8 (probabilities stay <= 2^8,
        // exact in fp32 and as precise in bf16).  A row's max exceeds it iff
        // one of its four lanes' does, so the wave-uniform test takes each
        // lane's own max; the row maxima are formed only when some row
        // rescales.
        // IEEE maximum (gfx950 v_maximum3_f32): unlike fmaxf it needs no
        // canonicalising v_max_f32 x, x per matrix-core result.  The scores
        // hold no NaN, where the two agree.
        auto vmax = [](float x, float y) { return __builtin_elementwise_maximum(x, y); };
        float bm = vmax(vmax(vmax(vmax(s[0], s[1]), s[2]), vmax(vmax(s[3], s[4]), s[5])), vmax(s[6], s[7])) * scale_log2;
        if (__builtin_amdgcn_ballot_w64(bm > m_run[t] + 8.f) != 0ull) {
            bm = max_across_rows(bm);
            const float mn = fmaxf(m_run[t], bm);
            const float alpha = m_run[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[t] - mn);
            l_run[t] *= alpha;
#pragma unroll
            for (int c = 0; c < NC16; ++c) o[t][c] *= alpha;  // o holds row n16 of this lane
            m_run[t] = mn;
        }
        const float mu = m_run[t] == -INFINITY ? 0.f : m_run[t];
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(s[e], scale_log2, -mu));
        const float rs = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        l_run[t] += rs;  // this lane's share of the row sum; the four shares are added at the end
        u32x4 pp;
        pp[0] = pack_bf16x2(p[0], p[1]);
        pp[1] = pack_bf16x2(p[2], p[3]);
        pp[2] = pack_bf16x2(p[4], p[5]);
        pp[3] = pack_bf16x2(p[6], p[7]);
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
        // Tile by tile: re-read the K fragments for the next tile rather than
        // keep them live (registers bound the waves per SIMD).
        if constexpr (!PHASED) asm volatile("" ::: "memory");
    }
}

// A segment's result for the 16-row tiles starting at row0, straight from
// registers: lane (n, q) holds row n of each tile (dims 16c + 4q .. +3 of O
// and the row's running max and sum).  The normalised output when the
// segment covers its slab, else the partial.
// NCW < D/16: o holds the column tiles c0 .. c0 + NCW - 1 only (a share of
// a merged result); with_ml: this caller stores the rows' (max, sum).
template <int D, int RT, bool BF16P = true, int NCW = D / 16>  // BF16P = false: the caller never stores bf16 partials
__device__ __forceinline__ void write_rows(const AttnArgs& a, const Seg& cur, int row0, const float (&m_run)[RT],
                                           const float (&l_run)[RT], const f32x4 (&o)[RT][NCW], int c0 = 0,
                                           bool with_ml = true) {
    const int lane = threadIdx.x & 63, n16 = lane & 15, q4 = lane >> 4;
    float l_row[RT];  // the row sums: the four lanes' shares added
#pragma unroll
    for (int t = 0; t < RT; ++t) l_row[t] = sum_across_rows(l_run[t]);
#pragma unroll
    for (int t = 0; t < RT; ++t) {
        const int r = row0 + t * 16 + n16;
        if (r >= a.R) continue;
        if (cur.direct) {
            const int node = r / a.G, hq = cur.g * a.G + r % a.G;
            const float inv = l_row[t] > 0.f ? 1.f / l_row[t] : 0.f;
            uint16_t* orow =
                static_cast<uint16_t*>(a.out) + ((static_cast<size_t>(cur.b) * a.N + node) * a.Hq + hq) * D;
#pragma unroll
            for (int c = 0; c < NCW; ++c) {
                uint2 pk;
                pk.x = pack_bf16x2(o[t][c][0] * inv, o[t][c][1] * inv);
                pk.y = pack_bf16x2(o[t][c][2] * inv, o[t][c][3] * inv);
                *reinterpret_cast<uint2*>(orow + 16 * (c0 + c) + 4 * q4) = pk;
            }
        } else {
            const size_t po = (static_cast<size_t>(cur.part) * a.R + r) * D;
            if (BF16P && a.bf16p) {  // half the bytes: the partials compete with the KV stream for HBM
                uint16_t* prow = reinterpret_cast<uint16_t*>(a.ws_o) + po;
#pragma unroll
                for (int c = 0; c < NCW; ++c)
                    *reinterpret_cast<uint2*>(prow + 16 * (c0 + c) + 4 * q4) =
                        make_uint2(pack_bf16x2(o[t][c][0], o[t][c][1]), pack_bf16x2(o[t][c][2], o[t][c][3]));
            } else {
                float* prow = a.ws_o + po;
#pragma unroll
                for (int c = 0; c < NCW; ++c) *reinterpret_cast<f32x4*>(prow + 16 * (c0 + c) + 4 * q4) = o[t][c];
            }
            if (with_ml && q4 == 0) a.ws_ml[static_cast<size_t>(cur.part) * a.R + r] = make_float2(m_run[t], l_row[t]);
        }
    }
}

// Blocks [f0, f1) of segment s taken by wave w of W: contiguous shares
// (empty when the segment has fewer blocks than W).
template <int W>
__device__ __forceinline__ void wave_share(const Seg& s, int w, int& f0, int& f1) {
    const int n = s.blk1 - s.blk0;
    f0 = s.blk0 + (w * n) / W;
    f1 = s.blk0 + ((w + 1) * n) / W;
}

// W = 1: one wavefront per workgroup streams its range.  W > 1 (small
// problems, where one-wave ranges would be a couple of blocks each and the
// partials would rival the KV bytes): W waves split every segment of the
// range into contiguous shares, then merge their softmax states exactly in
// LDS -- M = max of the waves' running maxima, O and the sums rescaled by
// 2^(m_w - M) and added -- so the workgroup writes one partial per segment.
template <int D, int RT, bool ROPE, int W = 1>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(RT <= 2 ? 2 : 1))) void attn_mfma(AttnArgs a) {
    constexpr int NC32 = D / 32;  // k-steps of the QK product
    constexpr int NC16 = D / 16;  // n-tiles of the PV product
    constexpr int CPR = D / 8;    // 16-byte chunks per cache row
    constexpr int KPL = KVBlock<D>::KPL;  // keys per lane in the V load (8 or 4)
    constexpr int KS_BYTES = 2 * NC32 * 64 * 16;  // K fragments of one block, lane-major
    constexpr int VT_BYTES = D * 64;              // V^T of one block
    constexpr int STAGE = KS_BYTES + VT_BYTES;
    // The merge's O of every wave reuses the stages; each wave stores whole column tiles.
    static_assert(W == 1 || (W * RT * NC16 * 64 * 16 <= W * STAGE && NC16 % W == 0), "merge layout");
    __shared__ __attribute__((aligned(16))) unsigned char s_stage[W * STAGE];
    __shared__ int s_cum[kMaxBalancedBatch + 1];
    __shared__ int s_len[kMaxBalancedBatch];
    __shared__ double s_rev[W][kRopeMaxPairs];
    __shared__ int s_depth[W][kMaxNodes];
    __shared__ float s_mw[W > 1 ? W * RT * 64 : 1];  // the waves' running maxima (merge)
    __shared__ float s_lw[W > 1 ? W * RT * 64 : 1];  // their rescaled sums

    int unit, rg;
    decode_unit(a, unit, rg);
    const int lane = threadIdx.x & 63, wave = W > 1 ? uniform(static_cast<int>(threadIdx.x >> 6)) : 0;
    const int n16 = lane & 15, q4 = lane >> 4;
    const int vch = lane % CPR, vkg = lane / CPR;
    if constexpr (ROPE) rope_table_to_lds<D>(a, s_rev[wave]);
    unsigned char* ks = s_stage + wave * STAGE;
    unsigned char* vt = ks + KS_BYTES;
    const uint16_t* kc = static_cast<const uint16_t*>(a.k);
    const uint16_t* vc = static_cast<const uint16_t*>(a.v);

    SegIter it;
    if constexpr (W > 1) {  // one wave scans the request block counts for all
        if (a.balanced && wave == 0) scan_request_blocks(a, s_cum, s_len);
        __syncthreads();
        it = begin_segments(a, unit, s_cum, s_len, false);
    } else {
        it = begin_segments(a, unit, s_cum, s_len);
    }
    Seg cur;
    if (!next_segment(a, it, s_cum, s_len, cur)) return;  // uniform over the workgroup
    int L = cur.L;
    int my0, my1;  // this wave's blocks of the current segment
    wave_share<W>(cur, wave, my0, my1);
    KVBlock<D> R;
    {
        const size_t head = (static_cast<size_t>(cur.b) * a.Hkv + cur.g) * a.cap * D;
        load_kv_block<D>(R, kc + head, vc + head, (my0 < my1 ? my0 : cur.blk0) * 32, L + a.N - 1, n16, q4, vch, vkg);
    }
    auto kread = [&](int h, int c) { return *reinterpret_cast<const u32x4*>(ks + ((h * NC32 + c) * 64 + lane) * 16); };
    for (;;) {
        const int b = cur.b, g = cur.g;
        const int Tk = L + a.N;
        const size_t head = (static_cast<size_t>(b) * a.Hkv + g) * a.cap * D;
        const uint16_t* kbase = kc + head;
        const uint16_t* vbase = vc + head;
        // The next segment, whose first block (of this wave's share) is
        // loaded during this one's last.
        Seg nxt;
        const bool more = next_segment(a, it, s_cum, s_len, nxt);
        const int Ln = more ? nxt.L : 0;
        const size_t nhead = more ? (static_cast<size_t>(nxt.b) * a.Hkv + nxt.g) * a.cap * D : head;
        int nmy0 = 0, nmy1 = 0;
        if (more) wave_share<W>(nxt, wave, nmy0, nmy1);
        const int nfirst = nmy0 < nmy1 ? nmy0 : nxt.blk0;  // (an empty share loads the segment's first block)

        bf16x8 qf[RT][NC32];
        uint64_t anc[RT];
        {
            const uint64_t node_anc = anc_mask(a, b);
            load_q<D, RT>(a, b, g, rg * RT * 16, node_anc, qf, anc);
            if constexpr (ROPE) {
                depths_to_lds(a, node_anc, s_depth[wave]);
                rope_q_frags<D, RT>(qf, anc, L, s_rev[wave]);
            }
        }
        float m_run[RT], l_run[RT];
        f32x4 o[RT][NC16];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            m_run[t] = -INFINITY;
            l_run[t] = 0.f;
#pragma unroll
            for (int c = 0; c < NC16; ++c) o[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }

        for (int xb = my0; xb < my1; ++xb) {
            const int kb = xb * 32;
            // Stage the block: K fragments as loaded (each lane reads back its
            // own), V transposed (row d holds the block's 32 keys); keys at
            // or past the slab end are zeroed so no stale value reaches P*V.
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int c = 0; c < NC32; ++c)
                    *reinterpret_cast<u32x4*>(ks + ((h * NC32 + c) * 64 + lane) * 16) = R.kf[h][c];
#pragma unroll
            for (int jj = 0; jj < KPL; ++jj)
                if (kb + vkg * KPL + jj >= Tk) R.vr[jj] = u32x4{0u, 0u, 0u, 0u};
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
                        wv[e] = __builtin_amdgcn_perm(R.vr[2 * e + 1][t >> 1], R.vr[2 * e][t >> 1], sel);
                    *reinterpret_cast<u32x4*>(dst) = wv;
                } else {
                    uint2 wv;
                    wv.x = __builtin_amdgcn_perm(R.vr[1][t >> 1], R.vr[0][t >> 1], sel);
                    wv.y = __builtin_amdgcn_perm(R.vr[3][t >> 1], R.vr[2][t >> 1], sel);
                    *reinterpret_cast<uint2*>(dst) = wv;
                }
            }
            // Tree keys of a fused-RoPE call: each lane turns the K rows of
            // its own staged fragments that are tree nodes, at L + depth
            // (the block's registers are free here, about to take the next
            // block's loads).
            if (ROPE && kb + 32 > L) {  // wave-uniform
                wave_lds_sync();
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int n = kb + 8 * (n16 >> 2) + 4 * h + (n16 & 3) - L;
                    if (n >= 0 && n < a.N) {
                        const int pos = L + s_depth[wave][n];
#pragma unroll
                        for (int c = 0; c < NC32 / 2; ++c) {
                            u32x4* lo = reinterpret_cast<u32x4*>(ks + ((h * NC32 + c) * 64 + lane) * 16);
                            u32x4* hi = reinterpret_cast<u32x4*>(ks + ((h * NC32 + c + NC32 / 2) * 64 + lane) * 16);
                            u32x4 x = *lo, y = *hi;
                            rope_bf16x8(x, y, pos, s_rev[wave], 32 * c + 8 * q4);
                            *lo = x;
                            *hi = y;
                        }
                    }
                }
            }
            // The registers are free: load the next block -- this segment's,
            // else the next segment's first, else this one again (a cache
            // hit).  The load is unconditional so the wait at the top of an
            // iteration never drains a prefetch early.
            asm volatile("" ::: "memory");
            {
                const bool here = xb + 1 < my1;
                const uint16_t* nk = here || !more ? kbase : kc + nhead;
                const uint16_t* nv = here || !more ? vbase : vc + nhead;
                const int nkb = here ? kb + 32 : (more ? nfirst * 32 : kb);
                const int nmax = here || !more ? Tk - 1 : Ln + a.N - 1;
                load_kv_block<D>(R, nk, nv, nkb, nmax, n16, q4, vch, vkg);
            }
            wave_lds_sync();
            block_update<D, RT, false>(kread, vt, qf, anc, kb, L, Tk, a.scale_log2, m_run, l_run, o);
            wave_lds_sync();
        }
        if constexpr (W > 1) {
            // A wave with no share here has not loaded the next segment's
            // first block yet.
            if (my0 >= my1 && more)
                load_kv_block<D>(R, kc + nhead, vc + nhead, nfirst * 32, Ln + a.N - 1, n16, q4, vch, vkg);
            // Merge: the running maxima first (every wave is past its last
            // stage read once they are all written); then every wave leaves
            // its rescaled O and sums in the stages, and wave w adds up and
            // stores column tiles [w*NCW, (w+1)*NCW) of the result.
#pragma unroll
            for (int t = 0; t < RT; ++t) s_mw[(wave * RT + t) * 64 + lane] = m_run[t];
            __syncthreads();
            f32x4* ob = reinterpret_cast<f32x4*>(s_stage);  // [W][RT][NC16][64 lanes]
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                float M = s_mw[t * 64 + lane];
#pragma unroll
                for (int w = 1; w < W; ++w) M = fmaxf(M, s_mw[(w * RT + t) * 64 + lane]);
                const float f = m_run[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[t] - M);
                s_lw[(wave * RT + t) * 64 + lane] = l_run[t] * f;
#pragma unroll
                for (int c = 0; c < NC16; ++c) ob[((wave * RT + t) * NC16 + c) * 64 + lane] = o[t][c] * f;
                m_run[t] = M;
            }
            __syncthreads();
            constexpr int NCW = NC16 / W;
            f32x4 os[RT][NCW];
#pragma unroll
            for (int t = 0; t < RT; ++t) {
                l_run[t] = 0.f;
#pragma unroll
                for (int c = 0; c < NCW; ++c) os[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int w = 0; w < W; ++w) {
                    l_run[t] += s_lw[(w * RT + t) * 64 + lane];
#pragma unroll
                    for (int c = 0; c < NCW; ++c) os[t][c] += ob[((w * RT + t) * NC16 + wave * NCW + c) * 64 + lane];
                }
            }
            write_rows<D, RT, true, NCW>(a, cur, rg * RT * 16, m_run, l_run, os, wave * NCW, wave == 0);
            __syncthreads();  // the stages and the merge arrays are free for the next segment
        } else {
            write_rows<D, RT>(a, cur, rg * RT * 16, m_run, l_run, o);
        }
        if (cur.table && rg == 0 && threadIdx.x == 0 && a.seg) a.seg[b * a.Hkv + g] = make_int2(cur.first, cur.count);
        if (!more) break;
        cur = nxt;
        L = Ln;
        my0 = nmy0;
        my1 = nmy1;
    }
}

// ----------------------------------------------------------------------------
// MFMA path for many query rows (bf16): WK waves share each KV block through
// LDS and wave w owns row tiles [w*RT, (w+1)*RT) of the workgroup's rows, so
// a block is read once per WK*RT*16 rows and no cross-wave merge is needed.
// The workgroup loads each 32-key block cooperatively (coalesced 16-byte
// chunks) into a double-buffered LDS stage, one block in LDS and the next in
// flight in registers; one barrier per block.
// ----------------------------------------------------------------------------
// K of one block in LDS: row-major 32 keys x D, 16-byte chunks XOR-swizzled
// so that the 16 rows one A-operand read touches (paired-half key order)
// fall on distinct banks (D = 128; two-way for D = 64).
__device__ __forceinline__ int k_swz(int row) { return (row & 3) | ((row >> 1) & 12); }

template <int D, int WK>
struct SharedKV {
    static constexpr int CPR = D / 8;
    static constexpr int NT = 64 * WK;
    static constexpr int KCH = 32 * CPR;    // K chunks of a block
    static constexpr int VTASK = 16 * CPR;  // (key pair, chunk) tasks of V
    // SPLIT: waves [0, WK/2) move V (one key pair each thread) and the rest
    // K (two chunks each), so no thread loads more than two chunks or any
    // chunk twice.  Otherwise every thread takes KPT K chunks and VPT V tasks.
    static constexpr bool SPLIT = NT == 2 * VTASK && KCH == 2 * VTASK;
    static constexpr int KPT = SPLIT ? 2 : KCH / NT;
    static constexpr int VPT = SPLIT ? 1 : (VTASK + NT - 1) / NT;
    static constexpr int NR = SPLIT ? 2 : KPT + 2 * VPT;
    static_assert(SPLIT || (KPT >= 1 && KPT * NT == KCH), "every thread loads whole K chunks");
    u32x4 r[NR];  // SPLIT: a V key pair or two K chunks; else K chunks, then V pairs
    int kb, Tk;   // the block's first key and its slab's key count
};

// Waves per shared-KV workgroup: eight for D = 128 (256 rows share each KV
// block); four for D = 64, where a 32-key block has 256 K chunks.
template <int D>
constexpr int wg_waves() {
    return D == 128 ? 8 : 4;
}

template <int D>
__device__ __forceinline__ u32x4 kv_chunk(const uint16_t* base, int kb, int r, int ch, int Tk) {
    const int row = min(kb + r, Tk - 1);
    return ld_stream(base + static_cast<size_t>(row) * D + ch * 8);
}

template <int D, int WK>
__device__ __forceinline__ void load_shared_kv(SharedKV<D, WK>& s, const uint16_t* kbase, const uint16_t* vbase, int kb,
                                               int Tk) {
    using S = SharedKV<D, WK>;
    const int tid = threadIdx.x;
    s.kb = kb;
    s.Tk = Tk;
    if constexpr (S::SPLIT) {
        if (tid < S::VTASK) {  // wave-uniform
            const int kp = tid / S::CPR, ch = tid % S::CPR;
            s.r[0] = kv_chunk<D>(vbase, kb, 2 * kp, ch, Tk);
            s.r[1] = kv_chunk<D>(vbase, kb, 2 * kp + 1, ch, Tk);
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int ci = tid - S::VTASK + S::VTASK * j;
                s.r[j] = kv_chunk<D>(kbase, kb, ci / S::CPR, ci % S::CPR, Tk);
            }
        }
    } else {
#pragma unroll
        for (int j = 0; j < S::KPT; ++j) {
            const int ci = tid + S::NT * j;
            s.r[j] = kv_chunk<D>(kbase, kb, ci / S::CPR, ci % S::CPR, Tk);
        }
#pragma unroll
        for (int j = 0; j < S::VPT; ++j) {
            const int vt = tid + S::NT * j;
            const int task = vt < S::VTASK ? vt : 0;  // spare lanes re-read task 0 and never stage it
            const int kp = task / S::CPR, ch = task % S::CPR;
            s.r[S::KPT + 2 * j] = kv_chunk<D>(vbase, kb, 2 * kp, ch, Tk);
            s.r[S::KPT + 2 * j + 1] = kv_chunk<D>(vbase, kb, 2 * kp + 1, ch, Tk);
        }
    }
}

// K row-major (swizzled chunks) and V transposed.  V keys at or past the
// slab end are zeroed so no stale value reaches P*V.
template <int D>
__device__ __forceinline__ void stage_k_chunk(unsigned char* ks, int ci, const u32x4& c) {
    constexpr int CPR = D / 8;
    const int row = ci / CPR, col = ci % CPR;
    *reinterpret_cast<u32x4*>(ks + row * (2 * D) + ((col ^ k_swz(row)) & (CPR - 1)) * 16) = c;
}

template <int D>
__device__ __forceinline__ void stage_v_pair(unsigned char* vt, int task, const u32x4& v0, const u32x4& v1, int kb,
                                             int Tk) {
    constexpr int CPR = D / 8;
    const int kp = task / CPR, ch = task % CPR;
    const int key0 = 2 * kp;
    auto put = [&](const u32x4& w0, const u32x4& w1) {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int d = 8 * ch + t;
            const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
            const uint32_t w = __builtin_amdgcn_perm(w1[t >> 1], w0[t >> 1], sel);
            *reinterpret_cast<uint32_t*>(vt + d * 64 + (((key0 >> 3) ^ vt_swz(d)) * 16) + (key0 & 7) * 2) = w;
        }
    };
    if (kb + 32 <= Tk) {  // workgroup-uniform: no key of the block is past the slab end
        put(v0, v1);
    } else {
        const u32x4 zero = {0u, 0u, 0u, 0u};
        put(kb + key0 < Tk ? v0 : zero, kb + key0 + 1 < Tk ? v1 : zero);
    }
}

template <int D, int WK>
__device__ __forceinline__ void stage_shared_kv(const SharedKV<D, WK>& s, unsigned char* ks, unsigned char* vt) {
    using S = SharedKV<D, WK>;
    const int tid = threadIdx.x;
    if constexpr (S::SPLIT) {
        if (tid < S::VTASK) {  // wave-uniform
            stage_v_pair<D>(vt, tid, s.r[0], s.r[1], s.kb, s.Tk);
        } else {
#pragma unroll
            for (int j = 0; j < 2; ++j) stage_k_chunk<D>(ks, tid - S::VTASK + S::VTASK * j, s.r[j]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < S::KPT; ++j) stage_k_chunk<D>(ks, tid + S::NT * j, s.r[j]);
#pragma unroll
        for (int j = 0; j < S::VPT; ++j) {
            const int vtask = tid + S::NT * j;
            if (vtask < S::VTASK) stage_v_pair<D>(vt, vtask, s.r[S::KPT + 2 * j], s.r[S::KPT + 2 * j + 1], s.kb, s.Tk);
        }
    }
}

template <int D, int RT, int WK, bool ROPE>
__global__ __launch_bounds__(64 * WK) __attribute__((amdgpu_waves_per_eu(2))) void attn_mfma_wg(AttnArgs a) {
    constexpr int NC32 = D / 32, NC16 = D / 16, CPR = D / 8;
    constexpr int KS_BYTES = 32 * D * 2;  // K of one block, row-major
    constexpr int VT_BYTES = D * 64;      // V^T of one block
    constexpr int STAGE = KS_BYTES + VT_BYTES;
    __shared__ __attribute__((aligned(16))) unsigned char s_stage[2 * STAGE];
    __shared__ int s_cum[kMaxBalancedBatch + 1];
    __shared__ int s_len[kMaxBalancedBatch];
    __shared__ double s_rev[kRopeMaxPairs];
    __shared__ int s_depth[kMaxNodes];

    int unit, rg;
    decode_unit(a, unit, rg);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n16 = lane & 15, q4 = lane >> 4;
    const uint16_t* kc = static_cast<const uint16_t*>(a.k);
    const uint16_t* vc = static_cast<const uint16_t*>(a.v);
    const int row0 = (rg * WK + wave) * RT * 16;
    if constexpr (ROPE) rope_table_to_lds<D>(a, s_rev);

    if (wave == 0) (void)begin_segments(a, unit, s_cum, s_len, true);
    __syncthreads();
    // Two cursors over the same segment walk: one computes, one loads ahead
    // (through segment ends too).
    SegIter it = begin_segments(a, unit, s_cum, s_len, false);
    SegIter lit = it;
    Seg cur, lseg;
    if (!next_segment(a, it, s_cum, s_len, cur)) return;
    (void)next_segment(a, lit, s_cum, s_len, lseg);
    int lb = lseg.blk0;
    bool lmore = true;
    auto load_next = [&](SharedKV<D, WK>& S) {
        const size_t head = (static_cast<size_t>(lseg.b) * a.Hkv + lseg.g) * a.cap * D;
        load_shared_kv<D, WK>(S, kc + head, vc + head, lb * 32, lseg.L + a.N);
        if (lb + 1 < lseg.blk1) {
            ++lb;
        } else if (lmore) {
            Seg t;
            lmore = next_segment(a, lit, s_cum, s_len, t);
            if (lmore) {
                lseg = t;
                lb = t.blk0;
            }
        }
    };
    // One register set: at block i it holds block i+1, which is staged into
    // the other LDS buffer, and then takes block i+2's loads, which have
    // block i+1's computation to land.
    SharedKV<D, WK> R;
    load_next(R);
    int bi = 0;
    stage_shared_kv<D, WK>(R, s_stage, s_stage + KS_BYTES);
    load_next(R);
    __syncthreads();

    for (;;) {
        const int b = cur.b, g = cur.g;
        const int L = cur.L, Tk = L + a.N;
        bf16x8 qf[RT][NC32];
        uint64_t anc[RT];
        {
            const uint64_t node_anc = anc_mask(a, b);
            load_q<D, RT>(a, b, g, row0, node_anc, qf, anc);
            if constexpr (ROPE) {
                depths_to_lds(a, node_anc, s_depth);  // every wave writes the same values
                rope_q_frags<D, RT>(qf, anc, L, s_rev);
            }
        }
        // Wait for the queries here, once per segment: left pending into the
        // block loop, the wait at the loop head would also cover the KV
        // prefetch issued after them (loads retire in order) on every block.
#pragma unroll
        for (int t = 0; t < RT; ++t) {
#pragma unroll
            for (int c = 0; c < NC32; ++c) asm volatile("" ::"v"(qf[t][c]));
            asm volatile("" ::"v"(anc[t]));
        }
        float m_run[RT], l_run[RT];
        f32x4 o[RT][NC16];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
            m_run[t] = -INFINITY;
            l_run[t] = 0.f;
#pragma unroll
            for (int c = 0; c < NC16; ++c) o[t][c] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int xb = cur.blk0; xb < cur.blk1; ++xb) {
            const unsigned char* ks = s_stage + bi * STAGE;
            const unsigned char* vt = ks + KS_BYTES;
            if (ROPE && xb * 32 + 32 > L) {  // workgroup-uniform: a block holding tree keys
                // Turn the staged K rows of tree nodes at L + depth: one
                // thread per (row, pair of 16-byte chunks D/2 apart).
                __syncthreads();  // the depths of this segment are in LDS
                unsigned char* kw = s_stage + bi * STAGE;
                for (int task = tid; task < 32 * (CPR / 2); task += 64 * WK) {
                    const int row = task / (CPR / 2), col = task % (CPR / 2);
                    const int n = xb * 32 + row - L;
                    if (n >= 0 && n < a.N) {
                        u32x4* lo = reinterpret_cast<u32x4*>(kw + row * (2 * D) + ((col ^ k_swz(row)) & (CPR - 1)) * 16);
                        u32x4* hi = reinterpret_cast<u32x4*>(kw + row * (2 * D) +
                                                             (((col + CPR / 2) ^ k_swz(row)) & (CPR - 1)) * 16);
                        u32x4 x = *lo, y = *hi;
                        rope_bf16x8(x, y, L + s_depth[n], s_rev, 8 * col);
                        *lo = x;
                        *hi = y;
                    }
                }
                __syncthreads();
            }
            auto kread = [&](int h, int c) {
                const int row = 8 * (n16 >> 2) + 4 * h + (n16 & 3);
                return *reinterpret_cast<const u32x4*>(ks + row * (2 * D) + (((4 * c + q4) ^ k_swz(row)) & (CPR - 1)) * 16);
            };
            block_update<D, RT, true>(kread, vt, qf, anc, xb * 32, L, Tk, a.scale_log2, m_run, l_run, o);
            // The next block into the other buffer (its previous block was
            // finished by every wave before the last barrier), then refill.
            unsigned char* nks = s_stage + (bi ^ 1) * STAGE;
            stage_shared_kv<D, WK>(R, nks, nks + KS_BYTES);
            load_next(R);
            __syncthreads();
            bi ^= 1;
        }
        write_rows<D, RT, false>(a, cur, row0, m_run, l_run, o);
        if (cur.table && rg == 0 && tid == 0 && a.seg) a.seg[b * a.Hkv + g] = make_int2(cur.first, cur.count);
        if (!next_segment(a, it, s_cum, s_len, cur)) break;
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
    // Row stride D + 4: 16-byte aligned rows, and the eight rows that a row
    // group's lanes read at once start on distinct banks.
    constexpr int DP = D + 4;
    constexpr int DPL = D / 8;            // dims per thread, contiguous
    constexpr int NV4 = 32 * D / 4 / 256;  // 16-byte vectors per thread of a 32-row tile
    __shared__ __attribute__((aligned(16))) float s_q[32][DP];
    __shared__ __attribute__((aligned(16))) float s_k[32][DP];
    __shared__ __attribute__((aligned(16))) float s_v[32][DP];
    __shared__ __attribute__((aligned(16))) float s_p[32][36];
    __shared__ uint64_t s_anc[kMaxNodes];
    __shared__ double s_rev[kRopeMaxPairs];

    int unit, rg;
    decode_unit(a, unit, rg);
    SegIter it;  // fixed splits only
    it.unit = unit;
    it.done = false;
    it.x = it.hi = it.nb_total = 0;
    Seg sg;
    if (!next_segment(a, it, nullptr, nullptr, sg)) return;
    const int b = sg.b, g = sg.g;
    const int L = sg.L;
    const int Tk = L + a.N;
    const int k0 = sg.blk0 * 32;
    const int k1 = min(sg.blk1 * 32, Tk);

    const int tid = threadIdx.x;
    if (tid < 64) {
        const uint64_t m = anc_mask(a, b);
        if (tid < a.N) s_anc[tid] = m;
    }
    if (a.rope) rope_table_to_lds<D>(a, s_rev);
    // Fused RoPE: rows of the LDS tile rot[0..32) turn at L + depth(node),
    // node(r) giving each row's node (or -1: left as is).
    auto rope_rows = [&](float (*rot)[DP], auto node_of) {
        for (int task = tid; task < 32 * (D / 2); task += 256) {
            const int row = task / (D / 2), j = task % (D / 2);
            const int n = node_of(row);
            if (n >= 0) {
                float c, sn;
                rope_cs(L + __popcll(s_anc[n]) - 1, s_rev[j], c, sn);
                float x = rot[row][j], y = rot[row][j + D / 2];
                rope_pair(x, y, c, sn);
                if constexpr (sizeof(T) == 2) {  // bf16 tensors: the rotated value rounded as the MFMA paths do
                    x = bf16_bits_to_f32(static_cast<uint16_t>(f32_to_bf16_bits(x)));
                    y = bf16_bits_to_f32(static_cast<uint16_t>(f32_to_bf16_bits(y)));
                }
                rot[row][j] = x;
                rot[row][j + D / 2] = y;
            }
        }
    };
    const T* qp = static_cast<const T*>(a.q);
    const size_t head = (static_cast<size_t>(b) * a.Hkv + g) * a.cap;
    const T* kp = static_cast<const T*>(a.k) + head * D;
    const T* vp = static_cast<const T*>(a.v) + head * D;
    // fp32: the K and V rows of one 32-key tile as 16-byte loads, all in
    // flight at once; the first tile's go out with the queries', and each
    // next tile's while the current one is computed.
    float4 kr[sizeof(T) == 4 ? NV4 : 1], vr[sizeof(T) == 4 ? NV4 : 1];
    auto load_tile = [&](int kb) {
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < NV4; ++i) {
                const int e4 = tid + 256 * i, kk = e4 / (D / 4), d4 = e4 % (D / 4);
                const size_t off = static_cast<size_t>(min(kb + kk, Tk - 1)) * D + 4 * d4;
                kr[i] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(kp) + off);
                vr[i] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(vp) + off);
            }
        }
    };
    if constexpr (sizeof(T) == 4) {
        // fp32: 16-byte loads, all of a thread's issued before its LDS stores
        float4 qr[NV4];
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
            const int e4 = tid + 256 * i, lr = e4 / (D / 4), d4 = e4 % (D / 4);
            const int r = min(rg * 32 + lr, a.R - 1);
            const int node = r / a.G, hq = g * a.G + r % a.G;
            qr[i] = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(qp) +
                                                     ((static_cast<size_t>(b) * a.N + node) * a.Hq + hq) * D + 4 * d4);
        }
        load_tile(k0);
#pragma unroll
        for (int i = 0; i < NV4; ++i) {
            const int e4 = tid + 256 * i, lr = e4 / (D / 4), d4 = e4 % (D / 4);
            *reinterpret_cast<float4*>(&s_q[lr][4 * d4]) = rg * 32 + lr < a.R ? qr[i] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    } else {
        for (int e = tid; e < 32 * D; e += 256) {
            const int lr = e / D, d = e % D;
            const int r = rg * 32 + lr;
            float x = 0.f;
            if (r < a.R) {
                const int node = r / a.G, hq = g * a.G + r % a.G;
                x = load_elem(qp, ((static_cast<size_t>(b) * a.N + node) * a.Hq + hq) * D + d);
            }
            s_q[lr][d] = x;
        }
    }
    __syncthreads();
    if (a.rope) {
        rope_rows(s_q, [&](int lr) { return rg * 32 + lr < a.R ? (rg * 32 + lr) / a.G : -1; });
        __syncthreads();
    }

    // Thread (sr, sk): query row sr of the tile, keys sk + 8*jj of each
    // 32-key tile, output dims sk*DPL .. sk*DPL + DPL - 1.
    const int sr = tid >> 3, sk = tid & 7;
    const int r = rg * 32 + sr;
    const bool rvalid = r < a.R;
    const uint64_t anc = rvalid ? s_anc[r / a.G] : ~0ull;
    float m_run = -INFINITY, l_run = 0.f;
    float o[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) o[j] = 0.f;

    for (int kb = k0; kb < k1; kb += 32) {
        __syncthreads();
        if constexpr (sizeof(T) == 4) {
#pragma unroll
            for (int i = 0; i < NV4; ++i) {
                const int e4 = tid + 256 * i, kk = e4 / (D / 4), d4 = e4 % (D / 4);
                // (component stores: a 16-byte store of the register array's
                // element made the compiler keep the array in scratch)
                float* kd = &s_k[kk][4 * d4];
                float* vd = &s_v[kk][4 * d4];
                kd[0] = kr[i].x;
                kd[1] = kr[i].y;
                kd[2] = kr[i].z;
                kd[3] = kr[i].w;
                vd[0] = vr[i].x;
                vd[1] = vr[i].y;
                vd[2] = vr[i].z;
                vd[3] = vr[i].w;
            }
            if (kb + 32 < k1) load_tile(kb + 32);  // workgroup-uniform
        } else {
            for (int e = tid; e < 32 * D; e += 256) {
                const int kk = e / D, d = e % D;
                const size_t row = static_cast<size_t>(min(kb + kk, Tk - 1));
                s_k[kk][d] = load_elem(kp, row * D + d);
                s_v[kk][d] = load_elem(vp, row * D + d);
            }
        }
        __syncthreads();
        if (a.rope && kb + 32 > L) {  // a tile holding tree keys
            rope_rows(s_k, [&](int kk) {
                const int n = kb + kk - L;
                return n >= 0 && n < a.N ? n : -1;
            });
            __syncthreads();
        }
        // Scores of keys sk + 8*jj: 16-byte LDS reads, the query row's
        // (a broadcast within the row's eight lanes) shared by the four keys.
        float dot[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
        for (int d = 0; d < D; d += 4) {
            const float4 qd = *reinterpret_cast<const float4*>(&s_q[sr][d]);
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float4 kv = *reinterpret_cast<const float4*>(&s_k[sk + 8 * jj][d]);
                dot[jj] = fmaf(qd.x, kv.x, dot[jj]);
                dot[jj] = fmaf(qd.y, kv.y, dot[jj]);
                dot[jj] = fmaf(qd.z, kv.z, dot[jj]);
                dot[jj] = fmaf(qd.w, kv.w, dot[jj]);
            }
        }
        float s[4];
        float bm = -INFINITY;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            const int key = kb + sk + 8 * jj;
            const bool ok = key < k1 && (key < L || ((anc >> (key - L)) & 1ull));
            s[jj] = ok ? dot[jj] * a.scale_log2 : -INFINITY;
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
        for (int j = 0; j < DPL; ++j) o[j] *= alpha;
        __syncthreads();
#pragma unroll 2
        for (int k4 = 0; k4 < 32; k4 += 4) {
            const float4 p4 = *reinterpret_cast<const float4*>(&s_p[sr][k4]);
            const float pk[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
                for (int j = 0; j < DPL; j += 4) {
                    const float4 vv = *reinterpret_cast<const float4*>(&s_v[k4 + u][sk * DPL + j]);
                    o[j] = fmaf(pk[u], vv.x, o[j]);
                    o[j + 1] = fmaf(pk[u], vv.y, o[j + 1]);
                    o[j + 2] = fmaf(pk[u], vv.z, o[j + 2]);
                    o[j + 3] = fmaf(pk[u], vv.w, o[j + 3]);
                }
            }
        }
    }
    if (sg.table && rg == 0 && tid == 0 && a.seg) a.seg[b * a.Hkv + g] = make_int2(sg.first, sg.count);
    if (!rvalid) return;
    const int node = r / a.G, hq = g * a.G + r % a.G;
    const bool bf16_out = sizeof(T) == 2;
    if (sg.direct) {
        const size_t ob = ((static_cast<size_t>(b) * a.N + node) * a.Hq + hq) * D + sk * DPL;
#pragma unroll
        for (int j = 0; j < DPL; ++j) store_out(a.out, bf16_out, ob + j, l_run > 0.f ? o[j] / l_run : 0.f);
    } else {
        const size_t pi = static_cast<size_t>(sg.part);
        float* prow = a.ws_o + (pi * a.R + r) * D + sk * DPL;
#pragma unroll
        for (int j = 0; j < DPL; j += 4) *reinterpret_cast<f32x4*>(prow + j) = f32x4{o[j], o[j + 1], o[j + 2], o[j + 3]};
        if (sk == 0) a.ws_ml[pi * a.R + r] = make_float2(m_run, l_run);
    }
}

// ----------------------------------------------------------------------------
// Split combine: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s over the
// partials of one slab.  One wavefront per (request, kv head, query row).
// ----------------------------------------------------------------------------
template <int D, int SB, bool BP>  // SB: partials whose loads are in flight together; BP: bf16 partials
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, int bf16_out) {
    constexpr int DPL = D / 64;  // output elements per lane: dims lane + 64 j (fp32), DPL * lane + j (bf16)
    const int lane = threadIdx.x & 63;
    const long id = static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
    if (id >= static_cast<long>(a.B) * a.Hkv * a.R) return;
    const int r = static_cast<int>(id % a.R);
    const int bg = static_cast<int>(id / a.R);
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    // The slab record and the prefix length are independent: both loads go out together.
    const int L = a.prefix_len[b];
    const int2 sp = a.seg[bg];
    __builtin_amdgcn_sched_barrier(0);
    if (request_blocks(a, L) == 0) return;  // outside the contract: out left unwritten
    const int first = sp.x, count = sp.y;
    if (count <= 1) return;  // written by its only segment
    // Running (max, sum, O) over batches of SB partials, each batch one round of loads.
    float M = -INFINITY, lsum = 0.f;
    float acc[DPL];
#pragma unroll
    for (int j = 0; j < DPL; ++j) acc[j] = 0.f;
    for (int s0 = 0; s0 < count; s0 += SB) {
        float2 ml[SB];
        float ov[SB][DPL];
        if constexpr (BP) {
            // DPL consecutive bf16 values per partial (one 4-byte or 2-byte
            // load) from clamped indexes, selected afterwards: no load under
            // a branch, so all SB are in flight together.
            uint32_t raw[SB];
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                const size_t pi = static_cast<size_t>(first + min(s0 + k, count - 1));
                ml[k] = a.ws_ml[pi * a.R + r];
                const uint16_t* prow = reinterpret_cast<const uint16_t*>(a.ws_o) + (pi * a.R + r) * D + DPL * lane;
                if constexpr (DPL == 2) raw[k] = *reinterpret_cast<const uint32_t*>(prow);
                else raw[k] = *prow;
            }
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                if (s0 + k >= count) ml[k] = make_float2(-INFINITY, 0.f);
                if constexpr (DPL == 2) {
                    ov[k][0] = __uint_as_float(raw[k] << 16);
                    ov[k][1] = __uint_as_float(raw[k] & 0xFFFF0000u);
                } else {
                    ov[k][0] = __uint_as_float(raw[k] << 16);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < SB; ++k) {
                const size_t pi = static_cast<size_t>(first + s0 + k);
                ml[k] = make_float2(-INFINITY, 0.f);
#pragma unroll
                for (int j = 0; j < DPL; ++j) ov[k][j] = 0.f;
                if (s0 + k < count) {
                    ml[k] = a.ws_ml[pi * a.R + r];
#pragma unroll
                    for (int j = 0; j < DPL; ++j) ov[k][j] = a.ws_o[(pi * a.R + r) * D + lane + 64 * j];
                }
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
    for (int j = 0; j < DPL; ++j) store_out(a.out, bf16_out != 0, ob + (BP ? DPL * lane + j : lane + 64 * j), acc[j] * inv);
}

// Split combine for slabs of few partials: a wavefront merges four rows at
// once (16 lanes per row, D/16 consecutive dims per lane), so the whole grid
// is resident in one round and every row pays the dependent chain (prefix
// length, slab record, partials, store) once, with SB partials of each of
// its four rows in flight together.  Loads come from clamped indexes and
// are selected afterwards (none under a branch).
template <int D, int SB, bool BP>  // BP: bf16 partials
__global__ __launch_bounds__(256) void attn_combine4(AttnArgs a, int bf16_out) {
    constexpr int EPL = D / 16;  // dims per lane
    constexpr int NV = EPL / 4;  // 16-byte vectors per lane
    const int lane = threadIdx.x & 63, grp = lane >> 4, sl = lane & 15;
    const long total = static_cast<long>(a.B) * a.Hkv * a.R;
    const long id = (static_cast<long>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * 4 + grp;
    const long idc = id < total ? id : total - 1;
    const int r = static_cast<int>(idc % a.R);
    const int bg = static_cast<int>(idc / a.R);
    const int b = bg / a.Hkv, g = bg % a.Hkv;
    const int2 sp = a.seg[bg];
    const bool live = id < total && request_blocks(a, a.prefix_len[b]) != 0 && sp.y > 1;
    // Rows outside the contract or of a directly written slab read partial 0
    // (their slab record may be stale) and store nothing.
    const int first = live ? sp.x : 0, count = live ? sp.y : 0;
    float M = -INFINITY, lsum = 0.f;
    float acc[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) acc[j] = 0.f;
    for (int s0 = 0; __builtin_amdgcn_ballot_w64(s0 < count) != 0ull; s0 += SB) {
        float2 ml[SB];
        f32x4 ov[SB][NV];
#pragma unroll
        for (int k = 0; k < SB; ++k) {
            const size_t pi = static_cast<size_t>(first + max(min(s0 + k, count - 1), 0));
            ml[k] = a.ws_ml[pi * a.R + r];
            if constexpr (BP) {  // EPL bf16 values: one 16-byte load (D = 128) or 8-byte load (D = 64)
                const uint16_t* prow = reinterpret_cast<const uint16_t*>(a.ws_o) + (pi * a.R + r) * D + sl * EPL;
                uint32_t w[EPL / 2];
                if constexpr (EPL == 8) {
                    const u32x4 u = *reinterpret_cast<const u32x4*>(prow);
                    w[0] = u[0];
                    w[1] = u[1];
                    w[2] = u[2];
                    w[3] = u[3];
                } else {
                    const uint2 u = *reinterpret_cast<const uint2*>(prow);
                    w[0] = u.x;
                    w[1] = u.y;
                }
#pragma unroll
                for (int v = 0; v < NV; ++v)
                    ov[k][v] = f32x4{__uint_as_float(w[2 * v] << 16), __uint_as_float(w[2 * v] & 0xFFFF0000u),
                                     __uint_as_float(w[2 * v + 1] << 16), __uint_as_float(w[2 * v + 1] & 0xFFFF0000u)};
            } else {
                const float* prow = a.ws_o + (pi * a.R + r) * D + sl * EPL;
#pragma unroll
                for (int v = 0; v < NV; ++v) ov[k][v] = *reinterpret_cast<const f32x4*>(prow + 4 * v);
            }
        }
        // Keep the scheduler from sinking the partials' loads towards their
        // uses (it would trade them for registers one round trip at a time).
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < SB; ++k)
            if (s0 + k >= count) ml[k] = make_float2(-INFINITY, 0.f);
        float Mn = M;
#pragma unroll
        for (int k = 0; k < SB; ++k) Mn = fmaxf(Mn, ml[k].x);
        const float Mu = Mn == -INFINITY ? 0.f : Mn;
        const float sc = exp2f(M - Mu);
        lsum *= sc;
#pragma unroll
        for (int j = 0; j < EPL; ++j) acc[j] *= sc;
#pragma unroll
        for (int k = 0; k < SB; ++k) {
            const float wgt = ml[k].x == -INFINITY ? 0.f : exp2f(ml[k].x - Mu);
            lsum += wgt * ml[k].y;
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[4 * v + e] += wgt * ov[k][v][e];
        }
        M = Mn;
    }
    if (!live) return;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const int node = r / a.G, hq = g * a.G + r % a.G;
    const size_t ob = ((static_cast<size_t>(b) * a.N + node) * a.Hq + hq) * D + sl * EPL;
    if (bf16_out) {
        uint32_t w[EPL / 2];
#pragma unroll
        for (int j = 0; j < EPL / 2; ++j) w[j] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
        uint16_t* o16 = static_cast<uint16_t*>(a.out) + ob;
#pragma unroll
        for (int v = 0; v < EPL / 8; ++v)
            *reinterpret_cast<u32x4*>(o16 + 8 * v) = u32x4{w[4 * v], w[4 * v + 1], w[4 * v + 2], w[4 * v + 3]};
        if constexpr (EPL % 8 != 0) *reinterpret_cast<uint2*>(o16) = make_uint2(w[0], w[1]);
    } else {
        float* o32 = static_cast<float*>(a.out) + ob;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            *reinterpret_cast<f32x4*>(o32 + 4 * v) =
                f32x4{acc[4 * v] * inv, acc[4 * v + 1] * inv, acc[4 * v + 2] * inv, acc[4 * v + 3] * inv};
    }
}

// ----------------------------------------------------------------------------
// Host side
// ----------------------------------------------------------------------------
// Upper bound on resident workgroups of one launch (4 per CU on 256 CUs);
// sizes the balanced-mode partials independently of the device.
constexpr int kMaxResident = 2048;
constexpr int kKeySplitWaves = 4;  // waves splitting one range (small problems, one row tile group)
constexpr long kKeySplitMinBlocks = 1024;

AttnPlan plan_attn(const spec_attn_desc& d, int max_prefix_len) {
    AttnPlan p{};
    const int G = d.num_q_heads / d.num_kv_heads;
    p.rows = d.num_nodes * G;
    const long slabs = static_cast<long>(d.batch) * d.num_kv_heads;
    const long keys_max = static_cast<long>(max_prefix_len) + d.num_nodes;
    const long blocks_max = (keys_max + 31) / 32;
    long min_blocks = 2;  // balanced mode: least blocks per range
    p.kwaves = 1;
    if (d.dtype == SPEC_BF16) {
        p.mfma = true;
        if (p.rows <= 64) {  // one wave holds every row
            p.row_tiles = (p.rows + 15) / 16;
            p.row_groups = 1;
            p.waves = 1;
            // Few blocks in all (under 8 per one-wave range at full
            // residency): the waves of a workgroup split each range so a
            // partial covers kKeySplitWaves times the blocks.  Below about
            // a thousand blocks the step is latency-bound and the merge's
            // barriers cost more than the partial traffic they save.
            const long nblk = slabs * blocks_max;
            if (p.row_tiles <= 2 && nblk >= kKeySplitMinBlocks && nblk < 8L * kMaxResident) p.kwaves = kKeySplitWaves;
        } else {  // wg_waves<D>() waves of 32 rows share each KV block
            p.row_tiles = 2;
            p.waves = d.head_dim == 128 ? wg_waves<128>() : wg_waves<64>();
            p.row_groups = (p.rows + 32 * p.waves - 1) / (32 * p.waves);
        }
    } else {
        p.mfma = false;
        p.row_tiles = 0;
        p.row_groups = (p.rows + 31) / 32;
        p.waves = 4;
    }
    p.max_keys = static_cast<int>(keys_max);
    long parts;
    // Balanced ranges index blocks in 32 bits.
    p.balanced = p.mfma && d.batch <= kMaxBalancedBatch &&
                 static_cast<long>(d.batch) * d.num_kv_heads * blocks_max < (1L << 30);
    if (p.balanced) {
        // P is picked per launch from the device (resident workgroups); the
        // workspace holds the most partials any device can ask for.
        if (d.kv_split_keys > 0) min_blocks = (d.kv_split_keys + 31) / 32;
        else if (p.kwaves > 1) min_blocks = p.kwaves;  // one block per wave
        long pcap = kMaxResident / p.row_groups / p.kwaves;
        if (pcap < 8) pcap = 8;
        const long by_work = (slabs * blocks_max + min_blocks - 1) / min_blocks;
        p.parts_max = static_cast<int>(by_work < pcap ? by_work : pcap);
        if (p.parts_max < 1) p.parts_max = 1;
        p.split_blocks = static_cast<int>(min_blocks);
        parts = p.parts_max > 1 ? p.parts_max + slabs : 0;
        p.nsplit_max = 0;
    } else {
        // Fixed splits: about 4096 units of work, at least 8 blocks each.
        const long units = slabs * p.row_groups;
        const long want = units >= 4096 ? 1 : (4096 + units - 1) / units;
        long chunk_blocks = (blocks_max + want - 1) / want;
        // At least 8 blocks per MFMA split; the VALU path (one tile per
        // barrier round) spreads small problems down to one block per split.
        const long min_split = d.kv_split_keys > 0 ? (d.kv_split_keys + 31) / 32 : (p.mfma ? 8 : 1);
        if (chunk_blocks < min_split) chunk_blocks = min_split;
        p.split_blocks = static_cast<int>(chunk_blocks);
        p.nsplit_max = static_cast<int>((blocks_max + chunk_blocks - 1) / chunk_blocks);
        if (p.nsplit_max < 1) p.nsplit_max = 1;
        p.parts_max = 0;
        parts = p.nsplit_max > 1 ? slabs * p.nsplit_max : 0;
    }
    if (parts > 0) {
        p.ws_bytes = align_up(static_cast<size_t>(parts) * p.rows * d.head_dim * sizeof(float), 256) +
                     align_up(static_cast<size_t>(parts) * p.rows * sizeof(float2), 256) +
                     align_up(static_cast<size_t>(slabs) * sizeof(int2), 256);
    } else {
        p.ws_bytes = 0;
    }
    return p;
}

template <typename K>
static int resident_per_cu(K kernel, int threads) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) n = 1;
    return n;
}

// Queried once and cached (atomics: host threads may launch concurrently;
// every thread computes the same value).
static int device_cus() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int D, int RT, bool ROPE, int W = 1>
static int mfma_resident() {
    static std::atomic<int> cached{0};
    int n = cached.load(std::memory_order_relaxed);
    if (n == 0) {
        n = resident_per_cu(attn_mfma<D, RT, ROPE, W>, 64 * W);
        cached.store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int D, bool ROPE>
static int mfma_wg_resident() {
    static std::atomic<int> cached{0};
    int n = cached.load(std::memory_order_relaxed);
    if (n == 0) {
        n = resident_per_cu(attn_mfma_wg<D, 2, wg_waves<D>(), ROPE>, 64 * wg_waves<D>());
        cached.store(n, std::memory_order_relaxed);
    }
    return n;
}

template <int D, bool ROPE>
static int mfma_resident_rt(int rt, int waves, int kwaves) {
    if (waves > 1) return mfma_wg_resident<D, ROPE>();
    if (kwaves > 1) return rt == 1 ? mfma_resident<D, 1, ROPE, kKeySplitWaves>() : mfma_resident<D, 2, ROPE, kKeySplitWaves>();
    switch (rt) {
        case 1: return mfma_resident<D, 1, ROPE>();
        case 2: return mfma_resident<D, 2, ROPE>();
        case 3: return mfma_resident<D, 3, ROPE>();
        default: return mfma_resident<D, 4, ROPE>();
    }
}

template <int D>
static int mfma_resident_rt(int rt, int waves, int kwaves, bool rope) {
    return rope ? mfma_resident_rt<D, true>(rt, waves, kwaves) : mfma_resident_rt<D, false>(rt, waves, kwaves);
}

// The rotating kernels are separate instantiations: the plain ones keep
// their register allocation (the rotation code in the block loop costs the
// one-wave kernel a spill).
template <int D, bool ROPE>
static void launch_mfma_rt(const AttnPlan& p, const AttnArgs& a, dim3 grid, hipStream_t st) {
    if (p.waves > 1) {
        hipLaunchKernelGGL((attn_mfma_wg<D, 2, wg_waves<D>(), ROPE>), grid, dim3(64 * wg_waves<D>()), 0, st, a);
        return;
    }
    if (p.kwaves > 1) {
        constexpr int W = kKeySplitWaves;
        if (p.row_tiles == 1)
            hipLaunchKernelGGL((attn_mfma<D, 1, ROPE, W>), grid, dim3(64 * W), 0, st, a);
        else
            hipLaunchKernelGGL((attn_mfma<D, 2, ROPE, W>), grid, dim3(64 * W), 0, st, a);
        return;
    }
    switch (p.row_tiles) {
        case 1: hipLaunchKernelGGL((attn_mfma<D, 1, ROPE>), grid, dim3(64), 0, st, a); break;
        case 2: hipLaunchKernelGGL((attn_mfma<D, 2, ROPE>), grid, dim3(64), 0, st, a); break;
        case 3: hipLaunchKernelGGL((attn_mfma<D, 3, ROPE>), grid, dim3(64), 0, st, a); break;
        default: hipLaunchKernelGGL((attn_mfma<D, 4, ROPE>), grid, dim3(64), 0, st, a); break;
    }
}

template <int D>
static void launch_mfma_rt(const AttnPlan& p, const AttnArgs& a, dim3 grid, hipStream_t st) {
    if (a.rope) launch_mfma_rt<D, true>(p, a, grid, st);
    else launch_mfma_rt<D, false>(p, a, grid, st);
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
    a.balanced = p.balanced ? 1 : 0;
    a.split_blocks = p.split_blocks;
    a.max_keys = p.max_keys;
    const float scale = d.softmax_scale > 0.f ? d.softmax_scale : 1.0f / sqrtf(static_cast<float>(d.head_dim));
    a.scale_log2 = scale * 1.4426950408889634f;
    a.rope = d.rope_base > 0.f ? 1 : 0;
    fill_rope_table(a.rope_tab, d.head_dim, a.rope ? d.rope_base : 1.f);
    const long slabs = static_cast<long>(d.batch) * d.num_kv_heads;
    long units;
    bool combine;
    if (p.balanced) {
        const bool rope = d.rope_base > 0.f;
        const int per_cu = d.head_dim == 128 ? mfma_resident_rt<128>(p.row_tiles, p.waves, p.kwaves, rope)
                                             : mfma_resident_rt<64>(p.row_tiles, p.waves, p.kwaves, rope);
        long P = static_cast<long>(per_cu) * device_cus() / p.row_groups;
        if (P > p.parts_max) P = p.parts_max;
        if (P >= 8) P = P / 8 * 8;
        if (P < 1) P = 1;
        a.nparts = static_cast<int>(P);
        units = P;
        combine = P > 1;
    } else {
        a.nparts = p.nsplit_max;
        units = slabs * p.nsplit_max;
        combine = p.nsplit_max > 1;
    }
    // Partials of the longest slab: its blocks over the blocks per range
    // (plus one for a range that starts inside it), or its splits.  Up to 24
    // (three rounds of eight) go to attn_combine4, which takes MFMA partials
    // in bf16.
    long most;
    if (p.balanced) {
        const long per = (slabs * ((static_cast<long>(p.max_keys) + 31) / 32)) / a.nparts;
        most = per > 0 ? ((p.max_keys + 31) / 32 + per - 1) / per + 1 : a.nparts;
    } else {
        most = p.nsplit_max;
    }
    const bool wide = most > 24;  // one row per wavefront, 32 partials per round (more registers)
    // (the many-row kernel keeps fp32 partials: the bf16 store path cost it
    // registers and time)
    a.bf16p = combine && p.mfma && p.waves == 1 ? 1 : 0;
    if (combine) {
        const long parts = p.balanced ? p.parts_max + slabs : slabs * p.nsplit_max;
        char* ws = static_cast<char*>(workspace);
        a.ws_o = reinterpret_cast<float*>(ws);
        ws += align_up(static_cast<size_t>(parts) * p.rows * d.head_dim * sizeof(float), 256);
        a.ws_ml = reinterpret_cast<float2*>(ws);
        ws += align_up(static_cast<size_t>(parts) * p.rows * sizeof(float2), 256);
        a.seg = reinterpret_cast<int2*>(ws);
    } else {
        a.ws_o = nullptr;
        a.ws_ml = nullptr;
        a.seg = nullptr;
    }
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
    if (combine) {
        const long rows = slabs * p.rows;
        const dim3 cgrid(static_cast<unsigned>((rows + 3) / 4));
        const int bf16_out = d.dtype == SPEC_BF16;
        if (!wide) {  // four rows per wavefront, the grid resident at once
            const dim3 cgrid4(static_cast<unsigned>((rows + 15) / 16));
            if (a.bf16p) {
                if (d.head_dim == 128)
                    hipLaunchKernelGGL((attn_combine4<128, 8, true>), cgrid4, dim3(256), 0, stream, a, bf16_out);
                else
                    hipLaunchKernelGGL((attn_combine4<64, 8, true>), cgrid4, dim3(256), 0, stream, a, bf16_out);
            } else if (d.head_dim == 128) {
                hipLaunchKernelGGL((attn_combine4<128, 8, false>), cgrid4, dim3(256), 0, stream, a, bf16_out);
            } else {
                hipLaunchKernelGGL((attn_combine4<64, 8, false>), cgrid4, dim3(256), 0, stream, a, bf16_out);
            }
        } else if (a.bf16p) {
            if (d.head_dim == 128)
                hipLaunchKernelGGL((attn_combine<128, 32, true>), cgrid, dim3(256), 0, stream, a, bf16_out);
            else
                hipLaunchKernelGGL((attn_combine<64, 32, true>), cgrid, dim3(256), 0, stream, a, bf16_out);
        } else if (d.head_dim == 128) {
            hipLaunchKernelGGL((attn_combine<128, 32, false>), cgrid, dim3(256), 0, stream, a, bf16_out);
        } else {
            hipLaunchKernelGGL((attn_combine<64, 32, false>), cgrid, dim3(256), 0, stream, a, bf16_out);
        }
        if (hipGetLastError() != hipSuccess) return SPEC_EHIP;
    }
    return SPEC_OK;
}

}  // namespace specv
