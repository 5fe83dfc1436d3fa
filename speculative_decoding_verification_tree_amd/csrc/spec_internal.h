// Host-side plumbing shared by the entry points and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/spec_verify.h"
#include "spec_common.h"

namespace specv {

constexpr int kTreeMaxNodes = 64;

// Execution plan of spec_verify_attn for one descriptor and prefix bound.
struct AttnPlan {
    bool mfma;        // bf16 MFMA path (else the VALU path)
    bool balanced;    // balanced block ranges (else fixed splits per slab)
    int rows;         // R = N * (Hq / Hkv): query rows per (request, kv head)
    int row_tiles;    // MFMA: 16-row tiles per wave
    int waves;        // wavefronts per workgroup (row tiles shared between them)
    int kwaves;       // one-wave MFMA path: waves splitting each range's blocks (merged in LDS)
    int row_groups;   // workgroups sharing one KV range (different query rows)
    int split_blocks; // fixed: 32-key blocks per split; balanced: least blocks per range
    int nsplit_max;   // fixed: splits of the longest request
    int parts_max;    // balanced: most ranges P a launch may use
    int max_keys;     // max_prefix_len + N
    size_t ws_bytes;  // partials + per-slab table (0 when no slab is ever split)
};

AttnPlan plan_attn(const spec_attn_desc& d, int max_prefix_len);

int launch_verify_attn(const spec_attn_desc& d, const AttnPlan& plan, const void* q, const void* k,
                       const void* v, const int32_t* prefix_len, const int32_t* parent, void* out,
                       void* workspace, hipStream_t stream);

struct AcceptPlan {
    int chunk;   // vocabulary entries per chunk
    int nchunk;
    size_t off_rowstat, off_dec, off_cstat, off_cslice, ws_bytes;
    // the truncation split over chunks, past ws_bytes
    size_t off_frec, off_fbins, off_fkeys, ws_filt_bytes;
};

AcceptPlan plan_accept(int B, int N, int V);
int max_accept_vocab();

int launch_accept(int rule, int B, int N, int V, const float* logits, const float* draft,
                  const int32_t* tokens, const int32_t* parent, const float* u_accept,
                  const float* u_sample, float temperature, float epsilon, float delta,
                  int32_t* accept_len, int32_t* path, int32_t* out_tokens, void* workspace,
                  const AcceptPlan& plan, hipStream_t stream, int top_k = 0, float top_p = 1.f,
                  bool split_filter = false);

size_t multidraft_workspace_bytes(int B, int V);
int launch_accept_multidraft(int B, int N, int V, const float* logits, const float* draft, const int32_t* tokens,
                             const int32_t* parent, const float* u_accept, const float* u_sample, float temperature,
                             int32_t* accept_len, int32_t* path, int32_t* out_tokens, void* workspace,
                             hipStream_t stream);

int launch_commit(const spec_attn_desc& d, void* k, void* v, int32_t* prefix_len, const int32_t* path,
                  const int32_t* accept_len, hipStream_t stream);

int launch_positions(int B, int N, const int32_t* prefix_len, const int32_t* parent, int32_t* pos,
                     hipStream_t stream);

int launch_validate(int B, int N, const int32_t* parent, int32_t* status, hipStream_t stream);

struct MedusaTreeArgs {
    int K, W, N;
    int widths[kTreeMaxNodes];
    int off[kTreeMaxNodes + 1];  // first node of each level (off[1] = 1)
    const int32_t* root;
    const int32_t* head;
    int32_t* parent;
    int32_t* tokens;
};

int launch_medusa_tree(const MedusaTreeArgs& a, int B, hipStream_t stream);

struct TreeRopeArgs {
    void* q;
    void* k;
    const int32_t* prefix_len;
    const int32_t* parent;
    int N, Hq, Hkv, D, cap;
    double log2_base;
};

int launch_tree_rope(const TreeRopeArgs& a, int B, bool bf16, hipStream_t stream);

inline size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// rev[j] = base^(-2j/D) / (2 pi), j < D/2: turns per position of rotary pair j.
inline void fill_rope_table(RopeTable& t, int D, float base) {
    const double two_pi = 6.283185307179586476925286766559;
    for (int j = 0; j < kRopeMaxPairs; ++j)
        t.rev[j] = j < D / 2 ? pow(static_cast<double>(base), -2.0 * j / D) / two_pi : 0.0;
}

// Linear-attention verification / commit (one launch, either or both phases).
struct LaArgs {
    float* state;  // [B][H][Dv][Dk] fp32
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const int32_t* parent;
    void* out;
    int B, N, H, Dk, Dv, bf16;
    // the accepted path committed before verification (or alone)
    int pN;
    const void* pk;
    const void* pv;
    const float* palpha;
    const int32_t* pparent;
    const int32_t* ppath;
    const int32_t* pacc;
    int do_commit, do_verify;
    int vec;  // every q, k, v row source 16-byte aligned (set by launch_la)
};
int launch_la(const LaArgs& a, hipStream_t stream);

}  // namespace specv
