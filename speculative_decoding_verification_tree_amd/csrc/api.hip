// extern "C" entry points: argument validation, then kernel launches.
// Nothing here allocates, frees or synchronises.
#include <math.h>

#include <mutex>

#include "spec_common.h"
#include "spec_internal.h"

using namespace specv;

static bool desc_ok(const spec_attn_desc* d, int* err) {
    if (!d) {
        *err = SPEC_EINVAL;
        return false;
    }
    if (d->batch < 0 || d->num_nodes < 1 || d->num_nodes > kMaxNodes || d->num_q_heads < 1 ||
        d->num_kv_heads < 1 || d->num_q_heads % d->num_kv_heads != 0 || d->kv_capacity < 1 || d->kv_split_keys < 0 ||
        !(d->softmax_scale == d->softmax_scale) || isinf(d->softmax_scale) || !(d->rope_base >= 0.f) ||
        isinf(d->rope_base)) {
        *err = SPEC_EINVAL;
        return false;
    }
    if (d->head_dim != 64 && d->head_dim != 128) {
        *err = d->head_dim > 0 ? SPEC_EUNSUPPORTED : SPEC_EINVAL;
        return false;
    }
    if (d->dtype != SPEC_F32 && d->dtype != SPEC_BF16) {
        *err = SPEC_EUNSUPPORTED;
        return false;
    }
    return true;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Scratch of spec_accept_reject_noalloc: one array per GPU, in the library's
// code object, held until the process ends.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels and copies get the device
// address that hipGetSymbolAddress returns for the current device, looked
// up once per device and cached.
constexpr int kMaxScratchDevices = 64;
static __device__ __align__(256) unsigned char scratch[SPEC_ACCEPT_NOALLOC_MAX_WORKSPACE];
static std::mutex g_scratch_mutex;
static void* g_scratch_ptr[kMaxScratchDevices] = {};

static int device_scratch(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return SPEC_EHIP;
    if (dev < 0 || dev >= kMaxScratchDevices) return SPEC_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPEC_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return SPEC_OK;
}

extern "C" {

size_t spec_verify_attn_workspace_bytes(const spec_attn_desc* desc, int32_t max_prefix_len) {
    int err;
    if (!desc_ok(desc, &err) || max_prefix_len < 0) return 0;
    if (desc->batch == 0) return 0;
    return plan_attn(*desc, max_prefix_len).ws_bytes;
}

int spec_verify_attn(const spec_attn_desc* desc, int32_t max_prefix_len, const void* q, const void* k_cache,
                     const void* v_cache, const int32_t* prefix_len, const int32_t* parent, void* out,
                     void* workspace, size_t workspace_bytes, void* stream) {
    int err;
    if (!desc_ok(desc, &err)) return err;
    if (desc->batch == 0) return SPEC_OK;
    if (max_prefix_len < 0 || static_cast<long>(max_prefix_len) + desc->num_nodes > desc->kv_capacity)
        return SPEC_EINVAL;
    if (!q || !k_cache || !v_cache || !prefix_len || !out) return SPEC_EINVAL;
    // the kernels move q, the caches, out and the partials in 16-byte vectors
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return SPEC_EINVAL;
    const AttnPlan plan = plan_attn(*desc, max_prefix_len);
    if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < plan.ws_bytes)) return SPEC_EWORKSPACE;
    if (plan.ws_bytes > 0 && !aligned16(workspace)) return SPEC_EINVAL;
    return launch_verify_attn(*desc, plan, q, k_cache, v_cache, prefix_len, parent, out, workspace,
                              static_cast<hipStream_t>(stream));
}

size_t spec_accept_workspace_bytes(int32_t batch, int32_t num_nodes, int32_t vocab) {
    if (batch < 1 || batch > 65535 || num_nodes < 1 || num_nodes > kMaxNodes || vocab < 1 ||
        vocab > max_accept_vocab())
        return 0;
    return plan_accept(batch, num_nodes, vocab).ws_bytes;
}

size_t spec_accept_filtered_workspace_bytes(int32_t batch, int32_t num_nodes, int32_t vocab) {
    if (batch < 1 || batch > 65535 || num_nodes < 1 || num_nodes > kMaxNodes || vocab < 1 ||
        vocab > max_accept_vocab())
        return 0;
    return plan_accept(batch, num_nodes, vocab).ws_filt_bytes;
}

size_t spec_accept_multidraft_workspace_bytes(int32_t batch, int32_t vocab) {
    if (batch < 1 || batch > 65535 || vocab < 1 || vocab > max_accept_vocab()) return 0;
    return multidraft_workspace_bytes(batch, vocab);
}

static int accept_common_checks(int32_t B, int32_t N, int32_t V, const float* logits, const int32_t* tokens,
                                int32_t* accept_len, int32_t* path, int32_t* out_tokens, float T) {
    if (B > 65535 || N < 1 || N > kMaxNodes || V < 1 || V > max_accept_vocab()) return SPEC_EINVAL;
    if (!(T >= 0.f) || isinf(T)) return SPEC_EINVAL;
    if (!logits || !tokens || !accept_len || !path || !out_tokens) return SPEC_EINVAL;
    return SPEC_OK;
}

int spec_accept_reject(int32_t batch, int32_t num_nodes, int32_t vocab, const float* target_logits,
                       const float* draft_probs, const int32_t* tokens, const int32_t* parent,
                       const float* u_accept, const float* u_sample, float temperature, int32_t* accept_len,
                       int32_t* path, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                       void* stream) {
    if (batch < 0) return SPEC_EINVAL;
    if (batch == 0) return SPEC_OK;
    int rc = accept_common_checks(batch, num_nodes, vocab, target_logits, tokens, accept_len, path, out_tokens,
                                  temperature);
    if (rc != SPEC_OK) return rc;
    if ((num_nodes > 1 && (!draft_probs || !u_accept)) || !u_sample) return SPEC_EINVAL;
    const AcceptPlan plan = plan_accept(batch, num_nodes, vocab);
    if (!workspace || workspace_bytes < plan.ws_bytes) return SPEC_EWORKSPACE;
    return launch_accept(0, batch, num_nodes, vocab, target_logits, draft_probs, tokens, parent, u_accept,
                         u_sample, temperature, 0.f, 0.f, accept_len, path, out_tokens, workspace, plan,
                         static_cast<hipStream_t>(stream));
}

int spec_accept_reject_noalloc(int32_t batch, int32_t num_nodes, int32_t vocab, const float* target_logits,
                               const float* draft_probs, const int32_t* tokens, const int32_t* parent,
                               const float* u_accept, const float* u_sample, float temperature, int32_t* accept_len,
                               int32_t* path, int32_t* out_tokens, void* stream) {
    if (batch < 0) return SPEC_EINVAL;
    if (batch == 0) return SPEC_OK;
    int rc = accept_common_checks(batch, num_nodes, vocab, target_logits, tokens, accept_len, path, out_tokens,
                                  temperature);
    if (rc != SPEC_OK) return rc;
    if ((num_nodes > 1 && (!draft_probs || !u_accept)) || !u_sample) return SPEC_EINVAL;
    const AcceptPlan plan = plan_accept(batch, num_nodes, vocab);
    if (plan.ws_bytes > SPEC_ACCEPT_NOALLOC_MAX_WORKSPACE) return SPEC_EWORKSPACE;
    void* ws = nullptr;
    rc = device_scratch(&ws);
    if (rc != SPEC_OK) return rc;
    return launch_accept(0, batch, num_nodes, vocab, target_logits, draft_probs, tokens, parent, u_accept,
                         u_sample, temperature, 0.f, 0.f, accept_len, path, out_tokens, ws, plan,
                         static_cast<hipStream_t>(stream));
}

int spec_accept_reject_filtered(int32_t batch, int32_t num_nodes, int32_t vocab, const float* target_logits,
                                const float* draft_probs, const int32_t* tokens, const int32_t* parent,
                                const float* u_accept, const float* u_sample, float temperature, int32_t top_k,
                                float top_p, int32_t* accept_len, int32_t* path, int32_t* out_tokens,
                                void* workspace, size_t workspace_bytes, void* stream) {
    if (batch < 0 || top_k < 0 || !(top_p > 0.f && top_p <= 1.f)) return SPEC_EINVAL;
    if (batch == 0) return SPEC_OK;
    int rc = accept_common_checks(batch, num_nodes, vocab, target_logits, tokens, accept_len, path, out_tokens,
                                  temperature);
    if (rc != SPEC_OK) return rc;
    if ((num_nodes > 1 && (!draft_probs || !u_accept)) || !u_sample) return SPEC_EINVAL;
    if (static_cast<long long>(batch) * num_nodes > 0x7fffffffLL) return SPEC_EUNSUPPORTED;
    const AcceptPlan plan = plan_accept(batch, num_nodes, vocab);
    if (!workspace || workspace_bytes < plan.ws_bytes) return SPEC_EWORKSPACE;
    // (the chunk kernels put the rows on the grid's second axis)
    const bool split = workspace_bytes >= plan.ws_filt_bytes && aligned16(workspace) &&
                       static_cast<long long>(batch) * num_nodes <= 65535;
    return launch_accept(0, batch, num_nodes, vocab, target_logits, draft_probs, tokens, parent, u_accept,
                         u_sample, temperature, 0.f, 0.f, accept_len, path, out_tokens, workspace, plan,
                         static_cast<hipStream_t>(stream), top_k, top_p, split);
}

int spec_accept_multidraft(int32_t batch, int32_t num_nodes, int32_t vocab, const float* target_logits,
                           const float* draft_probs, const int32_t* tokens, const int32_t* parent,
                           const float* u_accept, const float* u_sample, float temperature, int32_t* accept_len,
                           int32_t* path, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                           void* stream) {
    if (batch < 0) return SPEC_EINVAL;
    if (batch == 0) return SPEC_OK;
    int rc = accept_common_checks(batch, num_nodes, vocab, target_logits, tokens, accept_len, path, out_tokens,
                                  temperature);
    if (rc != SPEC_OK) return rc;
    if ((num_nodes > 1 && (!draft_probs || !u_accept)) || !u_sample) return SPEC_EINVAL;
    if (!workspace || workspace_bytes < multidraft_workspace_bytes(batch, vocab)) return SPEC_EWORKSPACE;
    return launch_accept_multidraft(batch, num_nodes, vocab, target_logits, draft_probs, tokens, parent, u_accept,
                                    u_sample, temperature, accept_len, path, out_tokens, workspace,
                                    static_cast<hipStream_t>(stream));
}

int spec_accept_typical(int32_t batch, int32_t num_nodes, int32_t vocab, const float* target_logits,
                        const int32_t* tokens, const int32_t* parent, float temperature, float epsilon,
                        float delta, int32_t* accept_len, int32_t* path, int32_t* out_tokens, void* workspace,
                        size_t workspace_bytes, void* stream) {
    if (batch < 0) return SPEC_EINVAL;
    if (batch == 0) return SPEC_OK;
    int rc = accept_common_checks(batch, num_nodes, vocab, target_logits, tokens, accept_len, path, out_tokens,
                                  temperature);
    if (rc != SPEC_OK) return rc;
    if (!(epsilon >= 0.f) || !(delta >= 0.f) || isinf(epsilon) || isinf(delta)) return SPEC_EINVAL;
    const AcceptPlan plan = plan_accept(batch, num_nodes, vocab);
    if (!workspace || workspace_bytes < plan.ws_bytes) return SPEC_EWORKSPACE;
    return launch_accept(1, batch, num_nodes, vocab, target_logits, nullptr, tokens, parent, nullptr, nullptr,
                         temperature, epsilon, delta, accept_len, path, out_tokens, workspace, plan,
                         static_cast<hipStream_t>(stream));
}

int spec_commit_kv(const spec_attn_desc* desc, void* k_cache, void* v_cache, int32_t* prefix_len,
                   const int32_t* path, const int32_t* accept_len, void* stream) {
    int err;
    if (!desc_ok(desc, &err)) return err;
    if (desc->batch == 0) return SPEC_OK;
    if (!k_cache || !v_cache || !prefix_len || !path || !accept_len) return SPEC_EINVAL;
    return launch_commit(*desc, k_cache, v_cache, prefix_len, path, accept_len, static_cast<hipStream_t>(stream));
}

int spec_tree_positions(int32_t batch, int32_t num_nodes, const int32_t* prefix_len, const int32_t* parent,
                        int32_t* positions, void* stream) {
    if (batch < 0 || num_nodes < 1 || num_nodes > kMaxNodes) return SPEC_EINVAL;
    if (batch == 0) return SPEC_OK;
    if (!prefix_len || !positions) return SPEC_EINVAL;
    return launch_positions(batch, num_nodes, prefix_len, parent, positions, static_cast<hipStream_t>(stream));
}

int spec_validate_tree(int32_t batch, int32_t num_nodes, const int32_t* parent, int32_t* status, void* stream) {
    if (batch < 0 || num_nodes < 1 || num_nodes > kMaxNodes) return SPEC_EINVAL;
    if (batch == 0) return SPEC_OK;
    if (!parent || !status) return SPEC_EINVAL;
    return launch_validate(batch, num_nodes, parent, status, static_cast<hipStream_t>(stream));
}

int32_t spec_medusa_tree_nodes(int32_t num_heads, const int32_t* widths, int32_t max_width) {
    if (num_heads < 1 || num_heads > kMaxNodes - 1 || !widths || max_width < 1) return 0;
    long n = 1, level = 1;
    for (int k = 0; k < num_heads; ++k) {
        if (widths[k] < 1 || widths[k] > max_width) return 0;
        level *= widths[k];
        n += level;
        if (n > kMaxNodes) return 0;
    }
    return static_cast<int32_t>(n);
}

int spec_medusa_tree(int32_t batch, int32_t num_heads, const int32_t* widths, int32_t max_width,
                     const int32_t* root_tokens, const int32_t* head_tokens, int32_t* parent, int32_t* tokens,
                     void* stream) {
    const int32_t N = spec_medusa_tree_nodes(num_heads, widths, max_width);
    if (batch < 0 || N == 0) return SPEC_EINVAL;
    if (batch == 0) return SPEC_OK;
    if (!root_tokens || !head_tokens || !parent || !tokens) return SPEC_EINVAL;
    MedusaTreeArgs a{};
    a.K = num_heads;
    a.W = max_width;
    a.N = N;
    a.off[0] = 0;
    a.off[1] = 1;
    long level = 1;
    for (int k = 0; k < num_heads; ++k) {
        a.widths[k] = widths[k];
        level *= widths[k];
        a.off[k + 2] = static_cast<int>(a.off[k + 1] + level);
    }
    a.root = root_tokens;
    a.head = head_tokens;
    a.parent = parent;
    a.tokens = tokens;
    return launch_medusa_tree(a, batch, static_cast<hipStream_t>(stream));
}

int spec_tree_rope(const spec_attn_desc* desc, void* q, void* k_cache, const int32_t* prefix_len,
                   const int32_t* parent, float rope_base, void* stream) {
    int err;
    if (!desc_ok(desc, &err)) return err;
    if (!(rope_base > 0.f) || isinf(rope_base)) return SPEC_EINVAL;
    if (desc->batch == 0) return SPEC_OK;
    if (!q || !k_cache || !prefix_len) return SPEC_EINVAL;
    TreeRopeArgs a;
    a.q = q;
    a.k = k_cache;
    a.prefix_len = prefix_len;
    a.parent = parent;
    a.N = desc->num_nodes;
    a.Hq = desc->num_q_heads;
    a.Hkv = desc->num_kv_heads;
    a.D = desc->head_dim;
    a.cap = desc->kv_capacity;
    a.log2_base = log2(static_cast<double>(rope_base));
    return launch_tree_rope(a, desc->batch, desc->dtype == SPEC_BF16, static_cast<hipStream_t>(stream));
}

const char* spec_status_string(int status) {
    switch (status) {
        case SPEC_OK: return "SPEC_OK";
        case SPEC_EINVAL: return "SPEC_EINVAL: invalid argument";
        case SPEC_EUNSUPPORTED: return "SPEC_EUNSUPPORTED: unsupported dtype or head_dim";
        case SPEC_EWORKSPACE: return "SPEC_EWORKSPACE: workspace too small";
        case SPEC_EHIP: return "SPEC_EHIP: kernel launch failed";
        default: return "unknown spec_status";
    }
}

static int la_desc_ok(const spec_la_desc* d) {
    if (!d) return SPEC_EINVAL;
    if (d->batch < 0 || d->batch > 65535 || d->num_heads < 1 || d->num_heads > 65535) return SPEC_EINVAL;
    if (d->dtype != SPEC_F32 && d->dtype != SPEC_BF16) return SPEC_EUNSUPPORTED;
    if ((d->key_dim != 64 && d->key_dim != 128) || (d->value_dim != 64 && d->value_dim != 128))
        return d->key_dim < 1 || d->value_dim < 1 ? SPEC_EINVAL : SPEC_EUNSUPPORTED;
    return SPEC_OK;
}

static bool la_factors_ok(const spec_la_factors* f) {
    return f && f->num_nodes >= 1 && f->num_nodes <= kMaxNodes && f->k && f->v && f->path && f->accept_len;
}

static LaArgs la_args(const spec_la_desc* d, float* state) {
    LaArgs a{};
    a.state = state;
    a.B = d->batch;
    a.H = d->num_heads;
    a.Dk = d->key_dim;
    a.Dv = d->value_dim;
    a.bf16 = d->dtype == SPEC_BF16;
    return a;
}

static void la_set_factors(LaArgs& a, const spec_la_factors* f) {
    a.pN = f->num_nodes;
    a.pk = f->k;
    a.pv = f->v;
    a.palpha = f->alpha;
    a.pparent = f->parent;
    a.ppath = f->path;
    a.pacc = f->accept_len;
    a.do_commit = 1;
}

int spec_la_verify(const spec_la_desc* desc, float* state, const void* q, const void* k, const void* v,
                   const float* alpha, const int32_t* parent, void* out, const spec_la_factors* pending,
                   void* stream) {
    int rc = la_desc_ok(desc);
    if (rc != SPEC_OK) return rc;
    if (desc->num_nodes < 1 || desc->num_nodes > kMaxNodes) return SPEC_EINVAL;
    if (desc->batch == 0) return SPEC_OK;
    if (!state || !q || !k || !v || !out) return SPEC_EINVAL;
    if (!aligned16(state)) return SPEC_EINVAL;  // the state moves in 16-byte vectors
    if (pending && !la_factors_ok(pending)) return SPEC_EINVAL;
    LaArgs a = la_args(desc, state);
    a.N = desc->num_nodes;
    a.q = q;
    a.k = k;
    a.v = v;
    a.alpha = alpha;
    a.parent = parent;
    a.out = out;
    a.do_verify = 1;
    if (pending) la_set_factors(a, pending);
    return launch_la(a, static_cast<hipStream_t>(stream));
}

int spec_la_commit(const spec_la_desc* desc, float* state, const spec_la_factors* accepted, void* stream) {
    int rc = la_desc_ok(desc);
    if (rc != SPEC_OK) return rc;
    if (desc->batch == 0) return SPEC_OK;
    if (!state || !la_factors_ok(accepted)) return SPEC_EINVAL;
    if (!aligned16(state)) return SPEC_EINVAL;
    LaArgs a = la_args(desc, state);
    la_set_factors(a, accepted);
    return launch_la(a, static_cast<hipStream_t>(stream));
}

}  // extern "C"
