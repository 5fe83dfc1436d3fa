/*
 * spec_verify.h -- C ABI of the MI355X (gfx950) speculative-decoding
 * verification step: tree-verify attention, rejection / typical acceptance
 * over the vocabulary, and the in-place KV commit of the accepted path.
 *
 * Conventions shared by every entry point
 *  - All tensor pointers are DEVICE memory owned by the caller.  The library
 *    never allocates, frees or synchronises; every call only enqueues kernels
 *    on `stream` (a hipStream_t; NULL = the null stream) and returns.
 *  - Calls are stateless and re-entrant.  Two calls that share a workspace or
 *    an output must not overlap in time (same rule as any stream work).
 *  - Row-major layouts; int32 indices; `B` = batch, `N` = tree nodes per
 *    request INCLUDING the root (a chain of K drafts has N = K + 1), `V` =
 *    vocabulary size.
 *  - Host-detectable argument errors return SPEC_EINVAL / SPEC_EUNSUPPORTED /
 *    SPEC_EWORKSPACE before anything is launched; a failed launch returns
 *    SPEC_EHIP.  Device-side contract violations (a malformed parent array, a
 *    token >= V, a uniform outside [0,1)) give undefined results but never an
 *    out-of-bounds access: the kernels clamp every index they read.
 *  - B == 0 is a no-op returning SPEC_OK.
 *
 * Tree model (MEDUSA section of the blog page "Fast Inference from
 * Transformers via Speculative Decoding", tree-attention paragraph): node 0 is
 * the root, the pending token whose logits give the depth-1 candidates; every
 * other node i has parent[i] < i.  A node attends to the verified prefix, its
 * ancestors and itself; its position is L_b + depth(i).  parent == NULL means
 * a chain (parent[i] = i - 1).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum spec_status {
    SPEC_OK = 0,
    SPEC_EINVAL = -1,       /* bad pointer, size or parameter value */
    SPEC_EUNSUPPORTED = -2, /* valid in principle but not built (dtype, head_dim) */
    SPEC_EWORKSPACE = -3,   /* workspace smaller than the matching *_workspace_bytes */
    SPEC_EHIP = -4          /* a kernel launch failed */
} spec_status;

typedef enum spec_dtype { SPEC_F32 = 0, SPEC_BF16 = 1 } spec_dtype;

/* Shape of the attention problem.  q/out are [B][N][Hq][D]; the caches are
 * [B][Hkv][kv_capacity][D].  Hq % Hkv == 0; query head h reads kv head
 * h / (Hq / Hkv).  head_dim is 64 or 128.  1 <= num_nodes <= 64.
 * softmax_scale <= 0 selects 1/sqrt(head_dim).
 * kv_split_keys: 0 lets the library choose how finely the KV axis is split
 * across workgroups; a positive value sets the least number of keys per KV
 * range (rounded up to whole 32-key blocks), for tuning and for tests that
 * need many short ranges.  It changes the work split and the workspace size,
 * not the result beyond rounding order.  Negative: SPEC_EINVAL.
 * rope_base: 0 means q and the tree's K rows arrive already rotated.  A
 * positive value fuses the depth-position rotary embedding (MEDUSA section,
 * tree-attention paragraph: position indices follow tree depth) into
 * spec_verify_attn and spec_commit_kv: q and the tree's K rows
 * [L_b, L_b + N) are given unrotated, the prefix rows [0, L_b) rotated at
 * their positions; the attention turns q of node i and the K row of node i
 * by position L_b + depth(i) as it reads them (the cache is not written),
 * and the commit writes the accepted K rows rotated at their new positions
 * L_b + d, so that the grown prefix is rotated.  The rotation is the one
 * spec_tree_rope applies (Llama rotate-half pairs (x_j, x_{j + D/2}) turned
 * by pos * rope_base^(-2j/D)); angles in fp64 turns, sine and cosine and the
 * products in fp32, rounded to the dtype.  V is never rotated.  Negative or
 * not finite: SPEC_EINVAL. */
typedef struct spec_attn_desc {
    int32_t batch;
    int32_t num_nodes;
    int32_t num_q_heads;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t kv_capacity; /* rows per (b, kv head); must be >= max_prefix_len + num_nodes */
    int32_t dtype;       /* spec_dtype of q, the caches and out */
    float softmax_scale;
    int32_t kv_split_keys; /* 0: automatic */
    float rope_base;       /* 0: inputs already rotated; > 0: fused depth-position RoPE */
} spec_attn_desc;

/* Workspace bytes spec_verify_attn needs for this shape and prefix bound
 * (split-KV partial results).  Returns 0 for an invalid descriptor or when no
 * workspace is needed (one KV split covers every request).  Contents need no
 * initialisation. */
size_t spec_verify_attn_workspace_bytes(const spec_attn_desc* desc, int32_t max_prefix_len);

/* Tree-verify attention (the parallel scoring pass of the verification step:
 * "Speculative Sampling" section -- all draft positions are scored in one
 * target pass -- with the MEDUSA tree mask).  For every (b, node i, q-head h):
 *   keys  = cache rows [0, L_b) and L_b + n for n on the root path of i;
 *   out   = softmax(scale * q k^T) v over those keys, fp32 accumulation.
 * Arguments
 *   max_prefix_len  host int >= every prefix_len[b] (sizes the KV split)
 *   q               [B][N][Hq][D] (dtype)
 *   k_cache,v_cache [B][Hkv][cap][D] (dtype); rows [0, L_b) are the verified
 *                   prefix, rows [L_b, L_b + N) the tree nodes' K/V (written
 *                   by the caller, node order); rows beyond are never read
 *   prefix_len      [B] int32, device
 *   parent          [B][N] int32 or NULL (chain)
 *   out             [B][N][Hq][D] (dtype), written
 *   workspace       >= spec_verify_attn_workspace_bytes(desc, max_prefix_len)
 * q, k_cache, v_cache, out and a non-empty workspace must be 16-byte aligned
 * (the kernels move them in 16-byte vectors), else SPEC_EINVAL. */
int spec_verify_attn(const spec_attn_desc* desc, int32_t max_prefix_len, const void* q,
                     const void* k_cache, const void* v_cache, const int32_t* prefix_len,
                     const int32_t* parent, void* out, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Workspace bytes for either acceptance entry point (per-chunk statistics;
 * contents need no initialisation).  0 for invalid sizes.  vocab <= 8388608,
 * batch <= 65535. */
size_t spec_accept_workspace_bytes(int32_t batch, int32_t num_nodes, int32_t vocab);

/* Rejection-rule acceptance ("Speculative Decoding" and "Speculative
 * Sampling" sections of the blog page "Fast Inference from Transformers via
 * Speculative Decoding").  p_u = softmax(target_logits[b][u] / T) (T == 0: the
 * one-hot lowest-index argmax).  Node i >= 1 with parent u and token x =
 * tokens[b][i] passes when u_accept[b][i] * draft_probs[b][i][x] < p_u(x); a
 * node is accepted when it and all its ancestors pass.  The stop node v is the
 * deepest accepted node (smallest index on ties), a = depth(v).  The last
 * token is drawn by inverse CDF (ascending token ids, uniform u_sample[b][v])
 * from norm(max(0, p_v - q_c)) when v has children (c = its smallest-index
 * child; p_v itself if that residual is all zero), else from p_v (the bonus
 * token).
 *   target_logits [B][N][V] fp32, row i = target logits at node i
 *   draft_probs   [B][N][V] fp32, row i = the distribution node i's token was
 *                 drawn from (already temperature-transformed); row 0 unused
 *   tokens        [B][N] int32 (entry 0 unused); parent [B][N] or NULL
 *   u_accept, u_sample [B][N] fp32 in [0, 1)
 *   temperature   >= 0, finite; batch <= 65535
 * Outputs: accept_len [B] = a; path [B][N] = root .. v then -1;
 *   out_tokens [B][N] = tokens of path[1..a], the drawn token, then -1. */
int spec_accept_reject(int32_t batch, int32_t num_nodes, int32_t vocab, const float* target_logits,
                       const float* draft_probs, const int32_t* tokens, const int32_t* parent,
                       const float* u_accept, const float* u_sample, float temperature,
                       int32_t* accept_len, int32_t* path, int32_t* out_tokens, void* workspace,
                       size_t workspace_bytes, void* stream);

/* spec_accept_reject without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same rule, arguments, outputs and
 * kernels as spec_accept_reject; the scratch it needs lives in one array per
 * GPU inside the library (SPEC_ACCEPT_NOALLOC_MAX_WORKSPACE bytes, held
 * until the process ends).  Shapes whose spec_accept_workspace_bytes exceeds
 * that return SPEC_EWORKSPACE before any launch.  Nothing is allocated or
 * freed.  Every call on one GPU uses that GPU's array: two calls that overlap
 * in time on one GPU (different streams, or other host threads) race and
 * give undefined results; calls ordered on one stream are safe.  Device: the
 * current HIP device (SPEC_EUNSUPPORTED for an ordinal >= 64). */
#define SPEC_ACCEPT_NOALLOC_MAX_WORKSPACE (8u << 20)
int spec_accept_reject_noalloc(int32_t batch, int32_t num_nodes, int32_t vocab, const float* target_logits,
                               const float* draft_probs, const int32_t* tokens, const int32_t* parent,
                               const float* u_accept, const float* u_sample, float temperature,
                               int32_t* accept_len, int32_t* path, int32_t* out_tokens, void* stream);

/* Rejection-rule acceptance on a truncated target (the "Speculative
 * Sampling" section of the same page lets top-k and nucleus sampling
 * transform the probabilities before the rule).  Every p_u of
 * spec_accept_reject is first truncated and renormalised: top-k keeps the
 * tokens whose logit is at least the k-th largest logit of the row (ties
 * kept); the nucleus then keeps, on the renormalised top-k distribution, the
 * tokens for which the mass of the tokens with a strictly larger logit is
 * below top_p.  The node tests, the residual and the bonus token use the
 * truncated p_u; draft_probs is taken as given (the caller's draft sampler
 * applies its own transform).  top_k == 0 or >= vocab: no top-k; top_p == 1:
 * no nucleus; at T == 0 both are no-ops (the argmax is always kept).  The
 * nucleus masses are summed in 2^-44 fixed point over fp32 terms, so a
 * boundary within about 1e-6 of top_p may fall either way.  Arguments and
 * outputs otherwise as spec_accept_reject.  workspace: at least
 * spec_accept_workspace_bytes; with top_k > 0, batch * num_nodes <= 65535
 * and at least spec_accept_filtered_workspace_bytes, each row's selection is
 * spread over the workgroups of its vocabulary chunks (each chunk leaves its
 * top digits' counts and keys in the workspace for the row's finishing
 * workgroup; nothing needs clearing), else, and for shapes of more than
 * 65,536 (row, chunk) pairs, one workgroup selects per row; the results are
 * identical.
 *   top_k >= 0; 0 < top_p <= 1, else SPEC_EINVAL */
/* Workspace bytes with which spec_accept_reject_filtered splits each row's
 * top-k selection over its vocabulary chunks: the plain acceptance
 * workspace, then per (row, chunk) a 16-byte record, 64 digit counts and 256
 * keys (1,296 bytes).  0 for shapes spec_accept_workspace_bytes rejects. */
size_t spec_accept_filtered_workspace_bytes(int32_t batch, int32_t num_nodes, int32_t vocab);

int spec_accept_reject_filtered(int32_t batch, int32_t num_nodes, int32_t vocab, const float* target_logits,
                                const float* draft_probs, const int32_t* tokens, const int32_t* parent,
                                const float* u_accept, const float* u_sample, float temperature, int32_t top_k,
                                float top_p, int32_t* accept_len, int32_t* path, int32_t* out_tokens,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Rejection over a tree with several drafts per node, by recursive
 * residuals (a reading: the "Speculative Sampling" section gives the
 * single-draft rule and the MEDUSA section says tree candidates can reuse
 * it, with no multi-draft scheme).  Starting at the root v, with r = p_v
 * (p as in spec_accept_reject): the children c of v are tested in ascending
 * index, c with token x passing when u_accept[b][c] * q_c(x) < r(x); a
 * rejected child replaces r by norm(max(0, r - q_c)) (r is kept if that is
 * all zero) and the next child is tested against it.  The first passing
 * child becomes v and the walk repeats from it.  When every child of v is
 * rejected the last token is drawn from r, and at a leaf from p_v (inverse
 * CDF, ascending token ids, uniform u_sample[b][v]).  Each emitted token is
 * then distributed as the target when every child's token was drawn from its
 * q (siblings may share one q, drawn i.i.d.), which the single-residual rule
 * of spec_accept_reject does not give for nodes with several children.  On
 * a chain both rules agree.  Arguments and outputs as spec_accept_reject;
 * workspace >= spec_accept_multidraft_workspace_bytes(batch, vocab) (two
 * residual rows and 2 KiB of tagged exchange records per request; contents
 * need no initialisation: the call clears the records' tags itself).
 * Each request's vocabulary is split over up to 64 workgroups that wait on
 * each other between passes, so the call assumes its grid runs at once (it
 * is sized from the device's occupancy; nothing else should fill the device
 * meanwhile); a request whose workgroups were not all running returns
 * accept_len = -1 after a bounded wait instead of hanging.  Calls that
 * overlap on one workspace race. */
size_t spec_accept_multidraft_workspace_bytes(int32_t batch, int32_t vocab);
int spec_accept_multidraft(int32_t batch, int32_t num_nodes, int32_t vocab, const float* target_logits,
                           const float* draft_probs, const int32_t* tokens, const int32_t* parent,
                           const float* u_accept, const float* u_sample, float temperature, int32_t* accept_len,
                           int32_t* path, int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Typical acceptance (MEDUSA section, typical-acceptance paragraph of the
 * same page).  Node i >= 1 with parent u and token x passes when
 * p_u(x) > min(epsilon, delta * exp(-H(p_u))), H in nats with p_u =
 * softmax(target_logits[b][u] / T).  The root is the previous step's greedy
 * token and is accepted unconditionally; acceptance, the stop node and the
 * outputs are as for spec_accept_reject except that the last token is
 * argmax p_v (lowest index on ties).  epsilon, delta >= 0, finite. */
int spec_accept_typical(int32_t batch, int32_t num_nodes, int32_t vocab, const float* target_logits,
                        const int32_t* tokens, const int32_t* parent, float temperature,
                        float epsilon, float delta, int32_t* accept_len, int32_t* path,
                        int32_t* out_tokens, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Commit of the accepted path (the rejected candidates are discarded, as the
 * speculative-decoding loop prescribes): for every request b and kv head the
 * cache rows L_b + path[b][d], d = 0..accept_len[b], move to L_b + d, in
 * place (all sources are read before they can be overwritten), then
 * prefix_len[b] += accept_len[b] + 1.  For a chain nothing moves.  With
 * desc->rope_base > 0 the K rows of the accepted path are also rotated at
 * their new positions L_b + d as they are written (every d, moved or not).
 * Uses the desc fields batch, num_nodes, num_kv_heads, head_dim,
 * kv_capacity, dtype and rope_base. */
int spec_commit_kv(const spec_attn_desc* desc, void* k_cache, void* v_cache, int32_t* prefix_len,
                   const int32_t* path, const int32_t* accept_len, void* stream);

/* Depth-based positions of the tree nodes (MEDUSA tree-attention paragraph):
 * positions[b][i] = prefix_len[b] + depth(i).  For callers that rotate q/k
 * before spec_verify_attn. */
int spec_tree_positions(int32_t batch, int32_t num_nodes, const int32_t* prefix_len,
                        const int32_t* parent, int32_t* positions, void* stream);

/* Debug check of a parent array: status[b] = 0 when parent[b][0] == -1 and
 * 0 <= parent[b][i] < i for all i >= 1, else 1 + the first offending node index. */
int spec_validate_tree(int32_t batch, int32_t num_nodes, const int32_t* parent, int32_t* status,
                       void* stream);

/* Candidate tree of Medusa heads (MEDUSA section, candidate-construction and
 * tree-attention paragraphs: head k proposes its top-s_k tokens, and the
 * candidates are the Cartesian product of the heads' proposals arranged as a
 * tree).  Node 0 is the root with token root_tokens[b].  The tree is built
 * breadth first: the children of a depth-(d-1) node are its extensions by
 * head d's candidates in rank order, parents visited in the order their level
 * was built.  Node (i_1..i_d) thus has parent (i_1..i_{d-1}) and token
 * head_tokens[b][d-1][i_d].
 * spec_medusa_tree_nodes returns N = 1 + sum_d prod_{k<=d} s_k, or 0 when
 * num_heads is outside [1, 63], a width is outside [1, max_width] or N > 64.
 * Arguments
 *   widths       host array of num_heads widths s_1..s_K
 *   max_width    row stride of head_tokens (>= every width)
 *   root_tokens  [B] int32, device
 *   head_tokens  [B][K][max_width] int32, device (entries past a width unread)
 *   parent, tokens [B][N] int32, device, written (parent[b][0] = -1)
 * Errors: SPEC_EINVAL for an invalid shape (as above) or a NULL pointer. */
int32_t spec_medusa_tree_nodes(int32_t num_heads, const int32_t* widths, int32_t max_width);
int spec_medusa_tree(int32_t batch, int32_t num_heads, const int32_t* widths, int32_t max_width,
                     const int32_t* root_tokens, const int32_t* head_tokens, int32_t* parent,
                     int32_t* tokens, void* stream);

/* Depth-position rotary embedding of the tree, in place (MEDUSA section,
 * tree-attention paragraph: position indices follow tree depth).  Node i of
 * request b sits at position pos = L_b + depth(i).  The rotation is the
 * Llama family's rotary embedding in its rotate-half layout: for j < D/2 the
 * pair (x_j, x_{j+D/2}) turns by pos * rope_base^(-2j/D)
 *   x_j' = x_j cos - x_{j+D/2} sin,   x_{j+D/2}' = x_j sin + x_{j+D/2} cos,
 * angles and products in fp64, rounded to fp32 (then to bf16).  Applied
 * to q[b][i][h] for every q head and to the tree's K rows
 * k_cache[b][g][L_b + i] for every kv head; the prefix rows and V are not
 * touched.  desc as for spec_verify_attn (softmax_scale unused); parent NULL
 * means a chain.  A request with L_b < 0 or L_b + N > cap is skipped.
 * Errors: SPEC_EINVAL for a bad descriptor, rope_base <= 0 or not finite, or
 * a NULL q / k_cache / prefix_len. */
int spec_tree_rope(const spec_attn_desc* desc, void* q, void* k_cache, const int32_t* prefix_len,
                   const int32_t* parent, float rope_base, void* stream);

/* Static string naming a spec_status value. */
const char* spec_status_string(int status);

/* Linear-attention verification (SpecLA paragraphs of the summary "SpecLA:
 * Efficient Speculative Decoding for Linear-Attention Models": the drafts of
 * a stateful linear-attention model are verified against its summary state,
 * a tree mask separating branches, and the state is recovered afterwards
 * from the accepted tokens' compact factors, the final update deferred to
 * the next step).  The summary gives no recurrence; the one implemented is a
 * matrix state per (request, head) with a scalar decay per token,
 *     S_t = alpha_t S_{t-1} + v_t k_t^T,   o_t = S_t q_t
 * (alpha = 1: plain linear attention), each tree node following its root
 * path from the committed state.  fp32 state and arithmetic. */
typedef struct {
    int32_t batch;
    int32_t num_nodes;   /* N, the nodes of this step's tree, 1..64 */
    int32_t num_heads;   /* H >= 1 */
    int32_t key_dim;     /* Dk: 64 or 128 */
    int32_t value_dim;   /* Dv: 64 or 128 */
    int32_t dtype;       /* spec_dtype of q, k, v and out: fp32 or bf16 */
} spec_la_desc;

/* The factors of one step's accepted path: that step's tree (its k, v,
 * decays and parents, num_nodes nodes) and its accepted path, as the
 * acceptance calls return it (path[b][0 .. accept_len[b]]). */
typedef struct {
    int32_t num_nodes;
    const void* k;          /* [B][N'][H][Dk] (dtype) */
    const void* v;          /* [B][N'][H][Dv] (dtype) */
    const float* alpha;     /* [B][N'][H] decays in (0, 1], or NULL (all 1) */
    const int32_t* parent;  /* [B][N'] or NULL (chain) */
    const int32_t* path;    /* [B][N'] */
    const int32_t* accept_len; /* [B] */
} spec_la_factors;

/* Outputs of every node of the tree: out[b][i][h] = A(-> i] S q_i +
 * sum over j on i's root path of A(j -> i] (q_i . k_j) v_j, where A(j -> i]
 * is the product of the decays of the path nodes after j up to i (A(-> i]:
 * the whole path root .. i).
 *   state  [B][H][Dv][Dk] fp32, device: the committed state (read); with
 *          pending != NULL it is first advanced in place by that step's
 *          accepted factors (the deferred commit), then read
 *   q, k   [B][N][H][Dk], v and out [B][N][H][Dv] (dtype), device; any
 *          alignment of the element type (16-byte aligned q, k, v and
 *          factor rows are read as 16-byte vectors, others element by
 *          element, with the same results)
 *   alpha  [B][N][H] fp32 decays in (0, 1] or NULL; parent [B][N] or NULL
 * Errors: SPEC_EINVAL (null pointers, sizes, a state pointer not 16-byte
 * aligned), SPEC_EUNSUPPORTED (Dk, Dv). */
int spec_la_verify(const spec_la_desc* desc, float* state, const void* q, const void* k, const void* v,
                   const float* alpha, const int32_t* parent, void* out, const spec_la_factors* pending,
                   void* stream);

/* The commit alone: state <- A(-> v] state + sum over j on the accepted path
 * of A(j -> v] v_j k_j^T (v the stop node), in place, from the factors; the
 * same update spec_la_verify applies for its pending argument.  desc gives
 * B, H, Dk, Dv and dtype (its num_nodes is not used).  state must be 16-byte
 * aligned, else SPEC_EINVAL. */
int spec_la_commit(const spec_la_desc* desc, float* state, const spec_la_factors* accepted, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
