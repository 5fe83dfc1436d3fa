/*
 * oracle.c -- plain, slow fp64 CPU reference of the speculative-decoding
 * verification step.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the benchmark's CPU-baseline leg call it; the product path never does.  It
 * shares no code with the HIP library.
 *
 * Every floating-point step is done in double precision on the exact input
 * values (bf16 and fp32 widen to double without rounding).  The loops follow
 * the definitions directly: no blocking, no fusion, no reordering.
 *
 * Sources (the pages this reference is written from):
 *  - "MEDUSA" section of "Fast Inference from Transformers via Speculative
 *    Decoding" blog post (taking-lying-flat.github.io, spec-decoding-i),
 *    tree attention paragraph: a node attends to itself, its ancestors and the
 *    verified prefix; positions follow tree depth; candidates are the
 *    Cartesian product of per-head top predictions.
 *  - Same page, "Speculative Decoding" / "Speculative Sampling" sections: the
 *    draft token x is kept when a uniform u satisfies u < p(x)/q(x); on the
 *    first rejection one token is drawn from norm(max(0, p - q)) and the rest
 *    are dropped; if every draft is kept one extra token is drawn from the
 *    target's distribution at the last position; sampling transforms such as
 *    temperature are applied to the probabilities first.
 *  - Same page, MEDUSA "typical acceptance" paragraph: a candidate token is
 *    accepted when p(x) > min(eps, delta * exp(-H(p))); the first token is
 *    greedy and always accepted; the output is the longest accepted prefix
 *    over all candidates; temperature 0 reduces to greedy.
 *
 * Readings where the pages are silent (their formulas were lost in
 * extraction):
 *  - node 0 is the root (the pending token from the previous step); its
 *    logits give the distribution of the depth-1 nodes; N rows = K + 1;
 *  - the rejection test is the strict u * q(x) < p(x);
 *  - every node is tested once with its own uniform u_accept[node]; the
 *    longest accepted root path wins, ties to the smallest stop-node index;
 *    the residual uses the smallest-index child of the stop node;
 *  - a draw from weights r with uniform u is the smallest token id x whose
 *    ascending cumulative sum exceeds u * sum(r) (fallback: the largest x with
 *    r_x > 0); a residual of zero total mass falls back to p itself;
 *  - typical rule: the entropy uses the natural log and the temperature-
 *    scaled p; the root is accepted unconditionally and the step's last token
 *    is argmax p at the stop node;
 *  - temperature 0 makes p one-hot at the lowest-index argmax;
 *  - top-k / nucleus truncation (rejection rule only, T > 0): top-k keeps
 *    every token whose logit is at least the k-th largest (ties kept); the
 *    nucleus then acts on the renormalised top-k distribution and keeps a
 *    token iff the mass of the tokens with a strictly larger logit is below
 *    top_p; the tests, residual and bonus use the renormalised result.
 */
#include <math.h>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1

static double load_elem(const void* base, int dtype, size_t idx) {
    if (dtype == ORACLE_F32) return (double)((const float*)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t*)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

static int parent_of(const int32_t* parent, int N, int b, int i) {
    if (i == 0) return -1;
    return parent ? parent[(size_t)b * N + i] : i - 1;
}

/* ---------------------------------------------------------------------------
 * Tree attention.  For query row (b, node i, q-head h), with kv-head
 * g = h / (Hq / Hkv):
 *   keys  = prefix rows [0, L_b)  plus tree rows L_b + n for every n on the
 *           root path of i (i itself included);
 *   s_j   = scale * <q, k_j>;  out = sum_j exp(s_j - max s) v_j / sum_j exp(s_j - max s).
 * sel == NULL computes every row into out[B][N][Hq][D]; otherwise sel holds
 * nsel (b, i, h) triples and out is [nsel][D].
 * ------------------------------------------------------------------------- */
int oracle_tree_attn(int B, int N, int Hq, int Hkv, int D, int cap, int dtype, double scale,
                     const void* q, const void* k, const void* v, const int32_t* prefix_len,
                     const int32_t* parent, int nsel, const int32_t* sel, double* out) {
    if (B < 0 || N < 1 || N > 64 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1) return -1;
    const int G = Hq / Hkv;
    const long total = sel ? (long)nsel : (long)B * N * Hq;
    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (long r = 0; r < total; ++r) {
        int b, i, h;
        if (sel) {
            b = sel[3 * r + 0];
            i = sel[3 * r + 1];
            h = sel[3 * r + 2];
        } else {
            b = (int)(r / ((long)N * Hq));
            i = (int)((r / Hq) % N);
            h = (int)(r % Hq);
        }
        const int g = h / G;
        const int L = prefix_len[b];
        int path[64], np = 0;
        for (int n = i; n >= 0; n = parent_of(parent, N, b, n)) path[np++] = n;
        const long nkeys = (long)L + np;
        if ((long)L + N > cap) {
#pragma omp atomic write
            err = 1;
            continue;
        }
        double* s = (double*)malloc(sizeof(double) * (size_t)nkeys);
        const size_t qoff = (((size_t)b * N + i) * Hq + h) * (size_t)D;
        const size_t kvbase = ((size_t)b * Hkv + g) * (size_t)cap;
        double m = -INFINITY;
        for (long j = 0; j < nkeys; ++j) {
            const long row = j < L ? j : (long)L + path[j - L];
            double dot = 0.0;
            for (int d = 0; d < D; ++d)
                dot += load_elem(q, dtype, qoff + d) * load_elem(k, dtype, (kvbase + row) * D + d);
            s[j] = scale * dot;
            if (s[j] > m) m = s[j];
        }
        double den = 0.0;
        for (long j = 0; j < nkeys; ++j) {
            s[j] = exp(s[j] - m);
            den += s[j];
        }
        double* o = out + (size_t)r * D;
        for (int d = 0; d < D; ++d) o[d] = 0.0;
        for (long j = 0; j < nkeys; ++j) {
            const long row = j < L ? j : (long)L + path[j - L];
            for (int d = 0; d < D; ++d) o[d] += s[j] * load_elem(v, dtype, (kvbase + row) * D + d);
        }
        for (int d = 0; d < D; ++d) o[d] /= den;
        free(s);
    }
    return err ? -1 : 0;
}

/* Lowest index of the largest value of a float row. */
static int row_argmax(const float* row, int V) {
    int best = 0;
    for (int x = 1; x < V; ++x)
        if (row[x] > row[best]) best = x;
    return best;
}

/* p = softmax(l / T) in fp64; T == 0 gives the one-hot at the argmax.
 * Also returns the entropy -sum p ln p (0 ln 0 = 0). */
static double target_probs(const float* row, int V, double T, double* p) {
    if (T == 0.0) {
        for (int x = 0; x < V; ++x) p[x] = 0.0;
        p[row_argmax(row, V)] = 1.0;
        return 0.0;
    }
    double m = -INFINITY;
    for (int x = 0; x < V; ++x) {
        const double z = (double)row[x] / T;
        if (z > m) m = z;
    }
    double S = 0.0;
    for (int x = 0; x < V; ++x) {
        p[x] = exp((double)row[x] / T - m);
        S += p[x];
    }
    double H = 0.0;
    for (int x = 0; x < V; ++x) {
        p[x] /= S;
        if (p[x] > 0.0) H -= p[x] * log(p[x]);
    }
    return H;
}

/* Top-k then nucleus (top-p) truncation of p = softmax(l / T), T > 0, in
 * place and renormalised: the "Speculative Sampling" section of the same page
 * lets top-k and nucleus sampling transform the probabilities before the
 * rejection rule.  top_k <= 0 or >= V: no top-k; top_p >= 1: no nucleus.
 * Top-k keeps every token whose logit is at least the k-th largest logit;
 * the nucleus, on the renormalised top-k distribution, keeps a token iff the
 * mass of the tokens with a strictly larger logit is below top_p (so tokens
 * of equal logit are kept or dropped together).  Returns the nucleus margin:
 * the smallest distance from top_p to the mass above a group of equal logits
 * (INFINITY without a nucleus). */
typedef struct {
    float l;
    int x;
} LogitIdx;

static int by_logit_desc(const void* a, const void* b) {
    const LogitIdx* p = (const LogitIdx*)a;
    const LogitIdx* q = (const LogitIdx*)b;
    if (p->l > q->l) return -1;
    if (p->l < q->l) return 1;
    return (p->x > q->x) - (p->x < q->x);
}

static double truncate_probs(const float* row, int V, int top_k, double top_p, double* p) {
    const int use_k = top_k > 0 && top_k < V, use_p = top_p < 1.0;
    if (!use_k && !use_p) return INFINITY;
    LogitIdx* s = (LogitIdx*)malloc(sizeof(LogitIdx) * (size_t)V);
    for (int x = 0; x < V; ++x) {
        s[x].l = row[x];
        s[x].x = x;
    }
    qsort(s, (size_t)V, sizeof(LogitIdx), by_logit_desc);
    int n = V; /* s[0 .. n) are kept */
    if (use_k) {
        n = top_k;
        while (n < V && s[n].l == s[top_k - 1].l) ++n;
    }
    double margin = INFINITY;
    if (use_p) {
        double W = 0.0;
        for (int i = 0; i < n; ++i) W += p[s[i].x];
        double above = 0.0;
        int kept = 0;
        for (int i = 0; i < n;) {
            int j = i;
            double g = 0.0;
            while (j < n && s[j].l == s[i].l) g += p[s[j++].x];
            const double A = above / W;
            if (fabs(A - top_p) < margin) margin = fabs(A - top_p);
            if (!(A < top_p)) break;
            above += g;
            kept = j;
            i = j;
        }
        n = kept;
    }
    char* keep = (char*)calloc((size_t)V, 1);
    for (int i = 0; i < n; ++i) keep[s[i].x] = 1;
    double S = 0.0;
    for (int x = 0; x < V; ++x) {
        if (!keep[x]) p[x] = 0.0;
        S += p[x];
    }
    for (int x = 0; x < V; ++x) p[x] /= S;
    free(keep);
    free(s);
    return margin;
}

/* Inverse-CDF draw from non-negative weights r (total S > 0) with uniform u.
 * *margin receives the distance, in the units of r, from u*S to the nearest
 * boundary of the chosen token's interval that borders another token of
 * non-zero weight (INFINITY when no such boundary exists). */
static int draw(const double* r, int V, double S, double u, double* margin) {
    const double t = u * S;
    double cum = 0.0;
    int x = -1;
    double lo = 0.0;
    for (int y = 0; y < V; ++y) {
        if (r[y] <= 0.0) continue;
        lo = cum;
        cum += r[y];
        if (cum > t) {
            x = y;
            break;
        }
    }
    if (x < 0) { /* rounding left u*S at or above the total */
        for (int y = V - 1; y >= 0; --y)
            if (r[y] > 0.0) {
                x = y;
                break;
            }
        *margin = 0.0;
        return x;
    }
    int any_below = 0, any_above = 0;
    for (int y = 0; y < x; ++y)
        if (r[y] > 0.0) {
            any_below = 1;
            break;
        }
    for (int y = x + 1; y < V; ++y)
        if (r[y] > 0.0) {
            any_above = 1;
            break;
        }
    double mg = INFINITY;
    if (any_below && t - lo < mg) mg = t - lo;
    if (any_above && cum - t < mg) mg = cum - t;
    *margin = mg;
    return x;
}

/* ---------------------------------------------------------------------------
 * Acceptance.  rule 0 = rejection rule, rule 1 = typical acceptance.
 * Per request b:
 *   p_u = softmax(l_u / T) for each node row u that has children (and the stop
 *   row); node i >= 1 with parent u, token x = tokens[i]:
 *     rejection: ok_i <=> u_accept[i] * q_i(x) < p_u(x)
 *     typical:   ok_i <=> p_u(x) > min(eps, delta * exp(-H(p_u)))
 *   acc_0 = 1, acc_i = ok_i && acc_parent(i); v = deepest accepted node
 *   (smallest index on ties); a = depth(v); path = root .. v.
 *   final token:
 *     typical: argmax p_v
 *     rejection, v has children: c = smallest child, r = max(0, p_v - q_c),
 *       r = p_v if sum r == 0, final = draw(r, u_sample[v]);
 *     rejection, v a leaf: final = draw(p_v, u_sample[v]).
 *   With top_k / top_p (rejection rule, T > 0) every p_u above is first
 *   truncated by truncate_probs.
 * Outputs accept_len[b] = a, path[b][0..a] then -1, out_tokens[b][0..a-1] =
 * tokens of path[1..a], out_tokens[b][a] = final, then -1.  margin[b] is the
 * smallest distance of any decision that can change the output from its
 * threshold (|min(1, p/q) - u|; |p - thr| / max(p, thr) for the typical
 * test; the draw margin in probability units; the nucleus margin of every
 * truncated row); stop[b] = v.
 * ------------------------------------------------------------------------- */
int oracle_accept_ex(int B, int N, int V, int rule, const float* logits, const float* draft,
                     const int32_t* tokens, const int32_t* parent, const float* u_accept,
                     const float* u_sample, double T, double eps, double delta, int top_k, double top_p,
                     int32_t* accept_len, int32_t* path, int32_t* out_tokens, double* margin,
                     int32_t* stop) {
    if (B < 0 || N < 1 || N > 64 || V < 1 || (rule != 0 && rule != 1) || !(T >= 0.0)) return -1;
    if (rule == 0 && N > 1 && !draft) return -1;
    if (top_k < 0 || !(top_p > 0.0 && top_p <= 1.0)) return -1;
    const int truncate = rule == 0 && T > 0.0 && ((top_k > 0 && top_k < V) || top_p < 1.0);
    if (rule == 1 && ((top_k > 0 && top_k < V) || top_p < 1.0)) return -1; /* rejection rule only */
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int par[64], depth[64], has_child[64], acc[64];
        for (int i = 0; i < N; ++i) has_child[i] = 0;
        for (int i = 0; i < N; ++i) {
            par[i] = parent_of(parent, N, b, i);
            depth[i] = i == 0 ? 0 : depth[par[i]] + 1;
            if (i > 0) has_child[par[i]] = 1;
        }
        double* P = (double*)calloc((size_t)N * V, sizeof(double));
        double H[64];
        int have[64];
        double mg = INFINITY;
        for (int u = 0; u < N; ++u) {
            have[u] = 0;
            if (has_child[u]) {
                H[u] = target_probs(logits + ((size_t)b * N + u) * V, V, T, P + (size_t)u * V);
                if (truncate) {
                    const double tm = truncate_probs(logits + ((size_t)b * N + u) * V, V, top_k, top_p,
                                                     P + (size_t)u * V);
                    if (tm < mg) mg = tm;
                }
                have[u] = 1;
            }
        }
        acc[0] = 1;
        for (int i = 1; i < N; ++i) {
            const int u = par[i];
            const int x = tokens[(size_t)b * N + i];
            const double pu = P[(size_t)u * V + x];
            int ok;
            if (rule == 0) {
                const double qx = draft[((size_t)b * N + i) * V + x];
                const double ua = u_accept[(size_t)b * N + i];
                ok = ua * qx < pu;
                if (acc[u]) {
                    const double ratio = qx > 0.0 ? pu / qx : (pu > 0.0 ? INFINITY : 0.0);
                    const double d = fabs(fmin(1.0, ratio) - ua);
                    if (d < mg) mg = d;
                }
            } else {
                const double thr = fmin(eps, delta * exp(-H[u]));
                ok = pu > thr;
                if (acc[u]) { /* relative: p and thr both carry relative rounding */
                    const double den = fmax(pu, thr);
                    const double d = den > 0.0 ? fabs(pu - thr) / den : INFINITY;
                    if (d < mg) mg = d;
                }
            }
            acc[i] = ok && acc[u];
        }
        int v = 0;
        for (int i = 1; i < N; ++i)
            if (acc[i] && depth[i] > depth[v]) v = i;
        const int a = depth[v];
        int32_t* pth = path + (size_t)b * N;
        int32_t* ot = out_tokens + (size_t)b * N;
        for (int i = 0; i < N; ++i) pth[i] = ot[i] = -1;
        for (int n = v, d = a; n >= 0; n = par[n], --d) pth[d] = n;
        for (int d = 1; d <= a; ++d) ot[d - 1] = tokens[(size_t)b * N + pth[d]];

        const float* lv = logits + ((size_t)b * N + v) * V;
        int final;
        if (rule == 1) {
            final = row_argmax(lv, V);
        } else {
            if (!have[v]) {
                target_probs(lv, V, T, P + (size_t)v * V);
                if (truncate) {
                    const double tm = truncate_probs(lv, V, top_k, top_p, P + (size_t)v * V);
                    if (tm < mg) mg = tm;
                }
            }
            const double* pv = P + (size_t)v * V;
            double* r = (double*)malloc(sizeof(double) * (size_t)V);
            double S = 0.0;
            if (has_child[v]) {
                int c = -1;
                for (int i = 1; i < N && c < 0; ++i)
                    if (par[i] == v) c = i;
                const float* qc = draft + ((size_t)b * N + c) * V;
                for (int x = 0; x < V; ++x) {
                    const double d = pv[x] - (double)qc[x];
                    r[x] = d > 0.0 ? d : 0.0;
                    S += r[x];
                }
            }
            if (S == 0.0) {
                S = 0.0;
                for (int x = 0; x < V; ++x) {
                    r[x] = pv[x];
                    S += r[x];
                }
            }
            double dm;
            final = draw(r, V, S, (double)u_sample[(size_t)b * N + v], &dm);
            if (dm < mg) mg = dm;
            free(r);
        }
        ot[a] = final;
        accept_len[b] = a;
        if (margin) margin[b] = mg;
        if (stop) stop[b] = v;
        free(P);
    }
    return 0;
}

int oracle_accept(int B, int N, int V, int rule, const float* logits, const float* draft,
                  const int32_t* tokens, const int32_t* parent, const float* u_accept,
                  const float* u_sample, double T, double eps, double delta, int32_t* accept_len,
                  int32_t* path, int32_t* out_tokens, double* margin, int32_t* stop) {
    return oracle_accept_ex(B, N, V, rule, logits, draft, tokens, parent, u_accept, u_sample, T, eps, delta, 0,
                            1.0, accept_len, path, out_tokens, margin, stop);
}

/* ---------------------------------------------------------------------------
 * Rejection over a tree with several drafts per node, by recursive residuals
 * (a reading: the pages give the single-draft rule and say that tree
 * candidates can reuse it, without a multi-draft scheme).  Per request b,
 * starting at the root v = 0:
 *   r = p_v = softmax(l_v / T);
 *   for the children c of v in ascending index, token x = tokens[c]:
 *     accept c iff u_accept[c] * q_c(x) < r(x); then v = c and repeat;
 *     else r = norm(max(0, r - q_c)) (r unchanged if that is all zero);
 *   every child rejected: final = draw(r, u_sample[v]); v a leaf: final =
 *   draw(p_v, u_sample[v]).
 * Each step emits a token distributed as p_v when the children's tokens are
 * drawn from their q (this is the point of the residual chain), and on a
 * chain the rule is the single-draft rule.  Outputs and margin as
 * oracle_accept (margins |min(1, r/q) - u| of the tests taken, and the draw).
 * ------------------------------------------------------------------------- */
int oracle_accept_multidraft(int B, int N, int V, const float* logits, const float* draft,
                             const int32_t* tokens, const int32_t* parent, const float* u_accept,
                             const float* u_sample, double T, int32_t* accept_len, int32_t* path,
                             int32_t* out_tokens, double* margin, int32_t* stop) {
    if (B < 0 || N < 1 || N > 64 || V < 1 || !(T >= 0.0)) return -1;
    if (N > 1 && !draft) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int b = 0; b < B; ++b) {
        int par[64];
        for (int i = 0; i < N; ++i) par[i] = parent_of(parent, N, b, i);
        double* p = (double*)malloc(sizeof(double) * (size_t)V);
        double* r = (double*)malloc(sizeof(double) * (size_t)V);
        double* t = (double*)malloc(sizeof(double) * (size_t)V);
        int32_t* pth = path + (size_t)b * N;
        int32_t* ot = out_tokens + (size_t)b * N;
        for (int i = 0; i < N; ++i) pth[i] = ot[i] = -1;
        pth[0] = 0;
        double mg = INFINITY;
        int v = 0, a = 0, final = -1;
        for (;;) {
            target_probs(logits + ((size_t)b * N + v) * V, V, T, p);
            for (int x = 0; x < V; ++x) r[x] = p[x];
            int next = -1, any_child = 0;
            for (int c = 1; c < N && next < 0; ++c) {
                if (par[c] != v) continue;
                any_child = 1;
                const int x = tokens[(size_t)b * N + c];
                const float* qc = draft + ((size_t)b * N + c) * V;
                const double qx = qc[x], ua = u_accept[(size_t)b * N + c];
                const double ratio = qx > 0.0 ? r[x] / qx : (r[x] > 0.0 ? INFINITY : 0.0);
                const double d = fabs(fmin(1.0, ratio) - ua);
                if (d < mg) mg = d;
                if (ua * qx < r[x]) {
                    next = c;
                    break;
                }
                double Z = 0.0;
                for (int y = 0; y < V; ++y) {
                    const double e = r[y] - (double)qc[y];
                    t[y] = e > 0.0 ? e : 0.0;
                    Z += t[y];
                }
                if (Z > 0.0)
                    for (int y = 0; y < V; ++y) r[y] = t[y] / Z;
            }
            if (next >= 0) {
                v = next;
                ++a;
                pth[a] = v;
                ot[a - 1] = tokens[(size_t)b * N + v];
                continue;
            }
            double S = 0.0;
            for (int x = 0; x < V; ++x) S += r[x];
            double dm;
            final = draw(r, V, S, (double)u_sample[(size_t)b * N + v], &dm);
            if (dm < mg) mg = dm;
            (void)any_child;
            break;
        }
        ot[a] = final;
        accept_len[b] = a;
        if (margin) margin[b] = mg;
        if (stop) stop[b] = v;
        free(p);
        free(r);
        free(t);
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Linear-attention verification and state commit (SpecLA paragraphs of the
 * gist.science summary "SpecLA: Efficient Speculative Decoding for
 * Linear-Attention Models": a stateful linear-attention model verifies a
 * chain or a tree of drafts against its summary state, with a tree mask for
 * branches, and afterwards recovers the state from compact factors).  The
 * pages give no recurrence; the reading is a matrix state per (request, head)
 * with a scalar decay per token:
 *     S_t = alpha_t S_{t-1} + v_t k_t^T,   o_t = S_t q_t
 * (alpha = 1: plain linear attention).  Node i of the tree follows its root
 * path: with A(j -> i] the product of alpha over the path nodes after j up
 * to i (and A(-> i] over the whole path root .. i),
 *     o_i = A(-> i] S q_i + sum_{j in anc(i)} A(j -> i] (q_i . k_j) v_j,
 * anc(i) including i.  The commit for accepted stop node v is S_v itself:
 *     S' = A(-> v] S + sum_{j on the path} A(j -> v] v_j k_j^T.
 * Layouts: S [B][H][Dv][Dk], q/k [B][N][H][Dk], v/out [B][N][H][Dv],
 * alpha [B][N][H] (NULL = 1), parent [B][N] (NULL = chain).
 * ------------------------------------------------------------------------- */
static double path_decay(const int* par, const double* al, int j, int i) {
    /* product of alpha over the path nodes after j up to i (j = -1: whole
       path); j must be an ancestor-or-self of i */
    double d = 1.0;
    for (int n = i; n != j; n = par[n]) d *= al[n];
    return d;
}

int oracle_la_verify(int B, int N, int H, int Dk, int Dv, int dtype, const float* state, const void* q,
                     const void* k, const void* v, const float* alpha, const int32_t* parent, double* out) {
    if (B < 0 || N < 1 || N > 64 || H < 1 || Dk < 1 || Dv < 1) return -1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            int par[64];
            double al[64];
            for (int i = 0; i < N; ++i) {
                par[i] = parent_of(parent, N, b, i);
                al[i] = alpha ? alpha[((size_t)b * N + i) * H + h] : 1.0;
            }
            const float* S = state + ((size_t)b * H + h) * Dv * Dk;
            for (int i = 0; i < N; ++i) {
                const size_t qo = (((size_t)b * N + i) * H + h) * Dk;
                double* o = out + (((size_t)b * N + i) * H + h) * Dv;
                const double Ai = path_decay(par, al, -1, i);
                for (int e = 0; e < Dv; ++e) {
                    double acc = 0.0;
                    for (int d = 0; d < Dk; ++d) acc += (double)S[(size_t)e * Dk + d] * load_elem(q, dtype, qo + d);
                    o[e] = Ai * acc;
                }
                for (int j = i; j >= 0; j = par[j]) {
                    const size_t ko = (((size_t)b * N + j) * H + h) * Dk;
                    const size_t vo = (((size_t)b * N + j) * H + h) * Dv;
                    double qk = 0.0;
                    for (int d = 0; d < Dk; ++d) qk += load_elem(q, dtype, qo + d) * load_elem(k, dtype, ko + d);
                    const double w = path_decay(par, al, j, i) * qk;
                    for (int e = 0; e < Dv; ++e) o[e] += w * load_elem(v, dtype, vo + e);
                }
            }
        }
    return 0;
}

/* In-place commit of the accepted path (path[b][0 .. accept_len[b]]) into
 * the state; the factors are the path nodes' k, v and alpha. */
int oracle_la_commit(int B, int N, int H, int Dk, int Dv, int dtype, float* state, const void* k, const void* v,
                     const float* alpha, const int32_t* parent, const int32_t* path, const int32_t* accept_len) {
    if (B < 0 || N < 1 || N > 64 || H < 1 || Dk < 1 || Dv < 1) return -1;
#pragma omp parallel for collapse(2) schedule(dynamic, 1)
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            int par[64];
            double al[64];
            for (int i = 0; i < N; ++i) {
                par[i] = parent_of(parent, N, b, i);
                al[i] = alpha ? alpha[((size_t)b * N + i) * H + h] : 1.0;
            }
            const int a = accept_len[b];
            const int vstop = path[(size_t)b * N + a];
            float* S = state + ((size_t)b * H + h) * Dv * Dk;
            const double Av = path_decay(par, al, -1, vstop);
            for (int e = 0; e < Dv; ++e)
                for (int d = 0; d < Dk; ++d) {
                    double acc = Av * (double)S[(size_t)e * Dk + d];
                    for (int t = 0; t <= a; ++t) {
                        const int j = path[(size_t)b * N + t];
                        acc += path_decay(par, al, j, vstop) *
                               load_elem(v, dtype, (((size_t)b * N + j) * H + h) * Dv + e) *
                               load_elem(k, dtype, (((size_t)b * N + j) * H + h) * Dk + d);
                    }
                    S[(size_t)e * Dk + d] = (float)acc;
                }
        }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Commit: for every request b and kv-head, the accepted path's rows
 * L_b + path[d] (d = 0..a) move to L_b + d; every source row is read before
 * any row is written.  prefix_len[b] becomes L_b + a + 1.  row_bytes = D *
 * element size; the caches are [B][Hkv][cap][row_bytes].
 * ------------------------------------------------------------------------- */
int oracle_commit(int B, int N, int Hkv, int cap, int row_bytes, uint8_t* k, uint8_t* v,
                  int32_t* prefix_len, const int32_t* path, const int32_t* accept_len) {
    for (int b = 0; b < B; ++b) {
        const int L = prefix_len[b];
        const int a = accept_len[b];
        if (a < 0 || a >= N || L + N > cap) return -1;
        uint8_t* tmp = (uint8_t*)malloc((size_t)(a + 1) * row_bytes);
        for (int which = 0; which < 2; ++which) {
            uint8_t* base = which ? v : k;
            for (int g = 0; g < Hkv; ++g) {
                uint8_t* head = base + ((size_t)b * Hkv + g) * (size_t)cap * row_bytes;
                for (int d = 0; d <= a; ++d)
                    memcpy(tmp + (size_t)d * row_bytes,
                           head + (size_t)(L + path[(size_t)b * N + d]) * row_bytes, row_bytes);
                for (int d = 0; d <= a; ++d)
                    memcpy(head + (size_t)(L + d) * row_bytes, tmp + (size_t)d * row_bytes, row_bytes);
            }
        }
        free(tmp);
        prefix_len[b] = L + a + 1;
    }
    return 0;
}

/* ---------------------------------------------------------------------------
 * Medusa candidate tree (MEDUSA section, candidate construction and tree
 * attention paragraphs): head k (k = 1..K) proposes its top-s_k tokens;
 * the candidates are the Cartesian product of the heads' proposals, arranged
 * as a tree.  Node 0 is the root (root_tokens[b]).  Reading: the tree is
 * built level by level (breadth first); the children of a depth-(d-1) node
 * are its extensions by head d's candidates in rank order, and the parents
 * of one level are visited in the order the previous level was built.  So
 * node (i_1, ..., i_d) has parent (i_1, ..., i_{d-1}) and token
 * head_tokens[b][d-1][i_d].  head_tokens is [B][K][max_width].
 * Returns the node count N (1 + sum over d of prod_{k<=d} s_k), or -1 if a
 * width is outside [1, max_width] or N exceeds max_nodes; parent and tokens
 * are [B][N].
 * ------------------------------------------------------------------------- */
int oracle_medusa_tree(int B, int K, const int32_t* widths, int max_width, int max_nodes,
                       const int32_t* root_tokens, const int32_t* head_tokens, int32_t* parent,
                       int32_t* tokens) {
    long n = 1, level = 1;
    for (int k = 0; k < K; ++k) {
        if (widths[k] < 1 || widths[k] > max_width) return -1;
        level *= widths[k];
        n += level;
        if (n > max_nodes) return -1;
    }
    const int N = (int)n;
    int* frontier = (int*)malloc(sizeof(int) * (size_t)N);
    int* next = (int*)malloc(sizeof(int) * (size_t)N);
    for (int b = 0; b < B; ++b) {
        int32_t* par = parent + (size_t)b * N;
        int32_t* tok = tokens + (size_t)b * N;
        par[0] = -1;
        tok[0] = root_tokens[b];
        int nf = 1, built = 1;
        frontier[0] = 0;
        for (int k = 0; k < K; ++k) {
            int nn = 0;
            for (int f = 0; f < nf; ++f)
                for (int c = 0; c < widths[k]; ++c) {
                    par[built] = frontier[f];
                    tok[built] = head_tokens[((size_t)b * K + k) * max_width + c];
                    next[nn++] = built++;
                }
            memcpy(frontier, next, sizeof(int) * (size_t)nn);
            nf = nn;
        }
    }
    free(frontier);
    free(next);
    return N;
}

/* ---------------------------------------------------------------------------
 * Depth-position rotary embedding of the tree (MEDUSA tree-attention
 * paragraph: position indices follow tree depth).  Node i of request b sits
 * at position pos = L_b + depth(i).  Reading: the rotary embedding of the
 * Llama family, in its rotate-half layout: for j < D/2 the pair
 * (x_j, x_{j+D/2}) is turned by the angle pos * base^(-2j/D):
 *   x_j'       = x_j cos - x_{j+D/2} sin
 *   x_{j+D/2}' = x_j sin + x_{j+D/2} cos.
 * Applied to q[b][i][h] (every q head) and to the tree's K rows
 * k_cache[b][g][L_b + i] (every kv head).  Outputs are fp64, unrounded:
 * q_out [B][N][Hq][D], k_out [B][Hkv][N][D].
 * ------------------------------------------------------------------------- */
static void rope_row(const void* src, int dtype, size_t off, int D, double pos, double base, double* out) {
    for (int j = 0; j < D / 2; ++j) {
        const double theta = pos * pow(base, -2.0 * j / D);
        const double c = cos(theta), sn = sin(theta);
        const double x = load_elem(src, dtype, off + j), y = load_elem(src, dtype, off + j + D / 2);
        out[j] = x * c - y * sn;
        out[j + D / 2] = x * sn + y * c;
    }
}

int oracle_tree_rope(int B, int N, int Hq, int Hkv, int D, int cap, int dtype, const void* q,
                     const void* k_cache, const int32_t* prefix_len, const int32_t* parent, double base,
                     double* q_out, double* k_out) {
    if (D % 2 != 0) return -1;
    for (int b = 0; b < B; ++b) {
        const int L = prefix_len[b];
        if (L < 0 || L + N > cap) return -1;
        for (int i = 0; i < N; ++i) {
            int depth = 0;
            for (int n = parent_of(parent, N, b, i); n >= 0; n = parent_of(parent, N, b, n)) ++depth;
            const double pos = (double)L + depth;
            for (int h = 0; h < Hq; ++h)
                rope_row(q, dtype, (((size_t)b * N + i) * Hq + h) * D, D, pos, base,
                         q_out + (((size_t)b * N + i) * Hq + h) * D);
            for (int g = 0; g < Hkv; ++g)
                rope_row(k_cache, dtype, (((size_t)b * Hkv + g) * cap + L + i) * D, D, pos, base,
                         k_out + (((size_t)b * Hkv + g) * N + i) * D);
        }
    }
    return 0;
}

/* Threads the OpenMP loops above use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the thread count of the OpenMP loops above (n >= 1); returns the
 * count now in effect. */
int oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#endif
    return oracle_num_threads();
}
