/*
 * sv_oracle.c -- plain CPU oracle for the tree-masked speculative verify step.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the slow, obviously-correct reference the
 * GPU library is checked against.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg load it; no product code path calls it.  It
 * shares no code, header, table or constant with the GPU library: its enums,
 * its bf16 decoding and its cache addressing are all written out here.
 *
 * Floating point is fp64 throughout (inputs are widened exactly from fp32 or
 * bf16); results are narrowed to fp32 with round-to-nearest-even at the end.
 * No blocking, fusion or reordering: each function follows the definition it
 * cites, loop by loop.
 *
 * Sources (web pages, cited by title and section):
 *  [ADR]  "ADR-037 -- EAGLE-3 with dynamic tree port" (hf2q docs): Phase status
 *         table rows E1.1-E1.5 (tree attention parity ladder, output layout
 *         [q_seq_len, num_heads, head_dim]), E4a (build_tree_mask from the
 *         parent array; global best-first expansion through one queue of
 *         pending candidates keyed by the fp64 cumulative log-probability),
 *         E4b.5b (NeoX RoPE at base position + tree depth, over the whole
 *         head), E4b.10a (top-K of the log-softmax, smaller token wins ties),
 *         E5a (tree-walk accept), E6 v2 (mask selects ancestors + self);
 *         section 4 Phase E1 (dynamic tree mask, apply_tree_attention), Phase
 *         E4 (expansion by cumulative log-probability up to a node budget) and
 *         Phase E5 (longest matching path from root; full accept picks the
 *         deepest).
 *  [HEADS] "Speculative-decoding heads: Medusa + EAGLE-2" (posttrainllm docs):
 *         "Why bother" (greedy verify accepts the longest matching argmax
 *         prefix), "Mechanism comparison" (EAGLE-2's dynamic candidate tree),
 *         "What's not implemented" item 1(c) (each tree node attends only to
 *         its ancestors).
 *  [ANE]  "Speculative decoding verify batches to amortize ANE dispatch"
 *         (llms-explorer): Facts on the commit rule (argmax decides, longest
 *         matching prefix plus one bonus token, accept(k) commits only the
 *         accepted prefix), on delayed KV write-through, and on Forge's sampled
 *         verification (a proposal is accepted with its target probability; on
 *         rejection the target distribution is sampled with it excluded).
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -shared -fPIC sv_oracle.c -lm
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Per-sequence tree status codes (oracle's own numbering). */
enum { OR_TREE_OK = 0, OR_TREE_BAD_ROOT = 1, OR_TREE_BAD_PARENT = 2 };
/* Element types of Q/K/V and the cache. */
enum { OR_F32 = 0, OR_BF16 = 1 };

/* ------------------------------------------------------------------------ */
/* Tree validity.  Reading: node 0 is the root (parent -1) and every other    */
/* node's parent precedes it (0 <= parent[i] < i), the order a best-first     */
/* expansion admits nodes in ([ADR] E4a).                                      */
static int tree_status(const int32_t *par, int T) {
    if (par[0] != -1) return OR_TREE_BAD_ROOT;
    for (int i = 1; i < T; ++i)
        if (par[i] < 0 || par[i] >= i) return OR_TREE_BAD_PARENT;
    return OR_TREE_OK;
}

/* ------------------------------------------------------------------------ */
/* Mask ([ADR] E4a build_tree_mask, E6 v2 "ancestors + self"; [HEADS] item    */
/* 1(c)).  Row i has bit j set iff node j is node i or one of its ancestors.  */
/* depth[i] = number of proper ancestors (root 0).  A malformed parent array  */
/* sets tree_err[b] and leaves every row self-only with depth 0.             */
int oracle_build_tree_mask(const int32_t *parents, int B, int T, uint64_t *mask,
                           int32_t *depth, int32_t *tree_err) {
    if (B < 0 || T < 1) return -1;
    const int W = (T + 63) / 64;
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parents + (int64_t)b * T;
        const int st = tree_status(par, T);
        tree_err[b] = st;
        for (int i = 0; i < T; ++i) {
            uint64_t *row = mask + ((int64_t)b * T + i) * W;
            for (int w = 0; w < W; ++w) row[w] = 0;
            int steps = 0;
            if (st != OR_TREE_OK) {
                row[i / 64] |= (uint64_t)1 << (i % 64);
            } else {
                int j = i;
                while (j != -1) {             /* walk to the root */
                    row[j / 64] |= (uint64_t)1 << (j % 64);
                    j = par[j];
                    ++steps;
                }
                steps -= 1;                   /* self is not an ancestor */
            }
            if (depth) depth[(int64_t)b * T + i] = steps;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
static double elem(const void *base, int dtype, int64_t idx) {
    if (dtype == OR_F32) return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;  /* bf16 = top half of fp32 */
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Cache addressing: position pos of sequence b, kv head h lives in block
 * table[b][pos / bs] at slot pos % bs.  Returns the element offset of the row,
 * or -1 when the table entry is outside [0, num_blocks). */
static int64_t cache_row(const int32_t *table, int bs, int max_blocks, int64_t block_stride,
                         int64_t head_stride, int64_t row_stride, int64_t num_blocks,
                         int b, int h, int64_t pos) {
    const int32_t blk = table[(int64_t)b * max_blocks + pos / bs];
    if (blk < 0 || blk >= num_blocks) return -1;
    return (int64_t)blk * block_stride + (int64_t)h * head_stride + (pos % bs) * row_stride;
}

/* ------------------------------------------------------------------------ */
/* Attention ([ADR] E1.1-E1.5 and section 4 Phase E1; [HEADS] item 1(c)).     */
/* For query row (b, h, i): kv head = h / (Hq/Hkv); keys are the P_b cached   */
/* prefix rows of that kv head in position order, then the tree rows j whose  */
/* mask bit is set in row i, in increasing j.  s = scale * <q, k>;            */
/* O = sum_k exp(s_k - max s) v_k / sum_k exp(s_k - max s), in fp64, stored   */
/* as fp32 at out[b][i][h][:] (layout [q_seq_len, num_heads, head_dim]).      */
/* P_b is clamped into [0, max_prefix_len]; prefix keys whose block-table     */
/* entry is out of range are left out.                                        */
/* With k_tree and v_tree NULL the tree rows live in the cache ([ADR] row E6  */
/* per-layer tree-verify block: K/V appended at [prefix_len, prefix_len +     */
/* tree_seq_len) before the attention reads them): tree row j is the cache    */
/* row at position P_b + j (left out if its block-table entry is out of       */
/* range).                                                                     */
/* rows: optional list of (b, h, i) triples; then out is [nrows][D].          */
static void attend_one(const void *q, const void *k_tree, const void *v_tree,
                       const void *k_cache, const void *v_cache, const int32_t *table, int bs,
                       int max_blocks, int64_t block_stride, int64_t head_stride,
                       int64_t row_stride, int64_t num_blocks, int dtype,
                       const int32_t *prefix_len, int max_prefix_len, const uint64_t *mask,
                       int Hq, int Hkv, int T, int D, double scale, int b, int h, int i,
                       double *s, const void **vsrc, int64_t *voff, double *num, float *dst) {
    const int W = (T + 63) / 64;
    const int G = Hq / Hkv;
    const int kvh = h / G;
    int64_t P = prefix_len[b];
    if (P < 0) P = 0;
    if (P > max_prefix_len) P = max_prefix_len;
    const int64_t qoff = (((int64_t)b * Hq + h) * T + i) * D;

    int64_t n = 0;
    for (int64_t p = 0; p < P; ++p) {
        const int64_t off = cache_row(table, bs, max_blocks, block_stride, head_stride,
                                      row_stride, num_blocks, b, kvh, p);
        if (off < 0) continue;
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += elem(q, dtype, qoff + d) * elem(k_cache, dtype, off + d);
        s[n] = scale * dot;
        vsrc[n] = v_cache;
        voff[n] = off;
        ++n;
    }
    const uint64_t *mrow = mask + ((int64_t)b * T + i) * W;
    for (int j = 0; j < T; ++j) {
        if (!((mrow[j / 64] >> (j % 64)) & 1)) continue;
        const void *ksrc = k_tree, *vsrc_j = v_tree;
        int64_t off = (((int64_t)b * Hkv + kvh) * T + j) * D;
        if (!k_tree) { /* tree rows kept in the cache: node j at position P + j */
            off = cache_row(table, bs, max_blocks, block_stride, head_stride, row_stride,
                            num_blocks, b, kvh, P + j);
            if (off < 0) continue;
            ksrc = k_cache;
            vsrc_j = v_cache;
        }
        double dot = 0.0;
        for (int d = 0; d < D; ++d) dot += elem(q, dtype, qoff + d) * elem(ksrc, dtype, off + d);
        s[n] = scale * dot;
        vsrc[n] = vsrc_j;
        voff[n] = off;
        ++n;
    }
    double m = -INFINITY;
    for (int64_t k = 0; k < n; ++k)
        if (s[k] > m) m = s[k];
    double den = 0.0;
    for (int d = 0; d < D; ++d) num[d] = 0.0;
    for (int64_t k = 0; k < n; ++k) {
        const double w = exp(s[k] - m);
        den += w;
        for (int d = 0; d < D; ++d) num[d] += w * elem(vsrc[k], dtype, voff[k] + d);
    }
    for (int d = 0; d < D; ++d) dst[d] = (float)(num[d] / den);
}

int oracle_tree_verify_attention(const void *q, const void *k_tree, const void *v_tree,
                                 const void *k_cache, const void *v_cache, const int32_t *table,
                                 int bs, int max_blocks, int64_t block_stride, int64_t head_stride,
                                 int64_t row_stride, int64_t num_blocks, int dtype,
                                 const int32_t *prefix_len, int max_prefix_len,
                                 const uint64_t *mask, int B, int Hq, int Hkv, int T, int D,
                                 double scale, const int32_t *rows, int64_t nrows, float *out,
                                 int nthreads) {
    if (Hkv <= 0 || Hq <= 0 || Hq % Hkv != 0 || T < 1 || D < 1 || B < 0) return -1;
    const int64_t total = rows ? nrows : (int64_t)B * Hq * T;
    const int64_t maxkeys = (int64_t)max_prefix_len + T;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    int bad = 0;
#pragma omp parallel
    {
        double *s = (double *)malloc(sizeof(double) * (size_t)maxkeys);
        const void **vsrc = (const void **)malloc(sizeof(void *) * (size_t)maxkeys);
        int64_t *voff = (int64_t *)malloc(sizeof(int64_t) * (size_t)maxkeys);
        double *num = (double *)malloc(sizeof(double) * (size_t)D);
        if (!s || !vsrc || !voff || !num) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t r = 0; r < total; ++r) {
                int b, h, i;
                float *dst;
                if (rows) {
                    b = rows[3 * r];
                    h = rows[3 * r + 1];
                    i = rows[3 * r + 2];
                    dst = out + r * D;
                } else {
                    b = (int)(r / ((int64_t)Hq * T));
                    h = (int)((r / T) % Hq);
                    i = (int)(r % T);
                    dst = out + (((int64_t)b * T + i) * Hq + h) * D;
                }
                attend_one(q, k_tree, v_tree, k_cache, v_cache, table, bs, max_blocks,
                           block_stride, head_stride, row_stride, num_blocks, dtype, prefix_len,
                           max_prefix_len, mask, Hq, Hkv, T, D, scale, b, h, i, s, vsrc, voff,
                           num, dst);
            }
        }
        free(s);
        free(vsrc);
        free(voff);
        free(num);
    }
    return bad ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* Argmax over the vocabulary ([ANE] commit rule: the target's argmax at each  */
/* row decides).  The smallest index holding the maximum wins ties ([ADR]     */
/* E4b.10a: smaller token wins).  NaN entries never win; an all-NaN row gives */
/* index 0.                                                                   */
static int32_t argmax_row(const float *x, int64_t V) {
    int64_t best = -1;
    float bv = 0.0f;
    for (int64_t v = 0; v < V; ++v) {
        if (isnan(x[v])) continue;
        if (best < 0 || x[v] > bv) {  /* strict: an equal later value does not replace */
            best = v;
            bv = x[v];
        }
    }
    return best < 0 ? 0 : (int32_t)best;
}

int oracle_argmax(const float *logits, int64_t R, int64_t V, int32_t *out, int nthreads) {
    if (R < 0 || V < 1) return -1;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) out[r] = argmax_row(logits + r * V, V);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Greedy acceptance ([ADR] E5a and Phase E5; [HEADS] "Why bother"; [ANE]     */
/* commit rule).  a[i] = argmax of row i.  Node 0 (the root) is always        */
/* accepted; node i >= 1 matches when its parent matches and its draft token  */
/* equals the parent's argmax.  The accepted node is the deepest matching     */
/* node (smallest index among equals); the path is root..that node,           */
/* L = its depth + 1, and the emitted tokens are a[] along the path (the last */
/* is the bonus / correction token).  An invalid tree (tree_err != 0 or a     */
/* malformed parent array) accepts nothing: L = 0, path and tokens -1.        */
int oracle_accept_longest_path(const float *logits, const int32_t *draft, const int32_t *parents,
                               const int32_t *tree_err, int B, int T, int64_t V,
                               int32_t *argmax_out, int32_t *accepted_len,
                               int32_t *accepted_nodes, int32_t *out_tokens) {
    if (B < 0 || T < 1 || V < 1) return -1;
    int32_t *a = (int32_t *)malloc(sizeof(int32_t) * (size_t)T);
    int32_t *dep = (int32_t *)malloc(sizeof(int32_t) * (size_t)T);
    unsigned char *match = (unsigned char *)malloc((size_t)T);
    int32_t *path = (int32_t *)malloc(sizeof(int32_t) * (size_t)T);
    if (!a || !dep || !match || !path) {
        free(a); free(dep); free(match); free(path);
        return -2;
    }
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parents + (int64_t)b * T;
        const int32_t *drf = draft + (int64_t)b * T;
        for (int i = 0; i < T; ++i) a[i] = argmax_row(logits + ((int64_t)b * T + i) * V, V);
        if (argmax_out)
            for (int i = 0; i < T; ++i) argmax_out[(int64_t)b * T + i] = a[i];
        int32_t *nodes = accepted_nodes + (int64_t)b * T;
        int32_t *toks = out_tokens + (int64_t)b * T;
        for (int j = 0; j < T; ++j) nodes[j] = toks[j] = -1;
        const int invalid = (tree_err && tree_err[b] != 0) || tree_status(par, T) != OR_TREE_OK;
        if (invalid) {
            accepted_len[b] = 0;
            continue;
        }
        match[0] = 1;
        dep[0] = 0;
        for (int i = 1; i < T; ++i) {
            dep[i] = dep[par[i]] + 1;
            match[i] = match[par[i]] && drf[i] == a[par[i]];
        }
        int best = 0;
        for (int i = 1; i < T; ++i)
            if (match[i] && dep[i] > dep[best]) best = i;
        const int L = dep[best] + 1;
        for (int j = L - 1, n = best; j >= 0; --j, n = par[n]) path[j] = n;
        for (int j = 0; j < L; ++j) {
            nodes[j] = path[j];
            toks[j] = a[path[j]];
        }
        accepted_len[b] = L;
    }
    free(a); free(dep); free(match); free(path);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Sampled acceptance ([ANE] Facts: Forge treats the drafted path as given,    */
/* accepts a proposal with its target probability, and on rejection samples   */
/* the target distribution with that proposal excluded).                       */
/* Target distribution of node v: p_v(x) = exp(l_v(x) / tau) / sum_y          */
/* exp(l_v(y) / tau) over logits row v (NaN and -inf entries have p = 0, +inf */
/* counts as the largest finite float; a row with no finite entry has p = 0   */
/* everywhere).                                                                */
/* Reading for a tree (the pages state the rule for one proposal): starting  */
/* at the root, the children of the current node v are tried in increasing    */
/* node index, each as one proposal from what is left of p_v.  With E the      */
/* tokens already rejected at v and R = 1 - sum_{x in E} p_v(x), child c with  */
/* token x is accepted when u_accept[c] * R < p_v(x) (x in E or outside the    */
/* vocabulary: p = 0); an accepted child becomes the current node.  When no    */
/* child is accepted (or v is a leaf), the emitted token is drawn from p_v     */
/* restricted to tokens outside E by inverse CDF: the smallest token y outside */
/* E with sum_{z <= y, z not in E} p_v(z) > u_sample[v] * R (token 0 if no     */
/* token outside E has probability).  Path and tokens: root..final node,       */
/* L = path length, out_tokens = the accepted children's draft tokens, then    */
/* the drawn token.  An invalid tree accepts nothing (L = 0, -1 entries).       */
static double logit_at(const float *row, int64_t y) {
    const float x = row[y];
    if (isnan(x)) return -INFINITY;
    if (isinf(x) && x > 0) return (double)FLT_MAX;
    return (double)x;
}

int oracle_accept_sampled(const float *logits, const int32_t *draft, const int32_t *parents,
                          const int32_t *tree_err, const float *u_accept, const float *u_sample,
                          double tau, int B, int T, int64_t V, int32_t *accepted_len,
                          int32_t *accepted_nodes, int32_t *out_tokens) {
    if (B < 0 || T < 1 || V < 1 || !(tau > 0)) return -1;
    double *p = (double *)malloc(sizeof(double) * (size_t)V);
    unsigned char *excl = (unsigned char *)malloc((size_t)V);
    int32_t *path = (int32_t *)malloc(sizeof(int32_t) * (size_t)T);
    if (!p || !excl || !path) {
        free(p); free(excl); free(path);
        return -2;
    }
    for (int b = 0; b < B; ++b) {
        const int32_t *par = parents + (int64_t)b * T;
        const int32_t *drf = draft + (int64_t)b * T;
        int32_t *nodes = accepted_nodes + (int64_t)b * T;
        int32_t *toks = out_tokens + (int64_t)b * T;
        for (int j = 0; j < T; ++j) nodes[j] = toks[j] = -1;
        if ((tree_err && tree_err[b] != 0) || tree_status(par, T) != OR_TREE_OK) {
            accepted_len[b] = 0;
            continue;
        }
        int v = 0, L = 0;
        path[L++] = 0;
        for (;;) {
            /* p_v */
            const float *row = logits + ((int64_t)b * T + v) * V;
            double m = -INFINITY;
            for (int64_t y = 0; y < V; ++y) {
                const double l = logit_at(row, y);
                if (l > m) m = l;
            }
            double Z = 0.0;
            for (int64_t y = 0; y < V; ++y) {
                const double l = logit_at(row, y);
                p[y] = l == -INFINITY ? 0.0 : exp((l - m) / tau);
                Z += p[y];
            }
            for (int64_t y = 0; y < V; ++y) p[y] = Z > 0.0 ? p[y] / Z : 0.0;
            memset(excl, 0, (size_t)V);
            /* children of v in increasing index */
            double R = 1.0;
            int next = -1;
            for (int c = v + 1; c < T && next < 0; ++c) {
                if (par[c] != v) continue;
                const int32_t x = drf[c];
                const int in_vocab = x >= 0 && (int64_t)x < V;
                const double px = (in_vocab && !excl[x]) ? p[x] : 0.0;
                if ((double)u_accept[(int64_t)b * T + c] * R < px) {
                    next = c;
                } else if (in_vocab && !excl[x]) {
                    excl[x] = 1;
                    R -= px;
                }
            }
            if (next >= 0) {
                toks[L - 1] = drf[next];
                path[L++] = next;
                v = next;
                continue;
            }
            /* draw from p_v without E */
            const double target = (double)u_sample[(int64_t)b * T + v] * R;
            double acc = 0.0;
            int32_t tok = -1;
            for (int64_t y = 0; y < V && tok < 0; ++y) {
                if (excl[y] || p[y] <= 0.0) continue;
                acc += p[y];
                if (acc > target) tok = (int32_t)y;
            }
            if (tok < 0) { /* rounding or no probability left: last eligible token, else 0 */
                tok = 0;
                for (int64_t y = V - 1; y >= 0; --y)
                    if (!excl[y] && p[y] > 0.0) { tok = (int32_t)y; break; }
            }
            toks[L - 1] = tok;
            break;
        }
        for (int j = 0; j < L; ++j) nodes[j] = path[j];
        accepted_len[b] = L;
    }
    free(p); free(excl); free(path);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Tree-position RoPE ([ADR] row E4b.5b: positions base_pos + tree depth, NeoX  */
/* style, the rotation covers the whole head).  For node i of sequence b,       */
/* pos = prefix_len[b] + depth[b][i]; for j < D/2 with f_j = theta^(-2j/D) and  */
/* a = pos * f_j:                                                               */
/*   x'[j]       = x[j] cos a - x[j + D/2] sin a                                */
/*   x'[j + D/2] = x[j + D/2] cos a + x[j] sin a                                */
/* applied in place to every head of Q [B][Hq][T][D] and of the tree keys       */
/* [B][Hkv][T][D]; each result is rounded to the tensor's type (to fp32 by     */
/* round-to-nearest-even, then to bf16 by round-to-nearest-even).              */
static void store_elem(void *base, int dtype, int64_t idx, double v) {
    float f = (float)v;
    if (dtype == OR_F32) {
        ((float *)base)[idx] = f;
        return;
    }
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    if ((bits & 0x7f800000u) == 0x7f800000u && (bits & 0x007fffffu)) {
        ((uint16_t *)base)[idx] = (uint16_t)((bits >> 16) | 0x40u);  /* NaN stays NaN */
        return;
    }
    const uint32_t lsb = (bits >> 16) & 1u;
    bits += 0x7fffu + lsb;                                             /* nearest, ties to even */
    ((uint16_t *)base)[idx] = (uint16_t)(bits >> 16);
}

static void rope_rows(void *x, int dtype, int64_t nheads, const int32_t *prefix_len,
                      const int32_t *depth, int B, int T, int D, double theta) {
    const int half = D / 2;
    for (int b = 0; b < B; ++b)
        for (int64_t h = 0; h < nheads; ++h)
            for (int i = 0; i < T; ++i) {
                const double pos = (double)prefix_len[b] + (double)depth[(int64_t)b * T + i];
                const int64_t row = (((int64_t)b * nheads + h) * T + i) * D;
                for (int j = 0; j < half; ++j) {
                    const double f = pow(theta, -2.0 * (double)j / (double)D);
                    const double a = pos * f;
                    const double c = cos(a), sn = sin(a);
                    const double x1 = elem(x, dtype, row + j), x2 = elem(x, dtype, row + j + half);
                    store_elem(x, dtype, row + j, x1 * c - x2 * sn);
                    store_elem(x, dtype, row + j + half, x2 * c + x1 * sn);
                }
            }
}

int oracle_rope_tree(void *q, void *k_tree, const int32_t *prefix_len, const int32_t *depth,
                     int B, int Hq, int Hkv, int T, int D, int dtype, double theta) {
    if (B < 0 || Hq < 1 || Hkv < 1 || T < 1 || D < 2 || (D & 1) || !(theta > 0) || isinf(theta))
        return -1;
    rope_rows(q, dtype, Hq, prefix_len, depth, B, T, D, theta);
    rope_rows(k_tree, dtype, Hkv, prefix_len, depth, B, T, D, theta);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Delayed KV write-through ([ANE] Facts: accept(k) commits only the accepted */
/* prefix; rejected drafts never touch the cache).  For each sequence with a  */
/* valid tree: cache row prefix_len[b] + j of every kv head receives tree row */
/* accepted_nodes[b][j] (K and V, byte copy), j < accepted_len[b]; then       */
/* new_prefix_len[b] = prefix_len[b] + accepted_len[b].  A sequence whose     */
/* request cannot be honoured in full (prefix_len outside                      */
/* [0, max_prefix_len], rows past capacity, a node index outside [0, T), a    */
/* block-table entry out of range) is left untouched and keeps its length.    */
int oracle_kv_commit(const void *k_tree, const void *v_tree, const int32_t *accepted_len,
                     const int32_t *accepted_nodes, const int32_t *tree_err, void *k_cache,
                     void *v_cache, const int32_t *table, int bs, int max_blocks,
                     int64_t block_stride, int64_t head_stride, int64_t row_stride,
                     int64_t num_blocks, int dtype, const int32_t *prefix_len, int max_prefix_len,
                     int32_t *new_prefix_len, int B, int Hkv, int T, int D) {
    if (B < 0 || Hkv < 1 || T < 1 || D < 1 || bs < 1 || max_blocks < 1) return -1;
    const size_t esz = dtype == OR_F32 ? 4 : 2;
    const int64_t cap = (int64_t)max_blocks * bs;
    for (int b = 0; b < B; ++b) {
        const int32_t P = prefix_len[b];
        const int32_t L = accepted_len[b];
        const int32_t *nodes = accepted_nodes + (int64_t)b * T;
        int ok = !(tree_err && tree_err[b] != 0);
        ok = ok && L >= 0 && L <= T && P >= 0 && P <= max_prefix_len && (int64_t)P + L <= cap;
        for (int j = 0; ok && j < L; ++j) {
            if (nodes[j] < 0 || nodes[j] >= T) ok = 0;
            else if (cache_row(table, bs, max_blocks, block_stride, head_stride, row_stride,
                               num_blocks, b, 0, (int64_t)P + j) < 0) ok = 0;
        }
        if (ok) {
            for (int h = 0; h < Hkv; ++h)
                for (int j = 0; j < L; ++j) {
                    const int64_t dst = cache_row(table, bs, max_blocks, block_stride, head_stride,
                                                  row_stride, num_blocks, b, h, (int64_t)P + j);
                    const int64_t src = (((int64_t)b * Hkv + h) * T + nodes[j]) * D;
                    memcpy((char *)k_cache + dst * esz, (const char *)k_tree + src * esz, esz * D);
                    memcpy((char *)v_cache + dst * esz, (const char *)v_tree + src * esz, esz * D);
                }
        }
        if (new_prefix_len) new_prefix_len[b] = ok ? P + L : P;
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Write-before-accept variant ([ADR] row E6 per-layer tree-verify block: the */
/* tree's K/V rows are appended to the cache at [prefix_len, prefix_len + T)  */
/* before the attention; [ADR] section 4 Phase E5 and row E5b: after the      */
/* acceptance, the cache is rolled back to the accepted path; [ANE] Facts on   */
/* KV write-before-accept, the trade-off delayed write-through avoids).        */
/* Append: for every sequence b with tree_err[b] == 0, if prefix_len[b] lies  */
/* in [0, max_prefix_len] and every position of [P, P + T) has a block-table  */
/* entry in range, tree row i of every kv head is copied to position P + i;   */
/* otherwise nothing is written and tree_err[b] becomes 3.                    */
int oracle_kv_append(const void *k_tree, const void *v_tree, int32_t *tree_err, void *k_cache,
                     void *v_cache, const int32_t *table, int bs, int max_blocks,
                     int64_t block_stride, int64_t head_stride, int64_t row_stride,
                     int64_t num_blocks, int dtype, const int32_t *prefix_len, int max_prefix_len,
                     int B, int Hkv, int T, int D) {
    if (B < 0 || Hkv < 1 || T < 1 || D < 1 || bs < 1 || max_blocks < 1 || !tree_err) return -1;
    const size_t esz = dtype == OR_F32 ? 4 : 2;
    const int64_t cap = (int64_t)max_blocks * bs;
    for (int b = 0; b < B; ++b) {
        if (tree_err[b] != 0) continue;
        const int32_t P = prefix_len[b];
        int ok = P >= 0 && P <= max_prefix_len && (int64_t)P + T <= cap;
        for (int i = 0; ok && i < T; ++i)
            if (cache_row(table, bs, max_blocks, block_stride, head_stride, row_stride, num_blocks,
                          b, 0, (int64_t)P + i) < 0)
                ok = 0;
        if (!ok) {
            tree_err[b] = 3;
            continue;
        }
        for (int h = 0; h < Hkv; ++h)
            for (int i = 0; i < T; ++i) {
                const int64_t dst = cache_row(table, bs, max_blocks, block_stride, head_stride,
                                              row_stride, num_blocks, b, h, (int64_t)P + i);
                const int64_t src = (((int64_t)b * Hkv + h) * T + i) * D;
                memcpy((char *)k_cache + dst * esz, (const char *)k_tree + src * esz, esz * D);
                memcpy((char *)v_cache + dst * esz, (const char *)v_tree + src * esz, esz * D);
            }
    }
    return 0;
}

/* Compaction: for every sequence b with tree_err[b] == 0 (or tree_err NULL),  */
/* L = accepted_len[b] in [0, T], path nodes in [0, T), P in                   */
/* [0, max_prefix_len] and every position of [P, P + T) with a block-table    */
/* entry in range: the cache row at P + j becomes the row that was at         */
/* P + accepted_nodes[b][j], for j < L (all rows are read before any is       */
/* written), and new_prefix_len[b] = P + L.  Otherwise nothing moves and      */
/* new_prefix_len[b] = P.  Rows from P + L on are left as they are.           */
int oracle_kv_compact(const int32_t *accepted_len, const int32_t *accepted_nodes,
                      const int32_t *tree_err, void *k_cache, void *v_cache, const int32_t *table,
                      int bs, int max_blocks, int64_t block_stride, int64_t head_stride,
                      int64_t row_stride, int64_t num_blocks, int dtype,
                      const int32_t *prefix_len, int max_prefix_len, int32_t *new_prefix_len,
                      int B, int Hkv, int T, int D) {
    if (B < 0 || Hkv < 1 || T < 1 || D < 1 || bs < 1 || max_blocks < 1) return -1;
    const size_t esz = dtype == OR_F32 ? 4 : 2;
    const int64_t cap = (int64_t)max_blocks * bs;
    char *tk = (char *)malloc(esz * (size_t)D * (size_t)T);
    char *tv = (char *)malloc(esz * (size_t)D * (size_t)T);
    if (!tk || !tv) {
        free(tk);
        free(tv);
        return -2;
    }
    for (int b = 0; b < B; ++b) {
        const int32_t P = prefix_len[b];
        const int32_t L = accepted_len[b];
        const int32_t *nodes = accepted_nodes + (int64_t)b * T;
        int ok = !(tree_err && tree_err[b] != 0);
        ok = ok && L >= 0 && L <= T && P >= 0 && P <= max_prefix_len && (int64_t)P + T <= cap;
        for (int j = 0; ok && j < L; ++j)
            if (nodes[j] < 0 || nodes[j] >= T) ok = 0;
        for (int i = 0; ok && i < T; ++i)
            if (cache_row(table, bs, max_blocks, block_stride, head_stride, row_stride, num_blocks,
                          b, 0, (int64_t)P + i) < 0)
                ok = 0;
        if (ok) {
            for (int h = 0; h < Hkv; ++h) {
                for (int j = 0; j < L; ++j) { /* read every source row first */
                    const int64_t src = cache_row(table, bs, max_blocks, block_stride, head_stride,
                                                  row_stride, num_blocks, b, h,
                                                  (int64_t)P + nodes[j]);
                    memcpy(tk + (size_t)j * D * esz, (const char *)k_cache + src * esz, esz * D);
                    memcpy(tv + (size_t)j * D * esz, (const char *)v_cache + src * esz, esz * D);
                }
                for (int j = 0; j < L; ++j) {
                    const int64_t dst = cache_row(table, bs, max_blocks, block_stride, head_stride,
                                                  row_stride, num_blocks, b, h, (int64_t)P + j);
                    memcpy((char *)k_cache + dst * esz, tk + (size_t)j * D * esz, esz * D);
                    memcpy((char *)v_cache + dst * esz, tv + (size_t)j * D * esz, esz * D);
                }
            }
        }
        if (new_prefix_len) new_prefix_len[b] = ok ? P + L : P;
    }
    free(tk);
    free(tv);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Top-K of a log-softmax row ([ADR] row E4b.10a: log_softmax of the row,   */
/* the K largest log-probabilities with the smaller token winning ties, and  */
/* the choice made on the unclamped values).  With l(y) = logit_at(row, y)   */
/* (NaN and -inf: -inf; +inf: the largest finite float), m = max_y l(y) and  */
/* Z = sum over finite l(y) of exp(l(y) - m):                                 */
/*   logp(y) = (l(y) - m) - log Z,  -inf where l(y) = -inf (and everywhere   */
/*   when the row has no finite entry).                                       */
/* logp increases strictly with l, so the K largest log-probabilities are     */
/* found by comparing l itself, which no rounding can merge: K times, the     */
/* token not chosen yet with the largest l, the smaller token on a tie.       */
/* Outputs are in that order (best first).                                    */
static void topk_row(const float *row, int64_t V, int K, int32_t *tok, double *logp,
                     unsigned char *taken) {
    double m = -INFINITY;
    for (int64_t y = 0; y < V; ++y) {
        const double l = logit_at(row, y);
        if (l > m) m = l;
    }
    double Z = 0.0;
    for (int64_t y = 0; y < V; ++y) {
        const double l = logit_at(row, y);
        if (l > -INFINITY) Z += exp(l - m);
    }
    memset(taken, 0, (size_t)V);
    for (int k = 0; k < K; ++k) {
        int64_t best = -1;
        double bl = 0.0;
        for (int64_t y = 0; y < V; ++y) {
            if (taken[y]) continue;
            const double l = logit_at(row, y);
            if (best < 0 || l > bl) {
                best = y;
                bl = l;
            }
        }
        taken[best] = 1;
        tok[k] = (int32_t)best;
        logp[k] = (bl == -INFINITY || Z == 0.0) ? -INFINITY : (bl - m) - log(Z);
    }
}

int oracle_topk_logprobs(const float *logits, int64_t R, int64_t V, int K, int32_t *tok,
                         double *logp, int nthreads) {
    if (R < 0 || V < 1 || K < 1 || (int64_t)K > V) return -1;
    if (nthreads > 0) omp_set_num_threads(nthreads);
    int fail = 0;
#pragma omp parallel
    {
        unsigned char *taken = (unsigned char *)malloc((size_t)V);
        if (!taken) {
#pragma omp atomic write
            fail = 1;
        }
#pragma omp for schedule(dynamic)
        for (int64_t r = 0; r < R; ++r)
            if (taken) topk_row(logits + r * V, V, K, tok + r * K, logp + r * K, taken);
        free(taken);
    }
    return fail ? -2 : 0;
}

/* ------------------------------------------------------------------------ */
/* EAGLE-2 global best-first tree expansion ([ADR] row E4a: one queue of     */
/* pending candidates keyed by the fp64 cumulative log-probability, admitted */
/* one node at a time, so that a grandchild of A can beat a sibling of A;     */
/* section 4 Phase E4: expand by cumulative log-probability until the node   */
/* budget is reached; [HEADS] "Mechanism comparison", EAGLE-2's dynamic      */
/* tree).  Per sequence b:                                                    */
/*   node 0 is the root: token root_token[b], cumulative log-prob 0, level 1. */
/*   Admitting node i runs the drafter on it.  The synthetic drafter's output */
/*   for the node admitted i-th is row i of drafter_logits[b]; its top-K     */
/*   (topk_row) offers K candidate children (token, key cum(i) + logp), best */
/*   first.  A node on level max_levels offers none, and neither does the    */
/*   node that completes the tree (so row T-1 is never read).                 */
/*   The pending candidate with the largest key is admitted next as node n:   */
/*   parent, token, cum(n) = key, level = parent's level + 1.  Ties go to the */
/*   candidate offered first (earlier parent, then better rank).             */
/*   Expansion stops at T nodes.                                              */
/* T must not exceed the nodes of a full K-ary tree of max_levels levels; the */
/* queue then never runs dry.                                                 */
int oracle_draft_tree(const float *drafter_logits, const int32_t *root_token, int B, int T,
                      int64_t V, int K, int max_levels, int32_t *parents, int32_t *tokens,
                      double *cum) {
    if (B < 0 || T < 1 || V < 1 || K < 1 || (int64_t)K > V || max_levels < 1) return -1;
    /* capacity: 1 + K + K^2 + ... over max_levels levels */
    int64_t cap = 0, width = 1;
    for (int lv = 0; lv < max_levels && cap < T; ++lv) {
        cap += width;
        width = width * K > T ? T : width * K;
    }
    if (cap < T) return -1;
    const int64_t np = (int64_t)T * K;
    double *ckey = (double *)malloc(sizeof(double) * (size_t)np);
    int32_t *cpar = (int32_t *)malloc(sizeof(int32_t) * (size_t)np);
    int32_t *ctok = (int32_t *)malloc(sizeof(int32_t) * (size_t)np);
    unsigned char *used = (unsigned char *)malloc((size_t)np);
    int32_t *level = (int32_t *)malloc(sizeof(int32_t) * (size_t)T);
    int32_t *ktok = (int32_t *)malloc(sizeof(int32_t) * (size_t)K);
    double *klp = (double *)malloc(sizeof(double) * (size_t)K);
    unsigned char *taken = (unsigned char *)malloc((size_t)V);
    int rc = 0;
    if (!ckey || !cpar || !ctok || !used || !level || !ktok || !klp || !taken) rc = -2;
    for (int b = 0; b < B && rc == 0; ++b) {
        const float *rows = drafter_logits + (int64_t)b * T * V;
        int32_t *par = parents + (int64_t)b * T;
        int32_t *tk = tokens + (int64_t)b * T;
        double *cm = cum + (int64_t)b * T;
        int64_t npend = 0;
        int n = 1;
        par[0] = -1;
        tk[0] = root_token[b];
        cm[0] = 0.0;
        level[0] = 1;
        int last = 0; /* the node admitted last, to be offered next */
        for (;;) {
            if (n < T && level[last] < max_levels) { /* the drafter runs on node `last` */
                topk_row(rows + (int64_t)last * V, V, K, ktok, klp, taken);
                for (int r = 0; r < K; ++r) {
                    ckey[npend] = cm[last] + klp[r];
                    cpar[npend] = last;
                    ctok[npend] = ktok[r];
                    used[npend] = 0;
                    ++npend;
                }
            }
            if (n == T) break;
            int64_t best = -1;
            for (int64_t q = 0; q < npend; ++q)
                if (!used[q] && (best < 0 || ckey[q] > ckey[best])) best = q;
            if (best < 0) {
                rc = -3;
                break;
            }
            used[best] = 1;
            par[n] = cpar[best];
            tk[n] = ctok[best];
            cm[n] = ckey[best];
            level[n] = level[cpar[best]] + 1;
            last = n++;
        }
    }
    free(ckey); free(cpar); free(ctok); free(used); free(level); free(ktok); free(klp); free(taken);
    return rc;
}
