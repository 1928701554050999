/*
 * sv.h -- C ABI of the tree-masked speculative verify library (libsv.so, gfx950).
 *
 * One verify step of speculative decoding, for a batch of B independent
 * sequences that each carry a draft token tree of T nodes:
 *
 *   1. sv_build_tree_mask        parent array -> ancestor-and-self bitmask
 *   2. sv_tree_verify_attention  tree rows attend to the cached prefix plus their
 *                                ancestors (split-KV, GQA, log-sum-exp merge)
 *   3. sv_accept_longest_path    vocab argmax per row -> longest matching root path
 *                                -> accepted nodes and emitted tokens
 *      (or sv_accept_sampled      target softmax per row -> proposals accepted with
 *                                their target probability, emitted token drawn)
 *   sv_rope_tree (before 2, when the caller's Q and tree keys are not yet rotated):
 *                                rotary embedding at base position + tree depth
 *   4. sv_kv_commit              copy only the accepted rows' K/V into the cache
 *
 * Write-before-accept variant: sv_kv_append puts the tree's K/V rows into the cache
 * before step 2, sv_tree_verify_attention then reads them there (NULL tree buffers),
 * and sv_kv_compact replaces step 4.
 *
 * Before the step, sv_draft_tree builds the draft tree itself from the drafter's
 * logits (top-K of each row's log-softmax, then EAGLE-2 global best-first
 * expansion); sv_topk_logprobs is its top-K on its own.
 *
 * Sources (web pages, by title and section):
 *   "ADR-037 -- EAGLE-3 with dynamic tree port" (hf2q docs): Phase status rows
 *     E1.1-E1.5 (tree attention; output layout [q_seq_len, num_heads, head_dim];
 *     head_dim 256/512), E4b.6 (the head_dim-128 retrofit of the tree attention),
 *     E1 review gate (dtype and byte-length validation), E4a
 *     (build_tree_mask from the parent array, checked overflow; best-first tree
 *     expansion), E4b.5b (tree-position RoPE), E4b.10a (top-K extraction), E5a
 *     (tree-walk accept), E5b (rollback to the accepted path), E6 (zero-head guard
 *     before the GQA modulo; the per-layer block that appends the tree's K/V to the
 *     cache before the attention), E6 v2 (ancestors + self); section 4, Phases E1,
 *     E4 and E5.
 *   "Speculative-decoding heads: Medusa + EAGLE-2" (posttrainllm docs): "Why
 *     bother" (greedy longest-matching-prefix verification), "Mechanism
 *     comparison" (EAGLE-2's dynamic tree) and "What's not implemented" item 1
 *     (ancestor-only tree attention, per-path argmax).
 *   "Speculative decoding verify batches to amortize ANE dispatch"
 *     (llms-explorer): Facts on the commit rule, on delayed KV write-through and on
 *     Forge's sampled verification.
 *
 * Conventions shared by every entry point:
 *   - Every data pointer is device memory owned by the caller.  The library
 *     allocates nothing, keeps no state between calls and never synchronises
 *     the stream.
 *   - Work is enqueued on `stream` (0 = the null stream) and runs in stream order.
 *   - Host-checkable argument errors return a negative sv_status before anything
 *     is enqueued; then no output is written.  SV_ERR_HIP reports a failed
 *     launch (hipGetLastError after the launch).
 *   - Data-dependent problems found on the device (a malformed parent array, an
 *     out-of-range block-table entry) never fault: they are reported through
 *     tree_err or handled as documented per function.
 *   - Integers are little-endian int32 unless stated; bf16 is stored as its
 *     16-bit pattern.
 */
#ifndef SV_H
#define SV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sv_status {
    SV_OK = 0,
    SV_ERR_NULL = -1,       /* a required pointer is NULL */
    SV_ERR_SHAPE = -2,      /* a size is negative/zero where not allowed, or inconsistent */
    SV_ERR_DTYPE = -3,      /* unknown dtype, or dtype not supported for this call */
    SV_ERR_GQA = -4,        /* Hkv <= 0, Hq <= 0 or Hq not a multiple of Hkv */
    SV_ERR_HEAD_DIM = -5,   /* head_dim not 128, 256 or 512 */
    SV_ERR_TREE_SIZE = -6,  /* T outside [1, 64] */
    SV_ERR_CAPACITY = -7,   /* max_prefix_len + T exceeds the rows the block table reserves */
    SV_ERR_OVERFLOW = -8,   /* a byte size does not fit in 64 bits / an index in 32 bits */
    SV_ERR_WORKSPACE = -9,  /* workspace NULL or smaller than the *_workspace_size result */
    SV_ERR_HIP = -10,       /* the HIP runtime reported an error */
    SV_ERR_ALIGN = -11,     /* a pointer or stride is not 16-byte aligned */
    SV_ERR_SCRATCH = -12    /* needs more scratch than the allocation-free entry point holds */
} sv_status;

typedef enum sv_dtype { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

/* Per-sequence tree status in tree_err[b]: written by sv_build_tree_mask, and set to
 * SV_TREE_NOT_APPENDED by sv_kv_append; every call that reads tree_err skips a sequence
 * whose status is not SV_TREE_OK. */
enum {
    SV_TREE_OK = 0,
    SV_TREE_BAD_ROOT = 1,
    SV_TREE_BAD_PARENT = 2,
    SV_TREE_NOT_APPENDED = 3  /* sv_kv_append could not place the tree rows in the cache */
};

/*
 * KV cache descriptor: one layout for contiguous and paged caches.
 *   Row `pos` of sequence b, kv head h starts at element
 *     block_table[b * max_blocks_per_seq + pos / block_size] * block_stride
 *       + h * head_stride + (pos % block_size) * row_stride
 *   of the K pool (and the same offset in the V pool); a row holds head_dim
 *   contiguous elements of `dtype`.
 *   Paged   [num_blocks][Hkv][block_size][D]: block_stride = Hkv*bs*D,
 *           head_stride = bs*D, row_stride = D.
 *   Contiguous [B][Hkv][cap][D]: block_size = cap, max_blocks_per_seq = 1,
 *           block_table[b] = b, same stride formulas.
 * Requirements: block_size a positive multiple of 16; strides multiples of 8
 * elements (16 bytes); k, v 16-byte aligned.  Block-table entries outside
 * [0, num_blocks) are never dereferenced (see each call).
 */
typedef struct sv_kv_cache {
    void *k;                     /* K pool, device */
    void *v;                     /* V pool, device */
    const int32_t *block_table;  /* [B][max_blocks_per_seq], device */
    int32_t block_size;          /* rows per block */
    int32_t max_blocks_per_seq;  /* row length of block_table */
    int64_t num_blocks;          /* blocks in each pool */
    int64_t block_stride;        /* elements */
    int64_t head_stride;         /* elements */
    int64_t row_stride;          /* elements */
    int32_t dtype;               /* sv_dtype; must equal the Q/K/V dtype */
} sv_kv_cache;

/*
 * Ancestor-and-self mask of each sequence's draft tree.
 * Defined by: ADR-037 Phase status rows E4a (build_tree_mask) and E6 v2
 * (ancestors + self); Medusa/EAGLE-2 page, "What's not implemented" 1(c).
 *
 *   parents  int32 [B][T]  node 0 is the root (parent -1); 0 <= parents[i] < i
 *   mask     uint64 [B][T][W], W = ceil(T/64) (= 1 since T <= 64): bit j of
 *            row i is set iff node j is node i or an ancestor of node i
 *   depth    int32 [B][T] or NULL: number of proper ancestors (root 0)
 *   tree_err int32 [B]: SV_TREE_OK, SV_TREE_BAD_ROOT (parents[0] != -1) or
 *            SV_TREE_BAD_PARENT (some parents[i] outside [0, i)).  A bad tree's
 *            rows are self-only with depth 0.
 * Errors: SV_ERR_NULL (parents, mask, tree_err), SV_ERR_SHAPE (B < 0),
 *         SV_ERR_TREE_SIZE (T outside [1, 64]), SV_ERR_HIP.
 */
int sv_build_tree_mask(const int32_t *parents, int32_t B, int32_t T, uint64_t *mask,
                       int32_t *depth, int32_t *tree_err, hipStream_t stream);

/*
 * Bytes of workspace sv_tree_verify_attention needs for this shape and split
 * count (num_splits 0 = automatic).  Returns 0 when the arguments would be
 * rejected by sv_tree_verify_attention's shape checks.
 */
size_t sv_tree_verify_attention_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t T,
                                               int32_t D, int32_t max_prefix_len, int32_t dtype,
                                               int32_t num_splits);

/*
 * Tree-masked attention of every tree node's query over its sequence's cached
 * prefix and its own ancestors plus itself.
 * Defined by: ADR-037 Phase status rows E1.1-E1.5 and section 4 Phase E1
 * (tree mask; tree = 1 equals decode, a chain equals causal attention);
 * Medusa/EAGLE-2 page "What's not implemented" 1(c).
 *
 * For query head h (kv head h / (Hq/Hkv)), node i of sequence b:
 *   keys  = cache rows 0 .. P_b-1 of that kv head, then tree rows j with bit j of
 *           mask[b][i] set;  P_b = prefix_len[b] clamped into [0, max_prefix_len]
 *   out[b][i][h][:] = softmax(scale * q . k) weighted sum of the matching values
 *   q       [B][Hq][T][D]   dtype (SV_BF16, or SV_F32)
 *   k_tree, v_tree [B][Hkv][T][D]  the tree nodes' own K/V (not yet in the cache),
 *           or both NULL when the tree rows are already in the cache (sv_kv_append):
 *           tree row j is then the cache row at position P_b + j (a row whose
 *           block-table entry is out of range is read from block 0 instead: its
 *           sequence was refused by sv_kv_append and marked in tree_err)
 *   cache   prefix K/V; cache->dtype must equal the Q/K/V dtype
 *   prefix_len int32 [B] device; max_prefix_len host upper bound of prefix_len
 *   mask    from sv_build_tree_mask
 *   out     float32 [B][T][Hq][D]   (layout [q_seq_len, num_heads, head_dim] per sequence)
 *   scale   softmax scale, usually 1/sqrt(D); must be positive and finite
 *   workspace  device, >= sv_tree_verify_attention_workspace_size(...) bytes,
 *              256-byte aligned; scratch for per-split partial results.  Its first
 *              256 KiB hold arrival counters of the chunk merge: they must be zero
 *              before the first call on a workspace (allocate it zero-filled, or clear
 *              it once), and every call leaves them zero again.  Do not write that
 *              region between calls; calls that share a workspace must not overlap
 *              in time (same stream, or ordered).
 *   num_splits 0 = automatic; otherwise the number of prefix chunks per sequence.
 *              Automatic splitting at head_dim 128 / 256 with bf16 may size the chunks
 *              from prefix_len on the device (so that sequences of different lengths
 *              share the CUs evenly); the result then depends on every sequence's
 *              length only through rounding of the chunked sums.
 * Arithmetic: bf16 (or fp32) operands, fp32 accumulation; the result matches
 * the exact softmax attention to within bf16 rounding of the probabilities.
 * Prefix rows whose block-table entry is outside [0, num_blocks) are left out.
 * Non-finite values: q, k_tree, v_tree and the cache rows a row attends to must be
 * finite (every tree row is attended to by its own node).  Anything else the cache
 * holds -- rows at positions >= P_b, blocks the table does not reach, the block an
 * out-of-range entry would have named -- may be anything, NaN included, without
 * affecting any output.  A non-finite value in an attended row gives an
 * unspecified (typically NaN) output for the rows that attend to it, and, on the
 * matrix-core paths (every bf16 call), possibly for the other rows of the same
 * sequence and kv head (0 * inf in the weighted sum).
 * Errors: SV_ERR_NULL, SV_ERR_SHAPE (B < 0, max_prefix_len < 0, block_size not a
 * positive multiple of 16, num_splits < 0, strides not positive, scale not
 * positive and finite),
 * SV_ERR_GQA, SV_ERR_HEAD_DIM, SV_ERR_TREE_SIZE, SV_ERR_DTYPE, SV_ERR_CAPACITY
 * (max_prefix_len + T > max_blocks_per_seq * block_size), SV_ERR_ALIGN,
 * SV_ERR_OVERFLOW, SV_ERR_WORKSPACE, SV_ERR_HIP.
 */
int sv_tree_verify_attention(const void *q, const void *k_tree, const void *v_tree,
                             const sv_kv_cache *cache, const int32_t *prefix_len,
                             int32_t max_prefix_len, const uint64_t *mask, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t T, int32_t D, float scale, float *out,
                             void *workspace, size_t workspace_bytes, int32_t num_splits,
                             hipStream_t stream);

/*
 * sv_tree_verify_attention without a workspace argument, for callers that cannot
 * allocate device memory around the call (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, results and errors as
 * sv_tree_verify_attention; its scratch is a 64 MiB array in the library's code object,
 * one per device, held until the process ends.  The call allocates nothing.
 *   - A call whose workspace_size would exceed 64 MiB returns SV_ERR_SCRATCH before
 *     anything is enqueued (the 32K-prefix batch of 16 x 8 kv heads needs ~61 MiB).
 *   - The first call on a device looks the array up and enqueues a small fill kernel on
 *     `stream` that clears its arrival counters (the only part that must start at zero;
 *     every call leaves them zero again).
 *   - All calls on one device share that device's array, which keeps the last call's
 *     contents: calls that overlap in time on one device (different streams, or host
 *     threads, without ordering) race and give unspecified results.
 * Errors: those of sv_tree_verify_attention except SV_ERR_WORKSPACE; SV_ERR_SCRATCH;
 * SV_ERR_HIP also when the array's device address cannot be obtained.
 */
int sv_tree_verify_attention_noalloc(const void *q, const void *k_tree, const void *v_tree,
                                     const sv_kv_cache *cache, const int32_t *prefix_len,
                                     int32_t max_prefix_len, const uint64_t *mask, int32_t B,
                                     int32_t Hq, int32_t Hkv, int32_t T, int32_t D, float scale,
                                     float *out, int32_t num_splits, hipStream_t stream);

/* Bytes of workspace sv_accept_longest_path needs (0 when the shape is invalid). */
size_t sv_accept_longest_path_workspace_size(int32_t B, int32_t T, int64_t V);

/*
 * Greedy acceptance.
 * Defined by: llms-explorer page Facts, commit rule (the target's argmax at each
 * draft row decides; longest matching prefix plus one bonus token); ADR-037 Phase
 * status row E5a and section 4 Phase E5 (longest matching path from the root;
 * full accept picks the deepest); row E4b.10a (smaller token wins ties);
 * Medusa/EAGLE-2 page "Why bother".
 *
 *   logits  float32 [B][T][V]; a[b][i] = smallest index of the row maximum, NaN
 *           never wins, an all-NaN row gives 0
 *   draft   int32 [B][T]: draft[b][i] is node i's token (draft[b][0] unused)
 *   parents int32 [B][T] (as for sv_build_tree_mask)
 *   tree_err int32 [B] or NULL: a non-zero entry (or a malformed parent array)
 *           makes that sequence accept nothing
 *   argmax_out int32 [B][T] or NULL: a[][]
 *   accepted_len int32 [B]: L = depth of the accepted node + 1 (0 if invalid)
 *   accepted_nodes int32 [B][T]: the path root..accepted node, then -1
 *   out_tokens int32 [B][T]: a[] along the path (L-1 accepted drafts + 1 bonus
 *           token), then -1
 * Node i >= 1 matches when its parent matches and draft[b][i] == a[b][parent];
 * the accepted node is the deepest matching node, the smallest index among equals.
 * Errors: SV_ERR_NULL, SV_ERR_SHAPE (B < 0, V < 1), SV_ERR_TREE_SIZE,
 * SV_ERR_OVERFLOW, SV_ERR_WORKSPACE, SV_ERR_HIP.
 */
int sv_accept_longest_path(const float *logits, const int32_t *draft, const int32_t *parents,
                           const int32_t *tree_err, int32_t B, int32_t T, int64_t V,
                           int32_t *argmax_out, int32_t *accepted_len, int32_t *accepted_nodes,
                           int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/* Bytes of workspace sv_accept_sampled needs (0 when the shape is invalid). */
size_t sv_accept_sampled_workspace_size(int32_t B, int32_t T, int64_t V);

/*
 * Sampled acceptance (temperature > 0), an alternative to sv_accept_longest_path
 * with the same outputs, for sv_kv_commit to consume.
 * Defined by: llms-explorer page Facts on Forge's sampled verification (the drafted
 * path is treated as given; a proposal is accepted with its target probability; on
 * rejection the target distribution is sampled with that proposal excluded, which
 * keeps the target distribution).  The pages state the rule for one proposal; for a
 * tree the children of a node are tried one after another as proposals from what is
 * left.
 *
 *   logits  float32 [B][T][V]; row v gives node v's target distribution
 *           p_v(x) = exp(l_v(x) / temperature) / sum_y exp(l_v(y) / temperature)
 *           (NaN and -inf entries have probability 0, +inf counts as FLT_MAX; a row
 *           without a finite entry has probability 0 everywhere)
 *   draft, parents, tree_err: as for sv_accept_longest_path
 *   u_accept float32 [B][T] in [0, 1): the draw for trying node c as a proposal
 *   u_sample float32 [B][T] in [0, 1): the draw for the emitted token at node v
 *           (the caller draws both; the library draws no random numbers)
 *   temperature > 0 and finite
 *   accepted_len, accepted_nodes, out_tokens: as for sv_accept_longest_path
 * Walk: start at the root.  At the current node v the children are tried in
 * increasing node index; with E the tokens rejected so far at v and
 * R = 1 - sum_{x in E} p_v(x), child c with token x is accepted when
 * u_accept[b][c] * R < p_v(x) (p = 0 for x in E or outside [0, V)) and becomes the
 * current node; a rejected token joins E.  When no child is accepted (or v is a
 * leaf) the emitted token is the smallest y not in E whose cumulative probability
 * over tokens not in E exceeds u_sample[b][v] * R (token 0 when no probability is
 * left).  out_tokens: the accepted children's draft tokens, then the emitted token.
 * Precision: fp32 (the row sums in chunks); a decision within a few 1e-7 of its
 * boundary can go either way, compared with an exact evaluation.
 * Errors: SV_ERR_NULL, SV_ERR_SHAPE (B < 0, V < 1, temperature not positive and
 * finite), SV_ERR_TREE_SIZE, SV_ERR_OVERFLOW, SV_ERR_WORKSPACE, SV_ERR_ALIGN,
 * SV_ERR_HIP.
 */
int sv_accept_sampled(const float *logits, const int32_t *draft, const int32_t *parents,
                      const int32_t *tree_err, const float *u_accept, const float *u_sample,
                      float temperature, int32_t B, int32_t T, int64_t V, int32_t *accepted_len,
                      int32_t *accepted_nodes, int32_t *out_tokens, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * Tree-position rotary embedding of the queries and tree keys, in place.
 * Defined by: ADR-037 Phase status row E4b.5b (RoPE on Q/K with tree positions
 * base position + tree depth, NeoX style, the rotation covers the whole head; rope
 * theta finite, head_dim even).
 *
 *   q       [B][Hq][T][D], k_tree [B][Hkv][T][D], float32 or bf16 (dtype), rotated
 *           in place
 *   prefix_len int32 [B]: base position of each sequence's root
 *   depth   int32 [B][T]: tree depth of each node (sv_build_tree_mask's output)
 *   theta   > 0 and finite (e.g. 10000)
 * Node i of sequence b sits at position prefix_len[b] + depth[b][i] (siblings share
 * a position; a chain gets consecutive ones).  For j < D/2, with
 * a = position * theta^(-2j/D):
 *   x[j] <- x[j] cos a - x[j + D/2] sin a,   x[j + D/2] <- x[j + D/2] cos a + x[j] sin a.
 * Angles, their cosines and sines and the rotation are evaluated in fp64 (an angle is
 * within about position * 2^-52 rad of exact, ~5e-7 at 2^31), each result is rounded
 * once to the tensor's type.
 * Errors: SV_ERR_NULL, SV_ERR_SHAPE (B < 0, Hq or Hkv < 1, D odd or outside
 * [2, 1024], theta not positive and finite), SV_ERR_TREE_SIZE, SV_ERR_DTYPE,
 * SV_ERR_OVERFLOW, SV_ERR_ALIGN, SV_ERR_HIP.
 */
int sv_rope_tree(void *q, void *k_tree, const int32_t *prefix_len, const int32_t *depth,
                 int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t D, int32_t dtype,
                 double theta, hipStream_t stream);

/*
 * Write-before-accept variant, step 1: the tree's K/V rows into the cache.
 * Defined by: ADR-037 Phase status row E6, per-layer tree-verify block (K/V
 * appended at [prefix_len, prefix_len + tree_seq_len) before the tree attention,
 * which then reads them from the cache); llms-explorer page Facts on KV
 * write-before-accept (the trade-off against delayed write-through).
 *
 * For every sequence b with tree_err[b] == 0: if prefix_len[b] lies in
 * [0, max_prefix_len] and every position of [P, P + T) has a block-table entry in
 * [0, num_blocks), tree row i of every kv head is copied to position P + i (byte
 * copy); otherwise nothing is written and tree_err[b] becomes
 * SV_TREE_NOT_APPENDED.  Sequences with tree_err[b] != 0 on entry are skipped.
 *   k_tree, v_tree [B][Hkv][T][D] (16-byte aligned), cache dtype
 *   tree_err int32 [B], read and updated (e.g. sv_build_tree_mask's output)
 * Then call sv_tree_verify_attention with k_tree = v_tree = NULL, accept as usual,
 * and sv_kv_compact instead of sv_kv_commit.
 * Errors: as sv_kv_commit (tree_err is required here).
 */
int sv_kv_append(const void *k_tree, const void *v_tree, int32_t *tree_err,
                 const sv_kv_cache *cache, const int32_t *prefix_len, int32_t max_prefix_len,
                 int32_t B, int32_t Hkv, int32_t T, int32_t D, hipStream_t stream);

/*
 * Write-before-accept variant, last step: compact the accepted path over the
 * appended rows.
 * Defined by: ADR-037 section 4 Phase E5 and Phase status row E5b (after the
 * acceptance the cache is rolled back to the accepted path).
 *
 * For every sequence b with tree_err[b] == 0 (or tree_err NULL), L =
 * accepted_len[b] in [0, T], accepted_nodes[b][j] in [0, T) for j < L, prefix_len[b]
 * in [0, max_prefix_len] and every position of [P, P + T) with a block-table entry
 * in range: the cache row at P + j becomes the row that was at
 * P + accepted_nodes[b][j], for j < L and every kv head (all moving rows are read
 * before any is written), and new_prefix_len[b] = P + L.  Otherwise nothing moves
 * and new_prefix_len[b] = P.  Rows from P + L on keep what they held.  With the
 * rows appended by sv_kv_append this leaves the same cache rows [0, P + L) and
 * prefix lengths as sv_kv_commit.  new_prefix_len may be NULL, or may alias
 * prefix_len.
 * Errors: SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_GQA, SV_ERR_TREE_SIZE, SV_ERR_HEAD_DIM,
 * SV_ERR_DTYPE, SV_ERR_CAPACITY, SV_ERR_ALIGN, SV_ERR_OVERFLOW, SV_ERR_HIP.
 */
int sv_kv_compact(const int32_t *accepted_len, const int32_t *accepted_nodes,
                  const int32_t *tree_err, const sv_kv_cache *cache, const int32_t *prefix_len,
                  int32_t max_prefix_len, int32_t *new_prefix_len, int32_t B, int32_t Hkv,
                  int32_t T, int32_t D, hipStream_t stream);

/*
 * Top-K of the log-softmax of each row.
 * Defined by: ADR-037 Phase status row E4b.10a (log_softmax of the row, the K
 * largest log-probabilities, the smaller token winning ties, the choice made on
 * unclamped values).
 *
 *   logits     float32 [R][V] (4-byte aligned)
 *   top_tokens int32 [R][K], top_logp float64 [R][K] (8-byte aligned): best first
 * With l(y) the logit (NaN and -inf read as -inf, +inf as FLT_MAX), m = max l and
 * Z = sum over finite l of exp(l - m): logp(y) = (l(y) - m) - log Z, evaluated in
 * fp64 (-inf where l is -inf, and for every token of a row without a finite
 * entry).  The K tokens are chosen by comparing l itself (logp increases strictly
 * with l), ties to the smaller token, so the tokens are exact; the log-probs
 * agree with an exact evaluation to about 1e-15 relative.
 * 1 <= K <= min(V, 64).  R = 0 is a no-op.
 * Errors: SV_ERR_NULL, SV_ERR_SHAPE (R < 0, V < 1, K out of range),
 * SV_ERR_OVERFLOW (V or R above INT_MAX), SV_ERR_ALIGN, SV_ERR_HIP.
 */

int sv_topk_logprobs(const float *logits, int64_t R, int64_t V, int32_t K, int32_t *top_tokens,
                     double *top_logp, hipStream_t stream);

/* Bytes of workspace sv_draft_tree needs (0 when the shape is invalid). */
size_t sv_draft_tree_workspace_size(int32_t B, int32_t T, int32_t K);

/*
 * Draft tree by EAGLE-2 global best-first expansion, from the drafter's logits.
 * Defined by: ADR-037 Phase status row E4a (one queue of pending candidates keyed
 * by the fp64 cumulative log-probability, admitted one node at a time, so that a
 * grandchild of A can come before a sibling of A), row E4b.10a (the top-K of each
 * drafter row), section 4 Phase E4 (expand by cumulative log-probability until the
 * node budget is reached); "Speculative-decoding heads: Medusa + EAGLE-2",
 * "Mechanism comparison" (EAGLE-2's dynamic candidate tree).
 *
 *   drafter_logits float32 [B][T][V]: row i of sequence b is the drafter's output
 *              for the node admitted i-th (row T-1 is never read)
 *   root_token int32 [B]: token of node 0 (the last committed token)
 *   K          candidates offered per expanded node, 1 <= K <= min(V, 64)
 *   max_levels levels of the tree, the root being level 1 (>= 1)
 *   parents    int32 [B][T]: parent of each node (node 0: -1; parent[i] < i)
 *   tokens     int32 [B][T]: draft token of each node (node 0: root_token)
 *   cum_logp   float64 [B][T]: cumulative log-probability of each node (root 0)
 * Node 0 is the root.  Admitting node i offers the K tokens of sv_topk_logprobs on
 * row i as candidate children with key cum_logp[i] + logp, best first, unless node
 * i is on level max_levels or is node T-1.  The pending candidate with the largest
 * key is admitted next, ties to the one offered first (earlier parent, then better
 * rank).  The output feeds sv_build_tree_mask (parents) and the acceptance calls
 * (tokens as draft).  Keys are compared in fp64; two keys within ~1e-15 relative of
 * each other may be ordered differently from an exact evaluation.
 * T must not exceed the nodes of a full K-ary tree of max_levels levels.
 * Errors: SV_ERR_NULL, SV_ERR_SHAPE (B < 0, V < 1, K or max_levels out of range, T
 * above that capacity), SV_ERR_TREE_SIZE (T outside [1, 64]), SV_ERR_OVERFLOW,
 * SV_ERR_WORKSPACE (when T > 1), SV_ERR_ALIGN, SV_ERR_HIP.
 */
int sv_draft_tree(const float *drafter_logits, const int32_t *root_token, int32_t B, int32_t T,
                  int64_t V, int32_t K, int32_t max_levels, int32_t *parents, int32_t *tokens,
                  double *cum_logp, void *workspace, size_t workspace_bytes,
                  hipStream_t stream);

/*
 * Delayed KV write-through: commit only the accepted rows.
 * Defined by: llms-explorer page Facts on Forge's accept(k) (only the accepted
 * prefix reaches the cache; rejected drafts never touch it) and on delayed KV
 * write-through (commit after the acceptance decision).
 *
 * For every sequence b with tree_err[b] == 0 (or tree_err NULL): for
 * j < accepted_len[b] and every kv head, cache row prefix_len[b] + j receives
 * tree row accepted_nodes[b][j] of k_tree and v_tree (byte copy); then
 * new_prefix_len[b] = prefix_len[b] + accepted_len[b].  A sequence whose request
 * cannot be honoured in full (prefix_len[b] outside [0, max_prefix_len],
 * accepted_len outside [0, T], a node index outside [0, T), a block-table entry
 * outside [0, num_blocks)) is left untouched and new_prefix_len[b] =
 * prefix_len[b].  new_prefix_len may be NULL, or may alias prefix_len.
 * Errors: SV_ERR_NULL, SV_ERR_SHAPE, SV_ERR_GQA (Hkv <= 0), SV_ERR_TREE_SIZE,
 * SV_ERR_HEAD_DIM, SV_ERR_DTYPE, SV_ERR_CAPACITY, SV_ERR_ALIGN, SV_ERR_OVERFLOW,
 * SV_ERR_HIP.
 */
int sv_kv_commit(const void *k_tree, const void *v_tree, const int32_t *accepted_len,
                 const int32_t *accepted_nodes, const int32_t *tree_err,
                 const sv_kv_cache *cache, const int32_t *prefix_len, int32_t max_prefix_len,
                 int32_t *new_prefix_len, int32_t B, int32_t Hkv, int32_t T, int32_t D,
                 hipStream_t stream);

/* Static description of a status code (never NULL). */
const char *sv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SV_H */
