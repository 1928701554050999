// sv_internal.h -- shared declarations of the gfx950 kernels behind include/sv.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sv.h"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kNumCU = 256;     // MI355X compute units (8 XCDs x 32)
constexpr int kNumXCD = 8;
constexpr int kKeyTile = 32;    // keys per attention tile; split sizes are multiples of it
constexpr int kMinChunk = 64;   // fewest prefix keys per chunk under automatic splitting
constexpr int kAttnMaxWaves = 8;  // wavefronts per attention workgroup

// Paged cache as seen by a kernel (element strides).
struct CacheView {
    const void *k;
    const void *v;
    const int32_t *table;
    int32_t bs;
    int32_t max_blocks;
    int64_t num_blocks;
    int64_t bstride;
    int64_t hstride;
    int64_t rstride;
};

// How one attention call is cut into workgroups.
struct AttnPlan {
    int mfma;          // 1: matrix-core kernel (bf16); 0: vector-ALU kernel (fp32)
    int R;             // query rows per kv head = (Hq / Hkv) * T, row r = g * T + i
    int rows_per_wg;   // rows one workgroup owns
    int n_rg;          // row groups per kv head
    int nthreads;      // threads per workgroup
    int S;             // prefix chunks (splits) per sequence, at most
    int C;             // keys per chunk, multiple of kKeyTile (unless balanced)
    int balanced;      // 1: the kernel sizes chunks from the actual prefix lengths and
                       // starts the largest first (attn_w4 kernel, B * S <= kBalancedChunks)
    int fused;         // 1: the attention kernel merges the chunks itself (attn_w4 and
                       // fp32 kernels, at most kMaxMergeUnits (sequence, kv head, row
                       // group) units); 0: the separate merge kernel does
    // Workspace layout: [arrival counters][header][partial (m, l)][partial O].  The
    // counters sit at offset 0 in a region of fixed size, so that they stay where they
    // were whatever the shapes of earlier calls on the same workspace.
    size_t ws_ml;      // bytes of partial (m, l)   [B][Hkv][S][R][2] fp32
    size_t ws_o;       // bytes of partial outputs  [B][Hkv][S][R][D] fp32
    size_t ws_total;
};

// Arrival counters of the in-kernel merge: int32 per (sequence, kv head, row group), in
// the first kCounterBytes of the workspace, zero before a call and zero after it.
constexpr size_t kCounterBytes = 256 * 1024;
constexpr int64_t kMaxMergeUnits = kCounterBytes / 4;
constexpr size_t kHeaderBytes = 256;  // the chunk length a balanced call chose
// Scratch of the allocation-free attention entry point, per device (counters included).
constexpr size_t kScratchBytes = (size_t)64 << 20;

// The most (sequence, chunk) pairs that a balanced call ranks by size.
constexpr int kBalancedChunks = 128;

struct AttnArgs {
    const void *q;
    const void *k_tree;
    const void *v_tree;
    CacheView cache;
    const int32_t *prefix_len;
    int32_t max_prefix_len;
    const uint64_t *mask;
    int32_t B, Hq, Hkv, T, D;
    float scale;
    float *out;
    float *ws_o;
    float *ws_ml;
    int32_t *ws_c;     // header: the chunk length of a balanced call
    int32_t *ws_cnt;   // arrival counters of the in-kernel merge
};

// Returns 0 and fills *p, or a negative sv_status for unsupported shapes.
int make_attn_plan(int B, int Hq, int Hkv, int T, int D, int max_prefix_len, int dtype,
                   int num_splits, AttnPlan *p);

hipError_t launch_tree_mask(const int32_t *parents, int B, int T, uint64_t *mask,
                            int32_t *depth, int32_t *tree_err, hipStream_t stream);
// Whether launch_attn_mfma runs the four-wavefront kernel (attn_w4) at this head_dim.
bool attn_w4_handles(int D);
hipError_t launch_attn_mfma(const AttnArgs &a, const AttnPlan &p, hipStream_t stream);
// head_dim 128 and 256, one wavefront per SIMD (called by launch_attn_mfma)
hipError_t launch_attn_w4(const AttnArgs &a, const AttnPlan &p, hipStream_t stream);
hipError_t launch_attn_valu(const AttnArgs &a, const AttnPlan &p, int dtype,
                            hipStream_t stream);
hipError_t launch_attn_reduce(const AttnArgs &a, const AttnPlan &p, hipStream_t stream);

// Vocab argmax in chunks: partial (value, index) pairs [rows][chunks].
struct ArgmaxPlan {
    int64_t chunk;     // elements per chunk
    int nchunks;       // chunks per row
    size_t ws_bytes;
};
int make_argmax_plan(int64_t rows, int64_t V, ArgmaxPlan *p);
hipError_t launch_argmax_partial(const float *logits, int64_t rows, int64_t V,
                                 const ArgmaxPlan &p, void *ws, hipStream_t stream);
hipError_t launch_accept(const void *ws, const ArgmaxPlan &p, const int32_t *draft,
                         const int32_t *parents, const int32_t *tree_err, int B, int T,
                         int32_t *argmax_out, int32_t *accepted_len, int32_t *accepted_nodes,
                         int32_t *out_tokens, hipStream_t stream);

// Sampled acceptance: per-chunk (max, sum) pairs [rows][chunks] in the workspace.
int make_sample_plan(int64_t rows, int64_t V, ArgmaxPlan *p);
hipError_t launch_accept_sampled(const float *logits, const int32_t *draft,
                                 const int32_t *parents, const int32_t *tree_err,
                                 const float *u_accept, const float *u_sample, float temperature,
                                 int B, int T, int64_t V, const ArgmaxPlan &p, void *ws,
                                 int32_t *accepted_len, int32_t *accepted_nodes,
                                 int32_t *out_tokens, hipStream_t stream);

hipError_t launch_rope_tree(void *q, void *k_tree, const int32_t *prefix_len,
                            const int32_t *depth, int B, int Hq, int Hkv, int T, int D, int dtype,
                            double theta, hipStream_t stream);

// Top-K of the log-softmax of rows: row r of the call reads logits row
// (r / rows_per_group) * group_stride + r % rows_per_group and writes [r][K].
hipError_t launch_topk_rows(const float *logits, int64_t rows, int64_t V, int K,
                            int rows_per_group, int64_t group_stride, int32_t *top_tok,
                            double *top_logp, hipStream_t stream);
// Best-first expansion from the top-K lists [B][T - 1][K] of each sequence's rows.
hipError_t launch_best_first(const int32_t *top_tok, const double *top_logp,
                             const int32_t *root_token, int B, int T, int K, int max_levels,
                             int32_t *parents, int32_t *tokens, double *cum, hipStream_t stream);

// The write-before-accept variant: tree rows into the cache at [P, P + T), then the
// accepted path compacted to [P, P + L).
hipError_t launch_kv_append(const void *k_tree, const void *v_tree, int32_t *tree_err,
                            void *k_cache, void *v_cache, const CacheView &c,
                            const int32_t *prefix_len, int32_t max_prefix_len, int B, int Hkv,
                            int T, int D, int esize, hipStream_t stream);
hipError_t launch_kv_compact(const int32_t *accepted_len, const int32_t *accepted_nodes,
                             const int32_t *tree_err, void *k_cache, void *v_cache,
                             const CacheView &c, const int32_t *prefix_len,
                             int32_t max_prefix_len, int32_t *new_prefix_len, int B, int Hkv,
                             int T, int D, int esize, hipStream_t stream);

hipError_t launch_kv_commit(const void *k_tree, const void *v_tree, const int32_t *accepted_len,
                            const int32_t *accepted_nodes, const int32_t *tree_err,
                            void *k_cache, void *v_cache, const CacheView &c,
                            const int32_t *prefix_len, int32_t max_prefix_len,
                            int32_t *new_prefix_len, int B, int Hkv, int T, int D, int esize,
                            hipStream_t stream);

}  // namespace sv
