// sv_api.hip -- the C ABI of include/sv.h: argument validation, work planning, launches.
//
// Every check that can be made on the host is made before anything is enqueued
// (the pages' validation culture: dtype and buffer-length checks, the zero-head
// guard before the GQA modulo, checked size arithmetic -- ADR-037 Phase status
// rows E1 review gate, E4a and E6).  Sizes are multiplied with overflow checks.
#include <limits.h>

#include <mutex>

#include "sv_internal.h"

namespace sv {
namespace {

bool mul_ok(int64_t a, int64_t b, int64_t *r) { return !__builtin_mul_overflow(a, b, r); }

bool prod_ok(std::initializer_list<int64_t> xs, int64_t *r) {
    int64_t acc = 1;
    for (int64_t x : xs)
        if (!mul_ok(acc, x, &acc)) return false;
    *r = acc;
    return true;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int esize_of(int dtype) { return dtype == SV_BF16 ? 2 : (dtype == SV_F32 ? 4 : 0); }

size_t round256(size_t x) { return (x + 255) / 256 * 256; }

int check_cache(const sv_kv_cache *c, int dtype, int64_t need_rows, int B) {
    if (c->block_size <= 0 || c->block_size % 16 != 0 || c->max_blocks_per_seq <= 0 ||
        c->num_blocks <= 0 || c->block_stride <= 0 || c->head_stride <= 0 || c->row_stride <= 0)
        return SV_ERR_SHAPE;
    if (c->dtype != dtype) return SV_ERR_DTYPE;
    int64_t cap;
    if (!mul_ok(c->max_blocks_per_seq, c->block_size, &cap)) return SV_ERR_OVERFLOW;
    if (need_rows > cap) return SV_ERR_CAPACITY;
    const int es = esize_of(dtype);
    if ((c->block_stride * es) % 16 || (c->head_stride * es) % 16 || (c->row_stride * es) % 16)
        return SV_ERR_ALIGN;
    if (!aligned16(c->k) || !aligned16(c->v)) return SV_ERR_ALIGN;
    int64_t tmp;
    if (!prod_ok({c->num_blocks, c->block_stride, es}, &tmp)) return SV_ERR_OVERFLOW;
    if (!prod_ok({(int64_t)B, c->max_blocks_per_seq}, &tmp)) return SV_ERR_OVERFLOW;
    return SV_OK;
}

CacheView view_of(const sv_kv_cache *c) {
    CacheView v;
    v.k = c->k;
    v.v = c->v;
    v.table = c->block_table;
    v.bs = c->block_size;
    v.max_blocks = c->max_blocks_per_seq;
    v.num_blocks = c->num_blocks;
    v.bstride = c->block_stride;
    v.hstride = c->head_stride;
    v.rstride = c->row_stride;
    return v;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SV_OK : SV_ERR_HIP; }

// Shape checks shared by the attention size query and the attention call.
int check_attn_shape(int B, int Hq, int Hkv, int T, int D, int max_prefix_len, int dtype,
                     int num_splits) {
    if (B < 0 || max_prefix_len < 0 || num_splits < 0) return SV_ERR_SHAPE;
    if (Hkv <= 0 || Hq <= 0) return SV_ERR_GQA;  // before the modulo
    if (Hq % Hkv != 0) return SV_ERR_GQA;
    if (D != 128 && D != 256 && D != 512) return SV_ERR_HEAD_DIM;
    if (T < 1 || T > 64) return SV_ERR_TREE_SIZE;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
    int64_t tmp;
    if (!prod_ok({(int64_t)B, Hq, T, D, 4}, &tmp)) return SV_ERR_OVERFLOW;
    if ((int64_t)max_prefix_len + T > INT_MAX) return SV_ERR_OVERFLOW;
    return SV_OK;
}

}  // namespace

int make_attn_plan(int B, int Hq, int Hkv, int T, int D, int max_prefix_len, int dtype,
                   int num_splits, AttnPlan *p) {
    const int rc = check_attn_shape(B, Hq, Hkv, T, D, max_prefix_len, dtype, num_splits);
    if (rc != SV_OK) return rc;
    const int R = (Hq / Hkv) * T;
    p->R = R;
    // bf16 always runs on the matrix cores; a kv head with fewer than 16 query rows
    // (single-node trees, small groups) pads its row block, which costs matrix-core time
    // but not latency.  fp32 runs on the vector ALUs.
    p->mfma = dtype == SV_BF16;
    if (p->mfma) {
        // 32-row blocks, each shared by D/256 wavefronts (one below 256); at most 8
        // wavefronts
        const int dsplit = D >= 256 ? D / 256 : 1;
        const int blocks = (R + 31) / 32;
        int nw = blocks * dsplit;
        nw = nw > kAttnMaxWaves ? kAttnMaxWaves : nw;
        p->rows_per_wg = (nw / dsplit) * 32;
        p->nthreads = 64 * nw;
    } else {
        p->rows_per_wg = 16;
        p->nthreads = 256;
    }
    p->n_rg = (R + p->rows_per_wg - 1) / p->rows_per_wg;
    int64_t units = (int64_t)(B > 0 ? B : 1) * Hkv * p->n_rg;
    int64_t want = num_splits > 0 ? num_splits : (kNumCU + units - 1) / units;
    const int64_t P = max_prefix_len > 0 ? max_prefix_len : 1;
    // automatic splitting keeps chunks of at least min_chunk keys: shorter ones cost more
    // in per-workgroup set-up and in merging partial results than they save (measured on
    // small calls: 64 keys on the matrix-core kernels, one 32-key chunk per workgroup on
    // the vector-ALU kernel)
    const int64_t min_chunk = p->mfma ? kMinChunk : kKeyTile;
    if (num_splits == 0 && want > (P + min_chunk - 1) / min_chunk) want = (P + min_chunk - 1) / min_chunk;
    if (want < 1) want = 1;
    int64_t C = (P + want - 1) / want;
    C = (C + kKeyTile - 1) / kKeyTile * kKeyTile;
    if (C < kKeyTile) C = kKeyTile;
    int64_t S = (max_prefix_len + C - 1) / C;
    if (S < 1) S = 1;
    // Prefix lengths that differ leave the chunks of a uniform cut unbalanced: when the
    // prefixes are split at all, the w4 kernel re-cuts the chunks from the actual lengths
    // and starts the largest first.  A grid that one chunk per sequence already fills is
    // not split further: the calls run at the board's power limit, where evening out the
    // finish times gains little and the partial results and their merge cost more.
    p->balanced = 0;
    if (p->mfma && attn_w4_handles(D) && num_splits == 0 && S > 1 &&
        (int64_t)B * S <= kBalancedChunks)
        p->balanced = 1;
    p->C = (int)C;
    p->S = (int)S;
    // In-kernel merge (head_dim 128/256): when each sequence is one chunk (no merge at
    // all, every workgroup writes its output), or when the grid fills the chip, so that
    // the merges of the many units run side by side.  A small call split into many chunks
    // merges faster in the separate kernel, which spreads the merge over many workgroups
    // instead of leaving each unit's to one.  The arrival counters must fit their region,
    // and one unit's partials must stay within a 31-bit byte offset.
    // The fp32 kernel merges inside itself whenever the counters and offsets allow: its
    // units are 16 rows, so one workgroup's merge is as short as the separate kernel's.
    const bool merge_fits = units <= kMaxMergeUnits && S * (int64_t)R * D * 4 < ((int64_t)1 << 31);
    p->fused = merge_fits && ((p->mfma && attn_w4_handles(D) && (S == 1 || units * S >= kNumCU)) ||
                              !p->mfma);
    int64_t work, o_elems, ml_elems;
    if (!prod_ok({units, S}, &work) || work > INT_MAX) return SV_ERR_OVERFLOW;
    if (!prod_ok({(int64_t)B, Hkv, S, R, D}, &o_elems)) return SV_ERR_OVERFLOW;
    if (!prod_ok({(int64_t)B, Hkv, S, R, 2}, &ml_elems)) return SV_ERR_OVERFLOW;
    // one chunk per sequence merged in the kernel: every workgroup writes its output
    // directly, and no partial results are stored
    const bool partials = !(p->fused && S == 1);
    p->ws_o = partials ? round256((size_t)o_elems * 4) : 0;
    p->ws_ml = partials ? round256((size_t)ml_elems * 4) : 0;
    p->ws_total = kCounterBytes + kHeaderBytes + p->ws_ml + p->ws_o;
    return SV_OK;
}

namespace {

// Every host-side check of an attention call except the workspace; *nothing when B == 0.
int check_attention(const void *q, const void *k_tree, const void *v_tree,
                    const sv_kv_cache *cache, const int32_t *prefix_len, int32_t max_prefix_len,
                    const uint64_t *mask, int32_t B, int32_t Hq, int32_t Hkv, int32_t T,
                    int32_t D, float scale, float *out, int32_t num_splits, AttnPlan *plan,
                    bool *nothing) {
    if (!cache) return SV_ERR_NULL;
    if (!(scale > 0.0f) || scale > 3.0e38f) return SV_ERR_SHAPE;  // positive and finite
    const int dtype = cache->dtype;
    int rc = make_attn_plan(B, Hq, Hkv, T, D, max_prefix_len, dtype, num_splits, plan);
    if (rc != SV_OK) return rc;
    *nothing = B == 0;
    if (B == 0) return SV_OK;
    // k_tree and v_tree both NULL: the tree rows are read from the cache at P + i
    if (!q || (!k_tree != !v_tree) || !prefix_len || !mask || !out || !cache->k || !cache->v ||
        !cache->block_table)
        return SV_ERR_NULL;
    rc = check_cache(cache, dtype, (int64_t)max_prefix_len + T, B);
    if (rc != SV_OK) return rc;
    if (!aligned16(q) || !aligned16(k_tree) || !aligned16(v_tree) || !aligned16(out))
        return SV_ERR_ALIGN;
    return SV_OK;
}

// Launches a checked attention call with its workspace laid out as the plan says.
int launch_attention(const AttnPlan &plan, const void *q, const void *k_tree, const void *v_tree,
                     const sv_kv_cache *cache, const int32_t *prefix_len, int32_t max_prefix_len,
                     const uint64_t *mask, int32_t B, int32_t Hq, int32_t Hkv, int32_t T,
                     int32_t D, float scale, float *out, void *workspace, hipStream_t stream) {
    AttnArgs a;
    a.q = q;
    a.k_tree = k_tree;
    a.v_tree = v_tree;
    a.cache = view_of(cache);
    a.prefix_len = prefix_len;
    a.max_prefix_len = max_prefix_len;
    a.mask = mask;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.T = T;
    a.D = D;
    a.scale = scale;
    a.out = out;
    char *ws = static_cast<char *>(workspace);
    a.ws_cnt = reinterpret_cast<int32_t *>(ws);
    a.ws_c = reinterpret_cast<int32_t *>(ws + kCounterBytes);
    a.ws_ml = reinterpret_cast<float *>(ws + kCounterBytes + kHeaderBytes);
    a.ws_o = reinterpret_cast<float *>(ws + kCounterBytes + kHeaderBytes + plan.ws_ml);
    hipError_t e = plan.mfma ? launch_attn_mfma(a, plan, stream)
                             : launch_attn_valu(a, plan, cache->dtype, stream);
    if (e != hipSuccess) return SV_ERR_HIP;
    if (plan.fused) return SV_OK;
    return hip_status(launch_attn_reduce(a, plan, stream));
}

// ---- scratch of the allocation-free attention entry point.  One array per device, in
// the code object, held until the process ends.  In host code `scratch` is a host-side
// stand-in for the symbol: its device address comes from hipGetSymbolAddress, once per
// device, and only that address is ever handed to kernels.
constexpr int kMaxDevices = 64;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];
void *g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

__global__ void zero_words_kernel(uint32_t *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0;
}

// The current device's scratch address; the first call on a device looks it up and
// clears the merge's arrival counters (a fill kernel on `stream`, so it is ordered before
// the attention kernels the call enqueues next).
int device_scratch(hipStream_t stream, void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SV_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return SV_ERR_HIP;
        hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, stream,
                           static_cast<uint32_t *>(ptr), kCounterBytes / 4);
        if (hipGetLastError() != hipSuccess) return SV_ERR_HIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return SV_OK;
}

}  // namespace

}  // namespace sv

using namespace sv;

extern "C" {

const char *sv_status_string(int status) {
    switch (status) {
        case SV_OK: return "ok";
        case SV_ERR_NULL: return "a required pointer is NULL";
        case SV_ERR_SHAPE: return "invalid or inconsistent size";
        case SV_ERR_DTYPE: return "unsupported or mismatched dtype";
        case SV_ERR_GQA: return "head counts must be positive with Hq a multiple of Hkv";
        case SV_ERR_HEAD_DIM: return "head_dim must be 128, 256 or 512";
        case SV_ERR_TREE_SIZE: return "tree size T must be in [1, 64]";
        case SV_ERR_CAPACITY: return "max_prefix_len + T exceeds the cache rows reserved per sequence";
        case SV_ERR_OVERFLOW: return "a size overflows";
        case SV_ERR_WORKSPACE: return "workspace missing or too small";
        case SV_ERR_HIP: return "HIP runtime error";
        case SV_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
        case SV_ERR_SCRATCH:
            return "the call needs more than the 64 MiB of scratch the allocation-free entry "
                   "point holds (use sv_tree_verify_attention with a workspace)";
        default: return "unknown status";
    }
}

int sv_build_tree_mask(const int32_t *parents, int32_t B, int32_t T, uint64_t *mask,
                       int32_t *depth, int32_t *tree_err, hipStream_t stream) {
    if (B < 0) return SV_ERR_SHAPE;
    if (T < 1 || T > 64) return SV_ERR_TREE_SIZE;
    if (B == 0) return SV_OK;
    if (!parents || !mask || !tree_err) return SV_ERR_NULL;
    return hip_status(launch_tree_mask(parents, B, T, mask, depth, tree_err, stream));
}

size_t sv_tree_verify_attention_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int32_t T,
                                               int32_t D, int32_t max_prefix_len, int32_t dtype,
                                               int32_t num_splits) {
    AttnPlan p;
    if (make_attn_plan(B, Hq, Hkv, T, D, max_prefix_len, dtype, num_splits, &p) != SV_OK)
        return 0;
    return p.ws_total;
}

int sv_tree_verify_attention(const void *q, const void *k_tree, const void *v_tree,
                             const sv_kv_cache *cache, const int32_t *prefix_len,
                             int32_t max_prefix_len, const uint64_t *mask, int32_t B, int32_t Hq,
                             int32_t Hkv, int32_t T, int32_t D, float scale, float *out,
                             void *workspace, size_t workspace_bytes, int32_t num_splits,
                             hipStream_t stream) {
    AttnPlan plan;
    bool nothing = false;
    int rc = check_attention(q, k_tree, v_tree, cache, prefix_len, max_prefix_len, mask, B, Hq,
                             Hkv, T, D, scale, out, num_splits, &plan, &nothing);
    if (rc != SV_OK || nothing) return rc;
    if (!workspace || workspace_bytes < plan.ws_total) return SV_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return SV_ERR_ALIGN;
    return launch_attention(plan, q, k_tree, v_tree, cache, prefix_len, max_prefix_len, mask, B,
                            Hq, Hkv, T, D, scale, out, workspace, stream);
}

int sv_tree_verify_attention_noalloc(const void *q, const void *k_tree, const void *v_tree,
                                     const sv_kv_cache *cache, const int32_t *prefix_len,
                                     int32_t max_prefix_len, const uint64_t *mask, int32_t B,
                                     int32_t Hq, int32_t Hkv, int32_t T, int32_t D, float scale,
                                     float *out, int32_t num_splits, hipStream_t stream) {
    AttnPlan plan;
    bool nothing = false;
    int rc = check_attention(q, k_tree, v_tree, cache, prefix_len, max_prefix_len, mask, B, Hq,
                             Hkv, T, D, scale, out, num_splits, &plan, &nothing);
    if (rc != SV_OK || nothing) return rc;
    if (plan.ws_total > kScratchBytes) return SV_ERR_SCRATCH;
    void *scratch_ptr = nullptr;
    rc = device_scratch(stream, &scratch_ptr);
    if (rc != SV_OK) return rc;
    return launch_attention(plan, q, k_tree, v_tree, cache, prefix_len, max_prefix_len, mask, B,
                            Hq, Hkv, T, D, scale, out, scratch_ptr, stream);
}

size_t sv_accept_longest_path_workspace_size(int32_t B, int32_t T, int64_t V) {
    if (B < 0 || T < 1 || T > 64 || V < 1 || V > INT_MAX) return 0;
    ArgmaxPlan p;
    if (make_argmax_plan((int64_t)B * T, V, &p) != 0) return 0;
    return round256(p.ws_bytes);
}

int sv_accept_longest_path(const float *logits, const int32_t *draft, const int32_t *parents,
                           const int32_t *tree_err, int32_t B, int32_t T, int64_t V,
                           int32_t *argmax_out, int32_t *accepted_len, int32_t *accepted_nodes,
                           int32_t *out_tokens, void *workspace, size_t workspace_bytes,
                           hipStream_t stream) {
    if (B < 0 || V < 1) return SV_ERR_SHAPE;
    if (T < 1 || T > 64) return SV_ERR_TREE_SIZE;
    int64_t tmp;
    if (V > INT_MAX || !prod_ok({(int64_t)B, T, V, 4}, &tmp)) return SV_ERR_OVERFLOW;
    if (B == 0) return SV_OK;
    if (!logits || !draft || !parents || !accepted_len || !accepted_nodes || !out_tokens)
        return SV_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(logits) & 3u) != 0) return SV_ERR_ALIGN;
    ArgmaxPlan p;
    const int rc = make_argmax_plan((int64_t)B * T, V, &p);
    if (rc != 0) return rc;
    if (!workspace || workspace_bytes < p.ws_bytes) return SV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SV_ERR_ALIGN;
    hipError_t e = launch_argmax_partial(logits, (int64_t)B * T, V, p, workspace, stream);
    if (e != hipSuccess) return SV_ERR_HIP;
    return hip_status(launch_accept(workspace, p, draft, parents, tree_err, B, T, argmax_out,
                                    accepted_len, accepted_nodes, out_tokens, stream));
}

size_t sv_accept_sampled_workspace_size(int32_t B, int32_t T, int64_t V) {
    if (B < 0 || T < 1 || T > 64 || V < 1 || V > INT_MAX) return 0;
    ArgmaxPlan p;
    if (make_sample_plan((int64_t)B * T, V, &p) != 0) return 0;
    return round256(p.ws_bytes);
}

int sv_accept_sampled(const float *logits, const int32_t *draft, const int32_t *parents,
                      const int32_t *tree_err, const float *u_accept, const float *u_sample,
                      float temperature, int32_t B, int32_t T, int64_t V, int32_t *accepted_len,
                      int32_t *accepted_nodes, int32_t *out_tokens, void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
    if (B < 0 || V < 1) return SV_ERR_SHAPE;
    if (T < 1 || T > 64) return SV_ERR_TREE_SIZE;
    if (!(temperature > 0.0f) || !(temperature < __builtin_huge_valf())) return SV_ERR_SHAPE;
    int64_t tmp;
    if (V > INT_MAX || !prod_ok({(int64_t)B, T, V, 4}, &tmp)) return SV_ERR_OVERFLOW;
    if (B == 0) return SV_OK;
    if (!logits || !draft || !parents || !u_accept || !u_sample || !accepted_len ||
        !accepted_nodes || !out_tokens)
        return SV_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(logits) & 3u) != 0) return SV_ERR_ALIGN;
    ArgmaxPlan p;
    const int rc = make_sample_plan((int64_t)B * T, V, &p);
    if (rc != 0) return rc;
    if (!workspace || workspace_bytes < p.ws_bytes) return SV_ERR_WORKSPACE;
    if (!aligned16(workspace)) return SV_ERR_ALIGN;
    return hip_status(launch_accept_sampled(logits, draft, parents, tree_err, u_accept, u_sample,
                                            temperature, B, T, V, p, workspace, accepted_len,
                                            accepted_nodes, out_tokens, stream));
}

int sv_rope_tree(void *q, void *k_tree, const int32_t *prefix_len, const int32_t *depth,
                 int32_t B, int32_t Hq, int32_t Hkv, int32_t T, int32_t D, int32_t dtype,
                 double theta, hipStream_t stream) {
    if (B < 0 || Hq < 1 || Hkv < 1 || D < 2 || D > 1024 || (D & 1)) return SV_ERR_SHAPE;
    if (!(theta > 0.0) || !(theta < __builtin_huge_val())) return SV_ERR_SHAPE;
    if (T < 1 || T > 64) return SV_ERR_TREE_SIZE;
    if (dtype != SV_F32 && dtype != SV_BF16) return SV_ERR_DTYPE;
    int64_t tmp;
    if (!prod_ok({(int64_t)B, (int64_t)Hq + Hkv, T, D, 4}, &tmp)) return SV_ERR_OVERFLOW;
    if (B == 0) return SV_OK;
    if (!q || !k_tree || !prefix_len || !depth) return SV_ERR_NULL;
    const uintptr_t al = dtype == SV_BF16 ? 1u : 3u;
    if ((reinterpret_cast<uintptr_t>(q) & al) || (reinterpret_cast<uintptr_t>(k_tree) & al))
        return SV_ERR_ALIGN;
    return hip_status(launch_rope_tree(q, k_tree, prefix_len, depth, B, Hq, Hkv, T, D, dtype,
                                       theta, stream));
}

int sv_kv_append(const void *k_tree, const void *v_tree, int32_t *tree_err,
                 const sv_kv_cache *cache, const int32_t *prefix_len, int32_t max_prefix_len,
                 int32_t B, int32_t Hkv, int32_t T, int32_t D, hipStream_t stream) {
    if (!cache) return SV_ERR_NULL;
    if (B < 0 || max_prefix_len < 0) return SV_ERR_SHAPE;
    if (Hkv <= 0) return SV_ERR_GQA;
    if (T < 1 || T > 64) return SV_ERR_TREE_SIZE;
    if (D != 128 && D != 256 && D != 512) return SV_ERR_HEAD_DIM;
    const int dtype = cache->dtype;
    const int es = esize_of(dtype);
    if (es == 0) return SV_ERR_DTYPE;
    int64_t tmp;
    if (!prod_ok({(int64_t)B, Hkv, T, D, es}, &tmp)) return SV_ERR_OVERFLOW;
    if ((int64_t)max_prefix_len + T > INT_MAX) return SV_ERR_OVERFLOW;
    if (B == 0) return SV_OK;
    if (!k_tree || !v_tree || !tree_err || !prefix_len || !cache->k || !cache->v ||
        !cache->block_table)
        return SV_ERR_NULL;
    int rc = check_cache(cache, dtype, (int64_t)max_prefix_len + T, B);
    if (rc != SV_OK) return rc;
    if (!aligned16(k_tree) || !aligned16(v_tree)) return SV_ERR_ALIGN;
    return hip_status(launch_kv_append(k_tree, v_tree, tree_err, cache->k, cache->v,
                                       view_of(cache), prefix_len, max_prefix_len, B, Hkv, T, D,
                                       es, stream));
}

int sv_kv_compact(const int32_t *accepted_len, const int32_t *accepted_nodes,
                  const int32_t *tree_err, const sv_kv_cache *cache, const int32_t *prefix_len,
                  int32_t max_prefix_len, int32_t *new_prefix_len, int32_t B, int32_t Hkv,
                  int32_t T, int32_t D, hipStream_t stream) {
    if (!cache) return SV_ERR_NULL;
    if (B < 0 || max_prefix_len < 0) return SV_ERR_SHAPE;
    if (Hkv <= 0) return SV_ERR_GQA;
    if (T < 1 || T > 64) return SV_ERR_TREE_SIZE;
    if (D != 128 && D != 256 && D != 512) return SV_ERR_HEAD_DIM;
    const int dtype = cache->dtype;
    const int es = esize_of(dtype);
    if (es == 0) return SV_ERR_DTYPE;
    int64_t tmp;
    if (!prod_ok({(int64_t)B, Hkv, T, D, es}, &tmp)) return SV_ERR_OVERFLOW;
    if ((int64_t)max_prefix_len + T > INT_MAX) return SV_ERR_OVERFLOW;
    if (B == 0) return SV_OK;
    if (!accepted_len || !accepted_nodes || !prefix_len || !cache->k || !cache->v ||
        !cache->block_table)
        return SV_ERR_NULL;
    int rc = check_cache(cache, dtype, (int64_t)max_prefix_len + T, B);
    if (rc != SV_OK) return rc;
    return hip_status(launch_kv_compact(accepted_len, accepted_nodes, tree_err, cache->k, cache->v,
                                        view_of(cache), prefix_len, max_prefix_len,
                                        new_prefix_len, B, Hkv, T, D, es, stream));
}

int sv_topk_logprobs(const float *logits, int64_t R, int64_t V, int32_t K, int32_t *top_tokens,
                     double *top_logp, hipStream_t stream) {
    if (R < 0 || V < 1 || K < 1 || K > 64 || (int64_t)K > V) return SV_ERR_SHAPE;
    int64_t tmp;
    if (V > INT_MAX || R > INT_MAX || !prod_ok({R, V, 4}, &tmp) || !prod_ok({R, K, 8}, &tmp))
        return SV_ERR_OVERFLOW;
    if (R == 0) return SV_OK;
    if (!logits || !top_tokens || !top_logp) return SV_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(logits) & 3u) || (reinterpret_cast<uintptr_t>(top_tokens) & 3u) ||
        (reinterpret_cast<uintptr_t>(top_logp) & 7u))
        return SV_ERR_ALIGN;
    return hip_status(launch_topk_rows(logits, R, V, K, 1, 1, top_tokens, top_logp, stream));
}

// Nodes of a full K-ary tree with `levels` levels, capped at 65.
static int64_t tree_capacity(int32_t K, int32_t levels) {
    int64_t cap = 0, width = 1;
    for (int32_t lv = 0; lv < levels && cap <= 64; ++lv) {
        cap += width;
        width = width * K > 65 ? 65 : width * K;
    }
    return cap;
}

static bool draft_shape_ok(int32_t B, int32_t T, int64_t V, int32_t K, int32_t max_levels) {
    return B >= 0 && V >= 1 && K >= 1 && K <= 64 && (int64_t)K <= V &&
           max_levels >= 1 && T >= 1 && T <= 64 && tree_capacity(K, max_levels) >= T;
}

size_t sv_draft_tree_workspace_size(int32_t B, int32_t T, int32_t K) {
    if (B < 0 || T < 1 || T > 64 || K < 1 || K > 64) return 0;
    const size_t n = (size_t)B * (size_t)(T - 1) * (size_t)K;
    return round256(n * sizeof(double)) + round256(n * sizeof(int32_t));
}

int sv_draft_tree(const float *drafter_logits, const int32_t *root_token, int32_t B, int32_t T,
                  int64_t V, int32_t K, int32_t max_levels, int32_t *parents, int32_t *tokens,
                  double *cum_logp, void *workspace, size_t workspace_bytes,
                  hipStream_t stream) {
    if (T < 1 || T > 64) return SV_ERR_TREE_SIZE;
    if (!draft_shape_ok(B, T, V, K, max_levels)) return SV_ERR_SHAPE;
    int64_t tmp;
    if (V > INT_MAX || !prod_ok({(int64_t)B, T, V, 4}, &tmp) || (int64_t)B * (T - 1) > INT_MAX)
        return SV_ERR_OVERFLOW;
    if (B == 0) return SV_OK;
    if (!drafter_logits || !root_token || !parents || !tokens || !cum_logp) return SV_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(drafter_logits) & 3u) ||
        (reinterpret_cast<uintptr_t>(cum_logp) & 7u))
        return SV_ERR_ALIGN;
    const size_t need = sv_draft_tree_workspace_size(B, T, K);
    if (T > 1 && (!workspace || workspace_bytes < need)) return SV_ERR_WORKSPACE;
    if (T > 1 && !aligned16(workspace)) return SV_ERR_ALIGN;
    const size_t n = (size_t)B * (size_t)(T - 1) * (size_t)K;
    double *lp = static_cast<double *>(workspace);
    int32_t *tk = reinterpret_cast<int32_t *>(static_cast<char *>(workspace) +
                                              round256(n * sizeof(double)));
    if (T > 1) {
        const int rc = hip_status(launch_topk_rows(drafter_logits, (int64_t)B * (T - 1), V, K,
                                                   T - 1, T, tk, lp, stream));
        if (rc != SV_OK) return rc;
    }
    return hip_status(launch_best_first(tk, lp, root_token, B, T, K, max_levels, parents, tokens,
                                        cum_logp, stream));
}

int sv_kv_commit(const void *k_tree, const void *v_tree, const int32_t *accepted_len,
                 const int32_t *accepted_nodes, const int32_t *tree_err,
                 const sv_kv_cache *cache, const int32_t *prefix_len, int32_t max_prefix_len,
                 int32_t *new_prefix_len, int32_t B, int32_t Hkv, int32_t T, int32_t D,
                 hipStream_t stream) {
    if (!cache) return SV_ERR_NULL;
    if (B < 0 || max_prefix_len < 0) return SV_ERR_SHAPE;
    if (Hkv <= 0) return SV_ERR_GQA;
    if (T < 1 || T > 64) return SV_ERR_TREE_SIZE;
    if (D != 128 && D != 256 && D != 512) return SV_ERR_HEAD_DIM;
    const int dtype = cache->dtype;
    const int es = esize_of(dtype);
    if (es == 0) return SV_ERR_DTYPE;
    int64_t tmp;
    if (!prod_ok({(int64_t)B, Hkv, T, D, es}, &tmp)) return SV_ERR_OVERFLOW;
    if ((int64_t)max_prefix_len + T > INT_MAX) return SV_ERR_OVERFLOW;
    if (B == 0) return SV_OK;
    if (!k_tree || !v_tree || !accepted_len || !accepted_nodes || !prefix_len || !cache->k ||
        !cache->v || !cache->block_table)
        return SV_ERR_NULL;
    int rc = check_cache(cache, dtype, (int64_t)max_prefix_len + T, B);
    if (rc != SV_OK) return rc;
    if (!aligned16(k_tree) || !aligned16(v_tree)) return SV_ERR_ALIGN;
    return hip_status(launch_kv_commit(k_tree, v_tree, accepted_len, accepted_nodes, tree_err,
                                       cache->k, cache->v, view_of(cache), prefix_len,
                                       max_prefix_len, new_prefix_len, B, Hkv, T, D, es,
                                       stream));
}

}  // extern "C"
