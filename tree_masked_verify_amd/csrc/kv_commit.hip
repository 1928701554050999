// kv_commit.hip -- delayed KV write-through of the accepted path.
//
// Rule (llms-explorer page Facts: Forge's accept(k) writes only the accepted prefix
// into the cache, rejected drafts never touch it; delayed write-through commits
// after the acceptance decision): row prefix_len[b] + j of every kv head receives
// tree row accepted_nodes[b][j], j < accepted_len[b].
//
// One workgroup per sequence.  It first checks the whole request (prefix length,
// accepted length, node indices, block-table entries; the path's node and block ids then
// stay in LDS for the copy) and either copies every row or none; a sequence it refuses
// keeps its prefix length.  All threads read
// prefix_len[b] before the barrier and one thread writes new_prefix_len[b] after
// it, so the two may alias.  Rows move as 16-byte vectors.
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kCommitThreads = 1024;

__global__ __launch_bounds__(kCommitThreads) void kv_commit_kernel(
    const unsigned char *__restrict__ k_tree, const unsigned char *__restrict__ v_tree,
    const int32_t *__restrict__ accepted_len, const int32_t *__restrict__ accepted_nodes,
    const int32_t *__restrict__ tree_err, unsigned char *__restrict__ k_cache,
    unsigned char *__restrict__ v_cache, CacheView c, int esize, const int32_t *prefix_len,
    int max_P, int32_t *new_prefix_len, int Hkv, int T, int row_bytes) {
    __shared__ int32_t s_node[64], s_blk[64];  // of path entry j (T <= 64)
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    // the path entries are read together with the lengths (entries past L are not used)
    const int P = prefix_len[b];
    const int L = accepted_len[b];
    const bool terr = tree_err && tree_err[b] != 0;
    const int node = tid < T ? accepted_nodes[(int64_t)b * T + tid] : -1;
    const int64_t cap = (int64_t)c.max_blocks * c.bs;

    bool ok = !terr && L >= 0 && L <= T && P >= 0 && P <= max_P && (int64_t)P + L <= cap;
    if (ok && tid < L) {
        const int pos = P + tid;
        const int32_t blk = c.table[(int64_t)b * c.max_blocks + pos / c.bs];
        ok = node >= 0 && node < T && blk >= 0 && blk < c.num_blocks;
        s_node[tid] = node;
        s_blk[tid] = blk;
    }
    const bool all_ok = __syncthreads_and(ok) != 0;

    if (all_ok && L > 0) {
        const int cpr = row_bytes / 16;  // 16-byte vectors per row
        const int units = Hkv * L * cpr;
        for (int u = tid; u < units; u += blockDim.x) {
            const int ch = u % cpr;
            const int t = u / cpr;
            const int j = t % L;
            const int h = t / L;
            const int pos = P + j;
            const int64_t src = (((int64_t)b * Hkv + h) * T + s_node[j]) * row_bytes + ch * 16;
            const int64_t dst = ((int64_t)s_blk[j] * c.bstride + (int64_t)h * c.hstride +
                                 (int64_t)(pos % c.bs) * c.rstride) * esize + ch * 16;
            *reinterpret_cast<u32x4 *>(k_cache + dst) = *reinterpret_cast<const u32x4 *>(k_tree + src);
            *reinterpret_cast<u32x4 *>(v_cache + dst) = *reinterpret_cast<const u32x4 *>(v_tree + src);
        }
    }
    if (tid == 0 && new_prefix_len) new_prefix_len[b] = all_ok ? P + L : P;
}

}  // namespace

hipError_t launch_kv_commit(const void *k_tree, const void *v_tree, const int32_t *accepted_len,
                            const int32_t *accepted_nodes, const int32_t *tree_err,
                            void *k_cache, void *v_cache, const CacheView &c,
                            const int32_t *prefix_len, int32_t max_prefix_len,
                            int32_t *new_prefix_len, int B, int Hkv, int T, int D, int esize,
                            hipStream_t stream) {
    if (B == 0) return hipSuccess;
    hipLaunchKernelGGL(kv_commit_kernel, dim3(B), dim3(kCommitThreads), 0, stream,
                       static_cast<const unsigned char *>(k_tree),
                       static_cast<const unsigned char *>(v_tree), accepted_len, accepted_nodes,
                       tree_err, static_cast<unsigned char *>(k_cache),
                       static_cast<unsigned char *>(v_cache), c, esize, prefix_len,
                       max_prefix_len, new_prefix_len, Hkv, T, D * esize);
    return hipGetLastError();
}

}  // namespace sv
