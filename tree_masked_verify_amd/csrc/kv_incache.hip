// kv_incache.hip -- the write-before-accept variant of the KV update: the tree's K/V rows
// go into the cache before the attention, and after the acceptance the accepted path is
// compacted down over them.
//
// Rules (ADR-037 Phase status row E6, per-layer tree-verify block: K/V appended at
// [prefix_len, prefix_len + tree_seq_len) before the tree attention; section 4 Phase E5
// and row E5b: the cache is rolled back to the accepted path; llms-explorer page Facts on
// KV write-before-accept and the delayed write-through that avoids it):
//   append:  tree row i of every kv head -> cache position prefix_len[b] + i, i < T;
//   compact: the row at P + accepted_nodes[b][j] -> position P + j, j < accepted_len[b];
//            new_prefix_len[b] = P + L.
//
// The append runs one workgroup per (sequence, kv head), the compaction one per sequence.
// Both first check the whole request (prefix length, block-table entries of [P, P + T),
// accepted length and nodes) and act on all of it or none of it; the block ids of
// [P, P + T) are staged in LDS once.  The compaction moves rows within the cache, and a path's source rows
// can be other rows' destinations (nodes 0, 2, 3 move rows 2 and 3 to 1 and 2), so it
// reads the moving rows' 16-byte pieces into registers, column by column over all kv heads,
// waits at a barrier, then writes them.
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kPer = 8;       // 16-byte pieces of each tensor a thread holds at once

// Byte offset of cache position pos (in [P, P + T)) of kv head h, with the block ids of
// [P, P + T) staged in LDS (blk[i] for position P + i).
__device__ __forceinline__ int64_t cache_byte(const CacheView &c, const int32_t *blk, int P,
                                              int h, int i, int esize) {
    const int pos = P + i;
    return ((int64_t)blk[(pos / c.bs) - (P / c.bs)] * c.bstride + (int64_t)h * c.hstride +
            (int64_t)(pos % c.bs) * c.rstride) * esize;
}

// Stages the block-table entries covering [P, P + T) in LDS and returns whether every one
// is in range (with `ok` false on entry, nothing is read and the answer is false).
__device__ __forceinline__ bool stage_blocks(const CacheView &c, int b, int P, int T, bool ok,
                                             int32_t *blk) {
    const int tid = threadIdx.x;
    const int nb = ok ? (P + T - 1) / c.bs - P / c.bs + 1 : 0;
    if (tid < nb) {
        const int32_t e = c.table[(int64_t)b * c.max_blocks + P / c.bs + tid];
        blk[tid] = e;
        ok = e >= 0 && e < c.num_blocks;
    }
    return __syncthreads_and(ok) != 0;
}

// One workgroup per (sequence, kv head); every workgroup of a sequence takes the same
// decision.  The one of kv head 0 records a refusal; the others' read of the status may
// see that record or not, and refuse either way.
__global__ __launch_bounds__(kThreads) void kv_append_kernel(
    const unsigned char *__restrict__ k_tree, const unsigned char *__restrict__ v_tree,
    int32_t *tree_err, unsigned char *__restrict__ k_cache, unsigned char *__restrict__ v_cache,
    CacheView c, int esize, const int32_t *__restrict__ prefix_len, int max_P, int Hkv, int T,
    int row_bytes) {
    __shared__ int32_t s_blk[65];
    const int b = blockIdx.x / Hkv;
    const int h = blockIdx.x - b * Hkv;
    const int tid = threadIdx.x;
    if (__atomic_load_n(&tree_err[b], __ATOMIC_RELAXED) != 0) return;   // uniform
    const int P = prefix_len[b];
    const int64_t cap = (int64_t)c.max_blocks * c.bs;
    const bool ok = stage_blocks(c, b, P, T, P >= 0 && P <= max_P && (int64_t)P + T <= cap, s_blk);
    if (!ok) {
        if (tid == 0 && h == 0) __atomic_store_n(&tree_err[b], 3, __ATOMIC_RELAXED);
        return;
    }
    // kPer pieces of K and of V per thread in flight: all loads of a batch, then its stores
    const int cpr = row_bytes / 16;
    const int units = T * cpr;
    const int64_t base = ((int64_t)b * Hkv + h) * T * row_bytes;
    for (int u0 = 0; u0 < units; u0 += kThreads * kPer) {
        u32x4 kb[kPer], vb[kPer];
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int u = u0 + e * kThreads + tid;
            if (u < units) {
                const int64_t src = base + (int64_t)u * 16;   // row u / cpr, piece u % cpr
                kb[e] = *reinterpret_cast<const u32x4 *>(k_tree + src);
                vb[e] = *reinterpret_cast<const u32x4 *>(v_tree + src);
            }
        }
#pragma unroll
        for (int e = 0; e < kPer; ++e) {
            const int u = u0 + e * kThreads + tid;
            if (u < units) {
                const int64_t dst = cache_byte(c, s_blk, P, h, u / cpr, esize) + (u % cpr) * 16;
                *reinterpret_cast<u32x4 *>(k_cache + dst) = kb[e];
                *reinterpret_cast<u32x4 *>(v_cache + dst) = vb[e];
            }
        }
    }
}

// One workgroup per sequence (new_prefix_len may alias prefix_len: every thread reads
// prefix_len[b] before the first barrier, one writes new_prefix_len[b] after the last).
__global__ __launch_bounds__(kThreads) void kv_compact_kernel(
    const int32_t *__restrict__ accepted_len, const int32_t *__restrict__ accepted_nodes,
    const int32_t *__restrict__ tree_err, unsigned char *k_cache, unsigned char *v_cache,
    CacheView c, int esize, const int32_t *prefix_len, int max_P, int32_t *new_prefix_len,
    int Hkv, int T, int row_bytes) {
    __shared__ int32_t s_blk[65];
    __shared__ int32_t s_move[64];   // destinations j whose source row differs
    __shared__ int32_t s_src[64];    // and their source nodes
    __shared__ int s_n;
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int P = prefix_len[b];
    const int L = accepted_len[b];
    const int64_t cap = (int64_t)c.max_blocks * c.bs;
    bool ok = !(tree_err && tree_err[b] != 0) && L >= 0 && L <= T && P >= 0 && P <= max_P &&
              (int64_t)P + T <= cap;
    int node = 0;
    if (ok && tid < L) {
        node = accepted_nodes[(int64_t)b * T + tid];
        ok = node >= 0 && node < T;
    }
    ok = __syncthreads_and(ok) != 0;
    const bool all_ok = stage_blocks(c, b, P, T, ok, s_blk);
    if (tid == 0) s_n = 0;
    __syncthreads();
    if (all_ok && tid < L && node != tid) {
        const int k = atomicAdd(&s_n, 1);
        s_move[k] = tid;
        s_src[k] = node;
    }
    __syncthreads();
    const int n = s_n;
    if (all_ok && n > 0) {
        // A round covers whole columns (a kv head's 16-byte piece position) of every moving
        // row: kcols columns, n pieces each, read before the barrier, written after it.
        // No round reads a piece an earlier round wrote.
        const int cpr = row_bytes / 16;
        const int ncols = Hkv * cpr;
        const int kcols = kThreads * kPer / n;   // >= 128
        for (int c0 = 0; c0 < ncols; c0 += kcols) {
            const int units = n * min(kcols, ncols - c0);
            u32x4 kb[kPer], vb[kPer];
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                const int u = e * kThreads + tid;
                if (u < units) {
                    const int col = c0 + u / n, m = u % n;
                    const int64_t src =
                        cache_byte(c, s_blk, P, col / cpr, s_src[m], esize) + (col % cpr) * 16;
                    kb[e] = *reinterpret_cast<const u32x4 *>(k_cache + src);
                    vb[e] = *reinterpret_cast<const u32x4 *>(v_cache + src);
                }
            }
            __syncthreads();   // every source piece of this round is read
#pragma unroll
            for (int e = 0; e < kPer; ++e) {
                const int u = e * kThreads + tid;
                if (u < units) {
                    const int col = c0 + u / n, m = u % n;
                    const int64_t dst =
                        cache_byte(c, s_blk, P, col / cpr, s_move[m], esize) + (col % cpr) * 16;
                    *reinterpret_cast<u32x4 *>(k_cache + dst) = kb[e];
                    *reinterpret_cast<u32x4 *>(v_cache + dst) = vb[e];
                }
            }
            __syncthreads();
        }
    }
    if (tid == 0 && new_prefix_len) new_prefix_len[b] = all_ok ? P + L : P;
}

}  // namespace

hipError_t launch_kv_append(const void *k_tree, const void *v_tree, int32_t *tree_err,
                            void *k_cache, void *v_cache, const CacheView &c,
                            const int32_t *prefix_len, int32_t max_prefix_len, int B, int Hkv,
                            int T, int D, int esize, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    hipLaunchKernelGGL(kv_append_kernel, dim3(B * Hkv), dim3(kThreads), 0, stream,
                       static_cast<const unsigned char *>(k_tree),
                       static_cast<const unsigned char *>(v_tree), tree_err,
                       static_cast<unsigned char *>(k_cache), static_cast<unsigned char *>(v_cache),
                       c, esize, prefix_len, max_prefix_len, Hkv, T, D * esize);
    return hipGetLastError();
}

hipError_t launch_kv_compact(const int32_t *accepted_len, const int32_t *accepted_nodes,
                             const int32_t *tree_err, void *k_cache, void *v_cache,
                             const CacheView &c, const int32_t *prefix_len,
                             int32_t max_prefix_len, int32_t *new_prefix_len, int B, int Hkv,
                             int T, int D, int esize, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    hipLaunchKernelGGL(kv_compact_kernel, dim3(B), dim3(kThreads), 0, stream, accepted_len,
                       accepted_nodes, tree_err, static_cast<unsigned char *>(k_cache),
                       static_cast<unsigned char *>(v_cache), c, esize, prefix_len,
                       max_prefix_len, new_prefix_len, Hkv, T, D * esize);
    return hipGetLastError();
}

}  // namespace sv
