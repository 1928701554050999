// accept.hip -- greedy acceptance: vocab argmax per tree row, then the longest root path
// whose draft tokens all equal their parent row's argmax, plus the bonus token.
//
// Rule (llms-explorer page Facts, commit rule; ADR-037 Phase status rows E5a and
// E4b.10a, section 4 Phase E5; Medusa/EAGLE-2 page "Why bother"):
//   a[i]   = smallest index of the maximum of logits row i (NaN never wins)
//   node i matches when every edge on its root path matches:
//          draft[c] == a[parent[c]] for each node c on the path below the root
//   accept the deepest matching node (smallest index among equals), emit
//   a[] along its path: L - 1 accepted drafts and one bonus token.
//
// argmax_partial_kernel streams each row chunk with 16-byte loads and reduces
// (value, index) pairs across the workgroup; accept_kernel (one wavefront per
// sequence, one lane per node) merges the chunk results in a fixed order and runs
// the path search with ballots and shuffles.
#include "sv_internal.h"

namespace sv {
namespace {

struct Best {
    float v;
    int32_t i;
};

constexpr int32_t kNone = 0x7fffffff;

// a beats b: larger value, or equal value at a smaller index.  NaN never beats.
__device__ __forceinline__ bool beats(float av, int32_t ai, float bv, int32_t bi) {
    return av > bv || (av == bv && ai < bi);
}

__device__ __forceinline__ void take(float &bv, int32_t &bi, float v, int32_t i) {
    if (beats(v, i, bv, bi)) {
        bv = v;
        bi = i;
    }
}

__global__ __launch_bounds__(256) void argmax_partial_kernel(const float *__restrict__ logits,
                                                             int64_t V, int64_t chunk,
                                                             int nchunks,
                                                             Best *__restrict__ out) {
    const int64_t row = blockIdx.x / nchunks;
    const int c = blockIdx.x - (int)row * nchunks;
    const int64_t lo = (int64_t)c * chunk;
    const int64_t hi = lo + chunk < V ? lo + chunk : V;
    const float *rp = logits + row * V;
    const int tid = threadIdx.x;

    float bv = -__builtin_huge_valf();
    int32_t bi = kNone;

    // body starts at the first 16-byte aligned element at or after lo
    const int64_t mis = (int64_t)((reinterpret_cast<uintptr_t>(rp + lo) >> 2) & 3);
    int64_t a0 = lo + ((4 - mis) & 3);
    if (a0 > hi) a0 = hi;
    const int64_t a1 = a0 + ((hi - a0) >> 2 << 2);
    if (lo + tid < a0) take(bv, bi, rp[lo + tid], (int32_t)(lo + tid));

    const f32x4 *vp = reinterpret_cast<const f32x4 *>(rp + a0);
    const int64_t nvec = (a1 - a0) >> 2;
    int64_t k = tid;
    // four independent 16-byte loads in flight per thread, non-temporal: every logit is
    // read once (the hint takes the 583 MB scan of the 32K batch from 106 to 92 us)
    for (; k + 3 * 256 < nvec; k += 4 * 256) {
        const f32x4 x0 = __builtin_nontemporal_load(vp + k),
                    x1 = __builtin_nontemporal_load(vp + k + 256),
                    x2 = __builtin_nontemporal_load(vp + k + 512),
                    x3 = __builtin_nontemporal_load(vp + k + 768);
        const int32_t e0 = (int32_t)(a0 + 4 * k);
        for (int j = 0; j < 4; ++j) take(bv, bi, x0[j], e0 + j);
        for (int j = 0; j < 4; ++j) take(bv, bi, x1[j], e0 + 1024 + j);
        for (int j = 0; j < 4; ++j) take(bv, bi, x2[j], e0 + 2048 + j);
        for (int j = 0; j < 4; ++j) take(bv, bi, x3[j], e0 + 3072 + j);
    }
    for (; k < nvec; k += 256) {
        const f32x4 x0 = __builtin_nontemporal_load(vp + k);
        const int32_t e0 = (int32_t)(a0 + 4 * k);
        for (int j = 0; j < 4; ++j) take(bv, bi, x0[j], e0 + j);
    }
    if (a1 + tid < hi) take(bv, bi, rp[a1 + tid], (int32_t)(a1 + tid));

    for (int off = 32; off > 0; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int32_t oi = __shfl_xor(bi, off, 64);
        take(bv, bi, ov, oi);
    }
    __shared__ Best part[4];
    const int w = tid >> 6;
    if ((tid & 63) == 0) part[w] = Best{bv, bi};
    __syncthreads();
    if (tid == 0) {
        for (int j = 1; j < (int)(blockDim.x >> 6); ++j) take(bv, bi, part[j].v, part[j].i);
        out[blockIdx.x] = Best{bv, bi};
    }
}

__global__ __launch_bounds__(256) void accept_kernel(const Best *__restrict__ part, int nchunks,
                                                     const int32_t *__restrict__ draft,
                                                     const int32_t *__restrict__ parents,
                                                     const int32_t *__restrict__ tree_err, int B,
                                                     int T, int32_t *__restrict__ argmax_out,
                                                     int32_t *__restrict__ accepted_len,
                                                     int32_t *__restrict__ accepted_nodes,
                                                     int32_t *__restrict__ out_tokens) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (b >= B) return;
    const bool in = lane < T;
    const int64_t row = (int64_t)b * T + lane;

    int32_t a = 0;
    if (in) {
        float bv = -__builtin_huge_valf();
        int32_t bi = kNone;
        for (int c = 0; c < nchunks; ++c) {
            const Best q = part[row * nchunks + c];
            take(bv, bi, q.v, q.i);
        }
        a = bi == kNone ? 0 : bi;
        if (argmax_out) argmax_out[row] = a;
    }

    const int p = in ? parents[row] : -1;
    const bool bad = (lane == 0 && p != -1) || (lane >= 1 && in && (p < 0 || p >= lane));
    const bool invalid = __ballot(bad) != 0ull || (tree_err && tree_err[b] != 0);
    if (invalid) {
        if (in) {
            accepted_nodes[row] = -1;
            out_tokens[row] = -1;
        }
        if (lane == 0) accepted_len[b] = 0;
        return;
    }

    // edge test of node `lane`: its draft token equals its parent's argmax
    const int32_t ap = __shfl(a, p < 0 ? 0 : p, 64);
    const bool edge = lane == 0 || (in && draft[row] == ap);
    const uint64_t E = __ballot(edge);

    // ancestors of node `lane` (self included) and its depth
    uint64_t anc = 1ull << lane;
    int depth = 0;
    int cur = p;
    for (int step = 0; step < T; ++step) {
        const bool live = cur >= 0;
        if (!__any(live)) break;
        if (live) {
            anc |= 1ull << cur;
            ++depth;
        }
        const int up = __shfl(p, live ? cur : 0, 64);
        cur = live ? up : -1;
    }
    const bool matched = in && (anc & ~E) == 0ull;

    // deepest matched node, smallest index among equals: maximise depth*64 + (63 - lane)
    int key = matched ? depth * 64 + (63 - lane) : -1;
    for (int off = 32; off > 0; off >>= 1) key = max(key, __shfl_xor(key, off, 64));
    const int best = 63 - (key & 63);
    const int L = (key >> 6) + 1;
    const uint64_t path = __shfl(anc, best, 64);

    if (in) {
        if ((path >> lane) & 1ull) {
            const int slot = __popcll(path & ((1ull << lane) - 1ull));
            accepted_nodes[(int64_t)b * T + slot] = lane;
            out_tokens[(int64_t)b * T + slot] = a;
        }
        if (lane >= L) {
            accepted_nodes[row] = -1;
            out_tokens[row] = -1;
        }
    }
    if (lane == 0) accepted_len[b] = L;
}

}  // namespace

int make_argmax_plan(int64_t rows, int64_t V, ArgmaxPlan *p) {
    if (rows < 0 || V < 1) return SV_ERR_SHAPE;
    // Rows are cut into chunks of at most 16384 logits (64 KB per workgroup), whatever the
    // row count: many short workgroups per CU keep the last round of a large call short.
    // (The 32K batch's 960 rows as 9600 workgroups; as 2880 workgroups of 200 KB the chip
    // ran 1.4 rounds of them, the second at 40% occupancy.)  Chunk starts stay 4 KB apart.
    const int64_t max_chunk = 16384;
    const int64_t n = (V + max_chunk - 1) / max_chunk;
    int64_t chunk = (V + n - 1) / n;
    chunk = (chunk + 1023) / 1024 * 1024;
    p->chunk = chunk;
    p->nchunks = (int)((V + chunk - 1) / chunk);
    // one workgroup per (row, chunk): the grid must stay within 2^31 - 1 workgroups
    if (rows > (int64_t)INT_MAX / p->nchunks) return SV_ERR_OVERFLOW;
    p->ws_bytes = (size_t)rows * p->nchunks * sizeof(Best);
    return 0;
}

hipError_t launch_argmax_partial(const float *logits, int64_t rows, int64_t V,
                                 const ArgmaxPlan &p, void *ws, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(argmax_partial_kernel, dim3((unsigned)(rows * p.nchunks)), dim3(256), 0,
                       stream, logits, V, p.chunk, p.nchunks, static_cast<Best *>(ws));
    return hipGetLastError();
}

hipError_t launch_accept(const void *ws, const ArgmaxPlan &p, const int32_t *draft,
                         const int32_t *parents, const int32_t *tree_err, int B, int T,
                         int32_t *argmax_out, int32_t *accepted_len, int32_t *accepted_nodes,
                         int32_t *out_tokens, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    const int per = 4;
    hipLaunchKernelGGL(accept_kernel, dim3((B + per - 1) / per), dim3(64 * per), 0, stream,
                       static_cast<const Best *>(ws), p.nchunks, draft, parents, tree_err, B, T,
                       argmax_out, accepted_len, accepted_nodes, out_tokens);
    return hipGetLastError();
}

}  // namespace sv
