// tree_mask.hip -- parent array -> ancestor-and-self bitmask, one wavefront per sequence.
//
// Rule: row i holds node i and every ancestor of node i (ADR-037 Phase status
// rows E4a and E6 v2; Medusa/EAGLE-2 page, "What's not implemented" 1(c)).
// Lane i owns node i (T <= 64 = the wavefront width) and climbs its own
// ancestor chain, reading each parent link from the lane that owns it; no lane
// waits on another's result, so the climb is at most depth steps.
#include "sv_internal.h"

namespace sv {
namespace {

__global__ __launch_bounds__(256) void tree_mask_kernel(const int32_t *__restrict__ parents,
                                                        int B, int T, uint64_t *__restrict__ mask,
                                                        int32_t *__restrict__ depth,
                                                        int32_t *__restrict__ tree_err) {
    const int lane = threadIdx.x & 63;
    const int b = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    if (b >= B) return;  // whole wavefront leaves together
    const int32_t *par = parents + (int64_t)b * T;
    const int p = lane < T ? par[lane] : -1;

    const bool bad_root = lane == 0 && p != -1;
    const bool bad_par = lane >= 1 && lane < T && (p < 0 || p >= lane);
    const int err = __ballot(bad_root) ? SV_TREE_BAD_ROOT
                                       : (__ballot(bad_par) ? SV_TREE_BAD_PARENT : SV_TREE_OK);

    uint64_t m = 1ull << lane;
    int d = 0;
    if (err == SV_TREE_OK) {
        // parents precede children, so every chain reaches -1 within T steps
        int cur = p;
        for (int step = 0; step < T; ++step) {
            const bool live = cur >= 0;
            if (!__any(live)) break;
            if (live) {
                m |= 1ull << cur;
                ++d;
            }
            const int up = __shfl(p, live ? cur : 0, 64);
            cur = live ? up : -1;
        }
    }
    if (lane < T) {
        mask[(int64_t)b * T + lane] = m;
        if (depth) depth[(int64_t)b * T + lane] = d;
    }
    if (lane == 0) tree_err[b] = err;
}

}  // namespace

hipError_t launch_tree_mask(const int32_t *parents, int B, int T, uint64_t *mask,
                            int32_t *depth, int32_t *tree_err, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    const int per_block = 4;  // sequences (wavefronts) per workgroup
    dim3 grid((B + per_block - 1) / per_block);
    hipLaunchKernelGGL(tree_mask_kernel, grid, dim3(64 * per_block), 0, stream, parents, B, T,
                       mask, depth, tree_err);
    return hipGetLastError();
}

}  // namespace sv
