// rope.hip -- tree-position rotary embedding of the verify step's queries and tree keys.
//
// Rule (ADR-037 Phase status row E4b.5b): NeoX style over the whole head; node i of
// sequence b sits at position prefix_len[b] + depth[b][i] (its base position plus its
// depth in the tree, depth from sv_build_tree_mask), so siblings share a position and a
// chain gets consecutive ones.  For j < D/2, f_j = theta^(-2j/D), a = pos * f_j:
//   x'[j] = x[j] cos a - x[j + D/2] sin a,   x'[j + D/2] = x[j + D/2] cos a + x[j] sin a.
//
// One workgroup per (sequence, node): its D/2 angles and their cosines and sines are
// formed in fp64 (positions reach 2^31; an fp32 angle would be off by ~1e-3 rad there;
// in fp64 the angle is within ~pos * 2^-52 rad) into LDS, then the threads rotate every
// Q head and every tree-key head of that node, consecutive threads on consecutive
// elements, in fp64, rounding once to the tensor's type.
#include "sv_internal.h"

namespace sv {
namespace {

template <bool kBF16>
__device__ __forceinline__ double load_x(const void *base, int64_t idx) {
    if (kBF16) return (double)(float)static_cast<const __bf16 *>(base)[idx];
    return (double)static_cast<const float *>(base)[idx];
}

template <bool kBF16>
__device__ __forceinline__ void store_x(void *base, int64_t idx, double v) {
    const float f = (float)v;  // nearest, ties to even
    if (kBF16)
        static_cast<__bf16 *>(base)[idx] = (__bf16)f;  // nearest, ties to even
    else
        static_cast<float *>(base)[idx] = f;
}

template <bool kBF16>
__global__ __launch_bounds__(256) void rope_tree_kernel(void *__restrict__ q, void *__restrict__ k,
                                                        const int32_t *__restrict__ prefix_len,
                                                        const int32_t *__restrict__ depth, int T,
                                                        int Hq, int Hkv, int D, double theta) {
    extern __shared__ double cs[];  // cos [D/2], then sin [D/2]
    const int b = blockIdx.x / T;
    const int i = blockIdx.x - b * T;
    const int half = D / 2;
    const double pos = (double)prefix_len[b] + (double)depth[(int64_t)b * T + i];
    for (int j = threadIdx.x; j < half; j += blockDim.x) {
        const double a = pos * pow(theta, -2.0 * (double)j / (double)D);
        // reduce a modulo 2 pi first, so that the sine and cosine see |r| <= pi: k = the
        // nearest integer to a / (2 pi), then a - k * 2 pi with 2 pi = kTwoPiHi + kTwoPiLo
        // (the double nearest 2 pi and the double nearest the remainder), each product
        // subtracted by one fused operation
        constexpr double kTwoPiHi = 0x1.921fb54442d18p+2;
        constexpr double kTwoPiLo = 0x1.1a62633145c07p-52;
        const double kq = rint(a * (1.0 / kTwoPiHi));
        const double r = fma(-kq, kTwoPiLo, fma(-kq, kTwoPiHi, a));
        double sn, c;
        sincos(r, &sn, &c);
        cs[j] = c;
        cs[half + j] = sn;
    }
    __syncthreads();
    const int nh = Hq + Hkv;
    for (int e = threadIdx.x; e < nh * half; e += blockDim.x) {
        const int h = e / half;
        const int j = e - h * half;
        void *base = h < Hq ? q : k;
        const int64_t row = h < Hq ? (((int64_t)b * Hq + h) * T + i) * D
                                   : (((int64_t)b * Hkv + (h - Hq)) * T + i) * D;
        const double x1 = load_x<kBF16>(base, row + j);
        const double x2 = load_x<kBF16>(base, row + j + half);
        const double c = cs[j], sn = cs[half + j];
        store_x<kBF16>(base, row + j, x1 * c - x2 * sn);
        store_x<kBF16>(base, row + j + half, x2 * c + x1 * sn);
    }
}

}  // namespace

hipError_t launch_rope_tree(void *q, void *k_tree, const int32_t *prefix_len,
                            const int32_t *depth, int B, int Hq, int Hkv, int T, int D, int dtype,
                            double theta, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    const size_t smem = (size_t)D * sizeof(double);
    const dim3 grid((unsigned)((int64_t)B * T));
    if (dtype == SV_BF16)
        hipLaunchKernelGGL(rope_tree_kernel<true>, grid, dim3(256), smem, stream, q, k_tree,
                           prefix_len, depth, T, Hq, Hkv, D, theta);
    else
        hipLaunchKernelGGL(rope_tree_kernel<false>, grid, dim3(256), smem, stream, q, k_tree,
                           prefix_len, depth, T, Hq, Hkv, D, theta);
    return hipGetLastError();
}

}  // namespace sv
