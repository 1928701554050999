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
// Q head and every tree-key head of that node in fp64 and round the result to the
// tensor's type (through fp32 for bf16, both steps to nearest even).  When D/2 holds
// whole 16-byte vectors and both tensors are 16-byte aligned, a thread moves 16 bytes of
// x[j..] and of x[j + D/2..] at a time and issues its first loads before the angles are
// formed, so that the memory latency hides behind the fp64 work.
#include "sv_internal.h"

namespace sv {
namespace {

template <bool kBF16>
__device__ __forceinline__ double load_x(const void *base, int64_t idx) {
    if (kBF16) return (double)(float)static_cast<const __bf16 *>(base)[idx];
    return (double)static_cast<const float *>(base)[idx];
}

// fp64 -> fp32, nearest with ties to even.  The empty statement keeps the compiler from
// fusing this rounding with a following fp32 -> bf16 one into a single fp64 -> bf16
// rounding (round to odd in between), which would differ from rounding twice to nearest
// and costs a compare-and-adjust sequence per element.
__device__ __forceinline__ float to_f32(double v) {
    float f = (float)v;
    asm volatile("" : "+v"(f));
    return f;
}

template <bool kBF16>
__device__ __forceinline__ void store_x(void *base, int64_t idx, double v) {
    const float f = to_f32(v);  // nearest, ties to even
    if (kBF16)
        static_cast<__bf16 *>(base)[idx] = (__bf16)f;  // nearest, ties to even
    else
        static_cast<float *>(base)[idx] = f;
}

// cos and sin of pos * theta^(-2j/D) for j < D/2 into cs[j], cs[D/2 + j]
__device__ __forceinline__ void rope_angles(double *cs, double pos, int D, double theta) {
    const int half = D / 2;
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
    rope_angles(cs, pos, D, theta);
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

// The 16-byte form: V = 16 / element size consecutive j per access (D/2 a multiple of V,
// 16-byte aligned tensors).  Pair e = (head h, group g) covers j = gV .. gV + V - 1.
template <bool kBF16>
struct RopeVec;
template <>
struct RopeVec<true> {
    using T = bf16x8;
    static constexpr int V = 8;
    static __device__ __forceinline__ double get(const T &x, int v) { return (double)(float)x[v]; }
    static __device__ __forceinline__ void put(T &x, int v, double r) {
        x[v] = (__bf16)to_f32(r);  // nearest even, twice
    }
};
template <>
struct RopeVec<false> {
    using T = f32x4;
    static constexpr int V = 4;
    static __device__ __forceinline__ double get(const T &x, int v) { return (double)x[v]; }
    static __device__ __forceinline__ void put(T &x, int v, double r) { x[v] = to_f32(r); }
};

template <bool kBF16>
__global__ __launch_bounds__(256) void rope_tree_vec_kernel(
    void *__restrict__ q, void *__restrict__ k, const int32_t *__restrict__ prefix_len,
    const int32_t *__restrict__ depth, int T, int Hq, int Hkv, int D, double theta) {
    using RV = RopeVec<kBF16>;
    using VT = typename RV::T;
    constexpr int V = RV::V;
    constexpr int kIt = 3;  // pairs a thread holds at once
    extern __shared__ double cs[];
    const int b = blockIdx.x / T;
    const int i = blockIdx.x - b * T;
    const int half = D / 2;
    const int ng = half / V;
    const int npairs = (Hq + Hkv) * ng;
    // pair e: its tensor and the vector index of its x[j] (x[j + D/2] is half / V further)
    const auto at = [&](int e, VT *&base, int &g) {
        const int h = e / ng;
        g = e - h * ng;
        const bool isq = h < Hq;
        base = static_cast<VT *>(isq ? q : k);
        const int64_t row = isq ? (((int64_t)b * Hq + h) * T + i) * D
                                : (((int64_t)b * Hkv + (h - Hq)) * T + i) * D;
        return row / V + g;
    };
    VT x1[kIt], x2[kIt];
    const auto load = [&](int e0) {
#pragma unroll
        for (int u = 0; u < kIt; ++u) {
            const int e = e0 + u * (int)blockDim.x;
            if (e < npairs) {
                VT *base;
                int g;
                const int64_t o = at(e, base, g);
                x1[u] = base[o];
                x2[u] = base[o + ng];
            }
        }
    };
    const auto rotate_store = [&](int e0) {
#pragma unroll
        for (int u = 0; u < kIt; ++u) {
            const int e = e0 + u * (int)blockDim.x;
            if (e < npairs) {
                VT *base;
                int g;
                const int64_t o = at(e, base, g);
                const int j0 = g * V;
                VT y1, y2;
#pragma unroll
                for (int v = 0; v < V; ++v) {
                    const double a1 = RV::get(x1[u], v), a2 = RV::get(x2[u], v);
                    const double c = cs[j0 + v], sn = cs[half + j0 + v];
                    RV::put(y1, v, a1 * c - a2 * sn);
                    RV::put(y2, v, a2 * c + a1 * sn);
                }
                base[o] = y1;
                base[o + ng] = y2;
            }
        }
    };
    const int step = kIt * (int)blockDim.x;
    load((int)threadIdx.x);
    const double pos = (double)prefix_len[b] + (double)depth[(int64_t)b * T + i];
    rope_angles(cs, pos, D, theta);
    __syncthreads();
    rotate_store((int)threadIdx.x);
    for (int e0 = (int)threadIdx.x + step; e0 < npairs; e0 += step) {
        load(e0);
        rotate_store(e0);
    }
}

}  // namespace

hipError_t launch_rope_tree(void *q, void *k_tree, const int32_t *prefix_len,
                            const int32_t *depth, int B, int Hq, int Hkv, int T, int D, int dtype,
                            double theta, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    const size_t smem = (size_t)D * sizeof(double);
    const dim3 grid((unsigned)((int64_t)B * T));
    const int V = dtype == SV_BF16 ? 8 : 4;
    const bool vec = (D / 2) % V == 0 && ((reinterpret_cast<uintptr_t>(q) |
                                           reinterpret_cast<uintptr_t>(k_tree)) & 15u) == 0;
    const auto kernel = dtype == SV_BF16 ? (vec ? rope_tree_vec_kernel<true> : rope_tree_kernel<true>)
                                         : (vec ? rope_tree_vec_kernel<false> : rope_tree_kernel<false>);
    hipLaunchKernelGGL(kernel, grid, dim3(256), smem, stream, q, k_tree, prefix_len, depth, T, Hq,
                       Hkv, D, theta);
    return hipGetLastError();
}

}  // namespace sv
