// attn_valu.hip -- tree-masked split-KV attention on the vector ALUs, for fp32 inputs
// and for kv heads with fewer than 16 query rows (single-node trees, small groups).
// Same partial-result format as attn_mfma.hip, so the same merge finishes it.
//
// Workgroup: 256 threads own 16 query rows of one (sequence, kv head, chunk); keys
// stream through LDS 16 at a time as fp32.  Thread (row = t / 16, sub = t % 16)
// scores key `sub` against its row, the 16 threads of a row reduce the max and sum
// by shuffles, and the same thread then accumulates head_dim entries sub, sub + 16,
// ... of the row's output.
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kRowsV = 16;
constexpr int kKeysV = 16;
constexpr float kNegInfV = -__builtin_huge_valf();

struct ValuParams {
    const void *q;
    const void *kt;
    const void *vt;
    const void *kc;
    const void *vc;
    const int32_t *table;
    int32_t bs, max_blocks;
    int64_t num_blocks, bstride, hstride, rstride;
    const int32_t *prefix_len;
    int max_P;
    const uint64_t *mask;
    int B, Hq, Hkv, T, G, R;
    float scale_log2;
    int S, C, n_rg, total;
    float *ws_o;
    float *ws_ml;
};

template <bool kBF16>
__device__ __forceinline__ float ld(const void *base, int64_t idx) {
    if (kBF16) {
        const uint16_t hbits = static_cast<const uint16_t *>(base)[idx];
        return __uint_as_float((uint32_t)hbits << 16);
    }
    return static_cast<const float *>(base)[idx];
}

template <int D, bool kBF16>
__global__ __launch_bounds__(256) void attn_valu_kernel(ValuParams p) {
    extern __shared__ __attribute__((aligned(16))) float fsm[];
    float *qs = fsm;                           // [16][D]
    float *ks = qs + kRowsV * D;               // [16][D + 1]
    float *vs = ks + kKeysV * (D + 1);         // [16][D]
    float *ps = vs + kKeysV * D;               // [16][16]

    const int n = gridDim.x;
    const int logical = (blockIdx.x % kNumXCD) * (n / kNumXCD) + blockIdx.x / kNumXCD;
    if (logical >= p.total) return;
    int t = logical;
    const int rg = t % p.n_rg;
    t /= p.n_rg;
    const int s = t % p.S;
    t /= p.S;
    const int kvh = t % p.Hkv;
    const int b = t / p.Hkv;

    int P = p.prefix_len[b];
    P = P < 0 ? 0 : (P > p.max_P ? p.max_P : P);
    const int start = s * p.C;
    if (s > 0 && start >= P) return;
    const int end = min(start + p.C, P);

    const int tid = threadIdx.x;
    const int rl = tid / kKeysV;        // local row
    const int sub = tid % kKeysV;
    const int row = rg * kRowsV + rl;
    const bool row_ok = row < p.R;
    const int g = row_ok ? row / p.T : 0;
    const int node = row_ok ? row - g * p.T : 0;

    // stage Q rows
    for (int e = tid; e < kRowsV * D; e += blockDim.x) {
        const int r = e / D, d = e - (e / D) * D;
        const int rr = rg * kRowsV + r;
        float v = 0.0f;
        if (rr < p.R) {
            const int gg = rr / p.T, ii = rr - (rr / p.T) * p.T;
            v = ld<kBF16>(p.q, (((int64_t)b * p.Hq + (int64_t)kvh * p.G + gg) * p.T + ii) * D + d);
        }
        qs[e] = v;
    }
    const uint64_t mrow = row_ok ? p.mask[(int64_t)b * p.T + node] : 0ull;

    constexpr int DPT = D / kKeysV;  // output entries per thread
    float o[DPT];
    for (int j = 0; j < DPT; ++j) o[j] = 0.0f;
    float m = kNegInfV, l = 0.0f;

    for (int pass = 0; pass < 2; ++pass) {
        const bool tree = pass == 1;
        if (tree && s != 0) break;
        const int lo = tree ? 0 : start;
        const int hi = tree ? p.T : end;
        for (int k0 = lo; k0 < hi; k0 += kKeysV) {
            __syncthreads();  // previous tile fully consumed (and Q staged)
            for (int e = tid; e < kKeysV * D; e += blockDim.x) {
                const int kk = e / D, d = e - (e / D) * D;
                const int pos = k0 + kk;
                float kv = 0.0f, vv = 0.0f;
                if (pos < hi) {
                    int64_t off = -1;
                    if (tree && p.kt) {
                        off = (((int64_t)b * p.Hkv + kvh) * p.T + pos) * D;
                    } else if (tree) {
                        // tree rows kept in the cache at P + pos (an out-of-range block
                        // entry reads block 0: such rows were never appended)
                        const int cpos = P + pos;
                        int32_t blk = p.table[(int64_t)b * p.max_blocks + cpos / p.bs];
                        blk = (blk >= 0 && blk < p.num_blocks) ? blk : 0;
                        off = (int64_t)blk * p.bstride + (int64_t)kvh * p.hstride +
                              (int64_t)(cpos % p.bs) * p.rstride;
                    } else {
                        const int32_t blk = p.table[(int64_t)b * p.max_blocks + pos / p.bs];
                        if (blk >= 0 && blk < p.num_blocks)
                            off = (int64_t)blk * p.bstride + (int64_t)kvh * p.hstride +
                                  (int64_t)(pos % p.bs) * p.rstride;
                    }
                    if (off >= 0) {
                        kv = ld<kBF16>(tree && p.kt ? p.kt : p.kc, off + d);
                        vv = ld<kBF16>(tree && p.kt ? p.vt : p.vc, off + d);
                    }
                }
                ks[kk * (D + 1) + d] = kv;
                vs[kk * D + d] = vv;
            }
            __syncthreads();

            // score of key `sub` for row `rl`
            const int pos = k0 + sub;
            bool ok = pos < hi;
            if (ok && !tree) {
                const int32_t blk = p.table[(int64_t)b * p.max_blocks + pos / p.bs];
                ok = blk >= 0 && blk < p.num_blocks;
            }
            if (tree) ok = ok && ((mrow >> pos) & 1ull);
            float dot = 0.0f;
            const float *qr = qs + rl * D;
            const float *kr = ks + sub * (D + 1);
            for (int d = 0; d < D; ++d) dot = fmaf(qr[d], kr[d], dot);
            const float x = ok ? dot * p.scale_log2 : kNegInfV;
            float mt = x;
            for (int off = 1; off < kKeysV; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off, 64));
            const float mnew = fmaxf(m, mt);
            const float alpha = mnew == kNegInfV ? 1.0f : exp2f(m - mnew);
            const float pr = x == kNegInfV ? 0.0f : exp2f(x - mnew);
            float lt = pr;
            for (int off = 1; off < kKeysV; off <<= 1) lt += __shfl_xor(lt, off, 64);
            l = l * alpha + lt;
            m = mnew;
            ps[rl * kKeysV + sub] = pr;
            __syncthreads();
            for (int j = 0; j < DPT; ++j) {
                const int d = sub + kKeysV * j;
                float acc = o[j] * alpha;
                for (int k = 0; k < kKeysV; ++k) acc = fmaf(ps[rl * kKeysV + k], vs[k * D + d], acc);
                o[j] = acc;
            }
        }
    }

    if (row_ok) {
        const int64_t base = (((int64_t)b * p.Hkv + kvh) * p.S + s) * p.R + row;
        for (int j = 0; j < DPT; ++j) p.ws_o[base * D + sub + kKeysV * j] = o[j];
        if (sub == 0) {
            p.ws_ml[base * 2 + 0] = m;
            p.ws_ml[base * 2 + 1] = l;
        }
    }
}

template <int D, bool kBF16>
hipError_t launch_v(const AttnArgs &a, const AttnPlan &pl, hipStream_t stream) {
    const size_t smem = sizeof(float) * ((size_t)kRowsV * D + (size_t)kKeysV * (D + 1) +
                                         (size_t)kKeysV * D + kRowsV * kKeysV);
    hipError_t e = hipFuncSetAttribute((const void *)attn_valu_kernel<D, kBF16>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    ValuParams p;
    p.q = a.q;
    p.kt = a.k_tree;
    p.vt = a.v_tree;
    p.kc = a.cache.k;
    p.vc = a.cache.v;
    p.table = a.cache.table;
    p.bs = a.cache.bs;
    p.max_blocks = a.cache.max_blocks;
    p.num_blocks = a.cache.num_blocks;
    p.bstride = a.cache.bstride;
    p.hstride = a.cache.hstride;
    p.rstride = a.cache.rstride;
    p.prefix_len = a.prefix_len;
    p.max_P = a.max_prefix_len;
    p.mask = a.mask;
    p.B = a.B;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.T = a.T;
    p.G = a.Hq / a.Hkv;
    p.R = pl.R;
    p.scale_log2 = a.scale * 1.4426950408889634f;
    p.S = pl.S;
    p.C = pl.C;
    p.n_rg = pl.n_rg;
    p.total = a.B * a.Hkv * pl.S * pl.n_rg;
    p.ws_o = a.ws_o;
    p.ws_ml = a.ws_ml;
    const int grid = (p.total + kNumXCD - 1) / kNumXCD * kNumXCD;
    hipLaunchKernelGGL((attn_valu_kernel<D, kBF16>), dim3(grid), dim3(256), smem, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_valu(const AttnArgs &a, const AttnPlan &pl, int dtype,
                            hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    const bool bf = dtype == SV_BF16;
    if (a.D == 128) return bf ? launch_v<128, true>(a, pl, stream) : launch_v<128, false>(a, pl, stream);
    if (a.D == 256) return bf ? launch_v<256, true>(a, pl, stream) : launch_v<256, false>(a, pl, stream);
    return bf ? launch_v<512, true>(a, pl, stream) : launch_v<512, false>(a, pl, stream);
}

}  // namespace sv
