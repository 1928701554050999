// attn_mfma.hip -- tree-masked split-KV attention on the gfx950 matrix cores (bf16 in,
// fp32 accumulate), for kv heads whose (GQA group x tree nodes) query rows fill at
// least one 16-row tile.
//
// What is computed (ADR-037 Phase status rows E1.1-E1.5, section 4 Phase E1;
// Medusa/EAGLE-2 page "What's not implemented" 1(c)): every query row (q head g of
// kv head kvh, tree node i) attends to the cached prefix of its sequence and to
// the tree rows its ancestor mask selects.  One workgroup covers one
// (sequence, kv head, prefix chunk, row group); it leaves an unnormalised partial
// output and its (reference max, sum) per row, merged afterwards by attn_reduce.
//
// Layout of the work inside a workgroup (up to 8 wavefronts, two per SIMD):
//   * a 32-row block of queries belongs to DSPLIT wavefronts (1 at head_dim 256,
//     2 at head_dim 512); each keeps the Q fragments of its share of head_dim in
//     registers and owns that share of the output;
//   * keys stream through LDS in tiles of 32 rows of K and V (rows padded by 16
//     bytes so the fragment reads below hit distinct banks);
//   * scores are formed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16 with keys
//     as M and query rows as N), so each lane holds one query row and 16 of the
//     tile's keys: the row max needs one swap between lane halves; with DSPLIT = 2
//     the two partial score tiles are summed through LDS first;
//   * the output is accumulated transposed, O^T = V^T P^T, so a lane keeps the
//     accumulators of the row it computed probabilities for; inside a 16-key step
//     the key order follows the score fragment's register order, so the P^T
//     fragment is the score registers as they stand;
//   * the reference max only moves when a tile raises it by more than 2^8, so the
//     accumulators are rarely rescaled (the merged result does not depend on the
//     reference values used).
#include "sv_internal.h"

namespace sv {
namespace {

template <int D>
struct MCfg {
    static constexpr int DSPLIT = D / 256;          // wavefronts sharing one row block
    static constexpr int DW = D / DSPLIT;           // head_dim share of one wavefront
    static constexpr int KS = DW / 16;              // k-steps of S^T = K Q^T
    static constexpr int DB = DW / 32;              // 32-wide d blocks of O^T
    static constexpr int CH = D / 8;                // 16-byte chunks per K/V row
    static constexpr int ROW_BYTES = D * 2 + 16;    // padded LDS row
    static constexpr int TILE_BYTES = kKeyTile * ROW_BYTES;
    static constexpr int XBYTES = DSPLIT > 1 ? 8 * 64 * 16 * 4 : 0;  // score exchange
    static constexpr int SMEM = 2 * TILE_BYTES + XBYTES;
};

struct MfmaParams {
    const __bf16 *q;
    const __bf16 *kt;
    const __bf16 *vt;
    const __bf16 *kc;
    const __bf16 *vc;
    const int32_t *table;
    int32_t bs, max_blocks;
    int64_t num_blocks, bstride, hstride, rstride;
    const int32_t *prefix_len;
    int max_P;
    const uint64_t *mask;
    int B, Hq, Hkv, T, G, R;
    float scale_log2;
    int S, C, n_rg, rows_per_wg, total;
    float *ws_o;
    float *ws_ml;
};

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kRescaleSlack = 8.0f;  // log2 units

__device__ __forceinline__ int xcd_logical_id() {
    // consecutive workgroup ids are dealt round-robin to the 8 XCDs; give each XCD a
    // contiguous range of logical ids, so the row groups of one (sequence, kv head,
    // chunk) run side by side under one L2
    const int n = gridDim.x;  // a multiple of kNumXCD
    const int x = blockIdx.x;
    return (x % kNumXCD) * (n / kNumXCD) + x / kNumXCD;
}

// Stage keys [k0, k0 + 32) of K and V into LDS (zero rows for keys out of range).
// Returns the validity bitmask of the 32 keys (the same in every wavefront).
template <int D, bool kTree>
__device__ __forceinline__ uint32_t stage_tile(const MfmaParams &p, int b, int kvh, int k0,
                                               int kend, unsigned char *ks, unsigned char *vs) {
    using Cf = MCfg<D>;
    const int tid = threadIdx.x;
    for (int c = tid; c < kKeyTile * Cf::CH; c += blockDim.x) {
        const int kk = c / Cf::CH;
        const int ch = c - kk * Cf::CH;
        const int pos = k0 + kk;
        u32x4 kv = {0u, 0u, 0u, 0u};
        u32x4 vv = {0u, 0u, 0u, 0u};
        if (pos < kend) {
            int64_t off = -1;
            if (kTree) {
                off = (((int64_t)b * p.Hkv + kvh) * p.T + pos) * D;
            } else {
                const int32_t blk = p.table[(int64_t)b * p.max_blocks + pos / p.bs];
                if (blk >= 0 && blk < p.num_blocks)
                    off = (int64_t)blk * p.bstride + (int64_t)kvh * p.hstride +
                          (int64_t)(pos % p.bs) * p.rstride;
            }
            if (off >= 0) {
                const __bf16 *ksrc = kTree ? p.kt : p.kc;
                const __bf16 *vsrc = kTree ? p.vt : p.vc;
                kv = *reinterpret_cast<const u32x4 *>(ksrc + off + ch * 8);
                vv = *reinterpret_cast<const u32x4 *>(vsrc + off + ch * 8);
            }
        }
        *reinterpret_cast<u32x4 *>(ks + kk * Cf::ROW_BYTES + ch * 16) = kv;
        *reinterpret_cast<u32x4 *>(vs + kk * Cf::ROW_BYTES + ch * 16) = vv;
    }
    const int lane = threadIdx.x & 63;
    const int pos = k0 + (lane & 31);
    bool ok = pos < kend;
    if (!kTree && ok) {
        const int32_t blk = p.table[(int64_t)b * p.max_blocks + pos / p.bs];
        ok = blk >= 0 && blk < p.num_blocks;
    }
    return (uint32_t)__ballot(ok);
}

template <int D, bool kTree>
__device__ __forceinline__ void tile_math(const unsigned char *ks, const unsigned char *vs,
                                          float *xs, uint32_t kvalid, int k0, int dpart,
                                          const bf16x8 (&qf)[MCfg<D>::KS], uint64_t mrow,
                                          f32x16 (&o)[MCfg<D>::DB], float &mref, float &lsum,
                                          float scale_log2) {
    using Cf = MCfg<D>;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;

    // ---- S^T = K Q^T over this wavefront's share of head_dim.
    //      lane (h, l32) receives query row l32, keys (r/4)*8 + 4h + r%4, r = 0..15
    f32x16 sacc;
    for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
    const unsigned char *kbase = ks + l32 * Cf::ROW_BYTES + dpart * Cf::DW * 2 + h * 16;
#pragma unroll
    for (int kstep = 0; kstep < Cf::KS; ++kstep) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kbase + kstep * 32);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kstep], sacc, 0, 0, 0);
    }
    if (Cf::DSPLIT > 1) {
        // add the partner wavefront's partial scores (same rows, other half of head_dim)
        f32x4 *mine = reinterpret_cast<f32x4 *>(xs + (w * 64 + lane) * 16);
        for (int v = 0; v < 4; ++v)
            mine[v] = f32x4{sacc[4 * v], sacc[4 * v + 1], sacc[4 * v + 2], sacc[4 * v + 3]};
        __syncthreads();
        const f32x4 *other = reinterpret_cast<const f32x4 *>(xs + ((w ^ 1) * 64 + lane) * 16);
        for (int v = 0; v < 4; ++v) {
            const f32x4 t = other[v];
            sacc[4 * v] += t[0];
            sacc[4 * v + 1] += t[1];
            sacc[4 * v + 2] += t[2];
            sacc[4 * v + 3] += t[3];
        }
    }

    // ---- mask, scale, online softmax; probabilities become bf16 P^T fragments
    float sv[16];
    float mt = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const int key = (r >> 2) * 8 + h * 4 + (r & 3);
        bool ok = (kvalid >> key) & 1u;
        if (kTree) ok = ok && ((mrow >> (k0 + key)) & 1ull);
        const float x = ok ? sacc[r] * scale_log2 : kNegInf;
        sv[r] = x;
        mt = fmaxf(mt, x);
    }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const bool raise = mt > mref + kRescaleSlack;
    if (__any(raise)) {
        const float mnew = fmaxf(mref, mt);
        const float alpha = mnew == kNegInf ? 1.0f : exp2f(mref - mnew);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < Cf::DB; ++db) o[db] *= alpha;
        mref = mnew;
    }
    bf16x8 pf[2];
    float add = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float pr = sv[r] == kNegInf ? 0.0f : exp2f(sv[r] - mref);
        const __bf16 pb = (__bf16)pr;
        add += (float)pb;  // the denominator sums exactly the weights the numerator uses
        pf[r >> 3][r & 7] = pb;
    }
    lsum += add;

    // ---- O^T += V^T P^T : A operand lane (h, l32) = V[key][d], d = dpart*DW + db*32 + l32,
    //      keys 16*kk2 + (j/4)*8 + 4h + j%4 (the score fragment's key order)
    const unsigned char *vbase = vs + h * 4 * Cf::ROW_BYTES + dpart * Cf::DW * 2 + l32 * 2;
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
#pragma unroll
        for (int db = 0; db < Cf::DB; ++db) {
            bf16x8 a;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int key0 = 16 * kk2 + (j >> 2) * 8 + (j & 3);
                a[j] = *reinterpret_cast<const __bf16 *>(vbase + key0 * Cf::ROW_BYTES + db * 64);
            }
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk2], o[db], 0, 0, 0);
        }
    }
}

template <int D>
__global__ __launch_bounds__(512) void attn_mfma_kernel(MfmaParams p) {
    using Cf = MCfg<D>;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    unsigned char *ks = smem;
    unsigned char *vs = smem + Cf::TILE_BYTES;
    float *xs = reinterpret_cast<float *>(smem + 2 * Cf::TILE_BYTES);

    const int logical = xcd_logical_id();
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
    if (s > 0 && start >= P) return;  // chunk past this sequence's prefix: nothing to merge
    const int end = min(start + p.C, P);

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int dpart = w % Cf::DSPLIT;
    const int row = rg * p.rows_per_wg + (w / Cf::DSPLIT) * 32 + l32;
    const bool valid = row < p.R;
    const int g = valid ? row / p.T : 0;
    const int i = valid ? row - g * p.T : 0;

    // Q fragments (B operand of S^T): lane holds row l32, d = dpart*DW + 16*kstep + 8h .. +8
    bf16x8 qf[Cf::KS];
    {
        const __bf16 *qp = p.q + (((int64_t)b * p.Hq + (int64_t)kvh * p.G + g) * p.T + i) * D +
                           dpart * Cf::DW + 8 * h;
#pragma unroll
        for (int kstep = 0; kstep < Cf::KS; ++kstep) {
            if (valid) {
                qf[kstep] = *reinterpret_cast<const bf16x8 *>(qp + 16 * kstep);
            } else {
                for (int j = 0; j < 8; ++j) qf[kstep][j] = (__bf16)0.0f;
            }
        }
    }
    const uint64_t mrow = valid ? p.mask[(int64_t)b * p.T + i] : 0ull;

    f32x16 o[Cf::DB];
#pragma unroll
    for (int db = 0; db < Cf::DB; ++db)
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float mref = kNegInf, lsum = 0.0f;

    for (int k0 = start; k0 < end; k0 += kKeyTile) {
        const uint32_t kvalid = stage_tile<D, false>(p, b, kvh, k0, end, ks, vs);
        __syncthreads();
        tile_math<D, false>(ks, vs, xs, kvalid, k0, dpart, qf, mrow, o, mref, lsum, p.scale_log2);
        __syncthreads();
    }
    if (s == 0) {
        for (int k0 = 0; k0 < p.T; k0 += kKeyTile) {
            const uint32_t kvalid = stage_tile<D, true>(p, b, kvh, k0, p.T, ks, vs);
            __syncthreads();
            tile_math<D, true>(ks, vs, xs, kvalid, k0, dpart, qf, mrow, o, mref, lsum,
                               p.scale_log2);
            __syncthreads();
        }
    }

    // ---- partial results: O (unnormalised), reference max (log2 units) and sum per row
    const float ltot = lsum + __shfl_xor(lsum, 32, 64);
    if (valid) {
        const int64_t base = (((int64_t)b * p.Hkv + kvh) * p.S + s) * p.R + row;
        float *op = p.ws_o + base * D + dpart * Cf::DW;
#pragma unroll
        for (int db = 0; db < Cf::DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 v = {o[db][4 * g4 + 0], o[db][4 * g4 + 1], o[db][4 * g4 + 2],
                                 o[db][4 * g4 + 3]};
                *reinterpret_cast<f32x4 *>(op + db * 32 + g4 * 8 + 4 * h) = v;
            }
        if (h == 0 && dpart == 0) {
            p.ws_ml[base * 2 + 0] = mref;
            p.ws_ml[base * 2 + 1] = ltot;
        }
    }
}

template <int D>
hipError_t launch_d(const AttnArgs &a, const AttnPlan &pl, hipStream_t stream) {
    using Cf = MCfg<D>;
    hipError_t e = hipFuncSetAttribute((const void *)attn_mfma_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, Cf::SMEM);
    if (e != hipSuccess) return e;
    MfmaParams p;
    p.q = static_cast<const __bf16 *>(a.q);
    p.kt = static_cast<const __bf16 *>(a.k_tree);
    p.vt = static_cast<const __bf16 *>(a.v_tree);
    p.kc = static_cast<const __bf16 *>(a.cache.k);
    p.vc = static_cast<const __bf16 *>(a.cache.v);
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
    p.rows_per_wg = pl.rows_per_wg;
    p.total = a.B * a.Hkv * pl.S * pl.n_rg;
    p.ws_o = a.ws_o;
    p.ws_ml = a.ws_ml;
    const int grid = (p.total + kNumXCD - 1) / kNumXCD * kNumXCD;
    hipLaunchKernelGGL(attn_mfma_kernel<D>, dim3(grid), dim3(pl.nthreads), Cf::SMEM, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs &a, const AttnPlan &pl, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return a.D == 256 ? launch_d<256>(a, pl, stream) : launch_d<512>(a, pl, stream);
}

}  // namespace sv
