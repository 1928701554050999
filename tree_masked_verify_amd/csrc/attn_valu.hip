// attn_valu.hip -- tree-masked split-KV attention on the vector ALUs, for fp32 inputs.
// A sequence whose prefix is one chunk writes its output directly; otherwise the chunks'
// partial results (the format attn_mfma.hip uses) are merged by the last chunk of each
// (sequence, kv head, row group) to finish, or by the separate merge kernel.
//
// What is computed (ADR-037 Phase status rows E1.1-E1.5, section 4 Phase E1): every
// query row (q head g of kv head kvh, tree node i) attends to the cached prefix of its
// sequence and to the tree rows its ancestor mask selects.
//
// Workgroup: 256 threads own 16 query rows of one (sequence, kv head, chunk); keys stream
// through LDS 16 at a time.  A tile is staged with 16-byte loads, one address computed
// per key, and the next tile's loads are issued into registers before the current tile
// is computed, so a tile costs one memory round trip that overlaps the arithmetic (the
// first tile's loads go out before Q is staged).  Thread (row = t / 16, sub = t % 16)
// scores key `sub` against its row (Q row broadcast from LDS, the key row read as 16-byte
// vectors from a padded LDS row); the 16 threads of a row, one row of 16 lanes, reduce the
// max and sum by DPP; the same thread then accumulates head_dim entries 4 sub .. 4 sub + 3
// of every 64 of the row's output, reading the V rows 16 bytes at a time.
#include "attn_common.h"

namespace sv {
namespace {

constexpr int kRowsV = 16;
constexpr int kKeysV = 16;
constexpr float kNegInfV = -__builtin_huge_valf();

// Maximum / sum over each row of 16 lanes, in every lane of the row (a row is the 16
// threads of one query row): DPP butterflies (quad_perm 1032 and 2301, row_half_mirror,
// row_mirror) instead of permutes through LDS.
template <int kCtrl>
__device__ __forceinline__ float dpp_row(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, 0xf, 0xf, false));
}
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, dpp_row<0xb1>(x));
    x = fmaxf(x, dpp_row<0x4e>(x));
    x = fmaxf(x, dpp_row<0x141>(x));
    return fmaxf(x, dpp_row<0x140>(x));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_row<0xb1>(x);
    x += dpp_row<0x4e>(x);
    x += dpp_row<0x141>(x);
    return x + dpp_row<0x140>(x);
}

struct ValuParams {
    const float *q;
    const float *kt;
    const float *vt;
    const float *kc;
    const float *vc;
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
    float *out;            // [B][T][Hq][D]
    int32_t *counters;     // arrivals per (sequence, kv head, row group); NULL: the
                           // separate merge kernel combines the chunks
};

template <int D>
struct VCfg {
    static constexpr int KROW = D + 4;                // padded K row (floats): 16-byte
                                                      // reads of 16 rows hit 64 banks
    static constexpr int PIECES = kKeysV * D / 4;     // 16-byte pieces per tile and tensor
    static constexpr int PER = PIECES / 256;          // per thread
    static constexpr int KS = 0;                      // [16][KROW]
    static constexpr int VS = KS + kKeysV * KROW;     // [16][D]
    static constexpr int PS = VS + kKeysV * D;        // [16][16] probabilities
    static constexpr int OK = PS + kRowsV * kKeysV;   // [16] key exists
    static constexpr int FLAG = OK + kKeysV;          // the merge's arrival flag
    static constexpr int FLOATS = FLAG + 1;
    static_assert(PIECES % 256 == 0, "tile pieces");
};

template <int D>
__global__ __launch_bounds__(256) void attn_valu_kernel(ValuParams p) {
    using Cf = VCfg<D>;
    extern __shared__ __attribute__((aligned(16))) float fsm[];
    float *ks = fsm + Cf::KS;
    float *vs = fsm + Cf::VS;
    float *ps = fsm + Cf::PS;
    int *okk = reinterpret_cast<int *>(fsm + Cf::OK);

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
    const int ntp = end > start ? (end - start + kKeysV - 1) / kKeysV : 0;   // prefix tiles
    const int ntt = s == 0 ? (p.T + kKeysV - 1) / kKeysV : 0;              // tree tiles
    const int nt = ntp + ntt;

    const int tid = threadIdx.x;
    const int rl = tid / kKeysV;        // local row
    const int sub = tid % kKeysV;
    const int row = rg * kRowsV + rl;
    const bool row_ok = row < p.R;
    const int node = row_ok ? row - (row / p.T) * p.T : 0;

    // Tile u: prefix keys start + 16u .. (u < ntp), else tree rows 16 (u - ntp) ...  This
    // thread's pieces j: key kk = (tid + 256 j) / (D / 4), 16-byte piece d4 of that key.
    // A key that does not exist (past the chunk or the tree, or behind an out-of-range
    // block entry) is staged as zeros and marked absent.
    f32x4 kreg[Cf::PER], vreg[Cf::PER];
    bool kok[Cf::PER];
    // The 16 keys of a prefix tile start at a multiple of 16 and so lie in one cache block
    // (block sizes are multiples of 16): one block-table entry per tile, read a tile ahead
    // of the fetch that uses it, so no fetch waits on the table.
    auto tile_block = [&](int u) -> int32_t {
        return u < ntp ? p.table[(int64_t)b * p.max_blocks + (start + u * kKeysV) / p.bs] : -1;
    };
    auto fetch = [&](int u, int32_t tblk) {
        const bool tree = u >= ntp;
        const int k0 = tree ? (u - ntp) * kKeysV : start + u * kKeysV;
#pragma unroll
        for (int j = 0; j < Cf::PER; ++j) {
            const int f = tid + 256 * j;
            const int kk = f / (D / 4), d4 = f - kk * (D / 4);
            const int pos = k0 + kk;
            int64_t off = -1;
            const float *kb = p.kc, *vb = p.vc;
            if (tree) {
                if (pos < p.T) {
                    if (p.kt) {
                        off = (((int64_t)b * p.Hkv + kvh) * p.T + pos) * D;
                        kb = p.kt;
                        vb = p.vt;
                    } else {
                        // tree rows kept in the cache at P + pos (an out-of-range block
                        // entry reads block 0: such rows were never appended)
                        const int cpos = P + pos;
                        int32_t blk = p.table[(int64_t)b * p.max_blocks + cpos / p.bs];
                        blk = (blk >= 0 && blk < p.num_blocks) ? blk : 0;
                        off = (int64_t)blk * p.bstride + (int64_t)kvh * p.hstride +
                              (int64_t)(cpos % p.bs) * p.rstride;
                    }
                }
            } else if (pos < end && tblk >= 0 && tblk < p.num_blocks) {
                off = (int64_t)tblk * p.bstride + (int64_t)kvh * p.hstride +
                      (int64_t)(pos % p.bs) * p.rstride;
            }
            kok[j] = off >= 0;
            kreg[j] = off >= 0 ? *reinterpret_cast<const f32x4 *>(kb + off + 4 * d4)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
            vreg[j] = off >= 0 ? *reinterpret_cast<const f32x4 *>(vb + off + 4 * d4)
                               : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    auto stash = [&]() {
#pragma unroll
        for (int j = 0; j < Cf::PER; ++j) {
            const int f = tid + 256 * j;
            const int kk = f / (D / 4), d4 = f - kk * (D / 4);
            *reinterpret_cast<f32x4 *>(ks + kk * Cf::KROW + 4 * d4) = kreg[j];
            *reinterpret_cast<f32x4 *>(vs + kk * D + 4 * d4) = vreg[j];
            if (d4 == 0) okk[kk] = kok[j];
        }
    };

    // Output entries of this thread: head_dim 4 sub + 64 jj + e (e < 4), DPT in all, so that
    // the V rows are read 16 bytes at a time.
    constexpr int DPT = D / kKeysV;
    constexpr int NV = D / 64;
    float o[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) o[j] = 0.0f;
    float m = kNegInfV, l = 0.0f;

    int32_t blk_next = tile_block(1);
    if (nt > 0) fetch(0, tile_block(0));
    // this thread's slice of its Q row (head_dim QW sub .. QW sub + QW - 1), kept in
    // registers, loaded while the first tile's loads are in flight
    constexpr int QW = D / kKeysV;
    f32x4 qreg[QW / 4];
    {
        const int gq = row_ok ? row / p.T : 0;
        const float *qp =
            p.q + (((int64_t)b * p.Hq + (int64_t)kvh * p.G + gq) * p.T + node) * D + QW * sub;
#pragma unroll
        for (int q4 = 0; q4 < QW / 4; ++q4)
            qreg[q4] = row_ok ? *reinterpret_cast<const f32x4 *>(qp + 4 * q4)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const uint64_t mrow = row_ok ? p.mask[(int64_t)b * p.T + node] : 0ull;
    for (int u = 0; u < nt; ++u) {
        const bool tree = u >= ntp;
        const int k0 = tree ? (u - ntp) * kKeysV : start + u * kKeysV;
        __syncthreads();  // previous tile fully consumed
        stash();
        __syncthreads();
        if (u + 1 < nt) {  // in flight while this tile is computed
            fetch(u + 1, blk_next);
            blk_next = tile_block(u + 2);
        }

        // score of key `sub` for row `rl`.  Each thread first forms the partial dot products
        // of its head_dim slice with all 16 keys, key (sub + j) % 16 in slot j (rotated, so
        // that the 16 lanes read 16 different K rows, on distinct banks); then a ring over
        // the row's 16 lanes (each step takes the neighbour's sum, row_ror 1, and adds one
        // slot) leaves lane sub with the sum over all slices for key sub.
        const int pos = k0 + sub;
        bool ok = okk[sub] != 0;
        if (tree) ok = ok && ((mrow >> pos) & 1ull);
        float vr[kKeysV];
#pragma unroll
        for (int j = 0; j < kKeysV; ++j) {
            const f32x4 *kr =
                reinterpret_cast<const f32x4 *>(ks + ((sub + j) & (kKeysV - 1)) * Cf::KROW + QW * sub);
            f32x4 a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q4 = 0; q4 < QW / 4; ++q4) {
                const f32x4 c = kr[q4];
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = fmaf(qreg[q4][e], c[e], a[e]);
            }
            vr[j] = (a[0] + a[1]) + (a[2] + a[3]);
        }
        float dot = vr[kKeysV - 1];
#pragma unroll
        for (int t = 1; t < kKeysV; ++t) dot = dpp_row<0x121>(dot) + vr[kKeysV - 1 - t];
        const float x = ok ? dot * p.scale_log2 : kNegInfV;
        const float mt = row16_max(x);
        const float mnew = fmaxf(m, mt);
        const float alpha = mnew == kNegInfV ? 1.0f : __builtin_amdgcn_exp2f(m - mnew);
        const float pr = x == kNegInfV ? 0.0f : __builtin_amdgcn_exp2f(x - mnew);
        const float lt = row16_sum(pr);
        l = l * alpha + lt;
        m = mnew;
        ps[rl * kKeysV + sub] = pr;
        __syncthreads();
        float pk[kKeysV];
#pragma unroll
        for (int k = 0; k < kKeysV; ++k) pk[k] = ps[rl * kKeysV + k];
#pragma unroll
        for (int jj = 0; jj < NV; ++jj) {
            f32x4 a2 = f32x4{o[4 * jj], o[4 * jj + 1], o[4 * jj + 2], o[4 * jj + 3]} * alpha;
#pragma unroll
            for (int k = 0; k < kKeysV; ++k) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(vs + k * D + 4 * sub + 64 * jj);
#pragma unroll
                for (int e = 0; e < 4; ++e) a2[e] = fmaf(pk[k], v[e], a2[e]);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) o[4 * jj + e] = a2[e];
        }
    }

    // chunks of this sequence: chunk 0, and every later one that starts inside the prefix
    const int nv = (int)min((int64_t)p.S, P > 0 ? ((int64_t)P + p.C - 1) / p.C : (int64_t)1);
    const int gg = row_ok ? row / p.T : 0;
    float *op = p.out + (((int64_t)b * p.T + node) * p.Hq + (int64_t)kvh * p.G + gg) * D;
    if (p.counters && nv == 1) {
        // the whole prefix in this chunk: the normalised output goes straight to out
        if (row_ok) {
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
#pragma unroll
            for (int jj = 0; jj < NV; ++jj)
                *reinterpret_cast<f32x4 *>(op + 4 * sub + 64 * jj) =
                    f32x4{o[4 * jj], o[4 * jj + 1], o[4 * jj + 2], o[4 * jj + 3]} * inv;
        }
        return;
    }
    const int64_t ubase = ((int64_t)b * p.Hkv + kvh) * p.S * (int64_t)p.R;  // slot (s, r)
    if (row_ok) {
        const int64_t base = ubase + (int64_t)s * p.R + row;
#pragma unroll
        for (int jj = 0; jj < NV; ++jj)
            *reinterpret_cast<f32x4 *>(p.ws_o + base * D + 4 * sub + 64 * jj) =
                f32x4{o[4 * jj], o[4 * jj + 1], o[4 * jj + 2], o[4 * jj + 3]};
        if (sub == 0) {
            p.ws_ml[base * 2 + 0] = m;
            p.ws_ml[base * 2 + 1] = l;
        }
    }
    if (!p.counters) return;  // merged by the separate merge kernel

    // The last of the nv chunks of this (sequence, kv head, row group) to finish merges
    // them, in chunk order.  Each thread waits until its partial stores have reached L2;
    // one thread then counts the arrival with a device-scope release (which writes this
    // XCD's L2 back, so the partials are visible from every XCD).  The last arrival resets
    // the counter for the next call and reads the partials with device-coherent loads.
    wait_loads<0>();
    __syncthreads();
    int *flag = reinterpret_cast<int *>(fsm + Cf::FLAG);
    if (tid == 0) {
        int32_t *cnt = p.counters + ((int64_t)b * p.Hkv + kvh) * p.n_rg + rg;
        const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == nv - 1;
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
    }
    __syncthreads();
    if (!*flag || !row_ok) return;
    // the 16 threads of the row: the chunks' reference maxima across them, then the
    // chunks four at a time with every load issued before any is used
    const uint32_t rows = (uint32_t)nv * (uint32_t)p.R;
    const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(p.ws_o + ubase * D, rows * D * 4);
    const __amdgpu_buffer_rsrc_t rml = coherent_rsrc(p.ws_ml + ubase * 2, rows * 8);
    float M = kNegInfV;
    for (int c = sub; c < nv; c += kKeysV)
        M = fmaxf(M, coherent_load1(rml, ((uint32_t)c * p.R + row) * 8));
    M = row16_max(M);
    constexpr int GRP = 4;
    f32x4 acc[NV];
#pragma unroll
    for (int jj = 0; jj < NV; ++jj) acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
    float L = 0.0f;
    for (int c0 = 0; c0 < nv; c0 += GRP) {
        float mc[GRP], lc[GRP];
        f32x4 oc[GRP][NV];
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            const int c = c0 + k < nv ? c0 + k : nv - 1;
            const uint32_t slot = (uint32_t)c * p.R + row;
            mc[k] = c0 + k < nv ? coherent_load1(rml, slot * 8) : kNegInfV;
            lc[k] = coherent_load1(rml, slot * 8 + 4);
#pragma unroll
            for (int jj = 0; jj < NV; ++jj)
                oc[k][jj] = coherent_load4(ro, (slot * D + 4 * sub + 64 * jj) * 4);
        }
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            const float wgt = mc[k] == kNegInfV ? 0.0f : __builtin_amdgcn_exp2f(mc[k] - M);
            L += wgt * lc[k];
#pragma unroll
            for (int jj = 0; jj < NV; ++jj) acc[jj] += wgt * oc[k][jj];
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int jj = 0; jj < NV; ++jj) *reinterpret_cast<f32x4 *>(op + 4 * sub + 64 * jj) = acc[jj] * inv;
}

template <int D>
hipError_t launch_v(const AttnArgs &a, const AttnPlan &pl, hipStream_t stream) {
    const size_t smem = sizeof(float) * VCfg<D>::FLOATS;
    hipError_t e = hipFuncSetAttribute((const void *)attn_valu_kernel<D>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
    ValuParams p;
    p.q = static_cast<const float *>(a.q);
    p.kt = static_cast<const float *>(a.k_tree);
    p.vt = static_cast<const float *>(a.v_tree);
    p.kc = static_cast<const float *>(a.cache.k);
    p.vc = static_cast<const float *>(a.cache.v);
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
    p.out = a.out;
    p.counters = pl.fused ? a.ws_cnt : nullptr;
    const int grid = (p.total + kNumXCD - 1) / kNumXCD * kNumXCD;
    hipLaunchKernelGGL(attn_valu_kernel<D>, dim3(grid), dim3(256), smem, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_valu(const AttnArgs &a, const AttnPlan &pl, int dtype,
                            hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    if (dtype != SV_F32) return hipErrorInvalidValue;  // bf16 runs on the matrix cores
    if (a.D == 128) return launch_v<128>(a, pl, stream);
    if (a.D == 256) return launch_v<256>(a, pl, stream);
    return launch_v<512>(a, pl, stream);
}

}  // namespace sv
