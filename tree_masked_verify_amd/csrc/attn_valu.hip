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
// is computed, so a tile costs one memory round trip that overlaps the arithmetic.
// Thread (row = t / 16, sub = t % 16) scores key `sub` against its row (Q row broadcast
// from LDS, the key row read as 16-byte vectors from a padded LDS row), the 16 threads
// of a row reduce the max and sum by shuffles, and the same thread then accumulates
// head_dim entries sub, sub + 16, ... of the row's output.
#include "attn_common.h"

namespace sv {
namespace {

constexpr int kRowsV = 16;
constexpr int kKeysV = 16;
constexpr float kNegInfV = -__builtin_huge_valf();

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
    static constexpr int QS = 0;                      // [16][D]
    static constexpr int KS = QS + kRowsV * D;        // [16][KROW]
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
    float *qs = fsm + Cf::QS;
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

    // stage Q rows (16-byte pieces)
    for (int e = tid; e < kRowsV * D / 4; e += blockDim.x) {
        const int r = e / (D / 4), d4 = e - r * (D / 4);
        const int rr = rg * kRowsV + r;
        f32x4 v = f32x4{0.f, 0.f, 0.f, 0.f};
        if (rr < p.R) {
            const int gg = rr / p.T, ii = rr - (rr / p.T) * p.T;
            v = *reinterpret_cast<const f32x4 *>(
                p.q + (((int64_t)b * p.Hq + (int64_t)kvh * p.G + gg) * p.T + ii) * D + 4 * d4);
        }
        *reinterpret_cast<f32x4 *>(qs + r * D + 4 * d4) = v;
    }
    const uint64_t mrow = row_ok ? p.mask[(int64_t)b * p.T + node] : 0ull;

    // Tile u: prefix keys start + 16u .. (u < ntp), else tree rows 16 (u - ntp) ...  This
    // thread's pieces j: key kk = (tid + 256 j) / (D / 4), 16-byte piece d4 of that key.
    // A key that does not exist (past the chunk or the tree, or behind an out-of-range
    // block entry) is staged as zeros and marked absent.
    f32x4 kreg[Cf::PER], vreg[Cf::PER];
    bool kok[Cf::PER];
    auto fetch = [&](int u) {
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
            } else if (pos < end) {
                const int32_t blk = p.table[(int64_t)b * p.max_blocks + pos / p.bs];
                if (blk >= 0 && blk < p.num_blocks)
                    off = (int64_t)blk * p.bstride + (int64_t)kvh * p.hstride +
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

    constexpr int DPT = D / kKeysV;  // output entries per thread
    float o[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) o[j] = 0.0f;
    float m = kNegInfV, l = 0.0f;

    if (nt > 0) fetch(0);
    for (int u = 0; u < nt; ++u) {
        const bool tree = u >= ntp;
        const int k0 = tree ? (u - ntp) * kKeysV : start + u * kKeysV;
        __syncthreads();  // previous tile fully consumed (and Q staged)
        stash();
        __syncthreads();
        if (u + 1 < nt) fetch(u + 1);  // in flight while this tile is computed

        // score of key `sub` for row `rl`: four independent partial sums over head_dim
        const int pos = k0 + sub;
        bool ok = okk[sub] != 0;
        if (tree) ok = ok && ((mrow >> pos) & 1ull);
        const f32x4 *qr = reinterpret_cast<const f32x4 *>(qs + rl * D);
        const f32x4 *kr = reinterpret_cast<const f32x4 *>(ks + sub * Cf::KROW);
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int d4 = 0; d4 < D / 4; ++d4) {
            const f32x4 a = qr[d4], c = kr[d4];
            acc[0] = fmaf(a[0], c[0], acc[0]);
            acc[1] = fmaf(a[1], c[1], acc[1]);
            acc[2] = fmaf(a[2], c[2], acc[2]);
            acc[3] = fmaf(a[3], c[3], acc[3]);
        }
        const float dot = (acc[0] + acc[1]) + (acc[2] + acc[3]);
        const float x = ok ? dot * p.scale_log2 : kNegInfV;
        float mt = x;
#pragma unroll
        for (int off = 1; off < kKeysV; off <<= 1) mt = fmaxf(mt, __shfl_xor(mt, off, 64));
        const float mnew = fmaxf(m, mt);
        const float alpha = mnew == kNegInfV ? 1.0f : exp2f(m - mnew);
        const float pr = x == kNegInfV ? 0.0f : exp2f(x - mnew);
        float lt = pr;
#pragma unroll
        for (int off = 1; off < kKeysV; off <<= 1) lt += __shfl_xor(lt, off, 64);
        l = l * alpha + lt;
        m = mnew;
        ps[rl * kKeysV + sub] = pr;
        __syncthreads();
        float pk[kKeysV];
#pragma unroll
        for (int k = 0; k < kKeysV; ++k) pk[k] = ps[rl * kKeysV + k];
#pragma unroll
        for (int j = 0; j < DPT; ++j) {
            const int d = sub + kKeysV * j;
            float a2 = o[j] * alpha;
#pragma unroll
            for (int k = 0; k < kKeysV; ++k) a2 = fmaf(pk[k], vs[k * D + d], a2);
            o[j] = a2;
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
            for (int j = 0; j < DPT; ++j) op[sub + kKeysV * j] = o[j] * inv;
        }
        return;
    }
    const int64_t ubase = ((int64_t)b * p.Hkv + kvh) * p.S * (int64_t)p.R;  // slot (s, r)
    if (row_ok) {
        const int64_t base = ubase + (int64_t)s * p.R + row;
#pragma unroll
        for (int j = 0; j < DPT; ++j) p.ws_o[base * D + sub + kKeysV * j] = o[j];
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
#pragma unroll
    for (int off = 1; off < kKeysV; off <<= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    constexpr int GRP = 4;
    float acc[DPT];
#pragma unroll
    for (int j = 0; j < DPT; ++j) acc[j] = 0.0f;
    float L = 0.0f;
    for (int c0 = 0; c0 < nv; c0 += GRP) {
        float mc[GRP], lc[GRP], oc[GRP][DPT];
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            const int c = c0 + k < nv ? c0 + k : nv - 1;
            const uint32_t slot = (uint32_t)c * p.R + row;
            mc[k] = c0 + k < nv ? coherent_load1(rml, slot * 8) : kNegInfV;
            lc[k] = coherent_load1(rml, slot * 8 + 4);
#pragma unroll
            for (int j = 0; j < DPT; ++j)
                oc[k][j] = coherent_load1(ro, (slot * D + sub + kKeysV * j) * 4);
        }
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            const float wgt = mc[k] == kNegInfV ? 0.0f : exp2f(mc[k] - M);
            L += wgt * lc[k];
#pragma unroll
            for (int j = 0; j < DPT; ++j) acc[j] += wgt * oc[k][j];
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
    for (int j = 0; j < DPT; ++j) op[sub + kKeysV * j] = acc[j] * inv;
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
