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
// Organisation (8 wavefronts per workgroup, two per SIMD, one workgroup per CU):
//   * a 32-row block of queries belongs to DSPLIT wavefronts (1 at head_dim 256,
//     2 at head_dim 512); each keeps the Q fragments of its share of head_dim in
//     registers and owns that share of the output;
//   * keys stream through an NST-deep ring of LDS stages, 32 keys of K and V per
//     stage, filled by direct global->LDS loads (global_load_lds_dwordx4) issued
//     NST-1 tiles ahead, so HBM latency hides behind the matrix work of the tiles
//     in between; one barrier per tile;
//   * LDS rows are padded (K by 16 bytes, V by 64 bytes) so that the K fragment reads
//     (ds_read_b128, 16 lanes per LDS cycle) and the V fragment reads
//     (ds_read_b64_tr_b16, a transposing read, 32 lanes per cycle) each touch 64
//     distinct banks, and every fragment address is one base register plus an
//     immediate;
//   * scores are formed transposed, S^T = K Q^T (v_mfma_f32_32x32x16_bf16 with keys
//     as M and query rows as N), so each lane holds one query row and 16 of the
//     tile's keys: the row max needs one swap between lane halves; with DSPLIT = 2
//     the two partial score tiles are summed through LDS first;
//   * the output is accumulated transposed, O^T = V^T P^T, so a lane keeps the
//     accumulators of the row it computed probabilities for; inside a 16-key step
//     the key order follows the score fragment's register order, so the P^T
//     fragment is the score registers as they stand, and the transposing read
//     delivers V^T in exactly that key order;
//   * the reference max only moves when a tile raises it by more than 2^8, so the
//     accumulators are rarely rescaled (the merged result does not depend on the
//     reference values used).
#include "sv_internal.h"

namespace sv {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;

template <int D>
struct MCfg {
    static constexpr int DSPLIT = D / 256;          // wavefronts sharing one row block
    static constexpr int DW = D / DSPLIT;           // head_dim share of one wavefront
    static constexpr int KS = DW / 16;              // k-steps of S^T = K Q^T
    static constexpr int DB = DW / 32;              // 32-wide d blocks of O^T
    static constexpr int KROW = D * 2 + 16;         // padded K row in LDS
    static constexpr int VROW = D * 2 + 64;         // padded V row in LDS
    static constexpr int KTILE = kKeyTile * KROW;
    static constexpr int STAGE_BYTES = kKeyTile * (KROW + VROW);  // K tile then V tile
    static constexpr int NST = D == 256 ? 4 : 2;    // ring depth
    static constexpr int NI = 2 * kKeyTile / kWaves;          // row loads per wavefront per tile
    static constexpr int XBYTES = DSPLIT > 1 ? kWaves / 2 * 64 * 16 * 4 : 0;  // score exchange
    static constexpr int SMEM = NST * STAGE_BYTES + XBYTES;
    static constexpr int ROWS_PER_WG = kWaves / DSPLIT * 32;
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
    int S, C, n_rg, total;
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

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Block-table entry of prefix position pos, or -1 when out of range.  The table is
// read through the constant address space: with a uniform pos this is a scalar load,
// which keeps the vector-memory counter free for the tile loads.
__device__ __forceinline__ int block_of(const MfmaParams &p, int b, int pos) {
    const __attribute__((address_space(4))) int32_t *tbl =
        (const __attribute__((address_space(4))) int32_t *)p.table;
    const int blk = tbl[(int64_t)b * p.max_blocks + pos / p.bs];
    return (blk >= 0 && blk < p.num_blocks) ? blk : -1;
}

// One 16-byte direct global->LDS load per lane: lane l's bytes land at LDS address
// lds_base + 16 * l.  Written as inline assembly so that the compiler does not see an
// LDS write it cannot disambiguate (it would then drain every load before each LDS
// read); completion is tracked explicitly with vmcnt.  M0 carries the LDS base; an
// SALU write of M0 needs one wait state before an LDS-DMA instruction reads it.
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 :
                 : "s"(lds_base), "v"(src)
                 : "memory", "m0");
}

// Workgroup barrier for LDS traffic only (no wait on the tile loads in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char *)p;
}

// Issue this wavefront's share of the direct global->LDS loads of one tile (keys
// [k0, k0 + 32) of K and V) into one ring stage: wavefronts 0-3 load K rows, 4-7 V
// rows, eight rows each, one row per load (rows are padded in LDS, so a load never
// spans two rows).  Keys past kend (and prefix keys whose block is out of range)
// load an in-range row instead; the score mask removes them.
template <int D>
__device__ __forceinline__ void issue_tile(const MfmaParams &p, int b, int kvh, bool tree,
                                           int k0, int kend, unsigned char *stage) {
    using Cf = MCfg<D>;
    constexpr int LANES = D / 8;  // 16-byte pieces per row: 32 or 64 lanes
    const int lane = threadIdx.x & 63;
    const int w = uni(threadIdx.x >> 6);
    const int tensor = w >> 2;            // 0: K, 1: V
    const int row0 = (w & 3) * Cf::NI;    // eight rows inside one 16-key group
    const __bf16 *src0;
    int64_t step;                         // elements between consecutive rows
    int pos0 = k0 + row0;
    pos0 = pos0 < kend ? pos0 : kend - 1;
    if (tree) {
        src0 = (tensor ? p.vt : p.kt) + (((int64_t)b * p.Hkv + kvh) * p.T + pos0) * D;
        step = D;
    } else {
        int blk = block_of(p, b, pos0);
        blk = blk < 0 ? 0 : blk;
        src0 = (tensor ? p.vc : p.kc) + (int64_t)blk * p.bstride + (int64_t)kvh * p.hstride +
               (int64_t)(pos0 % p.bs) * p.rstride;
        step = p.rstride;
    }
    unsigned char *dst0 = stage + (tensor ? Cf::KTILE + row0 * Cf::VROW : row0 * Cf::KROW);
    const int rowb = tensor ? Cf::VROW : Cf::KROW;
#pragma unroll
    for (int n = 0; n < Cf::NI; ++n) {
        int pos = k0 + row0 + n;
        pos = pos < kend ? pos : kend - 1;
        const __bf16 *src = src0 + (int64_t)(pos - pos0) * step + lane * 8;
        if (LANES == 64 || lane < LANES) dma16(src, lds_addr(dst0 + n * rowb));
    }
}

// Validity of the 32 keys of a tile (bit kk: key k0 + kk is real), from uniform values.
__device__ __forceinline__ uint32_t tile_valid(const MfmaParams &p, int b, bool tree, int k0,
                                               int kend) {
    uint32_t v = 0;
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
        const int pos = k0 + 16 * grp;
        if (pos < kend) {
            const int n = kend - pos < 16 ? kend - pos : 16;
            uint32_t bits = (n == 16 ? 0xffffu : ((1u << n) - 1u)) << (16 * grp);
            if (!tree && block_of(p, b, pos) < 0) bits = 0;
            v |= bits;
        }
    }
    return v;
}

template <int D>
__device__ __forceinline__ void tile_math(const unsigned char *ks, const unsigned char *vs,
                                          float *xs, uint32_t kvalid, bool tree, int k0,
                                          int dpart,
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
    const unsigned char *kbase = ks + l32 * Cf::KROW + dpart * Cf::DW * 2 + h * 16;
#pragma unroll
    for (int kstep = 0; kstep < Cf::KS; ++kstep) {
        const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kbase + kstep * 32);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kstep], sacc, 0, 0, 0);
    }
    if (Cf::DSPLIT > 1) {
        // sum the two partial score tiles of a wavefront pair (same rows, halves of
        // head_dim): the second half hands its scores over, the first adds and hands
        // the sum back, so both hold bit-identical scores
        f32x4 *slot = reinterpret_cast<f32x4 *>(xs + ((w >> 1) * 64 + lane) * 16);
        if (dpart == 1)
            for (int v = 0; v < 4; ++v)
                slot[v] = f32x4{sacc[4 * v], sacc[4 * v + 1], sacc[4 * v + 2], sacc[4 * v + 3]};
        lds_barrier();
        if (dpart == 0)
            for (int v = 0; v < 4; ++v) {
                const f32x4 t = slot[v];
                sacc[4 * v] += t[0];
                sacc[4 * v + 1] += t[1];
                sacc[4 * v + 2] += t[2];
                sacc[4 * v + 3] += t[3];
                slot[v] = f32x4{sacc[4 * v], sacc[4 * v + 1], sacc[4 * v + 2], sacc[4 * v + 3]};
            }
        lds_barrier();
        if (dpart == 1)
            for (int v = 0; v < 4; ++v) {
                const f32x4 t = slot[v];
                sacc[4 * v] = t[0];
                sacc[4 * v + 1] = t[1];
                sacc[4 * v + 2] = t[2];
                sacc[4 * v + 3] = t[3];
            }
    }

    // ---- mask, online softmax in log2 units; probabilities become bf16 P^T fragments.
    //      Full prefix tiles (the common case) need no masking at all.
    if (tree || kvalid != 0xffffffffu) {
        const uint32_t kv = kvalid >> (4 * h);                          // keys 4h + ...
        const uint64_t mt64 = tree ? (mrow >> (k0 + 4 * h)) : ~0ull;   // same key offset
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = (r >> 2) * 8 + (r & 3);
            const bool ok = ((kv >> off) & 1u) && ((mt64 >> off) & 1ull);
            sacc[r] = ok ? sacc[r] : kNegInf;
        }
    }
    float mt = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sacc[r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * scale_log2;   // row max over the tile, log2 units
    const bool raise = mt > mref + kRescaleSlack;
    if (__any(raise)) {
        const float mnew = fmaxf(mref, mt);
        const float alpha = mnew == kNegInf ? 1.0f : exp2f(mref - mnew);
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < Cf::DB; ++db) o[db] *= alpha;
        mref = mnew;
    }
    // exp2(s * scale_log2 - mref); a masked score (-inf) gives 0, and while a row has
    // seen no valid key its reference is taken as 0
    const float mneg = mref == kNegInf ? 0.0f : -mref;
    bf16x8 pf[2];
    float add = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, mneg));
        const __bf16 pb = (__bf16)pr;
        add += (float)pb;  // the denominator sums exactly the weights the numerator uses
        pf[r >> 3][r & 7] = pb;
    }
    lsum += add;

    // ---- O^T += V^T P^T.  The transposing read: in each 16-lane group, source lane
    //      4r + q points at 4 consecutive d of key row (16*kk2 + 8t + 4h + r); lane j of
    //      the group then receives that d column's 4 keys.
    const int g = lane >> 4;
    const int rr = (lane >> 2) & 3;
    const int qq = lane & 3;
    const unsigned char *vbase =
        vs + (4 * h + rr) * Cf::VROW + dpart * Cf::DW * 2 + ((g & 1) * 16 + 4 * qq) * 2;
#pragma unroll
    for (int kk2 = 0; kk2 < 2; ++kk2) {
#pragma unroll
        for (int db = 0; db < Cf::DB; ++db) {
            typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
            const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4 *)(vbase + (16 * kk2) * Cf::VROW + db * 64));
            const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
                (lds_bf16x4 *)(vbase + (16 * kk2 + 8) * Cf::VROW + db * 64));
            const bf16x8 a = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk2], o[db], 0, 0, 0);
        }
    }
}

// Wait until at most `left` tiles' loads of this wavefront are still in flight.
template <int NI>
__device__ __forceinline__ void wait_tiles_left(int left) {
    static_assert(2 * NI < 64, "vmcnt range");
    if (left >= 2) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * NI) : "memory");
    } else if (left == 1) {
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(NI) : "memory");
    } else {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
}

template <int D>
__global__ __launch_bounds__(512) void attn_mfma_kernel(MfmaParams p) {
    using Cf = MCfg<D>;
    static_assert(Cf::NST == 2 || Cf::NST == 4, "ring depth");
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
    float *xs = reinterpret_cast<float *>(smem + Cf::NST * Cf::STAGE_BYTES);

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
    const int ntp = end > start ? (end - start + kKeyTile - 1) / kKeyTile : 0;
    const int ntt = s == 0 ? (p.T + kKeyTile - 1) / kKeyTile : 0;
    const int nt = ntp + ntt;

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int h = lane >> 5;
    const int l32 = lane & 31;
    const int dpart = w % Cf::DSPLIT;
    const int row = rg * Cf::ROWS_PER_WG + (w / Cf::DSPLIT) * 32 + l32;
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
    // consume Q and the mask row here, so the loads are complete before the ring starts
    // and no wait for them lands inside the tile loop
#pragma unroll
    for (int kstep = 0; kstep < Cf::KS; ++kstep) asm volatile("" ::"v"(qf[kstep]));
    asm volatile("" ::"v"(mrow));

    // ring prologue: tiles 0 .. NST-2 in flight
#pragma unroll
    for (int u = 0; u < Cf::NST - 1; ++u) {
        if (u < nt) {
            const bool tr = u >= ntp;
            const int k0 = tr ? (u - ntp) * kKeyTile : start + u * kKeyTile;
            issue_tile<D>(p, b, kvh, tr, k0, tr ? p.T : end, smem + u * Cf::STAGE_BYTES);
        }
    }

    f32x16 o[Cf::DB];
#pragma unroll
    for (int db = 0; db < Cf::DB; ++db)
        for (int r = 0; r < 16; ++r) o[db][r] = 0.0f;
    float mref = kNegInf, lsum = 0.0f;

    for (int u = 0; u < nt; ++u) {
        // tiles issued after tile u that may still be in flight: min(NST - 2, nt - 1 - u)
        const int left = min(Cf::NST - 2, nt - 1 - u);
        wait_tiles_left<Cf::NI>(left);
        lds_barrier();  // tile u visible to all; stage of tile u-1 free for reuse
        const int un = u + Cf::NST - 1;
        if (un < nt) {
            const bool tr = un >= ntp;
            const int k0 = tr ? (un - ntp) * kKeyTile : start + un * kKeyTile;
            issue_tile<D>(p, b, kvh, tr, k0, tr ? p.T : end,
                          smem + (un % Cf::NST) * Cf::STAGE_BYTES);
        }
        const unsigned char *st = smem + (u % Cf::NST) * Cf::STAGE_BYTES;
        const bool tr = u >= ntp;
        const int k0 = tr ? (u - ntp) * kKeyTile : start + u * kKeyTile;
        const uint32_t kvalid = tile_valid(p, b, tr, k0, tr ? p.T : end);
        tile_math<D>(st, st + Cf::KTILE, xs, kvalid, tr, k0, dpart, qf, mrow, o, mref, lsum,
                     p.scale_log2);
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
    p.total = a.B * a.Hkv * pl.S * pl.n_rg;
    p.ws_o = a.ws_o;
    p.ws_ml = a.ws_ml;
    const int grid = (p.total + kNumXCD - 1) / kNumXCD * kNumXCD;
    hipLaunchKernelGGL(attn_mfma_kernel<D>, dim3(grid), dim3(64 * kWaves), Cf::SMEM, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_mfma(const AttnArgs &a, const AttnPlan &pl, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return a.D == 256 ? launch_d<256>(a, pl, stream) : launch_d<512>(a, pl, stream);
}

}  // namespace sv
