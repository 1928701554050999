// attn_mfma256.hip -- tree-masked split-KV attention for head_dim 256 on the gfx950
// matrix cores, one wavefront per SIMD.
//
// What is computed (ADR-037 Phase status rows E1.1-E1.5, section 4 Phase E1;
// Medusa/EAGLE-2 page "What's not implemented" 1(c)): every query row (q head g of
// kv head kvh, tree node i) attends to the cached prefix of its sequence and to
// the tree rows its ancestor mask selects.  One workgroup covers one
// (sequence, kv head, prefix chunk, row group); it leaves an unnormalised partial
// output and its (reference max, sum) per row, merged afterwards by attn_reduce.
//
// Organisation (4 wavefronts per workgroup, one per SIMD, one workgroup per CU):
//   * a wavefront owns 64 query rows as two 32-row blocks; their Q fragments stay in
//     registers (128 VGPRs) and their output accumulators in the accumulation
//     registers (256 AGPRs), so every K and V fragment read from LDS serves 64 rows;
//   * keys stream through a 4-deep ring of LDS stages, 32 keys of K and V per stage,
//     filled by direct global->LDS loads (global_load_lds_dwordx4, 1 KB per load)
//     issued two tiles ahead between the matrix instructions; one barrier per tile;
//   * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//     (32 keys x 32 rows per block): a lane holds 16 keys of one row, and the other
//     16 keys of that row sit in the lane 32 apart, so the row max is one lane swap;
//   * the output is accumulated transposed, O^T = V^T P^T, in 32 x 32 blocks over
//     16-key chunks; the chunk's key order follows the score registers, so the P^T
//     fragment is the score registers as they stand, and two transposing LDS reads
//     (ds_read_b64_tr_b16) deliver V^T in exactly that order;
//   * the softmax of tile u runs between the matrix instructions of the PV product of
//     tile u-1, so the one wavefront of a SIMD keeps the matrix core busy by itself;
//   * the reference max only moves when a tile raises it by more than 2^8, so the
//     accumulators are rarely rescaled (the merged result does not depend on the
//     reference values used).
#include "attn_common.h"

namespace sv {
namespace {

namespace w4 {

#ifndef SV_W4_KD
#define SV_W4_KD 5  // K fragments read ahead (k-steps)
#endif
#ifndef SV_W4_VD
#define SV_W4_VD 4  // V fragments read ahead (d blocks)
#endif

constexpr int D = 256;
constexpr int kW = 4;                    // wavefronts per workgroup
constexpr int kRowsPerWave = 64;
constexpr int kRowsPerWG = kW * kRowsPerWave;
constexpr int KS = D / 16;               // 16-wide k-steps of S^T = K Q^T
constexpr int DB = D / 32;               // 32-wide d blocks of O^T
// LDS tile: 16 units of 1 KB per tensor, unit p holding keys p and p + 16 side by side
// (one wavefront-wide direct load each).  K units are padded by 16 bytes (the K
// fragment read, 16 lanes x 16 bytes per LDS cycle, then touches 64 distinct banks),
// V units by 64 bytes (the transposing read, 32 lanes x 8 bytes per cycle over four
// units, likewise).
constexpr int UNITS = 16;
constexpr int KU = 1024 + 16;
constexpr int VU = 1024 + 64;
constexpr int KTILE = UNITS * KU;
constexpr int STAGE_BYTES = UNITS * (KU + VU);
constexpr int NST = 4;                   // ring depth
constexpr int LOOK = 2;                  // tiles loaded ahead
constexpr int NI = 2 * UNITS / kW;       // loads per wavefront per tile
constexpr int VMWAIT = NI * (LOOK - 1);  // loads left in flight at a wait
constexpr int kGrpMax = 2048;            // 16-key groups of one chunk in the LDS table
constexpr int GTAB_OFF = NST * STAGE_BYTES;
constexpr int MASK_OFF = GTAB_OFF + kGrpMax * 4;
constexpr uint32_t kNoGroup = 0xffffffffu;  // group table: block entry out of range
constexpr int SMEM = MASK_OFF + kRowsPerWG * 8;
static_assert(SMEM <= 160 * 1024, "LDS budget");

// LDS offset of key r of a tile (K or V unit stride u).
__device__ __forceinline__ int key_offset(int r, int u) { return (r & 15) * u + (r >> 4) * 512; }

// Issues the whole tree tile (rows past the last node read the last node, masked); the
// returned descriptor re-reads the last node (for repeat slots).
__device__ __forceinline__ TileLoad issue_tree(const MfmaParams &p, int b, int kvh, int k0,
                                               uint32_t stage) {
    const int w = uni(threadIdx.x >> 6);
    const int tensor = w >> 1;
    const int q = w & 1;
    const int half = (int)((threadIdx.x & 63) >> 5);
    const unsigned char *base = reinterpret_cast<const unsigned char *>(tensor ? p.vt : p.kt) +
                                ((int64_t)b * p.Hkv + kvh) * p.T * (D * 2) + (threadIdx.x & 31) * 16;
    const int row = k0 + 8 * q + 16 * half;
    TileLoad t;
    t.ustride = tensor ? VU : KU;
    t.lds = stage + (tensor ? KTILE : 0) + q * NI * t.ustride;
#pragma unroll
    for (int j = 0; j < NI; ++j)
        dma16(base + (int64_t)min(row + j, p.T - 1) * (D * 2), t.lds + j * t.ustride);
    t.src = base + (int64_t)(p.T - 1) * (D * 2);
    t.step = 0;
    t.spread = false;
    return t;
}

// Max over the two lanes of a row (lanes l and l ^ 32).
__device__ __forceinline__ float max_over_halves(float m) {
    const unsigned u = __float_as_uint(m);
    const auto c = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// The score product keeps its accumulators in VGPRs (the softmax reads them) while the
// output product keeps its 256 accumulators in AGPRs.  The compiler picks one register
// file for every matrix instruction of a function (the AGPR form here), so the score
// product's matrix instructions are written out.  Their operands come from LDS reads
// (ordered by the waits the compiler places before the statement) and from Q, loaded
// before the loop; consecutive products on one accumulator have another product
// between them, as in compiler-scheduled code.
__device__ __forceinline__ void mfma_vgpr_first(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}

__device__ __forceinline__ void mfma_vgpr(f32x16 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// A VALU read of a result needs 18 wait states after the (16-pass) matrix instruction
// that wrote it; the results pass through this statement, so every read follows it.
__device__ __forceinline__ void vgpr_read_guard(f32x16 &x, f32x16 &y) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" : "+v"(x), "+v"(y));
}

// S^T = K Q^T for one tile: A = K (32 keys x 16 d; lane: key l % 32, d 16 ks + 8 (l / 32)
// .. +8), B = Q^T (lane: row l % 32, same d).  sacc[rb] element r: row rb*32 + l % 32,
// key (r / 4) * 8 + (l / 32) * 4 + r % 4.  hook(ks) runs before each k-step's products.
template <class Hook>
__device__ __forceinline__ void tile_scores(const unsigned char *ks, const bf16x8 (&qf)[2][KS],
                                            f32x16 (&sacc)[2], Hook &&hook) {
    const int lane = threadIdx.x & 63;
    const unsigned char *kb = ks + key_offset(lane & 31, KU) + (lane >> 5) * 16;
    // K fragments are read KD k-steps ahead of their products; the reads sit before the
    // tile loads the hook issues (which the compiler does not move reads across)
    constexpr int KD = SV_W4_KD;
    bf16x8 a[KD + 1];
#pragma unroll
    for (int k = 0; k < KD; ++k) a[k] = *reinterpret_cast<const bf16x8 *>(kb + k * 32);
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        if (k + KD < KS) a[(k + KD) % (KD + 1)] = *reinterpret_cast<const bf16x8 *>(kb + (k + KD) * 32);
        hook(k);
        const bf16x8 &ak = a[k % (KD + 1)];
        if (k == 0) {
            mfma_vgpr_first(sacc[0], ak, qf[0][0]);
            mfma_vgpr_first(sacc[1], ak, qf[1][0]);
        } else {
            mfma_vgpr(sacc[0], ak, qf[0][k]);
            mfma_vgpr(sacc[1], ak, qf[1][k]);
        }
    }
    vgpr_read_guard(sacc[0], sacc[1]);
}

// Scores of keys that do not exist (past the chunk or the tree, or in an out-of-range
// block) or that the ancestor mask excludes become -inf.
__device__ __forceinline__ void mask_scores(f32x16 (&sacc)[2], uint32_t kvalid, bool tree, int k0,
                                            const uint64_t *mrow) {
    const int h = (threadIdx.x & 63) >> 5;
    const uint32_t kv = kvalid >> (4 * h);  // bit (r / 4) * 8 + r % 4: key of element r
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const uint64_t mt64 = tree ? (mrow[rb * 32] >> (k0 + 4 * h)) : ~0ull;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int off = (r >> 2) * 8 + (r & 3);
            const bool ok = ((kv >> off) & 1u) && ((mt64 >> off) & 1ull);
            sacc[rb][r] = ok ? sacc[rb][r] : kNegInf;
        }
    }
}

// Online softmax in log2 units, first half: the row max over the tile; the reference
// max of a row moves (to the tile max) only when the tile exceeds it by more than
// kRescaleSlack, and alpha is the factor the row's earlier sums and accumulators must
// take (1 when it did not move).  mneg = -reference (0 while a row has seen no valid key).
__device__ __forceinline__ void tile_max(const f32x16 (&sacc)[2], float (&mref)[2], float (&lsum)[2],
                                         float (&alpha)[2], float (&mneg)[2], float scale_log2) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        float m8[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) m8[j] = __builtin_fmaxf(sacc[rb][2 * j], sacc[rb][2 * j + 1]);
        float mt = __builtin_fmaxf(__builtin_fmaxf(__builtin_fmaxf(m8[0], m8[1]), __builtin_fmaxf(m8[2], m8[3])),
                                   __builtin_fmaxf(__builtin_fmaxf(m8[4], m8[5]), __builtin_fmaxf(m8[6], m8[7])));
        mt = max_over_halves(mt) * scale_log2;
        const bool raise = mt > mref[rb] + kRescaleSlack;
        const float mnew = raise ? mt : mref[rb];
        alpha[rb] = raise ? __builtin_amdgcn_exp2f(mref[rb] - mnew) : 1.0f;  // 0 when nothing seen yet
        mref[rb] = mnew;
        mneg[rb] = mnew == kNegInf ? 0.0f : -mnew;
        lsum[rb] *= alpha[rb];
    }
}

// Second half, for key chunk c: probabilities exp2(s * scale_log2 - mref) (a masked
// score, -inf, gives 0) as the bf16 P^T fragment pf[rb][c] (element j = score element
// 8c + j), and exactly those bf16 values added to the row sums.
__device__ __forceinline__ void tile_probs(const f32x16 (&sacc)[2], int c, const float (&mneg)[2],
                                           float (&lsum)[2], bf16x8 (&pf)[2][2], float scale_log2) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int j = 0; j < 8; j += 2) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[rb][8 * c + j], scale_log2, mneg[rb]));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[rb][8 * c + j + 1], scale_log2, mneg[rb]));
            const bf16x2 pk = {(__bf16)p0, (__bf16)p1};
            lsum[rb] = __builtin_amdgcn_fdot2_f32_bf16(pk, ones, lsum[rb], false);
            pf[rb][c][j] = pk[0];
            pf[rb][c][j + 1] = pk[1];
        }
    }
}

// O^T += V^T P^T over one 16-key chunk c of a tile (keys 16c .. 16c+15), whose V rows
// start at vc = the tile's V + 512 c; pc[rb] is the chunk's P^T fragment.  A = V^T (32 d x 16
// keys; lane l: d 32 db + l % 32, keys 16c + 4 (l / 32) + 0..3 and 16c + 8 + 4 (l / 32)
// + 0..3, the P^T fragment's order).  The transposing read: in each 16-lane group G,
// source lane 4r + q points at 4 consecutive d (32 db + 16 (G % 2) + 4q ..) of key
// 16c + 4 (G / 2) + r; lane j of the group then receives d 32 db + 16 (G % 2) + j of
// those 4 keys.
__device__ __forceinline__ void pv_one(const unsigned char *vc, const bf16x8 (&pc)[2], f32x16 (&o)[2][DB]) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4;
    const int r = (lane >> 2) & 3;
    const int q = lane & 3;
    const unsigned char *vb = vc + ((G >> 1) * 4 + r) * VU + (G & 1) * 32 + q * 8;
    // V^T fragments of the next VD d blocks are in flight while a block's products run
    constexpr int VD = SV_W4_VD;
    bf16x8 v[VD + 1];
    auto read = [&](int db) {
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(vb + db * 64));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4 *)(vb + 8 * VU + db * 64));
        v[db % (VD + 1)] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
#pragma unroll
    for (int db = 0; db < VD; ++db) read(db);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
        if (db + VD < DB) read(db + VD);
        o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[db % (VD + 1)], pc[0], o[0][db], 0, 0, 0);
        o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[db % (VD + 1)], pc[1], o[1][db], 0, 0, 0);
    }
}

__device__ __forceinline__ void pv_chunk(const unsigned char *vs, int c, const bf16x8 (&pf)[2][2],
                                         f32x16 (&o)[2][DB]) {
    const bf16x8 pc[2] = {pf[0][c], pf[1][c]};
    pv_one(vs + c * 512, pc, o);
}

// x *= s for an accumulator element held in an AGPR, without giving it a VGPR home (a
// VALU multiply on the accumulator tuples makes the register allocator move all 256
// accumulators into VGPRs, which do not hold them).
__device__ __forceinline__ float scale_agpr(float x, float s) {
    float t;
    asm("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
        : "+a"(x), "=&v"(t)
        : "v"(s));
    return x;
}

// Keeps the probabilities of chunk c computed before the (rarely taken) rescale branch
// rather than sunk past it, so that chunk 1's softmax stays between the matrix
// instructions of chunk 0's PV product.
__device__ __forceinline__ void settle(const bf16x8 (&pf)[2][2], int c) {
    asm volatile("" ::"v"(pf[0][c]), "v"(pf[1][c]));
}

// O *= alpha per row block, when any lane's reference max moved.  The accumulator
// reads are in assembly the compiler does not look into, so the 18 wait states after
// the last matrix instruction are given here, fenced against rescheduling.
__device__ __forceinline__ void rescale(f32x16 (&o)[2][DB], const float (&alpha)[2]) {
    if (__any(alpha[0] != 1.0f || alpha[1] != 1.0f)) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[rb][db][r] = scale_agpr(o[rb][db][r], alpha[rb]);
        // and 2 wait states before a matrix instruction reads what a VALU op wrote
        asm volatile("s_nop 1" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_w4_kernel(MfmaParams p) {
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];

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
    const int n = lane & 31;
    const int h = lane >> 5;
    const int row_base = rg * kRowsPerWG + w * kRowsPerWave + n;  // rows row_base + 32 rb

    // Q fragments (B operand of S^T): row rb*32 + n, d = 16 ks + 8 h .. +8; each row's
    // ancestor mask goes to LDS (read on tree tiles only)
    bf16x8 qf[2][KS];
    uint64_t *mrow = reinterpret_cast<uint64_t *>(smem + MASK_OFF) + w * kRowsPerWave + n;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = row_base + rb * 32;
        const bool valid = row < p.R;
        const int gh = valid ? row / p.T : 0;
        const int i = valid ? row - gh * p.T : 0;
        const __bf16 *qp = p.q + (((int64_t)b * p.Hq + (int64_t)kvh * p.G + gh) * p.T + i) * D + 8 * h;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            if (valid) {
                qf[rb][k] = *reinterpret_cast<const bf16x8 *>(qp + 16 * k);
            } else {
                for (int j = 0; j < 8; ++j) qf[rb][k][j] = (__bf16)0.0f;
            }
        }
        const uint64_t m = valid ? p.mask[(int64_t)b * p.T + i] : 0ull;
        if (h == 0) mrow[rb * 32] = m;
    }
    // consume Q here, so the loads are complete before the ring starts and no wait for
    // them lands inside the tile loop
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int k = 0; k < KS; ++k) asm volatile("" ::"v"(qf[rb][k]));

    // The chunk's 16-key groups: group j holds keys start + 16j .. +15, all in one cache
    // block.  When the chunk has at most kGrpMax groups and every group's row offset
    // fits (in 16-byte units), the offsets are staged in LDS (kNoGroup: block entry out
    // of range); otherwise groups are looked up in the block table directly.
    const int ngroups = ntp > 0 ? (end - start + 15) / 16 : 0;
    uint32_t *gtab = reinterpret_cast<uint32_t *>(smem + GTAB_OFF);
    bool staged = ngroups <= kGrpMax;
    bool all_ok = true;
    if (ntp > 0) {
        for (int j = (int)threadIdx.x; j < ngroups; j += blockDim.x) {
            const int pos = start + 16 * j;
            const int idx = pos / p.bs;
            const int blk = p.table[(int64_t)b * p.max_blocks + idx];
            const bool ok = blk >= 0 && blk < p.num_blocks;
            all_ok = all_ok && ok;
            const int64_t off16 = ok ? ((int64_t)blk * p.bstride + (int64_t)(pos - idx * p.bs) * p.rstride) / 8 : 0;
            staged = staged && off16 < (int64_t)kNoGroup;
            if (j < kGrpMax) gtab[j] = ok ? (uint32_t)off16 : kNoGroup;
        }
        // workgroup-wide flags, made visibly uniform (branches on them stay scalar)
        all_ok = uni(__syncthreads_and(all_ok)) != 0;
        staged = uni(__syncthreads_and(staged)) != 0;  // also publishes the LDS table
    }
    // byte offset (in the pool, head excluded) of group j's first row; false when its
    // block entry is out of range, and the offset is then that of block 0 (a valid
    // address whose keys the mask removes)
    auto group_off = [&](int j, int64_t &off) -> bool {
        if (staged) {
            const uint32_t v = gtab[j];
            off = v == kNoGroup ? 0 : (int64_t)v * 16;
            return v != kNoGroup;
        }
        const int pos = start + 16 * j;
        const int idx = pos / p.bs;
        const int blk = table_entry(p, b, idx);
        off = ((int64_t)(blk < 0 ? 0 : blk) * p.bstride + (int64_t)(pos - idx * p.bs) * p.rstride) * 2;
        return blk >= 0;
    };

    f32x16 o[2][DB];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[rb][db][r] = 0.0f;
    float mref[2] = {kNegInf, kNegInf};
    float lsum[2] = {0.0f, 0.0f};
    float alpha[2], mneg[2];
    bf16x8 pf[2][2];
    f32x16 sacc[2];

    // ---- tile loads.  Wavefront w loads tensor w / 2 (K, V), units (w % 2) * 8 + j of a
    // tile; lanes 0-31 carry key p of unit p, lanes 32-63 key p + 16.  Every tile slot
    // k < nt + LOOK issues exactly NI loads per wavefront (slots past the last tile repeat
    // the last tile's sources into a free stage), so "tile u has landed" is always the
    // same vmcnt, and the ring drains before exit.
    const uint32_t smem0 = lds_addr(smem);
    const int wq = uni(w & 1);
    const int tensor = uni(w >> 1);
    const int half = h;
    const int ustride = tensor ? VU : KU;
    const uint32_t lds_w = (tensor ? KTILE : 0) + wq * NI * ustride;
    const unsigned char *pool_w = reinterpret_cast<const unsigned char *>(tensor ? p.vc : p.kc) +
                                  (int64_t)kvh * p.hstride * 2;
    const int64_t step = p.rstride * 2;
    // per lane: its 16 bytes of the wavefront's first row inside a group
    const int64_t lane_off = (int64_t)(8 * wq) * step + (lane & 31) * 16;
    TileLoad tl;
    tl.ustride = ustride;
    auto prepare = [&](int k) {  // any tile slot
        const uint32_t stage = smem0 + (k & (NST - 1)) * STAGE_BYTES;
        if (k < ntp) {
            const int k0 = start + k * kKeyTile;
            int64_t off0, off1;
            group_off(2 * k, off0);
            if (k0 + 16 < end) {
                group_off(2 * k + 1, off1);
            } else {
                off1 = off0;  // group past the chunk end: re-read group 0 (masked)
            }
            tl.src = pool_w + (half ? off1 : off0) + lane_off;
            tl.step = step;
            tl.lds = stage + lds_w;
            tl.spread = true;
        } else if (k < nt) {
            tl = issue_tree(p, b, kvh, (k - ntp) * kKeyTile, stage);
        } else {
            tl.lds = stage + lds_w;
            tl.spread = true;
        }
    };
    auto issue = [&](int k) {
        prepare(k);
        if (tl.spread)
#pragma unroll
            for (int j = 0; j < NI; ++j) load_unit(tl, j);
    };
    // the NI loads of the prepared tile go between the k-steps of the score product
    auto load_in_scores = [&](int k) {
        constexpr int every = KS / NI;
        if (k % every == 0 && tl.spread) load_unit(tl, k / every);
    };

    // ---- one tile.  The PV products run one half-tile behind the softmax: tile u's
    // max and chunk-0 probabilities go between the matrix instructions of tile u-1's
    // chunk-1 PV product, and tile u's chunk-1 probabilities between those of its own
    // chunk-0 PV product.  Before the first tile the pending product adds zeros.
    bf16x8 pprev[2];  // P^T fragments of the pending chunk-1 product
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int j = 0; j < 8; ++j) pprev[rb][j] = (__bf16)0.0f;
    const unsigned char *vprev = smem + KTILE;  // V of the pending product (tile 0 at first)
    auto compute = [&](int u, bool masked, uint32_t kvalid, bool tree, int k0, auto &&hook) {
        const unsigned char *stg = smem + (u & (NST - 1)) * STAGE_BYTES;
        tile_scores(stg, qf, sacc, hook);
        if (masked) mask_scores(sacc, kvalid, tree, k0, mrow);
        pv_one(vprev, pprev, o);
        tile_max(sacc, mref, lsum, alpha, mneg, p.scale_log2);
        tile_probs(sacc, 0, mneg, lsum, pf, p.scale_log2);
        settle(pf, 0);
        rescale(o, alpha);
        pv_chunk(stg + KTILE, 0, pf, o);
        tile_probs(sacc, 1, mneg, lsum, pf, p.scale_log2);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) pprev[rb] = pf[rb][1];
        vprev = stg + KTILE + 512;
    };

    for (int k = 0; k < LOOK; ++k) issue(k);  // ring prologue
    int u = 0;
    if (staged && all_ok) {
        // full prefix tiles whose loads LOOK tiles ahead are full prefix tiles too: group
        // offsets read one tile early, no masking, no branches around the loads
        const int nfast = (end - start) / kKeyTile - LOOK;
        uint32_t gnext = nfast > 0 ? gtab[2 * LOOK + half] : 0;
        for (; u < nfast; ++u) {
            wait_loads<VMWAIT>();
            lds_barrier();  // tile u visible to all; stage of tile u - 2 free for reuse
            const uint32_t g = gnext;
            gnext = gtab[min(2 * (u + LOOK + 1) + half, kGrpMax - 1)];
            TileLoad f;
            f.src = pool_w + (int64_t)g * 16 + lane_off;
            f.step = step;
            f.lds = smem0 + ((u + LOOK) & (NST - 1)) * STAGE_BYTES + lds_w;
            f.ustride = ustride;
            compute(u, false, 0u, false, 0, [&](int k) {
                constexpr int every = KS / NI;
                if (k % every == 0) load_unit(f, k / every);
            });
        }
        tl = TileLoad{pool_w + lane_off, step, 0u, ustride, true};  // repeat-slot source
    }
    for (; u < nt; ++u) {
        wait_loads<VMWAIT>();
        lds_barrier();
        prepare(u + LOOK);
        const bool tr = u >= ntp;
        int k0;
        uint32_t kvalid;
        if (tr) {
            k0 = (u - ntp) * kKeyTile;
            kvalid = tree_valid(k0, p.T);
        } else {
            k0 = start + u * kKeyTile;
            kvalid = 0;
#pragma unroll
            for (int grp = 0; grp < 2; ++grp) {
                const int pos = k0 + 16 * grp;
                if (pos < end) {
                    int64_t off;
                    const int nk = end - pos < 16 ? end - pos : 16;
                    if (group_off(2 * u + grp, off))
                        kvalid |= (nk == 16 ? 0xffffu : ((1u << nk) - 1u)) << (16 * grp);
                }
            }
        }
        compute(u, tr || kvalid != 0xffffffffu, kvalid, tr, k0, load_in_scores);
    }
    pv_one(vprev, pprev, o);  // the last tile's chunk-1 product
    wait_loads<0>();  // the trailing repeat loads

    // ---- partial results: O (unnormalised), reference max (log2 units) and sum per row;
    //      accumulator element r of block (rb, db) is d = 32 db + 8 (r / 4) + 4 h + r % 4
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const float ltot = lsum[rb] + __shfl_xor(lsum[rb], 32, 64);
        const int row = row_base + rb * 32;
        if (row < p.R) {
            const int64_t base = (((int64_t)b * p.Hkv + kvh) * p.S + s) * p.R + row;
            float *op = p.ws_o + base * D + 4 * h;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    *reinterpret_cast<f32x4 *>(op + db * 32 + g4 * 8) =
                        f32x4{o[rb][db][4 * g4], o[rb][db][4 * g4 + 1], o[rb][db][4 * g4 + 2],
                              o[rb][db][4 * g4 + 3]};
            if (h == 0) {
                p.ws_ml[base * 2 + 0] = mref[rb];
                p.ws_ml[base * 2 + 1] = ltot;
            }
        }
    }
}

}  // namespace w4

}  // namespace

hipError_t launch_attn_mfma256(const AttnArgs &a, const AttnPlan &pl, hipStream_t stream) {
    using namespace w4;
    if (a.B == 0) return hipSuccess;
    hipError_t e = hipFuncSetAttribute((const void *)attn_w4_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, SMEM);
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
    hipLaunchKernelGGL(attn_w4_kernel, dim3(grid), dim3(64 * kW), SMEM, stream, p);
    return hipGetLastError();
}

}  // namespace sv
