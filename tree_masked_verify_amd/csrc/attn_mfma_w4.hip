// attn_mfma_w4.hip -- tree-masked split-KV attention for head_dim 128 and 256 on the
// gfx950 matrix cores, one wavefront per SIMD.
//
// What is computed (ADR-037 Phase status rows E1.1-E1.5, section 4 Phase E1, and row
// E4b.6 for head_dim 128; Medusa/EAGLE-2 page "What's not implemented" 1(c)): every query row (q head g of
// kv head kvh, tree node i) attends to the cached prefix of its sequence and to
// the tree rows its ancestor mask selects.  One workgroup covers one
// (sequence, kv head, prefix chunk, row group); it leaves an unnormalised partial
// output and its (reference max, sum) per row, merged afterwards by attn_reduce.
//
// Organisation (4 wavefronts per workgroup, one per SIMD, one workgroup per CU):
//   * a wavefront owns 64 query rows as two 32-row blocks; their Q fragments stay in
//     registers (D / 2 VGPRs) and their output accumulators in the accumulation
//     registers (D AGPRs), so every K and V fragment read from LDS serves 64 rows;
//   * keys stream through a 4-deep ring of LDS stages, 32 keys of K and V per stage,
//     filled by direct global->LDS loads (global_load_lds_dwordx4, two key rows per load)
//     issued three tiles ahead between the score product's matrix instructions; one
//     barrier per tile;
//   * scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16
//     (32 keys x 32 rows per block): a lane holds 16 keys of one row, and the other
//     16 keys of that row sit in the lane 32 apart, so the row max is one lane swap;
//   * the output is accumulated transposed, O^T = V^T P^T, in 32 x 32 blocks over
//     16-key chunks; the chunk's key order follows the score registers, so the P^T
//     fragment is the score registers as they stand, and two transposing LDS reads
//     (ds_read_b64_tr_b16) deliver V^T in exactly that order;
//   * the probabilities of a tile's second 16-key chunk are computed between the
//     matrix instructions of its first chunk's PV product;
//   * the reference max only moves when a tile raises it by more than 2^8, so the
//     accumulators are rarely rescaled (the merged result does not depend on the
//     reference values used);
//   * with automatic splitting (balanced plan) the chunk length comes from the actual
//     prefix lengths, about one chunk per CU in all, and the chunks start largest first
//     (balanced_item), so sequences of different lengths finish together.
#include "attn_common.h"

namespace sv {
namespace {

namespace w4 {

constexpr int kKD = 5;                   // K fragments read ahead (k-steps)
constexpr int kVD = 4;                   // V fragments read ahead (d blocks)
constexpr int kW = 4;                    // wavefronts per workgroup
constexpr int kRowsPerWave = 64;
constexpr int kRowsPerWG = kW * kRowsPerWave;
constexpr int UNITS = 16;                // LDS units per tensor and tile
constexpr int NST = 4;                   // ring depth
constexpr int LOOK = 3;                  // tiles loaded ahead (a stage is free once its PV is done)
constexpr int NI = 2 * UNITS / kW;       // loads per wavefront per tile
constexpr int VMWAIT = NI * (LOOK - 1);  // loads left in flight at a wait
constexpr int kGrpMax = 2048;            // 16-key groups of one chunk in the LDS table
constexpr uint32_t kNoGroup = 0xffffffffu;  // group table: block entry out of range

// LDS tile geometry for head_dim D: 16 units per tensor, unit p holding keys p and p + 16
// side by side, each unit filled by one direct load (D = 256: 1 KB, all 64 lanes; D = 128:
// 512 bytes, lanes 0-31).  K units are padded by 16 bytes (the K fragment read, 16 lanes
// x 16 bytes per LDS cycle, then touches 64 distinct banks: unit u starts at bank offset
// 16u mod 256), V units by 64 bytes (the transposing read, 32 lanes x 8 bytes per cycle
// over four units at bank offsets 0, 64, 128, 192, likewise).
template <int D>
struct Geo {
    static constexpr int KS = D / 16;            // 16-wide k-steps of S^T = K Q^T
    static constexpr int DB = D / 32;            // 32-wide d blocks of O^T
    static constexpr int KEYB = 2 * D;           // bytes of one key row
    static constexpr int LPK = KEYB / 16;        // lanes of a load per key row
    static constexpr int UNIT = 2 * KEYB;
    static constexpr int KU = UNIT + 16;
    static constexpr int VU = UNIT + 64;
    static constexpr int KTILE = UNITS * KU;
    static constexpr int STAGE_BYTES = UNITS * (KU + VU);
    static constexpr int GTAB_OFF = NST * STAGE_BYTES;
    static constexpr int MASK_OFF = GTAB_OFF + kGrpMax * 4;
    static constexpr int FLAG_OFF = MASK_OFF + kRowsPerWG * 8;  // the merge's arrival flag
    static constexpr int SMEM = FLAG_OFF + 16;
    static_assert(D == 128 || D == 256, "head_dim 128 or 256");
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    static_assert(NST * STAGE_BYTES >= kW * DB * 4 * 64 * 16, "stages hold the O staging");
    static_assert((KU % 256) == 16 && (VU % 256) == 64, "bank offsets");
};

// LDS offset of key r of a tile (K or V unit stride u).
template <int D>
__device__ __forceinline__ int key_offset(int r, int u) { return (r & 15) * u + (r >> 4) * Geo<D>::KEYB; }

// A unit load: every lane of the wavefront with D = 256, lanes 0-31 with D = 128 (the
// others would write past the unit).
template <int D, bool kNT = false>
__device__ __forceinline__ void unit_load(const unsigned char *src, uint32_t lds) {
    if (Geo<D>::LPK == 32 || (threadIdx.x & 63) < 2 * Geo<D>::LPK) dma16<kNT>(src, lds);
}

template <int D, bool kNT>
__device__ __forceinline__ void load_unit_d(const TileLoad &t, int j) {
    unit_load<D, kNT>(load_src(t, j), t.lds + j * t.ustride);
}

// Issues the whole tree tile (rows past the last node read the last node, masked); the
// returned descriptor re-reads the last node (for repeat slots).  kInCache: the tree rows
// sit in the cache at positions P + r instead of in the tree buffers.
template <int D, bool kInCache>
__device__ __forceinline__ TileLoad issue_tree(const MfmaParams &p, int b, int kvh, int P,
                                               int k0, uint32_t stage) {
    using G = Geo<D>;
    const int w = uni(threadIdx.x >> 6);
    const int tensor = w >> 1;
    const int q = w & 1;
    const int lane = threadIdx.x & 63;
    const int half = (lane / G::LPK) & 1;
    const int row = k0 + 8 * q + 16 * half;
    TileLoad t;
    t.ustride = tensor ? G::VU : G::KU;
    t.lds = stage + (tensor ? G::KTILE : 0) + q * NI * t.ustride;
    if constexpr (kInCache) {
        const unsigned char *pool =
            reinterpret_cast<const unsigned char *>(tensor ? p.vc : p.kc) + (lane % G::LPK) * 16;
#pragma unroll
        for (int j = 0; j < NI; ++j)
            unit_load<D>(tree_row_in_cache(pool, p, b, kvh, P, min(row + j, p.T - 1)),
                         t.lds + j * t.ustride);
        t.src = tree_row_in_cache(pool, p, b, kvh, P, p.T - 1);
    } else {
        const unsigned char *base =
            reinterpret_cast<const unsigned char *>(tensor ? p.vt : p.kt) +
            ((int64_t)b * p.Hkv + kvh) * p.T * (D * 2) + (lane % G::LPK) * 16;
#pragma unroll
        for (int j = 0; j < NI; ++j)
            unit_load<D>(base + (int64_t)min(row + j, p.T - 1) * (D * 2), t.lds + j * t.ustride);
        t.src = base + (int64_t)(p.T - 1) * (D * 2);
    }
    t.step = 0;
    t.spread = false;
    t.nvalid = NI;
    t.alt = t.src;
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
template <int D, class Hook>
__device__ __forceinline__ void tile_scores(const unsigned char *ks, const bf16x8 (&qf)[2][Geo<D>::KS],
                                            f32x16 (&sacc)[2], Hook &&hook) {
    constexpr int KS = Geo<D>::KS;
    const int lane = threadIdx.x & 63;
    const unsigned char *kb = ks + key_offset<D>(lane & 31, Geo<D>::KU) + (lane >> 5) * 16;
    // K fragments are read KD k-steps ahead of their products; the reads sit before the
    // tile loads the hook issues (which the compiler does not move reads across)
    constexpr int KD = kKD;
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
        // the loads the hook issues stay in their k-step
        __builtin_amdgcn_sched_barrier(0);
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

// Online softmax in log2 units, taken in 16 pieces that run between the steps of a PV
// product.  A single wavefront issues in order, so an operation that waits for the
// result of the one before it also holds up the next matrix instruction; the pieces are
// therefore arranged so that each one only uses results of earlier pieces (one step,
// two matrix instructions, apart):
//   0-2  row maxima of both row blocks: three levels of max3/max, then the lane swap
//        (the other 16 keys of a row sit in the lane 32 apart) and the log2 scaling;
//   3    reference updates: the reference max of a row moves (to the tile max) only
//        when the tile exceeds it by more than kRescaleSlack; alpha = exp2(old - new) is
//        the factor the row's earlier sum and accumulators must take, exactly 1 when the
//        reference did not move.  A row that has seen no valid key holds the finite
//        reference kNoRef (its sum and accumulators are 0), so that alpha needs no
//        special case;
//   4-15 probabilities exp2(s * scale_log2 - mref) of 16 element pairs (one pair of each
//        row block per piece), in five stages one piece apart: the fma, the exp2, the
//        rounding to bf16 into the P^T fragment (element j of fragment c is score element
//        8c + j), the sum of exactly those two bf16 values (widened by bit shifts), and
//        its addition to the row sum.  At head_dim 128, where half as many product steps
//        hide the pieces, the last two stages are one packed dot product of the pair with
//        (1, 1) into the row sum.  A masked score (-inf) gives 0.
constexpr float kNoRef = -1.0e30f;

struct RowState {
    float mref[2], lsum[2], alpha[2];
    bool raised[2];
};

struct SoftTmp {
    float m6[2][6], m2[2][2], mt[2];
    float x[16][2], y[16][2], t[16];
};

template <bool kDotSum>
__device__ __forceinline__ void softmax_piece(int k, const f32x16 (&sp)[2], RowState &rs, SoftTmp &t,
                                              bf16x8 (&pf)[2][2], float scale_log2) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const f32x16 &sr = sp[rb];
        if (k == 0) {
#pragma unroll
            for (int j = 0; j < 5; ++j)
                t.m6[rb][j] = __builtin_fmaxf(__builtin_fmaxf(sr[3 * j], sr[3 * j + 1]), sr[3 * j + 2]);
            t.m6[rb][5] = sr[15];
        }
        if (k == 1) {
            t.m2[rb][0] = __builtin_fmaxf(__builtin_fmaxf(t.m6[rb][0], t.m6[rb][1]), t.m6[rb][2]);
            t.m2[rb][1] = __builtin_fmaxf(__builtin_fmaxf(t.m6[rb][3], t.m6[rb][4]), t.m6[rb][5]);
        }
        if (k == 2) t.mt[rb] = max_over_halves(__builtin_fmaxf(t.m2[rb][0], t.m2[rb][1])) * scale_log2;
        if (k == 3) {
            rs.raised[rb] = t.mt[rb] > rs.mref[rb] + kRescaleSlack;
            const float mnew = rs.raised[rb] ? t.mt[rb] : rs.mref[rb];
            rs.alpha[rb] = __builtin_amdgcn_exp2f(rs.mref[rb] - mnew);
            rs.mref[rb] = mnew;
            rs.lsum[rb] *= rs.alpha[rb];
        }
        // pair q = 2 i + rb (i = 0..7): elements 2i, 2i + 1 of row block rb
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int q = 2 * i + rb;
            if (k == 4 + i) {
                t.x[q][0] = fmaf(sr[2 * i], scale_log2, -rs.mref[rb]);
                t.x[q][1] = fmaf(sr[2 * i + 1], scale_log2, -rs.mref[rb]);
            }
            if (k == 5 + i) {
                t.y[q][0] = __builtin_amdgcn_exp2f(t.x[q][0]);
                t.y[q][1] = __builtin_amdgcn_exp2f(t.x[q][1]);
            }
            if (k == 6 + i) {
                pf[rb][i >> 2][2 * (i & 3)] = (__bf16)t.y[q][0];
                pf[rb][i >> 2][2 * (i & 3) + 1] = (__bf16)t.y[q][1];
            }
            if (k == 7 + i) {
                const bf16x2 pk = {pf[rb][i >> 2][2 * (i & 3)], pf[rb][i >> 2][2 * (i & 3) + 1]};
                if constexpr (kDotSum) {
                    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
                    rs.lsum[rb] = __builtin_amdgcn_fdot2_f32_bf16(pk, one, rs.lsum[rb], false);
                } else {
                    const uint32_t wv = __builtin_bit_cast(uint32_t, pk);
                    t.t[q] = __uint_as_float(wv << 16) + __uint_as_float(wv & 0xffff0000u);
                }
            }
            if (!kDotSum && k == 8 + i) rs.lsum[rb] += t.t[q];
        }
    }
}

// O^T += V^T P^T over one tile (V at vs), in two 16-key chunks c (keys 16c .. 16c+15, V
// rows from vs + 512 c) with P^T fragments pf[rb][c].  A = V^T (32 d x 16
// keys; lane l: d 32 db + l % 32, keys 16c + 4 (l / 32) + 0..3 and 16c + 8 + 4 (l / 32)
// + 0..3, the P^T fragment's order).  The transposing read: in each 16-lane group G,
// source lane 4r + q points at 4 consecutive d (32 db + 16 (G % 2) + 4q ..) of key
// 16c + 4 (G / 2) + r; lane j of the group then receives d 32 db + 16 (G % 2) + j of
// those 4 keys.
template <int D, class Hook>
__device__ __forceinline__ void pv_tile(const unsigned char *vs, const bf16x8 (&pf)[2][2],
                                        f32x16 (&o)[2][Geo<D>::DB], Hook &&hook) {
    constexpr int DB = Geo<D>::DB, VU = Geo<D>::VU;
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const int lane = threadIdx.x & 63;
    const int G = lane >> 4;
    const int r = (lane >> 2) & 3;
    const int q = lane & 3;
    const unsigned char *vb = vs + ((G >> 1) * 4 + r) * VU + (G & 1) * 32 + q * 8;
    // V^T fragments of the next VD (chunk, d block) steps are in flight while a step's
    // products run
    constexpr int VD = kVD;
    constexpr int NSTEP = 2 * DB;
    bf16x8 v[VD + 1];
    auto read = [&](int i) {
        const unsigned char *a = vb + (i / DB) * Geo<D>::KEYB + (i % DB) * 64;
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)a);
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(a + 8 * VU));
        v[i % (VD + 1)] = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
    };
#pragma unroll
    for (int i = 0; i < VD; ++i) read(i);
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
        if (i + VD < NSTEP) read(i + VD);
        hook(i);
        const int c = i / DB, db = i % DB;
        o[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[i % (VD + 1)], pf[0][c], o[0][db], 0, 0, 0);
        o[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v[i % (VD + 1)], pf[1][c], o[1][db], 0, 0, 0);
        // the hook's work stays in its step, in the shadow of that step's products
        __builtin_amdgcn_sched_barrier(0);
    }
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

// Keeps a tile's softmax where it was written, between the matrix instructions of the
// PV product, rather than sunk past the (rarely taken) rescale branch into the next
// iteration.
__device__ __forceinline__ void settle(const bf16x8 (&pf)[2][2], const RowState &rs) {
    asm volatile("" ::"v"(pf[0][0]), "v"(pf[0][1]), "v"(pf[1][0]), "v"(pf[1][1]));
    asm volatile("" ::"v"(rs.lsum[0]), "v"(rs.lsum[1]), "v"(rs.mref[0]), "v"(rs.mref[1]));
}

// O *= alpha per row block, when any lane's reference max moved.  The accumulator
// reads are in assembly the compiler does not look into, so the 18 wait states after
// the last matrix instruction are given here, fenced against rescheduling.
template <int D>
__device__ __forceinline__ void rescale(f32x16 (&o)[2][Geo<D>::DB], const RowState &rs) {
    constexpr int DB = Geo<D>::DB;
    if (__any(rs.raised[0] || rs.raised[1])) {
        __builtin_amdgcn_sched_barrier(0);
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[rb][db][r] = scale_agpr(o[rb][db][r], rs.alpha[rb]);
        // and 2 wait states before a matrix instruction reads what a VALU op wrote
        asm volatile("s_nop 1" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Output row [b][i][h][:] of query row r (q head g = r / T of kv head kvh, node i).
__device__ __forceinline__ float *out_row(const MfmaParams &p, int b, int kvh, int r) {
    const int g = r / p.T;
    const int i = r - g * p.T;
    return p.out + (((int64_t)b * p.T + i) * p.Hq + (int64_t)kvh * p.G + g) * (int64_t)p.D;
}


// The merge of the nv chunks of one (sequence, kv head, row group), rows rbase and
// rbase + 32 of this lane (its half h of each 8-wide d piece), from their partials:
//   out = sum_c 2^(m_c - M) O_c / sum_c 2^(m_c - M) l_c,  M = max_c m_c,
// over the chunks c in order, so the result does not depend on which chunk merges.
// The loads go out in batches (four d blocks of two chunks at a time), so that the
// merge waits for a few memory round trips, not one per piece.  The unit's partials
// are nv * R rows from slot ubase (the launch keeps their bytes within 2^31).
template <int D>
__device__ __forceinline__ void merge_chunks(const MfmaParams &p, int b, int kvh, int64_t ubase,
                                             int rbase, int nv) {
    constexpr int DB = Geo<D>::DB;
    constexpr int QB = DB < 4 ? DB : 4;  // d blocks per batch
    const int h = (threadIdx.x & 63) >> 5;
    const uint32_t rows = (uint32_t)nv * (uint32_t)p.R;
    const __amdgpu_buffer_rsrc_t ro = coherent_rsrc(p.ws_o + ubase * D, rows * D * 4);
    const __amdgpu_buffer_rsrc_t rml = coherent_rsrc(p.ws_ml + ubase * 2, rows * 8);
    const uint32_t cs = (uint32_t)p.R;  // slots between consecutive chunks
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = rbase + rb * 32;
        if (row >= p.R) continue;
        auto mref = [&](int c) { return coherent_load1(rml, ((uint32_t)c * cs + row) * 8); };
        auto lsum = [&](int c) { return coherent_load1(rml, ((uint32_t)c * cs + row) * 8 + 4); };
        float M = kNegInf;
        for (int c = 0; c < nv; ++c) M = fmaxf(M, mref(c));
        float L = 0.0f;
        for (int c = 0; c < nv; ++c) {
            const float m2 = mref(c);
            const float wgt = m2 == kNegInf ? 0.0f : exp2f(m2 - M);
            L += wgt * lsum(c);
        }
        const float inv = L > 0.0f ? 1.0f / L : 0.0f;
        float *op = out_row(p, b, kvh, row) + 4 * h;
#pragma unroll
        for (int q = 0; q < DB / QB; ++q) {
            f32x4 acc[QB][4];
#pragma unroll
            for (int d = 0; d < QB; ++d)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) acc[d][g4] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int c = 0; c < nv; c += 2) {
                const bool two = c + 1 < nv;
                const float m0 = mref(c);
                const float m1 = two ? mref(c + 1) : kNegInf;
                const float w0 = m0 == kNegInf ? 0.0f : exp2f(m0 - M);
                const float w1 = m1 == kNegInf ? 0.0f : exp2f(m1 - M);
                f32x4 v0[QB][4], v1[QB][4];
#pragma unroll
                for (int d = 0; d < QB; ++d)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const uint32_t e = (((uint32_t)c * cs + row) * D + (q * QB + d) * 32 + g4 * 8 + 4 * h) * 4;
                        v0[d][g4] = coherent_load4(ro, e);
                        v1[d][g4] = two ? coherent_load4(ro, e + cs * D * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
                    }
#pragma unroll
                for (int d = 0; d < QB; ++d)
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        acc[d][g4] += w0 * v0[d][g4];
                        if (two) acc[d][g4] += w1 * v1[d][g4];
                    }
            }
#pragma unroll
            for (int d = 0; d < QB; ++d)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    *reinterpret_cast<f32x4 *>(op + (q * QB + d) * 32 + g4 * 8) = acc[d][g4] * inv;
        }
    }
}

template <int D, bool kInCache, bool kNT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_w4_kernel(MfmaParams p) {
    extern __shared__ __attribute__((aligned(1024))) unsigned char smem[];
    using G = Geo<D>;
    constexpr int KS = G::KS, DB = G::DB, KU = G::KU, VU = G::VU, KTILE = G::KTILE;
    constexpr int STAGE_BYTES = G::STAGE_BYTES, GTAB_OFF = G::GTAB_OFF, MASK_OFF = G::MASK_OFF;

    int b, kvh, s, rg, C;
    if (p.balanced) {
        C = balanced_chunk_len(p);
        // for the separate merge kernel (calls whose chunks are not merged in here)
        if (!p.counters && blockIdx.x == 0 && threadIdx.x == 0) *p.ws_c = C;
        if (!balanced_item(p, C, &b, &kvh, &s, &rg)) return;
    } else {
        const int logical = xcd_logical_id();
        if (logical >= p.total) return;
        int t = logical;
        rg = t % p.n_rg;
        t /= p.n_rg;
        s = t % p.S;
        t /= p.S;
        kvh = t % p.Hkv;
        b = t / p.Hkv;
        C = p.C;
    }

    const int P = clamp_prefix(p.prefix_len[b], p.max_P);
    const int start = s * C;
    if (s > 0 && start >= P) return;  // chunk past this sequence's prefix: nothing to merge
    const int end = min(start + C, P);
    const int ntp = end > start ? (end - start + kKeyTile - 1) / kKeyTile : 0;
    const int ntt = s == 0 ? (p.T + kKeyTile - 1) / kKeyTile : 0;
    const int nt = ntp + ntt;
    if (nt == 0) return;  // no rows (the host launches nothing for an empty tree)

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
    // Rows past the last query row get the reference +inf: their probabilities are 0 (the
    // PV products then multiply zeros, which costs the matrix cores less energy), and
    // their sums and accumulators, never stored, may hold NaN.
    RowState rs;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        rs.mref[rb] = row_base + rb * 32 < p.R ? kNoRef : __builtin_huge_valf();
        rs.lsum[rb] = 0.0f;
    }
    f32x16 sc[2];  // scores of the current tile
    // P^T fragments of even (set 0) and odd (set 1) tiles; set 1 starts as those of
    // "tile -1", zero, whose PV product adds nothing
    bf16x8 pf[2][2][2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) pf[1][rb][c][j] = (__bf16)0.0f;

    // ---- tile loads.  Wavefront w loads tensor w / 2 (K, V), units (w % 2) * 8 + j of a
    // tile; lanes 0-31 carry key p of unit p, lanes 32-63 key p + 16.  Iteration u of the
    // tile loop computes the scores of tile u and the PV product of tile u - 1, so K is
    // needed one iteration before V: in iteration u the K wavefronts load tile u + 3 and
    // the V wavefronts tile u + 2, both landing three iterations before their use.  Every
    // iteration (and the three of the prologue) issues exactly NI loads per wavefront
    // (past the last tile they repeat the last sources into a free stage; before tile 0
    // the V wavefronts read tile 0), so "iteration u's operands have landed" is always the
    // same vmcnt, and the ring drains before exit.
    const uint32_t smem0 = lds_addr(smem);
    const int wq = uni(w & 1);
    const int tensor = uni(w >> 1);
    const int ahead = tensor ? 2 : 3;
    const int half = (lane / G::LPK) & 1;  // the load's key row: p (0) or p + 16 (1)
    const int ustride = tensor ? VU : KU;
    const uint32_t lds_w = (tensor ? KTILE : 0) + wq * NI * ustride;
    const unsigned char *pool_w = reinterpret_cast<const unsigned char *>(tensor ? p.vc : p.kc) +
                                  (int64_t)kvh * p.hstride * 2;
    const int64_t step = p.rstride * 2;
    // per lane: its 16 bytes of the wavefront's first row inside a group
    const int64_t lane_off = (int64_t)(8 * wq) * step + (lane % G::LPK) * 16;
    // the first 16 bytes of tree row 0 of this kv head (finite by the caller's
    // contract), read by every lane in place of rows that hold no key
    const unsigned char *alt_w = uni_ptr(
        kInCache ? tree_row_in_cache(reinterpret_cast<const unsigned char *>(tensor ? p.vc : p.kc),
                                     p, b, kvh, P, 0)
                 : reinterpret_cast<const unsigned char *>(tensor ? p.vt : p.kt) +
                       ((int64_t)b * p.Hkv + kvh) * p.T * (D * 2));
    TileLoad tl;
    tl.ustride = ustride;
    auto prepare = [&](int k) {  // this wavefront's share of tile k (k >= -1)
        const uint32_t stage = smem0 + (k & (NST - 1)) * STAGE_BYTES;
        k = k < 0 ? 0 : k;
        if (k < ntp) {
            const int k0 = start + k * kKeyTile;
            int64_t off0, off1;
            const bool ok0 = group_off(2 * k, off0);
            bool ok1 = false;
            if (k0 + 16 < end) {
                ok1 = group_off(2 * k + 1, off1);
            } else {
                off1 = off0;  // group past the chunk end: no keys
            }
            // rows of this lane's loads: keys first .. first + NI - 1 of the chunk
            const int first = k0 + 16 * half + 8 * wq;
            const int left = end - first;
            tl.nvalid = (half ? ok1 : ok0) ? (left < 0 ? 0 : (left > NI ? NI : left)) : 0;
            tl.src = pool_w + (half ? off1 : off0) + lane_off;
            tl.alt = alt_w;
            tl.step = step;
            tl.lds = stage + lds_w;
            tl.spread = true;
        } else if (k < nt) {
            tl = issue_tree<D, kInCache>(p, b, kvh, P, (k - ntp) * kKeyTile, stage);
        } else {
            // repeat slot past the last tile (scores masked, probabilities 0)
            tl.src = alt_w;
            tl.alt = alt_w;
            tl.nvalid = 0;
            tl.step = 0;
            tl.lds = stage + lds_w;
            tl.spread = true;
        }
    };
    // the NI loads of the prepared tile go between the k-steps of the score product
    auto load_in_scores = [&](int k) {
        constexpr int every = KS / NI;
        if (k % every == 0 && tl.spread) load_unit_d<D, kNT>(tl, k / every);
    };

    // ---- iteration u: the score product of tile u (the hook issues loads between its
    // k-steps), its mask, then the PV product of tile u - 1 with the softmax of tile u in
    // pieces between its steps, and the rescale when a reference moved (after the PV
    // product of tile u - 1, before that of tile u).  Tile u's probabilities go to set
    // u % 2, a template constant, so the loops below run two iterations per trip.
    auto iteration = [&](auto cur_c, int u, auto &&loads, bool masked, uint32_t kvalid, bool tree, int k0) {
        constexpr int cur = decltype(cur_c)::value;
        tile_scores<D>(smem + (u & (NST - 1)) * STAGE_BYTES, qf, sc, loads);
        if (masked) mask_scores(sc, kvalid, tree, k0, mrow);
        SoftTmp tmp;
        pv_tile<D>(smem + ((u - 1) & (NST - 1)) * STAGE_BYTES + KTILE, pf[cur ^ 1], o, [&](int i) {
            // the softmax's 16 pieces over the product's 2 DB steps
            constexpr int per = 16 / (2 * DB);
#pragma unroll
            for (int r = 0; r < per; ++r) softmax_piece<D == 128>(i * per + r, sc, rs, tmp, pf[cur], p.scale_log2);
        });
        settle(pf[cur], rs);
        rescale<D>(o, rs);
    };
    using Set0 = std::integral_constant<int, 0>;
    using Set1 = std::integral_constant<int, 1>;

    for (int k = -3; k < 0; ++k) {  // ring prologue
        prepare(k + ahead);
        if (tl.spread)
#pragma unroll
            for (int j = 0; j < NI; ++j) load_unit_d<D, kNT>(tl, j);
    }
    int u = 0;
    if (staged && all_ok) {
        // full prefix tiles whose loads (up to 3 tiles ahead) are full prefix tiles too:
        // group offsets read one iteration early, no masking, no branches around the
        // loads; an even count, two iterations per trip
        const int nfull = (end - start) / kKeyTile;
        const int nfast = nfull > 3 ? (nfull - 3) & ~1 : 0;
        uint32_t gnext = nfast > 0 ? gtab[2 * ahead + half] : 0;
        auto fast = [&](auto cur_c, int uu) {
            wait_loads<VMWAIT>();
            lds_barrier();  // operands of iteration uu visible to all; load targets free
            const uint32_t g = gnext;
            gnext = gtab[min(2 * (uu + 1 + ahead) + half, kGrpMax - 1)];
            TileLoad f;
            f.src = pool_w + (int64_t)g * 16 + lane_off;
            f.step = step;
            f.lds = smem0 + ((uu + ahead) & (NST - 1)) * STAGE_BYTES + lds_w;
            f.ustride = ustride;
            f.nvalid = NI;  // full tiles in range: every row holds a key
            f.alt = alt_w;
            iteration(
                cur_c, uu,
                [&](int k) {
                    constexpr int every = KS / NI;
                    if (k % every == 0) load_unit_d<D, kNT>(f, k / every);
                },
                false, 0u, false, 0);
        };
        for (; u < nfast; u += 2) {
            fast(Set0{}, u);
            fast(Set1{}, u + 1);
        }
    }
    auto generic = [&](auto cur_c, int uu) {
        wait_loads<VMWAIT>();
        lds_barrier();
        prepare(uu + ahead);
        const bool tr = uu >= ntp && uu < nt;
        int k0 = 0;
        uint32_t kvalid = 0;
        if (uu >= nt) {
            // past the last tile: all keys masked
        } else if (tr) {
            k0 = (uu - ntp) * kKeyTile;
            kvalid = tree_valid(k0, p.T);
        } else {
            k0 = start + uu * kKeyTile;
            kvalid = 0;
#pragma unroll
            for (int grp = 0; grp < 2; ++grp) {
                const int pos = k0 + 16 * grp;
                if (pos < end) {
                    int64_t off;
                    const int nk = end - pos < 16 ? end - pos : 16;
                    if (group_off(2 * uu + grp, off))
                        kvalid |= (nk == 16 ? 0xffffu : ((1u << nk) - 1u)) << (16 * grp);
                }
            }
        }
        iteration(cur_c, uu, load_in_scores, tr || kvalid != 0xffffffffu, kvalid, tr, k0);
    };
    // iterations up to nt (the PV product of the last tile), two per trip from an even u;
    // iterations past the last tile compute the scores of repeat-slot data with every key
    // masked, so that their probabilities are zero and their PV products add nothing
    const int nit = (nt + 2) & ~1;
    for (; u < nit; u += 2) {
        generic(Set0{}, u);
        generic(Set1{}, u + 1);
    }
    wait_loads<0>();  // the trailing repeat loads

    // ---- results.  Accumulator element r of block (rb, db) is d = 32 db + 8 (r / 4) + 4 h
    //      + r % 4 of row row_base + 32 rb.  Each row has its reference max (log2 units;
    //      -inf when it saw no key) and the sum of its weights.
    float ltot[2], mfin[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        ltot[rb] = rs.lsum[rb] + __shfl_xor(rs.lsum[rb], 32, 64);
        mfin[rb] = rs.mref[rb] == kNoRef ? kNegInf : rs.mref[rb];
    }
    // recomputed here rather than kept live across the tile loop
    int rbase = row_base;
    asm volatile("" : "+v"(rbase));
    // chunks of this sequence: chunk 0, and every later one that starts inside the prefix
    const int64_t nv64 = P > 0 ? ((int64_t)P + C - 1) / C : 1;
    const int nv = (int)(nv64 < 1 ? 1 : (nv64 > p.S ? p.S : nv64));
    // the whole prefix in this chunk: the output goes straight to out (normalised
    // below); otherwise the chunk's partial result (O unnormalised, reference max, sum)
    const bool direct = p.counters && nv == 1;
    const int64_t ubase = ((int64_t)b * p.Hkv + kvh) * p.S * (int64_t)p.R;  // slot (s, r): ubase + s R + r
    if (direct) {
        // The whole prefix in this chunk: O is normalised on its way out.  Row block by row
        // block, the accumulators go to LDS (the ring's stages, free once every wavefront
        // is past its last tile: 8 KiB per d block and wavefront), straight from the
        // accumulation registers (only stores read those, which keeps the allocator from
        // moving them out), and come back one d block at a time to be scaled and stored.
        // (Writing O unnormalised to the output and rescaling it there wrote it to HBM
        // twice whenever L2 evicted the lines in between: 1.8x the output's bytes at the
        // batched 8K workload.)
        __syncthreads();
        f32x4 *lds_o = reinterpret_cast<f32x4 *>(smem) + w * (DB * 4 * 64);  // [db*4+g4][lane]
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    lds_o[(db * 4 + g4) * 64 + lane] =
                        f32x4{o[rb][db][4 * g4], o[rb][db][4 * g4 + 1], o[rb][db][4 * g4 + 2],
                              o[rb][db][4 * g4 + 3]};
            const int row = rbase + rb * 32;
            const float inv = ltot[rb] > 0.0f ? 1.0f / ltot[rb] : 0.0f;
            float *op = out_row(p, b, kvh, row < p.R ? row : 0) + 4 * h;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                asm volatile("" ::: "memory");  // one d block's lines in flight at a time
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const f32x4 v = lds_o[(db * 4 + g4) * 64 + lane];
                    if (row < p.R) *reinterpret_cast<f32x4 *>(op + db * 32 + g4 * 8) = v * inv;
                }
            }
            asm volatile("" ::: "memory");
        }
        return;
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = rbase + rb * 32;
        if (row < p.R) {
            const int64_t base = ubase + (int64_t)s * p.R + row;
            float *op = p.ws_o + base * D + 4 * h;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4)
                    *reinterpret_cast<f32x4 *>(op + db * 32 + g4 * 8) =
                        f32x4{o[rb][db][4 * g4], o[rb][db][4 * g4 + 1], o[rb][db][4 * g4 + 2],
                              o[rb][db][4 * g4 + 3]};
            if (h == 0) {
                p.ws_ml[base * 2 + 0] = mfin[rb];
                p.ws_ml[base * 2 + 1] = ltot[rb];
            }
        }
    }
    if (!p.counters) return;  // merged by the separate merge kernel

    // The last of the nv chunks of this (sequence, kv head, row group) to finish merges
    // them.  Each thread waits until its partial stores have reached L2; one thread then
    // counts the arrival with a device-scope release (which writes this XCD's L2 back, so
    // the partials are visible from every XCD).  The last arrival resets the counter for
    // the next call and reads the partials with device-coherent loads, which need no L2
    // invalidation (that would also evict the tiles other workgroups still share).
    wait_loads<0>();
    __syncthreads();
    int *flag = reinterpret_cast<int *>(smem + G::FLAG_OFF);
    if (threadIdx.x == 0) {
        int32_t *cnt = p.counters + ((int64_t)b * p.Hkv + kvh) * p.n_rg + rg;
        const int old = __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == nv - 1;
        if (last) __hip_atomic_store(cnt, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
    }
    __syncthreads();
    if (!*flag) return;
    merge_chunks<D>(p, b, kvh, ubase, rbase, nv);
}

}  // namespace w4

}  // namespace

namespace {
template <int D>
hipError_t launch_w4(const AttnArgs &a, const AttnPlan &pl, hipStream_t stream) {
    using namespace w4;
    constexpr int SMEM = Geo<D>::SMEM;
    // one row group per kv head: each workgroup streams its keys alone (non-temporal loads)
    const bool nt = pl.n_rg == 1;
    const auto kernel = a.k_tree ? (nt ? attn_w4_kernel<D, false, true> : attn_w4_kernel<D, false, false>)
                                 : (nt ? attn_w4_kernel<D, true, true> : attn_w4_kernel<D, true, false>);
    hipError_t e = hipFuncSetAttribute((const void *)kernel,
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
    p.balanced = pl.balanced;
    p.ws_o = a.ws_o;
    p.ws_ml = a.ws_ml;
    p.ws_c = a.ws_c;
    p.out = a.out;
    p.D = D;
    p.counters = pl.fused ? a.ws_cnt : nullptr;
    // balanced: whole blocks (n_rg workgroups) per XCD and round, see balanced_item
    const int grid = pl.balanced
                         ? (a.B * pl.S * a.Hkv + kNumXCD - 1) / kNumXCD * kNumXCD * pl.n_rg
                         : (p.total + kNumXCD - 1) / kNumXCD * kNumXCD;
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(64 * kW), SMEM, stream, p);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_attn_w4(const AttnArgs &a, const AttnPlan &pl, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    return a.D == 128 ? launch_w4<128>(a, pl, stream) : launch_w4<256>(a, pl, stream);
}

}  // namespace sv
