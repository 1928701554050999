// attn_mfma.hip -- tree-masked split-KV attention on the gfx950 matrix cores (bf16 in,
// fp32 accumulate) at head_dim 512, for kv heads whose (GQA group x tree nodes) query
// rows fill at least one 16-row tile.  (head_dim 128 and 256: attn_mfma_w4.hip.)
//
// What is computed (ADR-037 Phase status rows E1.1-E1.5, section 4 Phase E1;
// Medusa/EAGLE-2 page "What's not implemented" 1(c)): every query row (q head g of
// kv head kvh, tree node i) attends to the cached prefix of its sequence and to
// the tree rows its ancestor mask selects.  One workgroup covers one
// (sequence, kv head, prefix chunk, row group); it leaves an unnormalised partial
// output and its (reference max, sum) per row, merged afterwards by attn_reduce.
//
// Organisation (8 wavefronts per workgroup, two per SIMD, one workgroup per CU):
//   * a wavefront owns 32 query rows as two 16-row blocks, shared with a second
//     wavefront that takes the other half of head_dim; their Q fragments stay in
//     registers and the wavefront owns their output accumulators;
//   * keys stream through an NST-deep ring of LDS stages, 32 keys of K and V per
//     stage, filled by direct global->LDS loads (global_load_lds_dwordx4) issued
//     ahead of use, so HBM latency hides behind the matrix work; one barrier per tile;
//   * scores are formed transposed, S^T = K Q^T, as 2 x 2 blocks of
//     v_mfma_f32_16x16x32_bf16 (16 keys x 16 query rows each): four independent
//     accumulation chains.  A lane holds 8 of a row's 32 keys, so the row max takes
//     two lane swaps; the two half-head_dim partial score tiles of a wavefront pair
//     are summed through LDS first;
//   * the output is accumulated transposed, O^T = V^T P^T, in 16 x 16 blocks, so a
//     lane keeps the accumulators of the rows it computed probabilities for; the key
//     order inside the 32-key step follows the score registers, so the P^T fragment is
//     the score registers as they stand, and the transposing LDS read
//     (ds_read_b64_tr_b16) delivers V^T in exactly that key order;
//   * LDS rows are padded (K by 16 bytes, V by 32 bytes): the K fragment reads
//     (ds_read_b128, 16 lanes per LDS cycle) and the V fragment reads (32 lanes per
//     cycle) each touch 64 distinct banks, and every fragment address is one base
//     register plus an immediate;
//   * the reference max only moves when a tile raises it by more than 2^8, so the
//     accumulators are rarely rescaled (the merged result does not depend on the
//     reference values used).
#include "attn_common.h"

namespace sv {
namespace {

constexpr int kWaves = 8;

template <int D>
struct MCfg {
    static_assert(D == 512, "head_dim 512 (128 and 256: attn_mfma_w4.hip)");
    static constexpr int DSPLIT = 2;                // wavefronts sharing 32 rows
    static constexpr int DW = D / DSPLIT;           // head_dim share of one wavefront
    static constexpr int KS = DW / 32;              // 32-wide k-steps of S^T = K Q^T
    static constexpr int DB = DW / 16;              // 16-wide d blocks of O^T
    // An LDS tile is made of 1 KB units, each filled by one wavefront-wide direct load:
    // unit p holds key p.  Units are padded (K by 16 bytes, V by 32) so that the
    // fragment reads touch 64 distinct banks.
    static constexpr int UNITS = kKeyTile * D * 2 / 1024;    // 32
    static constexpr int KU = 1024 + 16;
    static constexpr int VU = 1024 + 32;
    static constexpr int KHALF = 16 * KU;                    // key r + 16 relative to key r
    static constexpr int VHALF = 16 * VU;
    static constexpr int KTILE = UNITS * KU;
    static constexpr int STAGE_BYTES = UNITS * (KU + VU);    // K tile then V tile
    static constexpr int NST = 2;                            // ring depth
    static constexpr int LOOK = NST - 1;                     // tiles loaded ahead
    static constexpr int NI = 2 * UNITS / kWaves;            // loads per wavefront per tile
    static constexpr int VMWAIT = NI * (LOOK - 1);           // loads left in flight at a wait
    static constexpr int ROWS_PER_WG = kWaves / DSPLIT * 32;
    static constexpr int XBYTES = kWaves / 2 * 64 * 16 * 4;  // score exchange
    static constexpr int TBL_OFF = NST * STAGE_BYTES + XBYTES;  // staged block-table entries
    static constexpr int MASK_OFF = TBL_OFF + kTblMax * 4;      // ancestor-mask rows
    static constexpr int SMEM = MASK_OFF + ROWS_PER_WG * 8;
    static_assert(KS % NI == 0 || NI % KS == 0, "load spacing");
};

// Lane layout of a load: all 64 lanes carry one key row (16 bytes each); wavefront q of
// a tensor loads keys 8 q .. 8 q + 7 of the tile, i.e. group q / 2.
__device__ __forceinline__ int load_lane_piece() { return (int)(threadIdx.x & 63); }

// Per lane: its 16 bytes of tree row 0 of kv head kvh (finite by the caller's contract),
// read in place of rows that hold no key.
template <int D, bool kInCache>
__device__ __forceinline__ const unsigned char *finite_row(const MfmaParams &p, int b, int kvh,
                                                           int P, int tensor) {
    if constexpr (kInCache)
        return tree_row_in_cache(reinterpret_cast<const unsigned char *>(tensor ? p.vc : p.kc) +
                                     load_lane_piece() * 16,
                                 p, b, kvh, P, 0);
    return reinterpret_cast<const unsigned char *>(tensor ? p.vt : p.kt) +
           ((int64_t)b * p.Hkv + kvh) * p.T * (D * 2) + load_lane_piece() * 16;
}

// This wavefront's loads of prefix tile k0 (chunk ending at `end`): rows past the end
// or in a block whose table entry is out of range read `alt`.
template <int D>
__device__ __forceinline__ TileLoad prepare_prefix(const MfmaParams &p, int kvh, const TileBlocks &tb,
                                                   int k0, int end, const unsigned char *alt,
                                                   uint32_t stage) {
    using Cf = MCfg<D>;
    const int w = uni(threadIdx.x >> 6);
    const int tensor = w >> 2;  // 0: K, 1: V
    const int q = w & 3;
    const int half = q >> 1;
    const int blk = half ? tb.blk[1] : tb.blk[0];
    // keys of one group stay inside its block: slot + 15 < block size
    const int row = (half ? tb.slot[1] : tb.slot[0]) + 8 * (q & 1);
    const int left = end - (k0 + 8 * q);
    TileLoad t;
    t.src = reinterpret_cast<const unsigned char *>(tensor ? p.vc : p.kc) +
            ((int64_t)blk * p.bstride + (int64_t)kvh * p.hstride + (int64_t)row * p.rstride) * 2 +
            load_lane_piece() * 16;
    t.step = p.rstride * 2;
    t.ustride = tensor ? Cf::VU : Cf::KU;
    t.lds = stage + (tensor ? Cf::KTILE : 0) + q * Cf::NI * t.ustride;
    t.spread = true;
    t.nvalid = (half ? tb.ok[1] : tb.ok[0]) ? (left < 0 ? 0 : (left > Cf::NI ? Cf::NI : left)) : 0;
    t.alt = alt;
    return t;
}

// Issues the whole tile; the returned descriptor re-reads the last node (for repeat
// slots).  kInCache: the tree rows sit in the cache at positions P + r instead of in the
// tree buffers.
template <int D, bool kInCache>
__device__ __forceinline__ TileLoad issue_tree(const MfmaParams &p, int b, int kvh, int P,
                                               int k0, uint32_t stage) {
    using Cf = MCfg<D>;
    const int w = uni(threadIdx.x >> 6);
    const int tensor = w >> 2;
    const int q = w & 3;
    const int row = k0 + 8 * q;
    TileLoad t;
    t.ustride = tensor ? Cf::VU : Cf::KU;
    t.lds = stage + (tensor ? Cf::KTILE : 0) + q * Cf::NI * t.ustride;
    if constexpr (kInCache) {
        const unsigned char *pool = reinterpret_cast<const unsigned char *>(tensor ? p.vc : p.kc) +
                                    load_lane_piece() * 16;
#pragma unroll
        for (int j = 0; j < Cf::NI; ++j)
            dma16(tree_row_in_cache(pool, p, b, kvh, P, min(row + j, p.T - 1)),
                  t.lds + j * t.ustride);
        t.src = tree_row_in_cache(pool, p, b, kvh, P, p.T - 1);
    } else {
        const unsigned char *base = reinterpret_cast<const unsigned char *>(tensor ? p.vt : p.kt) +
                                    ((int64_t)b * p.Hkv + kvh) * p.T * (D * 2) +
                                    load_lane_piece() * 16;
#pragma unroll
        for (int j = 0; j < Cf::NI; ++j)
            dma16(base + (int64_t)min(row + j, p.T - 1) * (D * 2), t.lds + j * t.ustride);
        t.src = base + (int64_t)(p.T - 1) * (D * 2);
    }
    t.step = 0;
    t.spread = false;
    t.nvalid = Cf::NI;
    t.alt = t.src;
    return t;
}

// Per-wavefront state of the online softmax: two 16-row blocks per lane (rows
// rb*16 + (lane & 15)), each with its reference max (log2 units) and partial sum.
template <int D>
struct RowState {
    f32x4 o[2][MCfg<D>::DB];   // O^T accumulators: [row block][16-wide d block]
    float mref[2];
    float lsum[2];
};

// Max over the four 16-lane groups (lanes n, n + 16, n + 32, n + 48 end up equal).
__device__ __forceinline__ float max_over_groups(float m) {
    // gfx950 row swaps: permlane16_swap exchanges rows 1 and 3 of its first operand
    // with rows 0 and 2 of its second, permlane32_swap the upper half of the first with
    // the lower half of the second; with both operands equal, the two results hold the
    // two partners of each lane pair.
    const unsigned u = __float_as_uint(m);
    const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned v = __float_as_uint(m);
    const auto c = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return fmaxf(__uint_as_float(c[0]), __uint_as_float(c[1]));
}

// First half of a tile: scores, mask, online softmax (rescaling the accumulators when
// the reference max moves); leaves the bf16 P^T fragments in pf[row block].
// Lane l = 16 g + n: score registers sacc[rb][kb][r] hold row rb*16 + n, key
// kb*16 + 4g + r.  hook(kstep) runs before the matrix products of each k-step (the
// caller issues tile loads there).
template <int D, class Hook>
__device__ __forceinline__ void tile_scores(const unsigned char *ks, float *xs, uint32_t kvalid,
                                            bool tree, int k0, int dpart,
                                            const bf16x8 (&qf)[2][MCfg<D>::KS],
                                            const uint64_t *mrow, RowState<D> &st,
                                            float scale_log2, bf16x8 (&pf)[2], Hook &&hook) {
    using Cf = MCfg<D>;
    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int g = lane >> 4;
    const int n = lane & 15;

    // ---- S^T = K Q^T over this wavefront's share of head_dim: A = K (16 keys x 32 d,
    //      lane: key kb*16 + n, d 32*ks + 8g .. +8), B = Q^T (lane: row rb*16 + n, same d)
    f32x4 sacc[2][2];
    for (int rb = 0; rb < 2; ++rb)
        for (int kb = 0; kb < 2; ++kb) sacc[rb][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
    const unsigned char *kbase = ks + n * Cf::KU + dpart * Cf::DW * 2 + g * 16;
#pragma unroll
    for (int kstep = 0; kstep < Cf::KS; ++kstep) {
        const bf16x8 a0 = *reinterpret_cast<const bf16x8 *>(kbase + kstep * 64);
        const bf16x8 a1 = *reinterpret_cast<const bf16x8 *>(kbase + Cf::KHALF + kstep * 64);
        hook(kstep);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            sacc[rb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, qf[rb][kstep], sacc[rb][0], 0, 0, 0);
            sacc[rb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, qf[rb][kstep], sacc[rb][1], 0, 0, 0);
        }
    }
    {
        // sum the two partial score tiles of a wavefront pair (same rows, halves of
        // head_dim): the second half hands its scores over, the first adds and hands
        // the sum back, so both hold bit-identical scores
        f32x4 *slot = reinterpret_cast<f32x4 *>(xs + ((w >> 1) * 64 + lane) * 16);
        if (dpart == 1)
            for (int v = 0; v < 4; ++v) slot[v] = sacc[v >> 1][v & 1];
        lds_barrier();
        if (dpart == 0)
            for (int v = 0; v < 4; ++v) {
                sacc[v >> 1][v & 1] += slot[v];
                slot[v] = sacc[v >> 1][v & 1];
            }
        lds_barrier();
        if (dpart == 1)
            for (int v = 0; v < 4; ++v) sacc[v >> 1][v & 1] = slot[v];
    }

    // ---- mask, online softmax in log2 units; probabilities become bf16 P^T fragments.
    //      Full prefix tiles (the common case) need no masking at all.
    if (tree || kvalid != 0xffffffffu) {
        const uint32_t kv = kvalid >> (4 * g);   // bit kb*16 + r: key kb*16 + 4g + r
#pragma unroll
        for (int rb = 0; rb < 2; ++rb) {
            const uint64_t mt64 = tree ? (mrow[rb * 16] >> (k0 + 4 * g)) : ~0ull;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int off = kb * 16 + r;
                    const bool ok = ((kv >> off) & 1u) && ((mt64 >> off) & 1ull);
                    sacc[rb][kb][r] = ok ? sacc[rb][kb][r] : kNegInf;
                }
        }
    }
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        float mt = fmaxf(fmaxf(fmaxf(sacc[rb][0][0], sacc[rb][0][1]),
                               fmaxf(sacc[rb][0][2], sacc[rb][0][3])),
                         fmaxf(fmaxf(sacc[rb][1][0], sacc[rb][1][1]),
                               fmaxf(sacc[rb][1][2], sacc[rb][1][3])));
        mt = max_over_groups(mt) * scale_log2;  // row max, log2 units
        const bool raise = mt > st.mref[rb] + kRescaleSlack;
        if (__any(raise)) {
            const float mnew = fmaxf(st.mref[rb], mt);
            const float alpha = mnew == kNegInf ? 1.0f : exp2f(st.mref[rb] - mnew);
            st.lsum[rb] *= alpha;
#pragma unroll
            for (int db = 0; db < Cf::DB; ++db) st.o[rb][db] *= alpha;
            st.mref[rb] = mnew;
        }
        // exp2(s * scale_log2 - mref); a masked score (-inf) gives 0, and while a row
        // has seen no valid key its reference is taken as 0
        const float mneg = st.mref[rb] == kNegInf ? 0.0f : -st.mref[rb];
        float add = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float pr = __builtin_amdgcn_exp2f(fmaf(sacc[rb][j >> 2][j & 3], scale_log2, mneg));
            const __bf16 pb = (__bf16)pr;
            add += (float)pb;  // the denominator sums exactly the weights the numerator uses
            pf[rb][j] = pb;
        }
        st.lsum[rb] += add;
    }
}

// Second half of a tile: O^T += V^T P^T in 16 x 16 blocks (A = V^T: 16 d x 32 keys,
// lane 16g + n holds d = db*16 + n and keys 4g + 0..3, 16 + 4g + 0..3, the P^T
// fragment's key order).  The transposing read: in each 16-lane group, source lane
// 4r + q points at 4 consecutive d of key row (16t + 4g + r); lane n of the group then
// receives column db*16 + n of those 4 keys.  hook(db) runs before each d block.
template <int D, class Hook>
__device__ __forceinline__ void tile_pv(const unsigned char *vs, int dpart,
                                        const bf16x8 (&pf)[2], RowState<D> &st, Hook &&hook) {
    using Cf = MCfg<D>;
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const int lane = threadIdx.x & 63;
    const int g = lane >> 4;
    const int rr = (lane >> 2) & 3;
    const int qq = lane & 3;
    const unsigned char *vbase = vs + (4 * g + rr) * Cf::VU + dpart * Cf::DW * 2 + qq * 8;
#pragma unroll
    for (int db = 0; db < Cf::DB; ++db) {
        const bf16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4 *)(vbase + db * 32));
        const bf16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
            (lds_bf16x4 *)(vbase + Cf::VHALF + db * 32));
        hook(db);
        const bf16x8 a = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
        st.o[0][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[0], st.o[0][db], 0, 0, 0);
        st.o[1][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf[1], st.o[1][db], 0, 0, 0);
    }
}

template <int D, bool kInCache>
__global__ __launch_bounds__(512) void attn_mfma_kernel(MfmaParams p) {
    using Cf = MCfg<D>;
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
    const int g = lane >> 4;
    const int n = lane & 15;
    const int dpart = w % Cf::DSPLIT;
    const int row_base = rg * Cf::ROWS_PER_WG + (w / Cf::DSPLIT) * 32 + n;

    // Q fragments (B operand of S^T): row rb*16 + n, d = dpart*DW + 32*kstep + 8g .. +8;
    // and each row's ancestor mask, kept in LDS (read on tree tiles only)
    bf16x8 qf[2][Cf::KS];
    uint64_t *mrow = reinterpret_cast<uint64_t *>(smem + Cf::MASK_OFF) + (w / Cf::DSPLIT) * 32 + n;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        const int row = row_base + rb * 16;
        const bool valid = row < p.R;
        const int gh = valid ? row / p.T : 0;
        const int i = valid ? row - gh * p.T : 0;
        const __bf16 *qp = p.q + (((int64_t)b * p.Hq + (int64_t)kvh * p.G + gh) * p.T + i) * D +
                           dpart * Cf::DW + 8 * g;
#pragma unroll
        for (int kstep = 0; kstep < Cf::KS; ++kstep) {
            if (valid) {
                qf[rb][kstep] = *reinterpret_cast<const bf16x8 *>(qp + 32 * kstep);
            } else {
                for (int j = 0; j < 8; ++j) qf[rb][kstep][j] = (__bf16)0.0f;
            }
        }
        const uint64_t m = valid ? p.mask[(int64_t)b * p.T + i] : 0ull;
        if (g == 0 && dpart == 0) mrow[rb * 16] = m;
    }
    // consume Q and the mask rows here, so the loads are complete before the ring
    // starts and no wait for them lands inside the tile loop
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
        for (int kstep = 0; kstep < Cf::KS; ++kstep) asm volatile("" ::"v"(qf[rb][kstep]));
    }

    // block-table entries this chunk touches: all in range? (then full tiles need no
    // masking); staged in LDS for the per-tile lookups when they fit
    const Cursor cstart = {start / p.bs, start % p.bs};
    const int nent = ntp > 0 ? (end - 1) / p.bs - cstart.idx + 1 : 0;
    BlockLookup bl{reinterpret_cast<const int *>(smem + Cf::TBL_OFF), cstart.idx, nent,
                   nent <= kTblMax, -1, -1000};
    bool all_ok = true;
    if (ntp > 0) {
        int *tbl = reinterpret_cast<int *>(smem + Cf::TBL_OFF);
        for (int i = (int)threadIdx.x; i < nent; i += blockDim.x) {
            const int blk = p.table[(int64_t)b * p.max_blocks + cstart.idx + i];
            const bool ok = blk >= 0 && blk < p.num_blocks;
            all_ok = all_ok && ok;
            if (bl.staged) tbl[i] = ok ? blk : -1;
        }
        all_ok = __syncthreads_and(all_ok) != 0;  // also publishes the LDS copy
    }

    RowState<D> rs;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        rs.mref[rb] = kNegInf;
        rs.lsum[rb] = 0.0f;
#pragma unroll
        for (int db = 0; db < Cf::DB; ++db) rs.o[rb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bf16x8 pf[2];

    // Tile loads.  Every tile slot k < nt + LOOK issues exactly NI loads per wavefront
    // (slots past the last tile repeat the last tile's sources into a free stage), so
    // "tile u has landed" is always the same vmcnt, and the ring drains before exit.
    const uint32_t smem0 = lds_addr(smem);
    Cursor cissue = cstart;   // prefix tile whose block entries tbn holds
    Cursor ccomp = cstart;    // next prefix tile to compute
    TileBlocks tbn = ntp > 0 ? lookup_blocks(p, b, bl, cissue, start, end)
                             : TileBlocks{{0, 0}, {0, 0}, {false, false}};
    const unsigned char *alt = finite_row<D, kInCache>(p, b, kvh, P, uni(threadIdx.x >> 6) >> 2);
    TileLoad tl;
    auto prepare = [&](int k) {
        const uint32_t stage = smem0 + (k % Cf::NST) * Cf::STAGE_BYTES;
        if (k < ntp) {
            tl = prepare_prefix<D>(p, kvh, tbn, start + k * kKeyTile, end, alt, stage);
            cissue = cursor_add(cissue, kKeyTile, p.bs);
            if (k + 1 < ntp) tbn = lookup_blocks(p, b, bl, cissue, start + (k + 1) * kKeyTile, end);
        } else if (k < nt) {
            tl = issue_tree<D, kInCache>(p, b, kvh, P, (k - ntp) * kKeyTile, stage);
        } else {
            tl.lds = stage + (tl.lds - smem0) % Cf::STAGE_BYTES;
            tl.spread = true;
        }
    };
    auto issue = [&](int k) {
        prepare(k);
        if (tl.spread)
#pragma unroll
            for (int j = 0; j < Cf::NI; ++j) load_unit(tl, j);
    };
    auto nohook = [](int) {};
    // spread the NI loads of the prepared tile over the k-steps of a score product
    auto load_in_scores = [&](int kstep) {
        constexpr int every = Cf::KS >= Cf::NI ? Cf::KS / Cf::NI : 1;
        constexpr int per = Cf::NI > Cf::KS ? Cf::NI / Cf::KS : 1;
        if (kstep % every == 0 && tl.spread)
#pragma unroll
            for (int j = 0; j < per; ++j) load_unit(tl, kstep / every * per + j);
    };
    auto scores = [&](int u, auto &&hook) {
        const unsigned char *stg = smem + (u % Cf::NST) * Cf::STAGE_BYTES;
        const bool tr = u >= ntp;
        int k0;
        uint32_t kvalid;
        if (tr) {
            k0 = (u - ntp) * kKeyTile;
            kvalid = tree_valid(k0, p.T);
        } else {
            k0 = start + u * kKeyTile;
            kvalid = prefix_valid(p, b, k0, ccomp, end, all_ok);
            ccomp = cursor_add(ccomp, kKeyTile, p.bs);
        }
        tile_scores<D>(stg, xs, kvalid, tr, k0, dpart, qf, mrow, rs, p.scale_log2, pf, hook);
    };
    auto pv = [&](int u, auto &&hook) {
        tile_pv<D>(smem + (u % Cf::NST) * Cf::STAGE_BYTES + Cf::KTILE, dpart, pf, rs, hook);
    };

    for (int k = 0; k < Cf::LOOK; ++k) issue(k);   // ring prologue
    for (int u = 0; u < nt; ++u) {
        wait_loads<Cf::VMWAIT>();
        lds_barrier();  // tile u visible to all; stage of tile u-1 free for reuse
        prepare(u + Cf::LOOK);
        scores(u, load_in_scores);
        pv(u, nohook);
    }
    wait_loads<0>();  // the trailing repeat loads

    // ---- partial results: O (unnormalised), reference max (log2 units) and sum per row
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
        float ltot = rs.lsum[rb] + __shfl_xor(rs.lsum[rb], 16, 64);
        ltot += __shfl_xor(ltot, 32, 64);
        const int row = row_base + rb * 16;
        if (row < p.R) {
            const int64_t base = (((int64_t)b * p.Hkv + kvh) * p.S + s) * p.R + row;
            float *op = p.ws_o + base * D + dpart * Cf::DW + 4 * g;
#pragma unroll
            for (int db = 0; db < Cf::DB; ++db)
                *reinterpret_cast<f32x4 *>(op + db * 16) = rs.o[rb][db];
            if (g == 0 && dpart == 0) {
                p.ws_ml[base * 2 + 0] = rs.mref[rb];
                p.ws_ml[base * 2 + 1] = ltot;
            }
        }
    }
}

template <int D>
hipError_t launch_d(const AttnArgs &a, const AttnPlan &pl, hipStream_t stream) {
    using Cf = MCfg<D>;
    const auto kernel = a.k_tree ? attn_mfma_kernel<D, false> : attn_mfma_kernel<D, true>;
    hipError_t e = hipFuncSetAttribute((const void *)kernel,
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
    hipLaunchKernelGGL(kernel, dim3(grid), dim3(64 * kWaves), Cf::SMEM, stream, p);
    return hipGetLastError();
}

}  // namespace

bool attn_w4_handles(int D) { return D == 128 || D == 256; }

hipError_t launch_attn_mfma(const AttnArgs &a, const AttnPlan &pl, hipStream_t stream) {
    if (a.B == 0) return hipSuccess;
    if (attn_w4_handles(a.D)) return launch_attn_w4(a, pl, stream);
    return launch_d<512>(a, pl, stream);
}

}  // namespace sv
