// attn_common.h -- device helpers shared by the attention kernels: the matrix-core
// kernels' parameters, direct global->LDS tile loads and their bookkeeping, LDS-only
// barriers, the paged-cache cursor and block-table lookups, key validity, and the
// device-coherent loads of the in-kernel chunk merges.
#pragma once

#include "sv_internal.h"

namespace sv {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kTblMax = 2048;  // block-table entries of one chunk that fit the LDS copy

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
    int balanced;          // chunks cut from the actual prefix lengths, largest first
    float *ws_o;
    float *ws_ml;
    int32_t *ws_c;         // where a balanced call leaves its chunk length (separate merge)
    float *out;            // [B][T][Hq][D]
    int D;
    int32_t *counters;     // arrivals per (sequence, kv head, row group); NULL: the
                           // separate merge kernel combines the chunks
};

// Tree rows kept in the cache (no tree buffers given): byte address of tree row r of
// sequence b, kv head kvh, at cache position P + r of a bf16 pool (plus the lane's byte
// offset already added to `pool`).  An out-of-range block-table entry reads block 0
// instead: the rows were then never appended, and the sequence is marked invalid.
__device__ __forceinline__ const unsigned char *tree_row_in_cache(const unsigned char *pool,
                                                                  const MfmaParams &p, int b,
                                                                  int kvh, int P, int r) {
    const int pos = P + r;
    int32_t blk = p.table[(int64_t)b * p.max_blocks + pos / p.bs];
    blk = (blk >= 0 && blk < p.num_blocks) ? blk : 0;
    return pool + ((int64_t)blk * p.bstride + (int64_t)kvh * p.hstride +
                   (int64_t)(pos % p.bs) * p.rstride) * 2;
}

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

// A pointer that is the same in every lane, made visibly uniform (kept in SGPRs).
__device__ __forceinline__ const unsigned char *uni_ptr(const unsigned char *p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const unsigned char *>(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ int clamp_prefix(int P, int max_P) {
    return P < 0 ? 0 : (P > max_P ? max_P : P);
}

// Keys of chunk s of a sequence with P prefix keys (chunks of C keys); the first chunk
// also holds the T tree keys.
__device__ __forceinline__ int chunk_keys(int P, int s, int C, int T) {
    const int start = s * C;
    const int n = start < P ? min(C, P - start) : 0;
    return s == 0 ? n + T : n;
}

// Balanced chunk length: the whole call's prefix keys, times the workgroups that read
// each of them (kv heads x row groups), over the compute units, so that about one
// chunk per CU remains; at least ceil(max_P / S) so that S chunks cover any sequence
// (the plan's own chunk length is at least that, so it fits an int), at most max_P;
// whole key tiles.  Same value in every wavefront that calls it.
__device__ __forceinline__ int balanced_chunk_len(const MfmaParams &p) {
    const int lane = threadIdx.x & 63;
    int64_t sum = 0;
    for (int b = lane; b < p.B; b += 64) sum += clamp_prefix(p.prefix_len[b], p.max_P);
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 64);
    const auto tiles = [](int64_t n) { return (n + kKeyTile - 1) / kKeyTile * kKeyTile; };
    const int64_t lower = tiles(((int64_t)p.max_P + p.S - 1) / p.S);
    int64_t upper = tiles(p.max_P);
    if (upper > INT_MAX / kKeyTile * kKeyTile) upper = INT_MAX / kKeyTile * kKeyTile;
    if (upper < lower) upper = lower;
    int64_t C = tiles((sum * p.Hkv * p.n_rg + kNumCU - 1) / kNumCU);
    C = C < lower ? lower : (C > upper ? upper : C);
    return uni((int)(C < kKeyTile ? kKeyTile : C));
}

// The work item of this workgroup in a balanced call.  The B * S chunks (id c = b S + s)
// are ranked by their keys, largest first (ties: smaller id); rank j has one block per kv
// head, and a block is n_rg workgroups (its row groups) that read the same keys.  Blocks
// are dealt to the XCDs in rank order, snaking (0..7, 7..0, ...), and each XCD starts its
// blocks in that order as CUs come free, so the smallest chunks fill in after the
// largest.  False when the workgroup has no item.
__device__ __forceinline__ bool balanced_item(const MfmaParams &p, int C, int *b, int *kvh,
                                              int *s, int *rg) {
    const int x = blockIdx.x % kNumXCD;
    const int pos = blockIdx.x / kNumXCD;
    const int k = pos / p.n_rg;
    *rg = pos - k * p.n_rg;
    const int gq = k * kNumXCD + ((k & 1) ? kNumXCD - 1 - x : x);
    const int N = p.B * p.S;  // <= kBalancedChunks
    if (gq >= N * p.Hkv) return false;
    const int j = gq / p.Hkv;
    *kvh = gq - j * p.Hkv;
    // lane l ranks chunks l and l + 64
    const int lane = threadIdx.x & 63;
    int sz[2], rk[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int c = lane + 64 * i;
        sz[i] = c < N ? chunk_keys(clamp_prefix(p.prefix_len[c / p.S], p.max_P), c % p.S, C, p.T)
                      : -1;
    }
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
        const int n2 = min(64, N - 64 * i2);
        for (int l2 = 0; l2 < n2; ++l2) {
            const int z = __builtin_amdgcn_readlane(sz[i2], l2);
            const int c2 = 64 * i2 + l2;
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c = lane + 64 * i;
                rk[i] += (z > sz[i] || (z == sz[i] && c2 < c)) ? 1 : 0;
            }
        }
    }
    int c = -1;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const uint64_t hit = __ballot(lane + 64 * i < N && rk[i] == j);
        if (hit) c = 64 * i + (int)__builtin_ctzll(hit);
    }
    c = uni(c);
    if (c < 0) return false;  // not reached: ranks 0 .. N-1 are all taken
    *b = c / p.S;
    *s = c - *b * p.S;
    return true;
}

// Block-table entry number `idx` of sequence b, or -1 when it is out of range.  The
// table is read through the constant address space: with a uniform index this is a
// scalar load, which keeps the vector-memory counter free for the tile loads.
__device__ __forceinline__ int table_entry(const MfmaParams &p, int b, int idx) {
    const __attribute__((address_space(4))) int32_t *tbl =
        (const __attribute__((address_space(4))) int32_t *)p.table;
    const int blk = tbl[(int64_t)b * p.max_blocks + idx];
    return (blk >= 0 && blk < p.num_blocks) ? blk : -1;
}

// Position of a prefix key inside the paged cache: (block number in the sequence's
// table, row inside the block).  Tiles advance by 32 keys, so positions are carried
// forward by additions instead of divisions by the block size (a multiple of 16).
struct Cursor {
    int idx;
    int slot;
};

__device__ __forceinline__ Cursor cursor_add(Cursor c, int n, int bs) {
    c.slot += n;
    while (c.slot >= bs) {  // n <= 32 and bs >= 16: at most two steps
        c.slot -= bs;
        ++c.idx;
    }
    return c;
}

// One 16-byte direct global->LDS load per lane: lane l's bytes land at LDS address
// lds_base + 16 * l.  Written as inline assembly so that the compiler does not see an
// LDS write it cannot disambiguate (it would then drain every load before each LDS
// read); completion is tracked explicitly with vmcnt, and the stages a load writes
// are ordered against their readers by the barriers (which carry memory clobbers).
// M0 carries the LDS base; an SALU write of M0 needs one wait state before an
// LDS-DMA instruction reads it.  M0 is listed as clobbered; the compiler reserves it (and
// warns about the clobber) but emits no use of M0 of its own in these kernels, so no value
// of it lives across the statement.  kNT adds the non-temporal hint (nt), for keys that one
// workgroup alone streams through once: at the board's power limit the call then takes
// ~2% less time.  Row groups that share a chunk go without it, as it makes them meet in
// L2 less often (+16% HBM reads at the batched 8K shape).
template <bool kNT = false>
__device__ __forceinline__ void dma16(const void *src, uint32_t lds_base) {
    if constexpr (kNT)
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
                     :
                     : "s"(lds_base), "v"(src)
                     : "m0");
    else
        asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                     :
                     : "s"(lds_base), "v"(src)
                     : "m0");
}

// Workgroup barrier for LDS traffic only (no wait on the tile loads in flight).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N of this wavefront's tile loads are still in flight (loads
// complete in issue order).
// Device-coherent reads of what other workgroups (possibly on other XCDs) wrote: buffer
// loads with the device-scope cache policy (sc1), through a resource covering `bytes`
// from `base` (reads past it return 0).
constexpr int kCoherent = 16;                       // sc1
constexpr uint32_t kRsrcWord3 = 0x00020000u;        // raw 32-bit buffer, gfx9 family
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ f32x4 coherent_load4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCoherent));
}
__device__ __forceinline__ float coherent_load1(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kCoherent));
}

template <int N>
__device__ __forceinline__ void wait_loads() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return (uint32_t)(size_t)(const __attribute__((address_space(3))) unsigned char *)p;
}

// Block-table entries of a chunk, checked against the pool size (-1: out of range),
// copied to LDS at kernel start when at most kTblMax of them; each wavefront then
// reads them through a 64-entry window held one entry per lane, so a lookup is a lane
// read, not a memory access.  Larger chunks read the table directly.
struct BlockLookup {
    const int *tbl;  // LDS copy, indexed relative to idx0
    int idx0;        // first table entry of the chunk
    int nent;        // entries the chunk touches
    bool staged;     // tbl holds all of them
    int win;         // lane i: relative entry wbase + i (-1 past the end)
    int wbase;
};

__device__ __forceinline__ int lookup_entry(const MfmaParams &p, int b, BlockLookup &bl, int idx) {
    if (!bl.staged) return table_entry(p, b, idx);
    const int rel = idx - bl.idx0;
    if (rel - bl.wbase >= 63) {  // lookups only move forward; keep rel and rel + 1 inside
        bl.wbase = rel;
        const int r = rel + (int)(threadIdx.x & 63);
        bl.win = r < bl.nent ? bl.tbl[r] : -1;
    }
    return __builtin_amdgcn_readlane(bl.win, rel - bl.wbase);
}

// Cache blocks of the two 16-key groups of a prefix tile (group 1 falls back to group
// 0 when it lies past the chunk end; an out-of-range entry reads block 0, whose keys
// the score mask removes).  Looked up one tile before the loads that use them.
struct TileBlocks {
    int blk[2];
    int slot[2];
    bool ok[2];  // the group's block-table entry is in range
};

__device__ __forceinline__ TileBlocks lookup_blocks(const MfmaParams &p, int b, BlockLookup &bl,
                                                    Cursor c, int k0, int kend) {
    TileBlocks tb;
    const int e0 = lookup_entry(p, b, bl, c.idx);
    tb.blk[0] = e0 < 0 ? 0 : e0;
    tb.slot[0] = c.slot;
    tb.ok[0] = e0 >= 0;
    tb.blk[1] = tb.blk[0];
    tb.slot[1] = c.slot;
    tb.ok[1] = tb.ok[0];
    if (k0 + 16 < kend) {
        // c.slot is a multiple of 16 below the block size (also a multiple of 16)
        if (c.slot + 16 < p.bs) {
            tb.slot[1] = c.slot + 16;
        } else {
            const int e1 = lookup_entry(p, b, bl, c.idx + 1);
            tb.blk[1] = e1 < 0 ? 0 : e1;
            tb.slot[1] = 0;
            tb.ok[1] = e1 >= 0;
        }
    }
    return tb;
}

// One wavefront's share of a tile's loads: NI loads of 1 KB, load j filling LDS unit
// (first unit + j) of the wavefront's tensor from row j (counted from each lane's first
// row) of the source.  Prefix tiles are issued one load at a time between matrix
// products of the tile before; tree tiles (rows past the last node clamped to it) and
// the trailing repeat slots are issued whole when prepared.
//
// A row that holds no key of the sequence (past the chunk end, in a block whose table
// entry is out of range, or a repeat slot) is read from `alt` instead: tree row 0 of
// the same kv head, an input the caller guarantees finite.  Such keys get probability 0,
// and a product 0 * v is 0 only for finite v, so reading whatever the cache holds there
// (possibly NaN) could otherwise leak into the output.
struct TileLoad {
    const unsigned char *src;   // per lane: its 16 bytes of the first row
    int64_t step;               // bytes between successive rows
    uint32_t lds;               // LDS address of the first unit
    int ustride;                // bytes between units
    bool spread;                // loads still to be issued one by one
    int nvalid;                 // per lane: rows 0 .. nvalid-1 come from src, the rest from alt
    const unsigned char *alt;   // per lane: its 16 bytes of a finite row
};

__device__ __forceinline__ const unsigned char *load_src(const TileLoad &t, int j) {
    return j < t.nvalid ? t.src + j * t.step : t.alt;
}

__device__ __forceinline__ void load_unit(const TileLoad &t, int j) {
    dma16(load_src(t, j), t.lds + j * t.ustride);
}

// Validity of the 32 keys of a prefix tile starting at cursor c (bit kk: key k0 + kk
// exists and its block-table entry is in range).
__device__ __forceinline__ uint32_t prefix_valid(const MfmaParams &p, int b, int k0, Cursor c,
                                                 int kend, bool all_blocks_ok) {
    if (all_blocks_ok && k0 + kKeyTile <= kend) return 0xffffffffu;
    uint32_t v = 0;
#pragma unroll
    for (int grp = 0; grp < 2; ++grp) {
        const int pos = k0 + 16 * grp;
        if (pos < kend) {
            const int n = kend - pos < 16 ? kend - pos : 16;
            uint32_t bits = (n == 16 ? 0xffffu : ((1u << n) - 1u)) << (16 * grp);
            const int idx = c.idx + (c.slot + 16 * grp >= p.bs ? 1 : 0);
            if (!all_blocks_ok && table_entry(p, b, idx) < 0) bits = 0;
            v |= bits;
        }
    }
    return v;
}

__device__ __forceinline__ uint32_t tree_valid(int k0, int T) {
    const int n = T - k0;
    return n >= 32 ? 0xffffffffu : ((1u << n) - 1u);
}

}  // namespace
}  // namespace sv
