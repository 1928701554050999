// accept_sampled.hip -- sampled acceptance: the target distribution of every tree row,
// then a walk from the root that accepts each proposal with its target probability and
// draws the emitted token from the target with the rejected proposals excluded.
//
// Rule (llms-explorer page Facts: Forge treats the drafted path as given, accepts a
// proposal with its target probability and, on rejection, samples the target
// distribution excluding it; ADR-037 row E4b.10a for the tie-free token order):
//   p_v(x) = exp2((l_v(x) - max l_v) * log2(e) / tau) / Z_v   (NaN, -inf: 0; +inf as the
//            largest finite float; a row without a finite entry has p = 0)
//   at the current node v the children are tried in increasing node index; with E the
//   tokens already rejected at v and R = 1 - sum_E p_v, child c (token x) is accepted
//   when u_accept[c] * R < p_v(x) (x in E or outside the vocabulary: p = 0), and becomes
//   the current node; when no child is accepted the emitted token is the smallest y
//   outside E whose cumulative probability (outside E) exceeds u_sample[v] * R.
//
// softmax_partial_kernel streams every row chunk once (online max and sum of exp2,
// 16-byte loads where aligned) into (max, sum) pairs.  sample_walk_kernel runs one
// workgroup per sequence: wave 0 merges the pairs of each row, checks the tree and
// walks it (one lane per node, proposals in order through a uniform loop); then the
// workgroup locates the drawn token: the chunk from the chunk pairs (a wave prefix scan),
// the 256-element tile inside it from tile sums (one coalesced pass over the chunk, which
// leaves the element weights in LDS), and the element inside the tile from a wavefront
// prefix scan over its 256 weights.  A lane the whole wavefront agrees on is read with
// readlane, and the prefix scans are DPP row shifts and broadcasts, not permutes through
// LDS.
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kTile = 256;      // elements per tile of the draw's in-chunk search
constexpr int kMaxTiles = 64;   // tiles per chunk at most (16384 elements)

struct MS {
    float m;  // running max (-inf: nothing seen)
    float s;  // sum of exp2((x - m) * k) over what was seen
};

// A logit as the rule reads it: NaN and -inf give -inf, +inf the largest finite float.
__device__ __forceinline__ float clean_logit(float x) {
    if (!(x > -__builtin_huge_valf())) return -__builtin_huge_valf();
    return x < 3.40282347e38f ? x : 3.40282347e38f;
}

__device__ __forceinline__ MS ms_merge(MS a, MS b, float k) {
    const float m = fmaxf(a.m, b.m);
    if (m == -__builtin_huge_valf()) return MS{m, 0.0f};
    return MS{m, a.s * __builtin_amdgcn_exp2f((a.m - m) * k) + b.s * __builtin_amdgcn_exp2f((b.m - m) * k)};
}

__device__ __forceinline__ void ms_add(MS &a, float x, float k) {
    if (!(x > -__builtin_huge_valf())) return;  // NaN, -inf: probability 0
    x = x < 3.40282347e38f ? x : 3.40282347e38f;
    if (x > a.m) {
        a.s = a.s * __builtin_amdgcn_exp2f((a.m - x) * k) + 1.0f;
        a.m = x;
    } else {
        a.s += __builtin_amdgcn_exp2f((x - a.m) * k);
    }
}

// One workgroup per (row, chunk): an online max and sum of exp2 per thread over 16-byte
// loads (scalar at the unaligned ends), merged across the workgroup.
__global__ __launch_bounds__(256) void softmax_partial_kernel(const float *__restrict__ logits,
                                                              int64_t V, int64_t chunk,
                                                              int nchunks, float k,
                                                              MS *__restrict__ out) {
    const int64_t row = blockIdx.x / nchunks;
    const int c = blockIdx.x - (int)row * nchunks;
    const int64_t lo = (int64_t)c * chunk;
    const int64_t hi = lo + chunk < V ? lo + chunk : V;
    const float *rp = logits + row * V;
    const int tid = threadIdx.x;
    MS a{-__builtin_huge_valf(), 0.0f};

    // body from the first 16-byte aligned element at or after lo
    const int64_t mis = (int64_t)((reinterpret_cast<uintptr_t>(rp + lo) >> 2) & 3);
    int64_t a0 = lo + ((4 - mis) & 3);
    if (a0 > hi) a0 = hi;
    const int64_t a1 = a0 + ((hi - a0) >> 2 << 2);
    if (lo + tid < a0) ms_add(a, rp[lo + tid], k);
    const f32x4 *vp = reinterpret_cast<const f32x4 *>(rp + a0);
    const int64_t nvec = (a1 - a0) >> 2;
    int64_t i = tid;
    for (; i + 3 * 256 < nvec; i += 4 * 256) {  // four 16-byte loads in flight per thread
        // non-temporal: every logit is read once here (the draw re-reads one chunk)
        const f32x4 x0 = __builtin_nontemporal_load(vp + i),
                    x1 = __builtin_nontemporal_load(vp + i + 256),
                    x2 = __builtin_nontemporal_load(vp + i + 512),
                    x3 = __builtin_nontemporal_load(vp + i + 768);
        for (int j = 0; j < 4; ++j) ms_add(a, x0[j], k);
        for (int j = 0; j < 4; ++j) ms_add(a, x1[j], k);
        for (int j = 0; j < 4; ++j) ms_add(a, x2[j], k);
        for (int j = 0; j < 4; ++j) ms_add(a, x3[j], k);
    }
    for (; i < nvec; i += 256) {
        const f32x4 x0 = __builtin_nontemporal_load(vp + i);
        for (int j = 0; j < 4; ++j) ms_add(a, x0[j], k);
    }
    if (a1 + tid < hi) ms_add(a, rp[a1 + tid], k);

    for (int off = 32; off > 0; off >>= 1) {
        const MS o{__shfl_xor(a.m, off, 64), __shfl_xor(a.s, off, 64)};
        a = ms_merge(a, o, k);
    }
    __shared__ MS part[4];
    if ((tid & 63) == 0) part[tid >> 6] = a;
    __syncthreads();
    if (tid == 0) {
        for (int j = 1; j < 4; ++j) a = ms_merge(a, part[j], k);
        out[blockIdx.x] = a;
    }
}

// Weight of a raw logit in a row whose max is m: exp2((l - m) * k), 0 for NaN / -inf.
__device__ __forceinline__ float weight_of(float raw, float m, float k) {
    const float l = clean_logit(raw);
    return l == -__builtin_huge_valf() ? 0.0f : __builtin_amdgcn_exp2f((l - m) * k);
}

// The value lane l holds, for a lane index every lane agrees on: a scalar read of one
// lane instead of a cross-lane permute through LDS.
__device__ __forceinline__ int lane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ float lane_f(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

// A float moved across lanes by one DPP control; lanes without a source, or outside the
// rows of kRowMask, read 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xf, true));
}

// Inclusive prefix sum over the 64 lanes (every lane active): shifts by 1, 2, 4 and 8
// lanes within each row of 16, then the last lane of row 0 (row 2) added to row 1 (row 3)
// and lane 31 to rows 2 and 3.
__device__ __forceinline__ float wave_incl_sum(float x) {
    x += dpp_f<0x111, 0xf>(x);
    x += dpp_f<0x112, 0xf>(x);
    x += dpp_f<0x114, 0xf>(x);
    x += dpp_f<0x118, 0xf>(x);
    x += dpp_f<0x142, 0xa>(x);
    x += dpp_f<0x143, 0xc>(x);
    return x;
}

constexpr int kWalkWaves = 16;  // wavefronts of the walk kernel's workgroup

__global__ __launch_bounds__(64 * kWalkWaves) void sample_walk_kernel(
    const float *__restrict__ logits, const MS *__restrict__ part, int64_t V, int64_t chunk,
    int nchunks, float k, const int32_t *__restrict__ draft, const int32_t *__restrict__ parents,
    const int32_t *__restrict__ tree_err, const float *__restrict__ u_accept,
    const float *__restrict__ u_sample, int T, int32_t *__restrict__ accepted_len,
    int32_t *__restrict__ accepted_nodes, int32_t *__restrict__ out_tokens) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;

    __shared__ int s_state[4];        // invalid flag, final node, path length, excluded count
    __shared__ float s_f[4];          // row max, draw target (weights), row sum
    __shared__ int32_t ex_tok[64];    // tokens rejected at the final node
    __shared__ float ex_w[64];        // and their weights
    __shared__ float tile_sum[kMaxTiles];    // per-tile weights of the chosen chunk
    __shared__ float red[kMaxTiles * 65];    // lane partials of the tile weights
    __shared__ float ew[kMaxTiles * kTile];  // the chosen chunk's element weights
    __shared__ int s_pick[2];         // chosen chunk, chosen tile
    __shared__ float s_r[2];          // residual target in the chunk, in the tile

    const int64_t row0 = (int64_t)b * T;
    if (w == 0) {
        const bool in = lane < T;
        const int p = in ? parents[row0 + lane] : -1;
        const int32_t x = in ? draft[row0 + lane] : -1;
        const bool xin = x >= 0 && (int64_t)x < V;
        // this node's token in its parent's row, fetched before the walk needs it (every
        // node at once, instead of one dependent load per level)
        const bool fetch = in && lane > 0 && p >= 0 && p < lane && xin;
        const float lx = fetch ? logits[(row0 + p) * V + x] : 0.0f;
        // row statistics of node `lane`
        MS st{-__builtin_huge_valf(), 0.0f};
        if (in) {
            const MS *pr = part + (row0 + lane) * nchunks;
            for (int c0 = 0; c0 < nchunks; c0 += 16) {  // sixteen pairs in flight
                MS q[16];
#pragma unroll
                for (int j = 0; j < 16; ++j)
                    q[j] = c0 + j < nchunks ? pr[c0 + j] : MS{-__builtin_huge_valf(), 0.0f};
#pragma unroll
                for (int j = 0; j < 16; ++j) st = ms_merge(st, q[j], k);
            }
        }
        const bool bad = (lane == 0 && p != -1) || (lane >= 1 && in && (p < 0 || p >= lane));
        const bool invalid = __ballot(bad) != 0ull || (tree_err && tree_err[b] != 0);
        if (invalid) {
            if (in) {
                accepted_nodes[row0 + lane] = -1;
                out_tokens[row0 + lane] = -1;
            }
            if (lane == 0) {
                accepted_len[b] = 0;
                s_state[0] = 1;
            }
        } else {
            const float ux = in ? u_accept[row0 + lane] : 1.0f;  // this node's draw as a proposal
            int v = 0, L = 1;
            uint64_t path = 1ull;
            float R = 1.0f;          // probability left at the current node
            bool rej = false;        // this lane's proposal was rejected at the final node
            float wx = 0.0f;         // weight of this lane's token in its parent's row
            for (;;) {
                R = 1.0f;
                const float mv = lane_f(st.m, v);
                const float zv = lane_f(st.s, v);
                const bool kid = in && p == v && lane > 0;
                wx = (kid && xin && zv > 0.0f) ? weight_of(lx, mv, k) : 0.0f;  // kid: p < lane
                const float px = zv > 0.0f ? wx / zv : 0.0f;
                rej = false;
                uint64_t kids = __ballot(kid);
                int next = -1;
                while (kids) {
                    const int c = __builtin_ctzll(kids);
                    kids &= kids - 1;
                    const int32_t xc = lane_i(x, c);
                    const bool okc = lane_i((int)xin, c) != 0;
                    const bool dup = __ballot(rej && x == xc) != 0ull;
                    const float pc = (okc && !dup) ? lane_f(px, c) : 0.0f;
                    const float u = lane_f(ux, c);
                    if (u * R < pc) {
                        next = c;
                        break;
                    }
                    if (okc && !dup) {
                        if (lane == c) rej = true;
                        R -= pc;
                    }
                }
                if (next < 0) break;
                const int32_t xn = lane_i(x, next);
                if (lane == 0) out_tokens[row0 + L - 1] = xn;
                path |= 1ull << next;
                ++L;
                v = next;
            }
            // path nodes in order (ancestors precede descendants in index order)
            if (in) {
                if ((path >> lane) & 1ull) accepted_nodes[row0 + __popcll(path & ((1ull << lane) - 1ull))] = lane;
                if (lane >= L) {
                    accepted_nodes[row0 + lane] = -1;
                    out_tokens[row0 + lane] = -1;
                }
            }
            // tokens rejected at the final node, compacted in node order
            const uint64_t rm = __ballot(rej);
            if (rej) {
                const int slot = __popcll(rm & ((1ull << lane) - 1ull));
                ex_tok[slot] = x;
                ex_w[slot] = wx;
            }
            const float mv = lane_f(st.m, v);
            const float zv = lane_f(st.s, v);
            if (lane == 0) {
                s_state[0] = 0;
                s_state[1] = v;
                s_state[2] = L;
                s_state[3] = __popcll(rm);
                s_f[0] = mv;
                s_f[1] = u_sample[row0 + v] * R * zv;
                s_f[2] = zv;
                accepted_len[b] = L;
            }
        }
    }
    __syncthreads();
    if (s_state[0]) return;
    const int v = s_state[1];
    const int L = s_state[2];
    const int nex = s_state[3];
    const float mv = s_f[0];
    const float target = s_f[1];
    const float zv = s_f[2];
    const float *row = logits + (row0 + v) * V;

    // chunk holding the target: chunk weights relative to mv less the excluded tokens,
    // 64 chunks at a time across the lanes of wave 0 (prefix scan, first crossing)
    if (w == 0) {
        int pick = -1, lastc = -1;
        float r = 0.0f, carry = 0.0f;
        if (zv > 0.0f) {
            for (int c0 = 0; c0 < nchunks && pick < 0; c0 += 64) {
                const int c = c0 + lane;
                float wc = 0.0f;
                if (c < nchunks) {
                    const MS q = part[(row0 + v) * nchunks + c];
                    wc = q.m == -__builtin_huge_valf() ? 0.0f : q.s * __builtin_amdgcn_exp2f((q.m - mv) * k);
                    const int64_t lo = (int64_t)c * chunk, hi = lo + chunk;
                    for (int j = 0; j < nex; ++j)
                        if (ex_tok[j] >= lo && ex_tok[j] < hi) wc -= ex_w[j];
                    wc = wc > 0.0f ? wc : 0.0f;
                }
                const float incl = wave_incl_sum(wc);  // inclusive prefix over the lanes
                const uint64_t hm = __ballot(wc > 0.0f && carry + incl > target);
                if (hm) {
                    const int hl = __builtin_ctzll(hm);
                    pick = c0 + hl;
                    r = target - (carry + lane_f(incl - wc, hl));
                } else {
                    const uint64_t pm = __ballot(wc > 0.0f);
                    if (pm) lastc = c0 + 63 - __builtin_clzll(pm);
                    carry += lane_f(incl, 63);
                }
            }
            if (pick < 0 && lastc >= 0) {  // rounding: the last chunk with weight, its end
                pick = lastc;
                r = __builtin_huge_valf();
            }
        }
        if (lane == 0) {
            s_pick[0] = pick;
            s_r[0] = r;
        }
    }
    __syncthreads();
    const int pc = s_pick[0];
    int32_t tok = 0;
    if (pc >= 0) {
        const int64_t lo = (int64_t)pc * chunk;
        const int64_t hi = lo + chunk < V ? lo + chunk : V;
        const int ntile = (int)((hi - lo + kTile - 1) / kTile);
        // tile weights: wave w owns tiles w, w + 16, w + 32, w + 48 and loads them in one
        // round (lane l: elements l, l + 64, l + 128, l + 192 of each, coalesced); the
        // element weights stay in LDS for the search inside the chosen tile, each lane's
        // partial sums go to LDS too (row stride 65: no bank conflicts), then thread t adds
        // up tile t's 64
        {
            static_assert(kMaxTiles == 4 * kWalkWaves, "four tiles per wavefront");
            float x[4][4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = w + kWalkWaves * j;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t y = lo + (int64_t)t * kTile + lane + 64 * q;
                    x[j][q] = t < ntile && y < hi ? row[y] : -__builtin_huge_valf();
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = w + kWalkWaves * j;
                float s = 0.0f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float l = clean_logit(x[j][q]);
                    const float wy =
                        l > -__builtin_huge_valf() ? __builtin_amdgcn_exp2f((l - mv) * k) : 0.0f;
                    s += wy;
                    if (t < ntile) ew[t * kTile + lane + 64 * q] = wy;
                }
                if (t < ntile) red[t * 65 + lane] = s;
            }
        }
        __syncthreads();
        if (tid < ntile) {
            float s = 0.0f;
            for (int j = 0; j < 64; ++j) s += red[tid * 65 + j];
            tile_sum[tid] = s;
        }
        __syncthreads();
        // tile holding the residual target: wave 0, lane l holds tiles 4l .. 4l + 3 (less the
        // excluded tokens' weights), a prefix scan across lanes, first crossing
        if (w == 0) {
            float tw[4], mine = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int t = 4 * lane + q;
                float x = t < ntile ? tile_sum[t] : 0.0f;
                for (int j = 0; j < nex; ++j)
                    if (ex_tok[j] >= lo && ex_tok[j] < hi && (ex_tok[j] - lo) / kTile == t) x -= ex_w[j];
                tw[q] = x > 0.0f ? x : 0.0f;
                mine += tw[q];
            }
            const float incl = wave_incl_sum(mine);
            const float r = s_r[0];
            float acc = incl - mine;
            int hit = -1, lastq = -1;
            float before_hit = 0.0f;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (tw[q] > 0.0f) {
                    if (hit < 0 && acc + tw[q] > r) {
                        hit = q;
                        before_hit = acc;
                    }
                    lastq = q;
                    acc += tw[q];
                }
            }
            int pick;
            float rr;
            const uint64_t hm = __ballot(hit >= 0);
            if (hm) {
                const int hl = __builtin_ctzll(hm);
                pick = 4 * hl + lane_i(hit, hl);
                rr = r - lane_f(before_hit, hl);
            } else {  // rounding: the last tile with weight, its end
                const uint64_t lm = __ballot(lastq >= 0);
                const int ll = lm ? 63 - __builtin_clzll(lm) : 0;
                pick = lm ? 4 * ll + lane_i(lastq, ll) : -1;
                rr = __builtin_huge_valf();
            }
            if (lane == 0) {
                s_pick[1] = pick;
                s_r[1] = rr;
            }
        }
        __syncthreads();
        const int tp = s_pick[1];
        if (w == 0 && tp >= 0) {
            // lane l owns elements 4l .. 4l+3 of the tile, in index order (their weights
            // from LDS; elements past the chunk hold 0)
            const int64_t base = lo + (int64_t)tp * kTile + 4 * lane;
            float e[4];
            for (int q = 0; q < 4; ++q) {
                const int64_t y = base + q;
                float wy = ew[tp * kTile + 4 * lane + q];
                for (int j = 0; j < nex; ++j)
                    if (ex_tok[j] == y) wy = 0.0f;
                e[q] = wy;
            }
            const float mine = e[0] + e[1] + e[2] + e[3];
            const float incl = wave_incl_sum(mine);  // inclusive prefix over lanes
            const float r = s_r[1];
            float acc = incl - mine;
            int hit = -1, lastpos = -1;
            for (int q = 0; q < 4; ++q) {
                if (e[q] > 0.0f) {
                    acc += e[q];
                    lastpos = q;
                    if (hit < 0 && acc > r) hit = q;
                }
            }
            const uint64_t hm = __ballot(hit >= 0);
            if (hm) {
                const int hl = __builtin_ctzll(hm);
                tok = lane_i((int)(base + (hit < 0 ? 0 : hit)), hl);
            } else {
                // rounding: the last element with weight in the tile
                const uint64_t lm = __ballot(lastpos >= 0);
                const int ll = lm ? 63 - __builtin_clzll(lm) : 0;
                tok = lane_i((int)(base + (lastpos < 0 ? 0 : lastpos)), ll);
                if (!lm) tok = 0;
            }
        }
    }
    if (tid == 0) {
        // the same value in lane 0 of wave 0 (tok was formed there when a chunk was picked)
        out_tokens[row0 + L - 1] = pc >= 0 ? tok : 0;
    }
}

}  // namespace

int make_sample_plan(int64_t rows, int64_t V, ArgmaxPlan *p) {
    const int rc = make_argmax_plan(rows, V, p);
    if (rc != 0) return rc;
    // the draw re-reads one chunk of the final node's row, by 256-element tiles: at most
    // kMaxTiles tiles a chunk keep that read to one round of loads, while the streaming
    // pass still has several workgroups per row
    const int64_t cap = (int64_t)kTile * kMaxTiles;
    if (p->chunk > cap) {
        p->chunk = cap;
        p->nchunks = (int)((V + cap - 1) / cap);
    }
    p->ws_bytes = (size_t)rows * p->nchunks * sizeof(MS);  // (max, sum) per row and chunk
    return 0;
}

hipError_t launch_accept_sampled(const float *logits, const int32_t *draft,
                                 const int32_t *parents, const int32_t *tree_err,
                                 const float *u_accept, const float *u_sample, float temperature,
                                 int B, int T, int64_t V, const ArgmaxPlan &p, void *ws,
                                 int32_t *accepted_len, int32_t *accepted_nodes,
                                 int32_t *out_tokens, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    const float k = 1.4426950408889634f / temperature;  // log2(e) / tau
    const int64_t rows = (int64_t)B * T;
    MS *part = static_cast<MS *>(ws);
    hipLaunchKernelGGL(softmax_partial_kernel, dim3((unsigned)(rows * p.nchunks)), dim3(256), 0,
                       stream, logits, V, p.chunk, p.nchunks, k, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(sample_walk_kernel, dim3((unsigned)B), dim3(64 * kWalkWaves), 0, stream,
                       logits, part,
                       V, p.chunk, p.nchunks, k, draft, parents, tree_err, u_accept, u_sample, T,
                       accepted_len, accepted_nodes, out_tokens);
    return hipGetLastError();
}

}  // namespace sv
