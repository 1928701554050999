// topk.hip -- top-K of the log-softmax of logits rows, and the global best-first
// expansion of a draft tree from the drafter's rows.
//
// Rules (ADR-037 Phase status rows E4b.10a and E4a; section 4 Phase E4):
//   l(y) = the logit, with NaN and -inf read as -inf and +inf as the largest finite float;
//   logp(y) = (l(y) - m) - log Z in fp64, m = max l, Z = sum over finite l of exp(l - m)
//   (every logp is -inf when the row has no finite entry).  The K largest log-probabilities
//   are chosen by comparing l itself (logp increases strictly with l, so no rounding can
//   merge two distinct values), ties to the smaller token, best first.
//   Best-first: node 0 is the root (cumulative log-prob 0, level 1).  The drafter's output
//   for the node admitted i-th is row i; admitting node i offers its K best tokens as
//   candidate children with key cum(i) + logp, unless node i is on the last allowed level
//   or completes the tree.  The pending candidate with the largest key (fp64) is admitted
//   next, ties to the one offered first; until T nodes.
//
// topk_rows_kernel: one workgroup of four wavefronts per row.  Every lane streams its
// 16-byte pieces once (buffer loads, each trip's loads in flight during the trip before)
// and keeps fp64 sums of exponentials (sum_small4 for pieces of logits below 31.5 in
// magnitude; otherwise an online max and exp_core, below).  Each wavefront keeps a candidate buffer in LDS: a piece's
// element enters it when it beats the wavefront's K-th best so far (while fewer than K
// entries exist, every element enters) and is not below the K-th best another wavefront
// has published.  When the buffer grows, the wavefront keeps its K best (K rounds of a
// 64-lane DPP max over (value, -index) keys), raises its threshold and publishes it.  At
// the end the four wavefronts' lists are merged the same way.
// best_first_kernel: one wavefront per sequence.  Lane j stands for admitted node j and
// holds its best child not admitted yet: a node's children come best first, so no other
// child of it can be next.  Each admission is a 64-lane max over those keys, ties to the
// lower lane (the earlier parent); the winner moves on to its next child and the lane of
// the new node starts on its own first child.
#include "sv_internal.h"

namespace sv {
namespace {

constexpr int kTkWaves = 4;                 // wavefronts per row
constexpr int kTkThreads = 64 * kTkWaves;
constexpr int kCap = 512;                   // candidate entries per wavefront
constexpr int kPiece = 256;                 // the most one piece (one 16-byte load per lane) adds
constexpr float kFltMax = 3.40282347e38f;
constexpr int kNonTemporal = 2;             // cache policy bits of a buffer load: nt
constexpr int kRsrcWord3 = 0x00020000;      // raw 32-bit buffer resource, gfx9 family

// exp(d) for d in [-700, 0] in fp64, callers clamp d into that range first.  Table-driven
// method (P. T. P. Tang, "Table-driven implementation of the exponential function in IEEE
// floating-point arithmetic", ACM TOMS 15(2), 1989): d = (256 k + j) ln2/256 + r with
// |r| <= ln2/512, so e^d = 2^k * 2^(j/256) * e^r; e^r - 1 is its Taylor polynomial of
// degree 4 (remainder below 2^-54 relative) and 2^(j/256) comes from a 256-entry table.
// n = 256 k + j is rounded by adding 1.5 * 2^52 (its low word then holds n).
__device__ __forceinline__ double exp_core(double d, const double *tab) {
    constexpr double kInvL = 0x1.71547652b82fep+8;    // 256 / ln 2
    constexpr double kL1 = 0x1.62e42fefa39efp-9;      // ln 2 / 256, leading part
    constexpr double kL2 = 0x1.abc9e3b39803fp-64;     // ln 2 / 256 - kL1
    constexpr double kRound = 0x1.8p52;
    const double nb = fma(d, kInvL, kRound);
    const double n = nb - kRound;
    const int ni = __double2loint(nb);
    double r = fma(-n, kL1, d);
    r = fma(-n, kL2, r);
    double q = fma(r, 1.0 / 24.0, 1.0 / 6.0);
    q = fma(q, r, 0.5);
    const double p = fma(r * r, q, r);                // e^r - 1
    const double t = tab[ni & 255];
    return ldexp(fma(t, p, t), ni >> 8);               // ni >> 8 = floor(n / 256)
}

// exp(x - m) for a raw logit x and a lane max m >= every finite x seen: NaN and -inf give
// 0, +inf gives 1 (it counts as the largest finite float, which then is m).
__device__ __forceinline__ double exp_term(float x, double md, const double *tab) {
    double d = (double)x - md;
    d = fmin(fmax(d, -700.0), 0.0);                    // fmax(NaN, -700) = -700
    return x > -__builtin_huge_valf() ? exp_core(d, tab) : 0.0;
}

// Adds e^x for four logits, each with |x| < 31.5, in fp64 from their fp32 values, to two
// running sums (logits 0 and 1 to s0, 2 and 3 to s1): n = round(1024 x) by the rounding
// trick in fp32 (adding 1.5 * 2^23 + 2^15 leaves 0x4B408000 + n in the bits), after which
// r = x - n/1024 is exact in fp32 with |r| <= 2^-11; with n = 256 k + j,
// e^x = e^(k/4) * (e^(j/1024) * e^r), the first two factors from tables indexed by bytes
// of those bits (t1[k + 128] by byte 1, t2[j] by byte 0) and e^r - 1 its Taylor polynomial
// of degree 3 (the remainder, r^4/24 and beyond, stays below 2^-48 relative: under the
// rounding of the fp64 sum of a row's terms, and one fp64 operation per logit fewer than
// degree 4).  Same table-driven method as exp_core, with
// no reduction step and no reference maximum.  The eight table reads are issued before the
// polynomials, which hide their latency.
__device__ __forceinline__ void sum_small4(const f32x4 &x, const double *t1, const double *t2,
                                           double &s0, double &s1) {
    constexpr float kMagic = 12615680.0f;              // 1.5 * 2^23 + 2^15
    double A[4], Bt[4], p[4];
    float rf[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float t = fmaf(x[e], 1024.0f, kMagic);
        rf[e] = fmaf(t - kMagic, -1.0f / 1024.0f, x[e]);
        const uint32_t b = __float_as_uint(t);
        A[e] = t1[(b >> 8) & 255u];
        Bt[e] = t2[b & 255u];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const double r = (double)rf[e];
        const double q = fma(r, 1.0 / 6.0, 0.5);
        p[e] = fma(r * r, q, r);                       // e^r - 1, to degree 3
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const double u = fma(Bt[e], p[e], Bt[e]);      // e^(j/1024) e^r
        if (e < 2) s0 = fma(A[e], u, s0);
        else s1 = fma(A[e], u, s1);
    }
}

// Whether all four logits are finite with |x| < 31.5 (the range of sum_small4), tested as
// a sum of squares below 31.5^2: rounding is monotone and every term is >= 0, so the
// rounded sum reaches 992.25 whenever one |x| does reach 31.5; inf gives inf and NaN fails
// the test.
__device__ __forceinline__ bool small_piece(const f32x4 &x) {
    const float q = fmaf(x[3], x[3], fmaf(x[2], x[2], fmaf(x[1], x[1], x[0] * x[0])));
    return q < 992.25f;
}

// A logit as the rule reads it: NaN and -inf give -inf, +inf the largest finite float, and
// -0 becomes +0 so that the two zeros compare equal as keys.
__device__ __forceinline__ float clean(float x) {
    x = fminf(fmaxf(x, -__builtin_huge_valf()), kFltMax);   // fmaxf(NaN, -inf) = -inf
    return x + 0.0f;
}

// The largest of four raw logits as the rule reads them (-inf when none is finite).  The
// max instructions ignore a quiet NaN operand; v_max_f32 x, x first quiets a signalling
// one.  (Inline assembly, so that these moves stay on the path that needs them.)
__device__ __forceinline__ float max4(const f32x4 &x) {
    float a, b;
    asm("v_max_f32 %0, %2, %2\n\t"
        "v_max_f32 %1, %3, %3\n\t"
        "v_max_f32 %0, %0, %1\n\t"
        "v_max_f32 %1, %4, %4\n\t"
        "v_max_f32 %0, %0, %1\n\t"
        "v_max_f32 %1, %5, %5\n\t"
        "v_max_f32 %0, %0, %1"
        : "=&v"(a), "=&v"(b) : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
    return fminf(fmaxf(a, -__builtin_huge_valf()), kFltMax);
}

// Order-preserving 64-bit key of (value, index): larger value first, then smaller index.
// 0 marks an empty slot (every real key is larger: ord(-inf) = 0x007fffff).
__device__ __forceinline__ uint64_t cand_key(float v, int32_t idx) {
    if (idx < 0) return 0;
    const uint32_t u = __float_as_uint(v);
    const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)o << 32) | (uint64_t)(0xffffffffu - (uint32_t)idx);
}
__device__ __forceinline__ float key_value(uint64_t k) {
    const uint32_t o = (uint32_t)(k >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
__device__ __forceinline__ int32_t key_index(uint64_t k) {
    return (int32_t)(0xffffffffu - (uint32_t)k);
}

// A 32-bit value moved across lanes by one DPP control; lanes without a source, or
// outside the rows of kRowMask, read 0.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, kRowMask, 0xf, true);
}

// Maximum over the wavefront of unsigned 32-bit values, in every lane: row_shr 1, 2, 4, 8
// leave each row's maximum in its lane 15; row_bcast 15 and 31 carry it into lane 63.
__device__ __forceinline__ uint32_t wave_max_dpp32(uint32_t x) {
    x = max(x, dpp_u32<0x111, 0xf>(x));
    x = max(x, dpp_u32<0x112, 0xf>(x));
    x = max(x, dpp_u32<0x114, 0xf>(x));
    x = max(x, dpp_u32<0x118, 0xf>(x));
    x = max(x, dpp_u32<0x142, 0xa>(x));
    x = max(x, dpp_u32<0x143, 0xc>(x));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// The lowest lane holding the largest nonzero 64-bit key, or -1 when every key is 0: a
// 32-bit maximum over the high words, then (only when several lanes share that word)
// over the low words of those lanes.
__device__ __forceinline__ int wave_argmax_key(uint64_t k) {
    const uint32_t hi = (uint32_t)(k >> 32);
    const uint32_t mhi = wave_max_dpp32(hi);
    const bool cand = k != 0 && hi == mhi;
    uint64_t bal = __ballot(cand);
    if (bal == 0) return -1;
    if (bal & (bal - 1)) {
        const uint32_t lo = cand ? (uint32_t)k : 0u;
        const uint32_t mlo = wave_max_dpp32(lo);
        bal = __ballot(cand && lo == mlo);
    }
    return (int)__builtin_ctzll(bal);
}

// Keeps the best min(n, K) of entries [0, n) (n <= 64 * kSlots) of a wavefront's (value,
// index) arrays in slots [0, min(n, K)), best first, and returns that count.  Entries with
// index -1 are empty.  Every lane reads its entries before any slot is written.
template <int kSlots>
__device__ int keep_best_n(float *cv, int32_t *ci, int n, int K, int lane) {
    uint64_t key[kSlots];
#pragma unroll
    for (int s = 0; s < kSlots; ++s) {
        const int q = s * 64 + lane;
        key[s] = q < n ? cand_key(cv[q], ci[q]) : 0;
    }
    const int m = n < K ? n : K;
    uint64_t mine = 0;
    for (int r = 0; r < m; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int s = 1; s < kSlots; ++s) best = key[s] > best ? key[s] : best;
        const int wl = wave_argmax_key(best);
        const uint64_t w =
            wl < 0 ? 0
                   : ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(best >> 32), wl)
                      << 32) |
                         (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)best, wl);
#pragma unroll
        for (int s = 0; s < kSlots; ++s) key[s] = key[s] == w ? 0 : key[s];
        mine = lane == r ? w : mine;
    }
    if (lane < m) {
        cv[lane] = key_value(mine);
        ci[lane] = mine ? key_index(mine) : -1;
    }
    return m;
}

// keep_best_n with as few slots per lane as n needs (n <= kCap).
__device__ int keep_best(float *cv, int32_t *ci, int n, int K, int lane) {
    if (n <= 64) return keep_best_n<1>(cv, ci, n, K, lane);
    if (n <= 256) return keep_best_n<4>(cv, ci, n, K, lane);
    return keep_best_n<kCap / 64>(cv, ci, n, K, lane);
}

struct WaveCands {
    float *cv;
    int32_t *ci;
    int cnt;      // entries in the buffer (wavefront-uniform)
    float tau;    // K-th best value once the buffer was cut to K, else -inf
    float *pub;   // every wavefront's last tau, in LDS (-inf before its first cut)
    float tsh;    // the largest of them when last read
};

__device__ __forceinline__ float uniform_f(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// Reads the wavefronts' published thresholds.  Another wavefront's K-th best u means K
// logits >= u exist, so a logit below u cannot be among the row's K best; one equal to u
// still can (ties go to the smaller token, and the wavefronts' tokens interleave), hence
// the test v >= tsh next to v > tau.  A stale value is an older, lower one: still a bound.
__device__ __forceinline__ void refresh_shared(WaveCands &wc) {
    float t = __hip_atomic_load(wc.pub, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
#pragma unroll
    for (int j = 1; j < kTkWaves; ++j)
        t = fmaxf(t, __hip_atomic_load(wc.pub + j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
    wc.tsh = uniform_f(t);
}

// After a cut back to K entries: the new threshold, published for the other wavefronts.
__device__ __forceinline__ void set_tau(WaveCands &wc, int w, int lane) {
    wc.tau = uniform_f(wc.cv[wc.cnt - 1]);
    if (lane == 0)
        __hip_atomic_store(wc.pub + w, wc.tau, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// One piece: up to four consecutive raw logits per lane (the first `nok` exist), all with
// larger indices than every entry already in the buffer, mx = max4 of them.  They are
// judged against the buffer as it stood before the piece.  Once the buffer holds K + 24
// entries it is cut back to K, so the threshold follows the running K-th best closely
// (each cut is K rounds of a 64-lane max over one slot per lane).
// Whether a logit of value m could enter the buffer now (the test of offer_piece).
__device__ __forceinline__ bool may_enter(const WaveCands &wc, float m, int K) {
    return (wc.cnt < K || m > wc.tau) && m >= wc.tsh;
}

__device__ __forceinline__ void offer_piece(WaveCands &wc, const f32x4 &x, float mx, int nok,
                                            int32_t idx0, int K, int w, int lane) {
    if (!__any(nok > 0 && may_enter(wc, mx, K))) return;
    bool full = wc.cnt >= K;
    if (wc.cnt + kPiece > kCap) {
        wc.cnt = __builtin_amdgcn_readfirstlane(keep_best(wc.cv, wc.ci, wc.cnt, K, lane));
        full = wc.cnt >= K;
        if (full) set_tau(wc, w, lane);
    }
    int cnt = wc.cnt;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float v = clean(x[e]);
        const bool pass = e < nok && (!full || v > wc.tau) && v >= wc.tsh;
        const uint64_t bal = __ballot(pass);
        if (bal) {
            const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi(
                                      (uint32_t)(bal >> 32),
                                      __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            if (pass) {
                wc.cv[pos] = v;
                wc.ci[pos] = idx0 + e;
            }
            cnt += __popcll(bal);
        }
    }
    wc.cnt = cnt;
    if (cnt >= K + 24) {
        wc.cnt = K;
        keep_best(wc.cv, wc.ci, cnt, K, lane);
        set_tau(wc, w, lane);
    }
}

// A lower bound of a row's K-th best logit from a wavefront's first trip: the K-th largest
// of its 64 lanes' maxima (K <= 64).  K distinct logits reach it, so a logit below it cannot
// be among the row's K best (one equal to it still can: ties go to the smaller token); the
// wavefront publishes it as it publishes its K-th best, which filters the rest of the trip
// instead of taking every logit of its first piece into the buffer.  K rounds of a 64-lane
// max over order-preserving keys, each taking out the lowest lane that holds the maximum.
__device__ __forceinline__ float kth_lane_max(float lm, int K, int lane) {
    const uint32_t u = __float_as_uint(lm);
    uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // lm is not NaN: key > 0
    uint32_t m = 0;
    for (int r = 0; r < K; ++r) {
        m = wave_max_dpp32(key);
        const uint64_t bal = __ballot(key == m);
        if (lane == (int)__builtin_ctzll(bal)) key = 0;
    }
    return __uint_as_float((m & 0x80000000u) ? (m & 0x7fffffffu) : ~m);
}

// The lane's share of sum_y exp(l(y)) in two parts: pieces whose logits all have |x| < 31.5
// add exp(x) directly (sf, sf2); any other piece goes, whole, to an online max m and a sum s of
// exp(x - m) (NaN and -inf add 0, +inf counts as the largest finite float).
struct RowSum {
    double sf;   // sum of exp(x) over the small pieces, in two parts
    double sf2;
    float m;     // running max over the other pieces (-FLT_MAX before the first)
    double md;   // m as a double
    double s;    // sum of exp(x - m) over the other pieces
};

// The largest of four values that are not NaN (so the max instructions need no quieting
// moves before them).
__device__ __forceinline__ float max4_ordered(const f32x4 &x) {
    float m;
    asm("v_max3_f32 %0, %1, %2, %3\n\tv_max_f32 %0, %0, %4"
        : "=&v"(m) : "v"(x[0]), "v"(x[1]), "v"(x[2]), "v"(x[3]));
    return m;
}

// Adds a piece to the lane's sums (entries beyond those that exist are -inf) and returns
// the largest of its logits as the rule reads them (max4).  Whether it takes the
// small-piece path is decided for the whole wavefront.
__device__ __forceinline__ float sum_piece(RowSum &a, const f32x4 &x, const double *tab,
                                           const double *t1, const double *t2) {
    if (__all(small_piece(x))) {
        sum_small4(x, t1, t2, a.sf, a.sf2);
        return max4_ordered(x);
    }
    const float mx = max4(x);
    if (mx > a.m) {
        const double mxd = (double)mx;
        a.s *= exp_core(fmax(a.md - mxd, -700.0), tab);
        a.m = mx;
        a.md = mxd;
    }
    const double e0 = exp_term(x[0], a.md, tab), e1 = exp_term(x[1], a.md, tab);
    const double e2 = exp_term(x[2], a.md, tab), e3 = exp_term(x[3], a.md, tab);
    a.s += (e0 + e1) + (e2 + e3);
    return mx;
}

__global__ __launch_bounds__(kTkThreads) void topk_rows_kernel(
    const float *__restrict__ logits, int64_t V, int K, int rows_per_group,
    int64_t group_stride, int32_t *__restrict__ top_tok, double *__restrict__ top_logp) {
    __shared__ float s_cv[kTkWaves][kCap];
    __shared__ int32_t s_ci[kTkWaves][kCap];
    __shared__ double s_tab[256];
    __shared__ double s_t1[256];
    __shared__ double s_t2[256];
    __shared__ double s_sf[kTkWaves];
    __shared__ float s_m[kTkWaves];
    __shared__ double s_s[kTkWaves];
    __shared__ float s_pub[kTkWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int64_t r = blockIdx.x;
    const int64_t src = (r / rows_per_group) * group_stride + r % rows_per_group;
    const float *rp = logits + src * V;
    constexpr float kNInf = -__builtin_huge_valf();

    // head: elements before the first 16-byte aligned one (wavefront 0, lanes 0..2)
    const int64_t mis = (int64_t)((reinterpret_cast<uintptr_t>(rp) >> 2) & 3);
    int64_t a0 = (4 - mis) & 3;
    if (a0 > V) a0 = V;
    const int64_t nvec = (V - a0) >> 2;
    const int64_t a1 = a0 + 4 * nvec;
    // body: 16-byte pieces, piece p = base + u * 256 + tid holds elements a0 + 4p .. + 3;
    // whole trips of four pieces per lane, then one trip with the pieces that are left
    const f32x4 *vp = reinterpret_cast<const f32x4 *>(rp + a0);
    constexpr int64_t kTrip = 4 * kTkThreads;
    const int64_t nfull = nvec / kTrip * kTrip;
    // one trip's loads: buffer loads from the trip's start (kept in scalar registers) at
    // 32-bit lane offsets; non-temporal, since every logit is read once
    auto fetch = [&](f32x4 (&raw)[4], int64_t base) __attribute__((always_inline)) {
        const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<f32x4 *>(vp + base), 0,
                                                          (int)(kTrip * 16), kRsrcWord3);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            raw[u] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rs, (u * kTkThreads + tid) * 16, 0, kNonTemporal));
    };
    // the first trip's loads go out before the tables are built
    f32x4 ra[4], rb[4];
    if (nfull > 0) fetch(ra, 0);

    s_tab[tid] = exp2((double)tid / 256.0);
    s_t1[tid] = exp((double)(tid - 128) * 0.25);
    s_t2[tid] = exp((double)tid / 1024.0);
    if (tid < kTkWaves) s_pub[tid] = kNInf;
    __syncthreads();

    WaveCands wc{s_cv[w], s_ci[w], 0, kNInf, s_pub, kNInf};
    RowSum acc{0.0, 0.0, -kFltMax, (double)-kFltMax, 0.0};

    // the head's elements, before the first 16-byte aligned one
    if (w == 0) {
        const int nok = lane < a0 ? 1 : 0;
        const f32x4 x{nok ? rp[lane] : kNInf, kNInf, kNInf, kNInf};
        const float mx = sum_piece(acc, x, s_tab, s_t1, s_t2);
        offer_piece(wc, x, mx, nok, lane, K, w, lane);
    }

    // one trip's sums and offers.  The common case, every piece small, is one block, so
    // that its sixteen exponentials interleave.  Most trips hold no logit that could enter
    // (one test for the four pieces); the others offer their pieces one at a time.  The
    // first trip first publishes the K-th largest of its lane maxima (kth_lane_max).
    auto trip = [&](const f32x4 (&raw)[4], int64_t base) __attribute__((always_inline)) {
        float mx[4];
        // (all four tested, without short-circuit branches: a bitwise and of the lane masks)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Wbitwise-instead-of-logical"
        const bool all_small = small_piece(raw[0]) & small_piece(raw[1]) & small_piece(raw[2]) &
                               small_piece(raw[3]);
#pragma clang diagnostic pop
        if (__all(all_small)) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                sum_small4(raw[u], s_t1, s_t2, acc.sf, acc.sf2);
                mx[u] = max4_ordered(raw[u]);
            }
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) mx[u] = sum_piece(acc, raw[u], s_tab, s_t1, s_t2);
        }
        const float tmax = max4_ordered(f32x4{mx[0], mx[1], mx[2], mx[3]});
        if (base == 0) {
            const float th = kth_lane_max(tmax, K, lane);
            if (lane == 0) __hip_atomic_store(wc.pub + w, th, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        refresh_shared(wc);
        if (!__any(may_enter(wc, tmax, K))) return;
        f32x4 r0 = raw[0], r1 = raw[1], r2 = raw[2], r3 = raw[3];
        float m0 = mx[0], m1 = mx[1], m2 = mx[2], m3 = mx[3];
#pragma unroll 1
        for (int u = 0; u < 4; ++u) {
            offer_piece(wc, r0, m0, 4, (int32_t)(a0 + 4 * (base + u * kTkThreads + tid)), K, w,
                        lane);
            r0 = r1; r1 = r2; r2 = r3;
            m0 = m1; m1 = m2; m2 = m3;
        }
    };
    // two buffers: each trip's loads are in flight during the trip before.  The loads are
    // issued unconditionally (past the last trip they re-read the trip before, in bounds)
    // so that the wait before a trip's math counts that trip's loads only.
    for (int64_t base = 0; base < nfull; base += 2 * kTrip) {
        const bool two = base + kTrip < nfull;
        fetch(rb, two ? base + kTrip : base);
        trip(ra, base);
        if (!two) break;
        fetch(ra, base + 2 * kTrip < nfull ? base + 2 * kTrip : base);
        trip(rb, base + kTrip);
    }
    if (nfull < nvec) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t p = nfull + u * kTkThreads + tid;
            const f32x4 x = p < nvec ? vp[p] : f32x4{kNInf, kNInf, kNInf, kNInf};
            const float mx = sum_piece(acc, x, s_tab, s_t1, s_t2);
            offer_piece(wc, x, mx, p < nvec ? 4 : 0, (int32_t)(a0 + 4 * p), K, w, lane);
        }
    }

    // tail: the last V - a1 (< 4) elements (wavefront 0), larger than every index above
    if (w == 0) {
        const int nok = a1 + lane < V ? 1 : 0;
        const f32x4 x{nok ? rp[a1 + lane] : kNInf, kNInf, kNInf, kNInf};
        const float mx = sum_piece(acc, x, s_tab, s_t1, s_t2);
        offer_piece(wc, x, mx, nok, (int32_t)(a1 + lane), K, w, lane);
    }

    // each wavefront's K best, then the max and sum of the wavefront
    const int c = keep_best(wc.cv, wc.ci, wc.cnt, K, lane);
    for (int k = c + lane; k < K; k += 64) wc.ci[k] = -1;
    float M = acc.m;
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    double S = acc.s * exp_core(fmax(acc.md - (double)M, -700.0), s_tab);
    double SF = acc.sf + acc.sf2;
    for (int off = 32; off > 0; off >>= 1) {
        S += __shfl_xor(S, off, 64);
        SF += __shfl_xor(SF, off, 64);
    }
    if (lane == 0) {
        s_m[w] = M;
        s_s[w] = S;
        s_sf[w] = SF;
    }
    __syncthreads();
    // the other three lists move behind wavefront 0's, which then keeps the best K of 4K
    for (int q = tid; q < (kTkWaves - 1) * K; q += kTkThreads) {
        const int ww = 1 + q / K, k = q - (ww - 1) * K;
        s_cv[0][K + q] = s_cv[ww][k];
        s_ci[0][K + q] = s_ci[ww][k];
    }
    __syncthreads();
    if (w != 0) return;
    const int kept = keep_best(s_cv[0], s_ci[0], kTkWaves * K, K, lane);
    (void)kept;  // = K: the row holds V >= K elements
    // logp(y) = (l(y) - R) - log(SF e^-R + S e^(M-R)), the sum of exp(l - R) over the row,
    // with R = 0 when only small pieces added anything, M when only the others did, else
    // max(M, 0) (so both factors are <= 1 and l - R is exact)
    M = s_m[0];
    for (int j = 1; j < kTkWaves; ++j) M = fmaxf(M, s_m[j]);
    S = 0.0;
    SF = 0.0;
    for (int j = 0; j < kTkWaves; ++j) {
        S += s_s[j] * exp_core(fmax((double)s_m[j] - (double)M, -700.0), s_tab);
        SF += s_sf[j];
    }
    double R = 0.0, logS = log(SF);
    if (S > 0.0 && SF > 0.0) {
        R = fmax((double)M, 0.0);
        logS = log(SF * exp_core(fmax(-R, -700.0), s_tab) +
                   S * exp_core(fmax((double)M - R, -700.0), s_tab));
    } else if (S > 0.0) {
        R = (double)M;
        logS = log(S);
    }
    for (int k = lane; k < K; k += 64) {
        const float v = s_cv[0][k];
        top_tok[r * K + k] = s_ci[0][k];
        top_logp[r * K + k] = v > kNInf ? ((double)v - R) - logS : -__builtin_huge_val();
    }
}

__device__ __forceinline__ uint64_t ord_f64(double x) {
    const uint64_t u = (uint64_t)__double_as_longlong(x);
    return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

__device__ __forceinline__ double readlane_f64(double x, int lane) {
    const int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
    const int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
    return __hiloint2double(hi, lo);
}

// Maximum over the wavefront of unsigned 32-bit values, in every lane: within each row of
// 16 lanes by DPP butterflies (quad_perm 1032 and 2301, row_half_mirror, row_mirror), then
// across rows by the gfx950 row swaps (permlane16_swap exchanges rows 1 and 3 of its first
// operand with rows 0 and 2 of its second, permlane32_swap the upper half of the first
// with the lower half of the second; with both operands equal the two results hold the
// two partners of each lane pair).
__device__ __forceinline__ uint32_t wave_max_all_u32(uint32_t x) {
    x = max(x, dpp_u32<0xb1, 0xf>(x));
    x = max(x, dpp_u32<0x4e, 0xf>(x));
    x = max(x, dpp_u32<0x141, 0xf>(x));
    x = max(x, dpp_u32<0x140, 0xf>(x));
    const auto a = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    x = max((uint32_t)a[0], (uint32_t)a[1]);
    const auto c = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return max((uint32_t)c[0], (uint32_t)c[1]);
}

// One wavefront per sequence (T <= 64: one lane per node).  Row i's lists sit at
// [b][i][K] for i < T - 1, staged in LDS.  Each lane keeps its head child (the best one not
// admitted yet) and the one after it in registers; an admission is a wavefront maximum of
// the high words of the order-preserving keys (the low words only break a tie), read-lane
// broadcasts of the winner, and branch-free updates; every lane then re-reads the child
// after its head, which the next admission needs only after its own maximum.
__global__ __launch_bounds__(64) void best_first_kernel(
    const int32_t *__restrict__ top_tok, const double *__restrict__ top_logp,
    const int32_t *__restrict__ root_token, int T, int K, int max_levels,
    int32_t *__restrict__ parents, int32_t *__restrict__ tokens, double *__restrict__ cum) {
    extern __shared__ double s_lp[];              // [(T - 1) * K] log-probs, then tokens
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int nr = T - 1;
    int32_t *s_tk = reinterpret_cast<int32_t *>(s_lp + (size_t)nr * K);
    const int64_t off = (int64_t)b * nr * K;
    for (int q = lane; q < nr * K; q += 64) {
        s_lp[q] = top_logp[off + q];
        s_tk[q] = top_tok[off + q];
    }
    __syncthreads();

    const int lrow = (lane < nr ? lane : 0) * K;  // this lane's row (row 0 for lanes past it)
    int rank = 0;                                 // rank of the head child
    double hlp = 0.0, nlp = 0.0;                  // log-probs of the head child and the next
    int32_t htok = -1, ntok = -1;
    if (nr > 0) {
        hlp = s_lp[lrow];
        htok = s_tk[lrow];
        nlp = s_lp[lrow + min(1, K - 1)];
        ntok = s_tk[lrow + min(1, K - 1)];
    }
    int32_t par = -1, tok = lane == 0 ? root_token[b] : -1;
    double cj = 0.0;                              // this node's cumulative log-prob
    int level = 1;
    bool live = lane == 0 && nr > 0 && max_levels > 1;   // has a pending child
    for (int n = 1; n < T; ++n) {
        const double key = cj + hlp;
        const uint64_t ok = live ? ord_f64(key) : 0;
        // (the maxima run in every lane: the row swaps and DPP reads need all lanes active)
        const uint32_t hi = (uint32_t)(ok >> 32);
        const uint32_t mhi = wave_max_all_u32(hi);
        const bool cand = ok != 0 && hi == mhi;
        uint64_t bal = __ballot(cand);
        if (bal == 0) break;    // nothing pending: excluded by the caller's shape check
        if (bal & (bal - 1)) {  // several keys share the high word
            const uint32_t lo = cand ? (uint32_t)ok : 0u;
            const uint32_t mlo = wave_max_all_u32(lo);
            bal = __ballot(cand && lo == mlo);
        }
        const int win = (int)__builtin_ctzll(bal);
        const double wkey = readlane_f64(key, win);
        const int32_t wtok = __builtin_amdgcn_readlane(htok, win);
        const int wlevel = __builtin_amdgcn_readlane(level, win);
        const bool won = lane == win;
        rank += won ? 1 : 0;
        live = won ? rank < K : live;
        hlp = won ? nlp : hlp;
        htok = won ? ntok : htok;
        const bool fresh = lane == n;
        par = fresh ? win : par;
        tok = fresh ? wtok : tok;
        cj = fresh ? wkey : cj;
        level = fresh ? wlevel + 1 : level;
        live = fresh ? (n < nr && wlevel + 1 < max_levels) : live;
        const int nx = lrow + min(rank + 1, K - 1);
        nlp = s_lp[nx];
        ntok = s_tk[nx];
    }
    if (lane < T) {
        parents[(int64_t)b * T + lane] = par;
        tokens[(int64_t)b * T + lane] = tok;
        cum[(int64_t)b * T + lane] = cj;
    }
}

}  // namespace

hipError_t launch_topk_rows(const float *logits, int64_t rows, int64_t V, int K,
                            int rows_per_group, int64_t group_stride, int32_t *top_tok,
                            double *top_logp, hipStream_t stream) {
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)rows), dim3(kTkThreads), 0, stream,
                       logits, V, K, rows_per_group, group_stride, top_tok, top_logp);
    return hipGetLastError();
}

hipError_t launch_best_first(const int32_t *top_tok, const double *top_logp,
                             const int32_t *root_token, int B, int T, int K, int max_levels,
                             int32_t *parents, int32_t *tokens, double *cum, hipStream_t stream) {
    if (B == 0) return hipSuccess;
    const size_t smem = (size_t)(T - 1) * K * (sizeof(double) + sizeof(int32_t));
    hipLaunchKernelGGL(best_first_kernel, dim3((unsigned)B), dim3(64), smem, stream, top_tok,
                       top_logp, root_token, T, K, max_levels, parents, tokens, cum);
    return hipGetLastError();
}

}  // namespace sv
