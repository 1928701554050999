// attn_reduce.hip -- merge the per-chunk partial attention results of each query row.
//
// Chunk s of a row left an unnormalised output O_s, its reference max m_s (log2
// units) and the sum l_s of its exp2(score - m_s) weights; the chunks of C keys that
// exist for the row's prefix length took part (C from the plan, or from the workspace
// header when the attention kernel chose it).  With M = max_s m_s:
//   out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s,
// the split-then-merge scheme the pages' flash_attn_vec_reduce plays (ADR-037
// Phase status row E1.2 and the E6 full-layer rows).  One wavefront per output row
// (b, i, h), chunks in a fixed order, no atomics: the result is deterministic.
// The output is laid out [B][T][Hq][D] (ADR-037 row E1.3).
#include "sv_internal.h"

namespace sv {
namespace {

constexpr float kNegInfR = -__builtin_huge_valf();

template <int D>
__global__ __launch_bounds__(256) void attn_reduce_kernel(const float *__restrict__ ws_o,
                                                          const float *__restrict__ ws_ml,
                                                          const int32_t *__restrict__ prefix_len,
                                                          int max_P, int B, int Hq, int Hkv,
                                                          int T, int R, int S, int C,
                                                          const int32_t *__restrict__ c_hdr,
                                                          float *__restrict__ out) {
    constexpr int NV4 = D / 4;                 // float4 vectors per row
    constexpr int VPL = (NV4 + 63) / 64;       // per lane (lanes past NV4 idle at D = 128)
    const int lane = threadIdx.x & 63;
    const int64_t x = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nrows = (int64_t)B * T * Hq;
    if (x >= nrows) return;
    const int h = (int)(x % Hq);
    const int i = (int)((x / Hq) % T);
    const int b = (int)(x / ((int64_t)Hq * T));
    const int G = Hq / Hkv;
    const int kvh = h / G;
    const int r = (h - kvh * G) * T + i;

    int P = prefix_len[b];
    P = P < 0 ? 0 : (P > max_P ? max_P : P);
    if (c_hdr) C = *c_hdr;  // the chunk length the attention kernel chose
    int nv = (P + C - 1) / C;
    nv = nv < 1 ? 1 : (nv > S ? S : nv);

    const int64_t base0 = ((int64_t)b * Hkv + kvh) * S * (int64_t)R + r;
    // the chunks' reference maxima across the lanes (lane s: chunk s, then s + 64, ...):
    // their maximum M in one round trip per 64 chunks
    float M = kNegInfR;
    for (int s = lane; s < nv; s += 64) M = fmaxf(M, ws_ml[(base0 + (int64_t)s * R) * 2]);
    for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));

    // chunks in groups of eight whose loads are all issued before any is used, so that
    // the merge waits for one memory round trip per group, not per chunk; the sums run
    // over the chunks in order
    constexpr int GRP = 8;
    f32x4 acc[VPL];
    for (int v = 0; v < VPL; ++v) acc[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    float L = 0.0f;
    for (int s0 = 0; s0 < nv; s0 += GRP) {
        float m[GRP], l[GRP];
        f32x4 src[GRP][VPL];
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            const int s = s0 + k < nv ? s0 + k : nv - 1;
            const int64_t base = base0 + (int64_t)s * R;
            m[k] = s0 + k < nv ? ws_ml[base * 2] : kNegInfR;
            l[k] = ws_ml[base * 2 + 1];
            const f32x4 *o = reinterpret_cast<const f32x4 *>(ws_o + base * D);
#pragma unroll
            for (int v = 0; v < VPL; ++v)
                src[k][v] = lane + 64 * v < NV4 ? o[lane + 64 * v] : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k = 0; k < GRP; ++k) {
            const float wgt = m[k] == kNegInfR ? 0.0f : exp2f(m[k] - M);
            L += wgt * l[k];
#pragma unroll
            for (int v = 0; v < VPL; ++v) acc[v] += wgt * src[k][v];
        }
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    f32x4 *dst = reinterpret_cast<f32x4 *>(out + (((int64_t)b * T + i) * Hq + h) * D);
    for (int v = 0; v < VPL; ++v)
        if (lane + 64 * v < NV4) dst[lane + 64 * v] = acc[v] * inv;
}

}  // namespace

hipError_t launch_attn_reduce(const AttnArgs &a, const AttnPlan &pl, hipStream_t stream) {
    const int64_t nrows = (int64_t)a.B * a.T * a.Hq;
    if (nrows == 0) return hipSuccess;
    const int per = 4;
    const int32_t *c_hdr = pl.balanced ? a.ws_c : nullptr;
    dim3 grid((unsigned)((nrows + per - 1) / per));
    if (a.D == 128)
        hipLaunchKernelGGL(attn_reduce_kernel<128>, grid, dim3(64 * per), 0, stream, a.ws_o,
                           a.ws_ml, a.prefix_len, a.max_prefix_len, a.B, a.Hq, a.Hkv, a.T,
                           pl.R, pl.S, pl.C, c_hdr, a.out);
    else if (a.D == 256)
        hipLaunchKernelGGL(attn_reduce_kernel<256>, grid, dim3(64 * per), 0, stream, a.ws_o,
                           a.ws_ml, a.prefix_len, a.max_prefix_len, a.B, a.Hq, a.Hkv, a.T,
                           pl.R, pl.S, pl.C, c_hdr, a.out);
    else
        hipLaunchKernelGGL(attn_reduce_kernel<512>, grid, dim3(64 * per), 0, stream, a.ws_o,
                           a.ws_ml, a.prefix_len, a.max_prefix_len, a.B, a.Hq, a.Hkv, a.T,
                           pl.R, pl.S, pl.C, c_hdr, a.out);
    return hipGetLastError();
}

}  // namespace sv
