// attn.hip -- sparse decode attention over selected rows on gfx950.
//
// Method: "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
// Recallable Compression", section 背景知识与设计原则 / 长上下文推理与KV缓存压缩
// (long-context inference and KV compression): the decode output is
// approximated by softmax(q K_S^T / sqrt(d)) V_S over the B selected rows.
//
// Two kernels per decode step, HBM-bound: every selected K and V row (256 B
// each in bf16) is read once, and the G query heads of a KV head share that
// gather.
//  * partial, grid (splits, KV heads): a workgroup takes R = 64 consecutive
//    entries of idx, the idx and then all K/V/q loads of a thread in flight
//    at once; scores for the G heads (bf16: one MFMA tile per wave; fp32:
//    16 lanes per row), split max, exp, weighted V sum (bf16: each wave
//    stages 16 V rows in an LDS tile and one wave per query head sums all 64
//    rows in order; fp32: 16 lanes per row) -> (m, l, acc[d]) per query head;
//  * combine, one workgroup per query head: o = sum_s e^{m_s - M} acc_s /
//    sum_s e^{m_s - M} l_s, summed in split order.
// A kernel boundary hands the partials over: on this multi-XCD part a
// per-workgroup device-scope release fence costs more than a launch.
// bf16 inputs compute in fp32; fp32 inputs compute in fp64.
#include "attn_dev.h"

namespace ckv {

// partial, fp32: the rows of split s come from idx (thread (slot, q8) takes
// split rows slot + 16 k); everything else is attn_rows_f32. idx is read
// without waiting for n_sel.
template <int G>
__global__ __launch_bounds__(256) void k_attn_partial_f32(
    const float *__restrict__ q, const float *__restrict__ K, const float *__restrict__ V,
    int64_t kv_head_stride, int64_t kv_rows, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ n_sel, int B, double scale, double *__restrict__ part, int H,
    int S) {
    __shared__ double zs[G][kAttnRows];
    __shared__ double red[4][G][kD + 1];
    int h, s;
    xcd_head_unit(blockIdx.x, S, h, s);
    if (h >= H) return;
    const int slot = threadIdx.x >> 4;
    int tk[kRowsPerSlot];
#pragma unroll
    for (int k = 0; k < kRowsPerSlot; ++k) {
        const int r = s * kAttnRows + slot + 16 * k;
        tk[k] = idx[(int64_t)h * B + (r < B ? r : B - 1)];
    }
    int n = n_sel[h];
    n = n < 0 ? 0 : (n > B ? B : n);
    attn_rows_f32<G>(q, K, V, kv_head_stride, kv_rows, h, s, tk, n, scale, part, S, zs, red);
}

// partial, bf16: the rows of split s come from idx (the V row of lane l is
// split row l, the score row of lane l of wave w is split row 16w + (l & 15));
// everything else is attn_rows_bf16.
template <int G, bool VTILE>
__global__ __launch_bounds__(256) void k_attn_partial_bf16(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t kv_head_stride, int64_t kv_rows,
    const int32_t *__restrict__ idx, const int32_t *__restrict__ n_sel, int B, double scale,
    float *__restrict__ part, int H, int S) {
    __shared__ float zs[G][kAttnRows];
    __shared__ uint32_t sv[kAttnRows][kAttnRows];
    int h, s;
    xcd_head_unit(blockIdx.x, S, h, s);
    if (h >= H) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15;
    const int r0 = s * kAttnRows;
    const int32_t *ih = idx + (int64_t)h * B;
    // clamped reads, not waiting for n_sel
    const int rV = r0 + lane, rK = r0 + 16 * wave + col;
    const int tkV = ih[rV < B ? rV : B - 1];
    const int tkK = ih[rK < B ? rK : B - 1];
    int n = n_sel[h];
    n = n < 0 ? 0 : (n > B ? B : n);
    const bool okK = rK < n && tkK >= 0 && (int64_t)tkK < kv_rows;
    const bool okV = rV < n && tkV >= 0 && (int64_t)tkV < kv_rows;
    attn_rows_bf16<G, false, VTILE>(q, K, V, kv_head_stride, h, okK ? tkK : 0, okK,
                                    okV ? tkV : 0, (float)scale, part, S, s, zs, sv);
}

// combine: one workgroup per query head, thread j owns channel j; the
// split records are read in batches with every load of a batch in flight.
template <typename A>
__global__ __launch_bounds__(128) void k_attn_combine(const A *__restrict__ part, int S,
                                                      float *__restrict__ o, int H, int G) {
    constexpr int PW = kD + 2;
    constexpr int NB = 16;
    int h, g;
    xcd_head_unit(blockIdx.x, G, h, g);
    if (h >= H) return;
    const int hq = h * G + g, j = threadIdx.x;
    const A *p = part + (int64_t)hq * S * PW;
    // one pass: records in batches of NB, every load of a batch in flight
    // (addresses clamped, values masked); the running max rescales the sums
    // batch by batch, so the result equals the two-pass merge up to rounding
    A M = (A)(-INFINITY), Ls = (A)0, a = (A)0;
    for (int s0 = 0; s0 < S; s0 += NB) {
        A m[NB], l[NB], v[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            const int sp = s0 + k < S ? s0 + k : S - 1;
            const A *rec = p + (int64_t)sp * PW;
            m[k] = rec[0];
            l[k] = rec[1];
            v[k] = rec[2 + j];
        }
        A bm = M;
#pragma unroll
        for (int k = 0; k < NB; ++k)
            if (s0 + k < S) bm = m[k] > bm ? m[k] : bm;
        if (bm > (A)(-INFINITY)) {
            const A sc = (M > (A)(-INFINITY)) ? ex(M - bm) : (A)0;
            Ls *= sc;
            a *= sc;
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const A w = (s0 + k < S && m[k] > (A)(-INFINITY)) ? ex(m[k] - bm) : (A)0;
                Ls += w * l[k];
                a += w * v[k];
            }
            M = bm;
        }
    }
    const float out = (Ls > (A)0) ? (float)(a / Ls) : 0.f;
    o[(int64_t)hq * kD + j] = out;
}

template <typename T, int G>
static void launch_g(const AttnPlan &p, const void *q, const void *K, const void *V,
                     const int32_t *idx, const int32_t *n_sel, float *o, hipStream_t s) {
    typedef typename Acc<T>::type A;
    if (sizeof(T) == 2)
        hipLaunchKernelGGL((p.host_kv ? &k_attn_partial_bf16<G, false>
                                      : &k_attn_partial_bf16<G, true>),
                           dim3(xcd_head_grid(p.H, p.S)), dim3(256), 0, s, (const uint16_t *)q,
                           (const uint16_t *)K, (const uint16_t *)V, p.kv_head_stride, p.kv_rows,
                           idx, n_sel, p.B, p.scale, (float *)p.partials, p.H, p.S);
    else
        hipLaunchKernelGGL((k_attn_partial_f32<G>), dim3(xcd_head_grid(p.H, p.S)), dim3(256), 0,
                           s, (const float *)q, (const float *)K, (const float *)V,
                           p.kv_head_stride, p.kv_rows, idx, n_sel, p.B, p.scale,
                           (double *)p.partials, p.H, p.S);
}

template <typename T>
static void launch_t(const AttnPlan &p, const void *q, const void *K, const void *V,
                     const int32_t *idx, const int32_t *n_sel, float *o, hipStream_t s) {
    switch (p.G) {
        case 1: launch_g<T, 1>(p, q, K, V, idx, n_sel, o, s); break;
        case 2: launch_g<T, 2>(p, q, K, V, idx, n_sel, o, s); break;
        case 3: launch_g<T, 3>(p, q, K, V, idx, n_sel, o, s); break;
        case 4: launch_g<T, 4>(p, q, K, V, idx, n_sel, o, s); break;
        case 5: launch_g<T, 5>(p, q, K, V, idx, n_sel, o, s); break;
        case 6: launch_g<T, 6>(p, q, K, V, idx, n_sel, o, s); break;
        case 7: launch_g<T, 7>(p, q, K, V, idx, n_sel, o, s); break;
        default: launch_g<T, 8>(p, q, K, V, idx, n_sel, o, s); break;
    }
}

hipError_t launch_attn_combine(const AttnPlan &p, float *o, hipStream_t s) {
    if (p.dtype == 1)
        hipLaunchKernelGGL(k_attn_combine<float>, dim3(xcd_head_grid(p.H, p.G)), dim3(128), 0,
                           s, (const float *)p.partials, p.S, o, p.H, p.G);
    else
        hipLaunchKernelGGL(k_attn_combine<double>, dim3(xcd_head_grid(p.H, p.G)), dim3(128), 0,
                           s, (const double *)p.partials, p.S, o, p.H, p.G);
    return hipGetLastError();
}

hipError_t launch_attn(const AttnPlan &p, const void *q, const void *K, const void *V,
                       const int32_t *idx, const int32_t *n_sel, float *o, hipStream_t s) {
    if (p.dtype == 1)
        launch_t<uint16_t>(p, q, K, V, idx, n_sel, o, s);
    else
        launch_t<float>(p, q, K, V, idx, n_sel, o, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_attn_combine(p, o, s);
}

}  // namespace ckv
