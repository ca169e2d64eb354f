// decode.hip -- one decode step as selection + attention with one launch
// fewer than ckv_select followed by ckv_sparse_attn, on gfx950.
//
// Method: "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
// Recallable Compression": cluster-granular selection (section
// 核心方法细节 / 语义聚类粒度的选择, and 选择与索引机制 with Fig. 8) followed by
// the sparse decode attention softmax(q K_S^T / sqrt(d)) V_S (section
// 背景知识与设计原则 / 长上下文推理与KV缓存压缩).
//
// Launches: k_sel_score (as in ckv_select), then k_sel_attn_bf16 (fp32 rows:
// k_sel_attn_f32, the same selection with the fp64 attention core), whose
// workgroup (h, s) finds the cut of head h on its own, turns slots
// [64 s, 64 s + 64) of the head's idx row into token ids (and writes them),
// and right away runs the attention partial of that split on those rows;
// then the split combine of ckv_sparse_attn. The idx round trip through
// memory and one launch of the separate calls disappear. The selection and
// the attention are the same device code as the separate calls, so idx,
// n_sel and o are bitwise the same.
#include "attn_dev.h"
#include "sel_dev.h"

namespace ckv {

template <int CMAX, int G, bool VTILE>
__global__ __launch_bounds__(kCutThreads) void k_sel_attn_bf16(
    const double *__restrict__ scores, int C, const int32_t *__restrict__ offsets, int c_cap,
    const int32_t *__restrict__ tokens, int64_t t_cap, int n_sink, int64_t pending_begin,
    int64_t n_pending, int B, int32_t *__restrict__ idx, int32_t *__restrict__ n_sel,
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ K,
    const uint16_t *__restrict__ V, int64_t kv_head_stride, int64_t kv_rows, float fscale,
    float *__restrict__ part, int H, int NS) {
    static_assert(kSelSlice == kAttnRows, "one selection window per attention split");
    // the selection's LDS is dead once the slot is known: the V tile reuses it
    __shared__ union {
        SelLds<CMAX> sel;
        uint32_t sv[kAttnRows][kAttnRows];
    } U;
    SelLds<CMAX> &S = U.sel;
    __shared__ float zs[G][kAttnRows];
    int h, s;
    xcd_head_unit(blockIdx.x, NS, h, s);
    if (h >= H) return;
    const SelSlot r = sel_cut_emit<CMAX>(S, scores + (int64_t)h * C, C,
                                         offsets + (int64_t)h * (c_cap + 1),
                                         tokens + (int64_t)h * t_cap, t_cap, n_sink,
                                         pending_begin, n_pending, B, s);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = s * kSelSlice + lane;
    if (wave == 0 && e < B) idx[(int64_t)h * B + e] = r.val;
    if (s == 0 && tid == 0) n_sel[h] = r.n_sel;
    // every wave holds the token of split row `lane`; the score row of lane l
    // is split row 16 wave + (l & 15)
    const int n = r.n_sel < B ? r.n_sel : B;
    const bool okV = e < n && r.val >= 0 && (int64_t)r.val < kv_rows;
    const int rowV = okV ? r.val : 0;
    const int rk = 16 * wave + (lane & 15);
    const int tkK = __shfl(r.val, rk);
    const bool okK = s * kSelSlice + rk < n && tkK >= 0 && (int64_t)tkK < kv_rows;
    attn_rows_bf16<G, true, VTILE>(q, K, V, kv_head_stride, h, okK ? tkK : 0, okK, rowV, fscale,
                                   part, NS, s, zs, U.sv);
}

// fp32 rows: the same selection, then attn_rows_f32 on the window's rows
// (fp64 arithmetic); the selection's LDS is dead once the slot is known, so
// the attention's reduction buffer reuses it.
template <int CMAX, int G>
__global__ __launch_bounds__(kCutThreads) void k_sel_attn_f32(
    const double *__restrict__ scores, int C, const int32_t *__restrict__ offsets, int c_cap,
    const int32_t *__restrict__ tokens, int64_t t_cap, int n_sink, int64_t pending_begin,
    int64_t n_pending, int B, int32_t *__restrict__ idx, int32_t *__restrict__ n_sel,
    const float *__restrict__ q, const float *__restrict__ K, const float *__restrict__ V,
    int64_t kv_head_stride, int64_t kv_rows, double scale, double *__restrict__ part, int H,
    int NS) {
    static_assert(kSelSlice == kAttnRows, "one selection window per attention split");
    __shared__ union {
        SelLds<CMAX> sel;
        double red[4][G][kD + 1];
    } U;
    __shared__ double zs[G][kAttnRows];
    int h, s;
    xcd_head_unit(blockIdx.x, NS, h, s);
    if (h >= H) return;
    const SelSlot r = sel_cut_emit<CMAX>(U.sel, scores + (int64_t)h * C, C,
                                         offsets + (int64_t)h * (c_cap + 1),
                                         tokens + (int64_t)h * t_cap, t_cap, n_sink,
                                         pending_begin, n_pending, B, s);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int e = s * kSelSlice + lane;
    if (wave == 0 && e < B) idx[(int64_t)h * B + e] = r.val;
    if (s == 0 && tid == 0) n_sel[h] = r.n_sel;
    // every wave holds the token of split row `lane`; thread (slot, q8) takes
    // split rows slot + 16 k
    const int slot = tid >> 4;
    int tk[kRowsPerSlot];
#pragma unroll
    for (int k = 0; k < kRowsPerSlot; ++k) tk[k] = __shfl(r.val, slot + 16 * k);
    const int n = r.n_sel < 0 ? 0 : (r.n_sel < B ? r.n_sel : B);
    attn_rows_f32<G>(q, K, V, kv_head_stride, kv_rows, h, s, tk, n, scale, part, NS, zs, U.red);
}

template <int CMAX, int G>
static void launch_fused_f32_g(const SelectPlan &sp, const AttnPlan &ap, const void *q,
                               const int32_t *offsets, const int32_t *tokens, const void *K,
                               const void *V, int32_t *idx, int32_t *n_sel, hipStream_t s) {
    hipLaunchKernelGGL((k_sel_attn_f32<CMAX, G>), dim3(xcd_head_grid(sp.H, ap.S)),
                       dim3(kCutThreads), 0, s, sp.scores, sp.C, offsets, sp.c_cap, tokens,
                       sp.t_cap, sp.n_sink, sp.pending_begin, sp.n_pending, sp.B, idx, n_sel,
                       (const float *)q, (const float *)K, (const float *)V, ap.kv_head_stride,
                       ap.kv_rows, ap.scale, (double *)ap.partials, sp.H, ap.S);
}

template <int CMAX, int G>
static void launch_fused_g(const SelectPlan &sp, const AttnPlan &ap, const void *q,
                           const int32_t *offsets, const int32_t *tokens, const void *K,
                           const void *V, int32_t *idx, int32_t *n_sel, hipStream_t s) {
    // pinned host K/V: the V gather that keeps more requests in flight on the link
    hipLaunchKernelGGL((ap.host_kv ? &k_sel_attn_bf16<CMAX, G, false>
                                   : &k_sel_attn_bf16<CMAX, G, true>),
                       dim3(xcd_head_grid(sp.H, ap.S)),
                       dim3(kCutThreads), 0, s, sp.scores, sp.C, offsets, sp.c_cap, tokens,
                       sp.t_cap, sp.n_sink, sp.pending_begin, sp.n_pending, sp.B, idx, n_sel,
                       (const uint16_t *)q, (const uint16_t *)K, (const uint16_t *)V,
                       ap.kv_head_stride, ap.kv_rows, (float)ap.scale, (float *)ap.partials,
                       sp.H, ap.S);
}

template <int CMAX, bool F32, int G>
static void launch_fused(const SelectPlan &sp, const AttnPlan &ap, const void *q,
                         const int32_t *offsets, const int32_t *tokens, const void *K,
                         const void *V, int32_t *idx, int32_t *n_sel, hipStream_t s) {
    if constexpr (F32)
        launch_fused_f32_g<CMAX, G>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s);
    else
        launch_fused_g<CMAX, G>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s);
}

template <int CMAX, bool F32>
static void launch_fused_c(const SelectPlan &sp, const AttnPlan &ap, const void *q,
                           const int32_t *offsets, const int32_t *tokens, const void *K,
                           const void *V, int32_t *idx, int32_t *n_sel, hipStream_t s) {
    switch (sp.G) {
        case 1: launch_fused<CMAX, F32, 1>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s); break;
        case 2: launch_fused<CMAX, F32, 2>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s); break;
        case 3: launch_fused<CMAX, F32, 3>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s); break;
        case 4: launch_fused<CMAX, F32, 4>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s); break;
        case 5: launch_fused<CMAX, F32, 5>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s); break;
        case 6: launch_fused<CMAX, F32, 6>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s); break;
        case 7: launch_fused<CMAX, F32, 7>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s); break;
        default: launch_fused<CMAX, F32, 8>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s); break;
    }
}

hipError_t launch_select_attn(const SelectPlan &sp, const AttnPlan &ap, const void *q,
                              const float *cent, const int32_t *offsets, const int32_t *tokens,
                              const void *K, const void *V, int32_t *idx, int32_t *n_sel,
                              float *o, hipStream_t s) {
    hipError_t e = launch_sel_score(sp, q, cent, s);
    if (e != hipSuccess) return e;
    const bool f32 = sp.dtype != 1;             // fp32: fp64 attention arithmetic
    if (sp.C <= 512 && f32)
        launch_fused_c<512, true>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s);
    else if (sp.C <= 512)
        launch_fused_c<512, false>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s);
    else if (f32)
        launch_fused_c<kMaxC, true>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s);
    else
        launch_fused_c<kMaxC, false>(sp, ap, q, offsets, tokens, K, V, idx, n_sel, s);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_attn_combine(ap, o, s);
}

}  // namespace ckv
