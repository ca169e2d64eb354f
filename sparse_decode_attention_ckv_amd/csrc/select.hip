// select.hip -- decode-time cluster-granular selection on gfx950.
//
// Method: "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
// Recallable Compression", section 核心方法细节 / 语义聚类粒度的选择
// (score q.mu_i, admit clusters in descending score until the budget) and
// section 选择与索引机制 (Fig. 8: sizes, prefix sums, the cut, the trim of the
// last cluster, token indices). The device logic of both steps lives in
// sel_dev.h; this file holds the two kernels of ckv_select:
//  * k_sel_score: fp64 scores of 32 clusters per workgroup, 8 lanes per
//    cluster, grid placed so that every workgroup of a head shares an XCD;
//  * k_sel_cut: one 256-thread workgroup per 64 slots of a head's idx row;
//    each finds the cut from the scores on its own and writes its slots.
#include "sel_dev.h"

namespace ckv {

// s_c = q_g . mu_c for clusters [32 j, 32 j + 32) of KV head h into
// scores[h][c]. Lane lam (< 8) of a cluster holds the fma runs r = lam + 8i,
// i < 4 (channels 4r .. 4r + 3); the tree levels +16 and +8 stay inside the
// lane, +4, +2 and +1 cross lanes (commutative adds: every lane ends with
// the same value).
template <bool BF16>
__global__ __launch_bounds__(kScoreThreads) void k_sel_score(
    const void *__restrict__ q, int G, const float *__restrict__ cent, int C, int c_cap, int H,
    int S, double *__restrict__ scores) {
    __shared__ double qg[kD];
    int h, j;
    xcd_head_unit(blockIdx.x, S, h, j);
    if (h >= H) return;
    const int tid = threadIdx.x, lam = tid & (kScoreLanes - 1), slot = tid / kScoreLanes;
    const int c = j * kScoreChunk + slot;
    const float *row = cent + ((int64_t)h * c_cap + (c < C ? c : C - 1)) * kD;
    u32x4 w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = *(const u32x4 *)(row + 4 * (lam + 8 * i));
    float qv[8];
    if (tid < kD) {
        sel_q_load<BF16>(q, G, h, tid, qv);
        qg[tid] = sel_q_sum(qv, G);
    }
    __syncthreads();
    double run[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const double *qr = qg + 4 * (lam + 8 * i);
        double a = 0.0;
        a = __fma_rn(qr[0], (double)__uint_as_float(w[i].x), a);
        a = __fma_rn(qr[1], (double)__uint_as_float(w[i].y), a);
        a = __fma_rn(qr[2], (double)__uint_as_float(w[i].z), a);
        a = __fma_rn(qr[3], (double)__uint_as_float(w[i].w), a);
        run[i] = a;
    }
    // runs lam, lam + 8, lam + 16, lam + 24: level +16 pairs (0, 2) and (1, 3),
    // level +8 joins them
    double v = (run[0] + run[2]) + (run[1] + run[3]);
    v = v + __shfl_xor(v, 4);
    v = v + __shfl_xor(v, 2);
    v = v + __shfl_xor(v, 1);
    if (lam == 0 && c < C) scores[(int64_t)h * C + c] = v;
}

template <int CMAX>
__global__ __launch_bounds__(kCutThreads) void k_sel_cut(
    const double *__restrict__ scores, int C, const int32_t *__restrict__ offsets, int c_cap,
    const int32_t *__restrict__ tokens, int64_t t_cap, int n_sink, int64_t pending_begin,
    int64_t n_pending, int B, int32_t *__restrict__ idx, int32_t *__restrict__ n_sel, int H,
    int NS) {
    __shared__ SelLds<CMAX> S;
    int h, s;
    xcd_head_unit(blockIdx.x, NS, h, s);
    if (h >= H) return;
    const SelSlot r = sel_cut_emit<CMAX>(S, scores + (int64_t)h * C, C,
                                         offsets + (int64_t)h * (c_cap + 1),
                                         tokens + (int64_t)h * t_cap, t_cap, n_sink,
                                         pending_begin, n_pending, B, s);
    const int tid = threadIdx.x;
    const int e = s * kSelSlice + tid;
    if (tid < kSelSlice && e < B) idx[(int64_t)h * B + e] = r.val;
    if (s == 0 && tid == 0) n_sel[h] = r.n_sel;
}

hipError_t launch_sel_score(const SelectPlan &p, const void *q, const float *cent,
                            hipStream_t s) {
    const int S = (p.C + kScoreChunk - 1) / kScoreChunk;
    if (p.dtype == 1)
        hipLaunchKernelGGL(k_sel_score<true>, dim3(xcd_head_grid(p.H, S)), dim3(kScoreThreads),
                           0, s, q, p.G, cent, p.C, p.c_cap, p.H, S, p.scores);
    else
        hipLaunchKernelGGL(k_sel_score<false>, dim3(xcd_head_grid(p.H, S)), dim3(kScoreThreads),
                           0, s, q, p.G, cent, p.C, p.c_cap, p.H, S, p.scores);
    return hipGetLastError();
}

hipError_t launch_select(const SelectPlan &p, const void *q, const float *cent,
                         const int32_t *offsets, const int32_t *tokens, int32_t *idx,
                         int32_t *n_sel, hipStream_t s) {
    hipError_t e = launch_sel_score(p, q, cent, s);
    if (e != hipSuccess) return e;
    const int NS = (p.B + kSelSlice - 1) / kSelSlice;
    const dim3 grid(xcd_head_grid(p.H, NS));
    if (p.C <= 512)
        hipLaunchKernelGGL(k_sel_cut<512>, grid, dim3(kCutThreads), 0, s, p.scores, p.C, offsets,
                           p.c_cap, tokens, p.t_cap, p.n_sink, p.pending_begin, p.n_pending,
                           p.B, idx, n_sel, p.H, NS);
    else
        hipLaunchKernelGGL(k_sel_cut<kMaxC>, grid, dim3(kCutThreads), 0, s, p.scores, p.C,
                           offsets, p.c_cap, tokens, p.t_cap, p.n_sink, p.pending_begin,
                           p.n_pending, p.B, idx, n_sel, p.H, NS);
    return hipGetLastError();
}

}  // namespace ckv
