// select.hip -- decode-time cluster-granular selection on gfx950.
//
// Method: "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
// Recallable Compression", section 核心方法细节 / 语义聚类粒度的选择
// (cluster-granular selection: score q.mu_i, sort descending, admit the
// clusters' tokens until the budget B is reached) and section 选择与索引机制
// (selection and indexing, Fig. 8: sort, gather and reorder the cluster
// sizes, prefix-sum them, find where the budget falls, trim the last
// cluster, emit the token indices).
//
// Two kernels per step:
//   score      s_c = q_g . mu_c in fp64, many workgroups per head (the
//              centroids are the bytes that matter: HBM-bound GEMV)
//   sort_cut   one workgroup per head: bitonic sort of (s desc, id asc) in
//              LDS, prefix sum of the sizes in rank order, cut at the budget,
//              and a parallel emission of idx (binary search per slot).
#include "ckv_dev.h"

namespace ckv {

// score: a half-wave (32 lanes) per cluster; lane r holds channels
// 4r..4r+3 (one 16-byte fp32 load), runs a 4-step fp64 fma chain from 0,
// and the 32 run sums are added pairwise (lane r + lane r+16, +8, ..., +1)
// with xor shuffles; lane 0 then holds the score. q_g is the fp64 sum of the
// G query rows in row order.
constexpr int kScoreClusters = 32;   // clusters per workgroup (4 passes of 8)

template <bool BF16>
__global__ __launch_bounds__(256) void k_score(const void *__restrict__ q, int G,
                                               const float *__restrict__ cent, int C,
                                               int c_cap, double *__restrict__ scores) {
    const int h = blockIdx.y;
    const int tid = threadIdx.x, half = tid >> 5, r = tid & 31;
    double qg[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        double a = 0.0;
        for (int g = 0; g < G; ++g) {
            const int64_t idx = ((int64_t)h * G + g) * kD + 4 * r + e;
            a += BF16 ? (double)bf16_to_f32(((const uint16_t *)q)[idx])
                      : (double)((const float *)q)[idx];
        }
        qg[e] = a;
    }
#pragma unroll
    for (int k = 0; k < kScoreClusters / 8; ++k) {
        const int c = blockIdx.x * kScoreClusters + 8 * k + half;
        double a = 0.0;
        if (c < C) {
            const u32x4 w = *(const u32x4 *)(cent + ((int64_t)h * c_cap + c) * kD + 4 * r);
            a = __fma_rn(qg[0], (double)__uint_as_float(w.x), a);
            a = __fma_rn(qg[1], (double)__uint_as_float(w.y), a);
            a = __fma_rn(qg[2], (double)__uint_as_float(w.z), a);
            a = __fma_rn(qg[3], (double)__uint_as_float(w.w), a);
        }
#pragma unroll
        for (int w = 16; w >= 1; w >>= 1) a = a + __shfl_xor(a, w, 32);
        if (c < C && r == 0) scores[(int64_t)h * C + c] = a;
    }
}

// "a comes before b" in rank order
__device__ __forceinline__ bool before(double sa, int ia, double sb, int ib) {
    return sa > sb || (sa == sb && ia < ib);
}

// sort_cut: P = power of two >= C, T = P/2 threads (at least 64).
__global__ __launch_bounds__(1024) void k_sort_cut(
    const double *__restrict__ scores, int C, int P, const int32_t *__restrict__ offsets,
    int c_cap, const int32_t *__restrict__ tokens, int64_t t_cap, int n_sink,
    int64_t pending_begin, int64_t n_pending, int B, int32_t *__restrict__ idx,
    int32_t *__restrict__ n_sel) {
    extern __shared__ double smem[];
    double *sc = smem;                           // [P]
    int32_t *id = (int32_t *)(sc + P);           // [P]
    int32_t *sz = id + P;                        // [P]  sizes in rank order
    int32_t *inc = sz + P;                       // [P]  inclusive prefix
    __shared__ int wsum[17];
    const int h = blockIdx.x, tid = threadIdx.x, T = blockDim.x;
    const int32_t *off = offsets + (int64_t)h * (c_cap + 1);
    const int32_t *tok = tokens + (int64_t)h * t_cap;

    for (int e = tid; e < P; e += T) {
        sc[e] = (e < C) ? scores[(int64_t)h * C + e] : -INFINITY;
        id[e] = e;
    }
    __syncthreads();
    for (int k = 2; k <= P; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int pr = tid; pr < (P >> 1); pr += T) {
                const int i = 2 * pr - (pr & (j - 1));
                const int l = i + j;
                const bool up = (i & k) == 0;
                const double si = sc[i], sl = sc[l];
                const int ii = id[i], il = id[l];
                const bool sw = up ? before(sl, il, si, ii) : before(si, ii, sl, il);
                if (sw) {
                    sc[i] = sl; sc[l] = si;
                    id[i] = il; id[l] = ii;
                }
            }
            __syncthreads();
        }
    }
    // sizes in rank order, clamped offsets
    for (int e = tid; e < P; e += T) {
        const int c = id[e];
        int n = 0;
        if (c < C) {
            int64_t b0 = off[c], b1 = off[c + 1];
            b0 = b0 < 0 ? 0 : (b0 > t_cap ? t_cap : b0);
            b1 = b1 < b0 ? b0 : (b1 > t_cap ? t_cap : b1);
            n = (int)(b1 - b0);
        }
        sz[e] = n;
    }
    __syncthreads();
    // inclusive prefix of sz: each thread owns P/T consecutive entries
    const int per = P / T;
    int loc = 0;
    for (int u = 0; u < per; ++u) loc += sz[tid * per + u];
    const int lane = tid & 63, wave = tid >> 6, nw = (T + 63) >> 6;
    int x = loc;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63 || tid == T - 1) wsum[wave] = x;
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int w = 0; w < nw; ++w) {
            const int t = wsum[w];
            wsum[w] = run;
            run += t;
        }
    }
    __syncthreads();
    int run = wsum[wave] + x - loc;
    for (int u = 0; u < per; ++u) {
        run += sz[tid * per + u];
        inc[tid * per + u] = run;
    }
    __syncthreads();

    const int64_t beff = (int64_t)B - n_sink - n_pending;
    const int64_t total = inc[P - 1];
    const int64_t ntake = beff < total ? beff : total;
    const int64_t head = (int64_t)n_sink + n_pending;
    int32_t *out = idx + (int64_t)h * B;
    for (int e = tid; e < B; e += T) {
        int32_t v;
        if (e < n_sink) {
            v = e;
        } else if (e < head) {
            v = (int32_t)(pending_begin + (e - n_sink));
        } else if (e - head < ntake) {
            const int p = (int)(e - head);
            int lo = 0, hi = P - 1;        // smallest rank with inc > p
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (inc[mid] > p) hi = mid; else lo = mid + 1;
            }
            const int c = id[lo];
            int64_t b0 = off[c];
            b0 = b0 < 0 ? 0 : (b0 > t_cap ? t_cap : b0);
            v = tok[b0 + (p - (inc[lo] - sz[lo]))];
        } else {
            v = -1;
        }
        out[e] = v;
    }
    if (tid == 0) n_sel[h] = (int32_t)(head + ntake);
}

hipError_t launch_select(const SelectPlan &p, const void *q, const float *cent,
                         const int32_t *offsets, const int32_t *tokens, int32_t *idx,
                         int32_t *n_sel, hipStream_t s) {
    dim3 g1((p.C + kScoreClusters - 1) / kScoreClusters, p.H);
    if (p.dtype == 1)
        hipLaunchKernelGGL(k_score<true>, g1, dim3(256), 0, s, q, p.G, cent, p.C, p.c_cap,
                           p.scores);
    else
        hipLaunchKernelGGL(k_score<false>, g1, dim3(256), 0, s, q, p.G, cent, p.C, p.c_cap,
                           p.scores);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int P = 128;
    while (P < p.C) P <<= 1;
    const int T = P / 2;
    const size_t lds = (size_t)P * (sizeof(double) + 3 * sizeof(int32_t));
    hipLaunchKernelGGL(k_sort_cut, dim3(p.H), dim3(T), lds, s, p.scores, p.C, P, offsets,
                       p.c_cap, tokens, p.t_cap, p.n_sink, p.pending_begin, p.n_pending, p.B,
                       idx, n_sel);
    return hipGetLastError();
}

}  // namespace ckv
