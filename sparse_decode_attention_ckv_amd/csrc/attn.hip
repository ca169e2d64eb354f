// attn.hip -- sparse decode attention over selected rows on gfx950.
//
// Method: "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
// Recallable Compression", section 背景知识与设计原则 / 长上下文推理与KV缓存压缩
// (long-context inference and KV compression): the decode output is
// approximated by softmax(q K_S^T / sqrt(d)) V_S over the B selected rows.
//
// The step is HBM-bound: every selected K and V row (256 B each in bf16) is
// read once, and the G query heads of a KV head share that gather.
//   partial  grid (splits, KV heads): a workgroup takes R = 32 consecutive
//            entries of idx; 16 lanes per row, 16 bytes per lane; scores for
//            the G heads, max, exp, weighted V sum -> (m, l, acc[d]) per head
//   combine  one workgroup per query head merges the splits:
//            o = sum_s e^{m_s - M} acc_s / sum_s e^{m_s - M} l_s
// bf16 inputs compute in fp32; fp32 inputs compute in fp64.
#include "ckv_dev.h"

namespace ckv {

constexpr int kAttnRows = 32;   // rows of idx per workgroup (split)

template <typename T> struct Acc;
template <> struct Acc<uint16_t> { typedef float type; };
template <> struct Acc<float> { typedef double type; };

__device__ __forceinline__ float ex(float x) { return __expf(x); }
__device__ __forceinline__ double ex(double x) { return exp(x); }

template <typename T>
__device__ __forceinline__ void load8(const T *p, typename Acc<T>::type *f);

template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t *p, float *f) {
    unpack8(*(const u32x4 *)p, f);
}
template <>
__device__ __forceinline__ void load8<float>(const float *p, double *f) {
    const u32x4 a = *(const u32x4 *)p, b = *(const u32x4 *)(p + 4);
    f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y);
    f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
    f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y);
    f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
}

template <typename T, int G>
__global__ __launch_bounds__(256) void k_attn_partial(
    const T *__restrict__ q, const T *__restrict__ K, const T *__restrict__ V,
    int64_t kv_head_stride, int64_t kv_rows, const int32_t *__restrict__ idx,
    const int32_t *__restrict__ n_sel, int B, int S, double scale,
    typename Acc<T>::type *__restrict__ part) {
    typedef typename Acc<T>::type A;
    __shared__ A zs[G][kAttnRows];
    __shared__ A red[4][G][kD + 1];
    const int s = blockIdx.x, h = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = tid >> 4, q8 = tid & 15;
    int n = n_sel[h];
    n = n < 0 ? 0 : (n > B ? B : n);
    const int r0 = s * kAttnRows;

    // rows slot and slot + 16 of this split
    int64_t row[2];
    bool ok[2];
    A kf[2][8], vf[2][8];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int r = r0 + slot + 16 * k;
        const int64_t t = (r < n) ? (int64_t)idx[(int64_t)h * B + r] : -1;
        ok[k] = t >= 0 && t < kv_rows;
        row[k] = ok[k] ? t : 0;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (ok[k]) {
            const int64_t base = (int64_t)h * kv_head_stride + row[k] * kD + 8 * q8;
            load8<T>(K + base, kf[k]);
            load8<T>(V + base, vf[k]);
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) kf[k][e] = vf[k][e] = (A)0;
        }
    }
    A qf[G][8];
#pragma unroll
    for (int g = 0; g < G; ++g) load8<T>(q + ((int64_t)h * G + g) * kD + 8 * q8, qf[g]);

    A z[2][G];
#pragma unroll
    for (int k = 0; k < 2; ++k)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            A a = (A)0;
#pragma unroll
            for (int e = 0; e < 8; ++e) a += qf[g][e] * kf[k][e];
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) a += __shfl_xor(a, m);
            z[k][g] = ok[k] ? a * (A)scale : (A)(-INFINITY);
        }
    if (q8 == 0) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
#pragma unroll
            for (int g = 0; g < G; ++g) zs[g][slot + 16 * k] = z[k][g];
    }
    __syncthreads();
    A mx[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        A m = (A)(-INFINITY);
        for (int r = 0; r < kAttnRows; ++r) m = zs[g][r] > m ? zs[g][r] : m;
        mx[g] = m;
    }
    A acc[G][8], l[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = (A)0;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = (A)0;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const A p = ok[k] ? ex(z[k][g] - mx[g]) : (A)0;
            l[g] += p;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] += p * vf[k][e];
        }
    }
    // combine the 4 slots of the wave (lanes q8, q8+16, q8+32, q8+48)
#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] += __shfl_xor(l[g], 16);
        l[g] += __shfl_xor(l[g], 32);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            acc[g][e] += __shfl_xor(acc[g][e], 16);
            acc[g][e] += __shfl_xor(acc[g][e], 32);
        }
    }
    if (lane < 16) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red[wave][g][8 * lane + e] = acc[g][e];
            if (lane == 0) red[wave][g][kD] = l[g];
        }
    }
    __syncthreads();
    // write (m, l, acc) per query head: thread j < d handles channel j
    for (int w = tid; w < G * (kD + 1); w += 256) {
        const int g = w / (kD + 1), j = w % (kD + 1);
        const A v = ((red[0][g][j] + red[1][g][j]) + red[2][g][j]) + red[3][g][j];
        A *dst = part + (((int64_t)h * G + g) * S + s) * (kD + 2);
        if (j == kD) {
            dst[0] = mx[g];
            dst[1] = v;
        } else {
            dst[2 + j] = v;
        }
    }
}

template <typename A>
__global__ __launch_bounds__(128) void k_attn_combine(const A *__restrict__ part, int S,
                                                      float *__restrict__ o) {
    const int hq = blockIdx.x, j = threadIdx.x;
    const A *p = part + (int64_t)hq * S * (kD + 2);
    A M = (A)(-INFINITY);
    for (int s = 0; s < S; ++s) M = p[s * (kD + 2)] > M ? p[s * (kD + 2)] : M;
    float out = 0.f;
    if (M > (A)(-INFINITY)) {
        A Ls = (A)0, a = (A)0;
        for (int s = 0; s < S; ++s) {
            const A m = p[s * (kD + 2)];
            const A w = (m > (A)(-INFINITY)) ? ex(m - M) : (A)0;
            Ls += w * p[s * (kD + 2) + 1];
            a += w * p[s * (kD + 2) + 2 + j];
        }
        out = (float)(a / Ls);
    }
    o[(int64_t)hq * kD + j] = out;
}

template <typename T, int G>
static void launch_partial(const AttnPlan &p, const void *q, const void *K, const void *V,
                           const int32_t *idx, const int32_t *n_sel, hipStream_t s) {
    typedef typename Acc<T>::type A;
    hipLaunchKernelGGL((k_attn_partial<T, G>), dim3(p.S, p.H), dim3(256), 0, s,
                       (const T *)q, (const T *)K, (const T *)V, p.kv_head_stride, p.kv_rows,
                       idx, n_sel, p.B, p.S, p.scale, (A *)p.partials);
}

template <typename T>
static void launch_partial_g(const AttnPlan &p, const void *q, const void *K, const void *V,
                             const int32_t *idx, const int32_t *n_sel, hipStream_t s) {
    switch (p.G) {
        case 1: launch_partial<T, 1>(p, q, K, V, idx, n_sel, s); break;
        case 2: launch_partial<T, 2>(p, q, K, V, idx, n_sel, s); break;
        case 3: launch_partial<T, 3>(p, q, K, V, idx, n_sel, s); break;
        case 4: launch_partial<T, 4>(p, q, K, V, idx, n_sel, s); break;
        case 5: launch_partial<T, 5>(p, q, K, V, idx, n_sel, s); break;
        case 6: launch_partial<T, 6>(p, q, K, V, idx, n_sel, s); break;
        case 7: launch_partial<T, 7>(p, q, K, V, idx, n_sel, s); break;
        default: launch_partial<T, 8>(p, q, K, V, idx, n_sel, s); break;
    }
}

hipError_t launch_attn(const AttnPlan &p, const void *q, const void *K, const void *V,
                       const int32_t *idx, const int32_t *n_sel, float *o, hipStream_t s) {
    if (p.dtype == 1)
        launch_partial_g<uint16_t>(p, q, K, V, idx, n_sel, s);
    else
        launch_partial_g<float>(p, q, K, V, idx, n_sel, s);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (p.dtype == 1)
        hipLaunchKernelGGL(k_attn_combine<float>, dim3(p.H * p.G), dim3(128), 0, s,
                           (const float *)p.partials, p.S, o);
    else
        hipLaunchKernelGGL(k_attn_combine<double>, dim3(p.H * p.G), dim3(128), 0, s,
                           (const double *)p.partials, p.S, o);
    return hipGetLastError();
}

}  // namespace ckv
