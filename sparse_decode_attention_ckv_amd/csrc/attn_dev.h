// attn_dev.h -- device core of the split-K decode attention (bf16 and fp32), shared by
// the attention kernel (attn.hip) and the fused selection + attention kernel
// (decode.hip). Internal; include/ckv.h is the public ABI.
//
// Method: "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
// Recallable Compression", section 背景知识与设计原则 / 长上下文推理与KV缓存压缩
// (long-context inference and KV compression): the decode output is
// approximated by softmax(q K_S^T / sqrt(d)) V_S over the selected rows.
#pragma once

#include "ckv_dev.h"

namespace ckv {

constexpr int kAttnRows = kAttnSplitRows;   // rows of idx per workgroup (split)
constexpr int kAttnPW = kD + 2;             // partial record: m, l, acc[d]

constexpr int kRowsPerSlot = kAttnRows / 16;

template <typename T> struct Acc;
template <> struct Acc<uint16_t> { typedef float type; };
template <> struct Acc<float> { typedef double type; };

__device__ __forceinline__ float ex(float x) { return __expf(x); }
__device__ __forceinline__ double ex(double x) { return exp(x); }

// 8 consecutive elements held as 16-byte chunks (1 for bf16, 2 for fp32)
template <typename T>
__device__ __forceinline__ void unpack_chunks(const u32x4 *w, typename Acc<T>::type *f);
template <>
__device__ __forceinline__ void unpack_chunks<uint16_t>(const u32x4 *w, float *f) {
    unpack8(w[0], f);
}
template <>
__device__ __forceinline__ void unpack_chunks<float>(const u32x4 *w, double *f) {
    f[0] = __uint_as_float(w[0].x); f[1] = __uint_as_float(w[0].y);
    f[2] = __uint_as_float(w[0].z); f[3] = __uint_as_float(w[0].w);
    f[4] = __uint_as_float(w[1].x); f[5] = __uint_as_float(w[1].y);
    f[6] = __uint_as_float(w[1].z); f[7] = __uint_as_float(w[1].w);
}

// One split of 64 selected fp32 rows of KV head h for its G query heads, in
// fp64, 256 threads: thread (slot = tid >> 4, q8 = tid & 15) holds channels
// 8 q8 .. 8 q8 + 7 of split rows slot + 16 k (k < 4), whose tokens are tk[k];
// a row is valid if its split position 64 s + slot + 16 k is below n and its
// token lies in [0, kv_rows). Scores are 16-lane dot products, then the split
// max, exp and the weighted V sum, reduced over the slots in a fixed order
// (lane butterflies, then the four waves in order); the partial (m, l,
// acc[128]) of query head hG + g goes to part[((hG + g) S + s) * kAttnPW ...].
// Every K, V and q chunk of a thread is requested before the first is used.
// zs and red are LDS; red is first written after a barrier that every thread
// reaches after its own loads, so it may share LDS with data the caller read
// before the call.
template <int G>
__device__ __forceinline__ void attn_rows_f32(const float *__restrict__ q,
                                              const float *__restrict__ K,
                                              const float *__restrict__ V, int64_t kv_head_stride,
                                              int64_t kv_rows, int h, int s,
                                              const int (&tk)[kRowsPerSlot], int n, double scale,
                                              double *__restrict__ part, int S,
                                              double (&zs)[G][kAttnRows],
                                              double (&red)[4][G][kD + 1]) {
    constexpr int PW = kAttnPW;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int slot = tid >> 4, q8 = tid & 15;
    const int r0 = s * kAttnRows;
    int64_t row[kRowsPerSlot];
    bool ok[kRowsPerSlot];
#pragma unroll
    for (int k = 0; k < kRowsPerSlot; ++k) {
        const int r = r0 + slot + 16 * k;
        ok[k] = r < n && tk[k] >= 0 && (int64_t)tk[k] < kv_rows;
        row[k] = ok[k] ? tk[k] : 0;
    }
    // raw 16-byte chunks: K and V rows, then q; the scheduling barrier keeps
    // every one of these loads ahead of the first use
    constexpr int NV = 2;                         // 16-byte chunks per 8 fp32 elements
    u32x4 kr[kRowsPerSlot][NV], vr[kRowsPerSlot][NV], qr[G][NV];
#pragma unroll
    for (int k = 0; k < kRowsPerSlot; ++k) {
        const int64_t base = (int64_t)h * kv_head_stride + row[k] * kD + 8 * q8;
#pragma unroll
        for (int c = 0; c < NV; ++c) {
            kr[k][c] = *(const u32x4 *)(K + base + c * 4);
            vr[k][c] = *(const u32x4 *)(V + base + c * 4);
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int c = 0; c < NV; ++c)
            qr[g][c] = *(const u32x4 *)(q + ((int64_t)h * G + g) * kD + 8 * q8 + c * 4);
    __builtin_amdgcn_sched_barrier(0);
    double kf[kRowsPerSlot][8], vf[kRowsPerSlot][8], qf[G][8];
#pragma unroll
    for (int k = 0; k < kRowsPerSlot; ++k) {
        unpack_chunks<float>(kr[k], kf[k]);
        unpack_chunks<float>(vr[k], vf[k]);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kf[k][e] = ok[k] ? kf[k][e] : (double)0;
            vf[k][e] = ok[k] ? vf[k][e] : (double)0;
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) unpack_chunks<float>(qr[g], qf[g]);

    double z[kRowsPerSlot][G];
#pragma unroll
    for (int k = 0; k < kRowsPerSlot; ++k)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            double a = 0.0;
#pragma unroll
            for (int e = 0; e < 8; ++e) a += qf[g][e] * kf[k][e];
#pragma unroll
            for (int m = 8; m >= 1; m >>= 1) a += __shfl_xor(a, m);
            z[k][g] = ok[k] ? a * (double)scale : (double)(-INFINITY);
        }
    if (q8 == 0) {
#pragma unroll
        for (int k = 0; k < kRowsPerSlot; ++k)
#pragma unroll
            for (int g = 0; g < G; ++g) zs[g][slot + 16 * k] = z[k][g];
    }
    __syncthreads();
    double mx[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        double m = (double)(-INFINITY);
#pragma unroll 8
        for (int r = 0; r < kAttnRows; ++r) m = zs[g][r] > m ? zs[g][r] : m;
        mx[g] = m;
    }
    double acc[G][8], l[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = (double)0;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[g][e] = (double)0;
#pragma unroll
        for (int k = 0; k < kRowsPerSlot; ++k) {
            const double p = ok[k] ? ex(z[k][g] - mx[g]) : (double)0;
            l[g] += p;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] += p * vf[k][e];
        }
    }
    // the 4 slots of a wave (lanes q8, q8+16, q8+32, q8+48), then the 4 waves
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
    for (int w = tid; w < G * (kD + 1); w += 256) {
        const int g = w / (kD + 1), j = w % (kD + 1);
        const double v = ((red[0][g][j] + red[1][g][j]) + red[2][g][j]) + red[3][g][j];
        double *dst = part + (((int64_t)h * G + g) * S + s) * PW;
        if (j == kD) {
            dst[0] = mx[g];
            dst[1] = v;
        } else {
            dst[2 + j] = v;
        }
    }
}

// One split of 64 selected rows of KV head h for its G query heads, 256
// threads (4 waves). Partial (m, l, acc[128]) of query head hG + g goes to
// part[((hG + g) S + s) * kAttnPW ...].
//   rowK/okK: the row (and whether it is valid) of split row
//             16 * wave + (lane & 15), the row this lane scores;
//   rowV/okV: the row of split row `lane` (rowV is read from every lane).
// Scores: one MFMA tile per wave, v_mfma_f32_16x16x32_bf16 with the query
// heads on M (rows 0..G-1 of the A tile, the rest zero) and the wave's 16
// rows on N: lane l supplies, for k step t, channels 32t + 8(l>>4) .. +7 of
// head (l & 15) (A) and of its score row (B), and receives the scores of
// heads 4(l>>4) + i for that row. V: wave w loads split rows 16w .. 16w + 15
// only, 16 bytes per lane (lane l: row 16w + 4i + (l >> 4), channels
// 8(l & 15) .. + 7), into the LDS tile sv, so each row crosses from L2 once
// and no V words wait in registers. Softmax and V: wave w takes the heads
// g = w, w+4; lane l owns channels 2l, 2l+1 (word l of every sv row) and row l
// of the split, so the max and the sum of p are 64-lane wave reductions and
// the V sum runs over the rows in order with p_r taken from lane r
// (readlane): no cross-lane reduction of the accumulators. Every K fragment,
// q fragment and V chunk of a thread is requested before the first is used.
// SYNC: sv shares LDS with data the caller read before the call, so a barrier
// precedes the first write to it. VTILE false (K/V in host memory read over
// the host link): every wave instead requests all 64 V rows itself, 4 bytes
// per lane into 64 VGPRs, which keeps four times as many requests in flight on
// the link's long round trip; the V sum is the same arithmetic in the same
// order, so the result is the same.
template <int G, bool SYNC, bool VTILE = true>
__device__ __forceinline__ void attn_rows_bf16(const uint16_t *__restrict__ q,
                                               const uint16_t *__restrict__ K,
                                               const uint16_t *__restrict__ V,
                                               int64_t kv_head_stride, int h, int rowK, bool okK,
                                               int rowV, float fscale, float *__restrict__ part,
                                               int S, int s, float (&zs)[G][kAttnRows],
                                               uint32_t (&sv)[kAttnRows][kAttnRows]) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int col = lane & 15, kq = lane >> 4;    // MFMA fragment coordinates
    const uint16_t *Kh = K + (int64_t)h * kv_head_stride;
    const uint16_t *Vh = V + (int64_t)h * kv_head_stride;
    const uint16_t *qrow = q + ((int64_t)h * G + (col < G ? col : 0)) * kD;
    int vrow[4];
    if constexpr (VTILE) {
#pragma unroll
        for (int i = 0; i < 4; ++i) vrow[i] = __shfl(rowV, 16 * wave + 4 * i + kq);
    }
    u32x4 kb[4], qa[4], vb[4];
    uint32_t vv[VTILE ? 1 : kAttnRows];
#pragma unroll
    for (int t = 0; t < 4; ++t) kb[t] = *(const u32x4 *)(Kh + (int64_t)rowK * kD + 32 * t + 8 * kq);
#pragma unroll
    for (int t = 0; t < 4; ++t) qa[t] = *(const u32x4 *)(qrow + 32 * t + 8 * kq);
    if constexpr (VTILE) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            vb[i] = *(const u32x4 *)(Vh + (int64_t)vrow[i] * kD + 8 * col);
    } else {
#pragma unroll
        for (int r = 0; r < kAttnRows; ++r) {
            const int row = __builtin_amdgcn_readlane(rowV, r);
            vv[r] = *(const uint32_t *)(Vh + (int64_t)row * kD + 2 * lane);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if (SYNC) __syncthreads();

    f32x4 acc4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const u32x4 a = col < G ? qa[t] : (u32x4){0u, 0u, 0u, 0u};
        acc4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, kb[t]), acc4,
                                                       0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int g = 4 * kq + i;
        if (g < G) zs[g][16 * wave + col] = okK ? acc4[i] * fscale : -INFINITY;
    }
    if constexpr (VTILE) {
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4 *)&sv[16 * wave + 4 * i + kq][4 * col] = vb[i];
    }
    __syncthreads();

    for (int g = wave; g < G; g += 4) {
        const float z = zs[g][lane];
        float m = z;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float y = __shfl_xor(m, o);
            m = y > m ? y : m;
        }
        const float p = (z > -INFINITY) ? __expf(z - m) : 0.f;
        float l = p;
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
        float a0 = 0.f, a1 = 0.f;
#pragma unroll
        for (int r = 0; r < kAttnRows; ++r) {
            const float pr = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(p), r));
            const uint32_t vw = VTILE ? sv[r][lane] : vv[VTILE ? 0 : r];
            a0 += pr * bf16_lo(vw);
            a1 += pr * bf16_hi(vw);
        }
        float *dst = part + (((int64_t)h * G + g) * S + s) * kAttnPW;
        if (lane == 0) {
            dst[0] = m;
            dst[1] = l;
        }
        *(float2 *)(dst + 2 + 2 * lane) = make_float2(a0, a1);
    }
}

}  // namespace ckv
