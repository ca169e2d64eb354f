// attn_dev.h -- device core of the bf16 split-K decode attention, shared by
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
