// ckv_dev.h -- internal declarations of libckv: device helpers shared by the
// kernels, and the plans and launchers of the decode kernels (cluster_dev.h
// and cache_dev.h hold the others).
// Not part of the public ABI; include/ckv.h is.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ckv {

constexpr int kD = 128;               // supported head dimension
constexpr int kMaxC = 2048;           // max clusters per call (LDS-sized kernels)
constexpr int kAttnSplitRows = 64;    // idx entries per attention workgroup
constexpr int kMaxSplits = 512;       // attention splits per head -> B <= 32768

// ---- element types ------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// fp32 -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Unpack 8 bf16 held in a u32x4 into floats (element j of the chunk).
__device__ __forceinline__ void unpack8(const u32x4 &w, float *f) {
    f[0] = bf16_lo(w.x); f[1] = bf16_hi(w.x);
    f[2] = bf16_lo(w.y); f[3] = bf16_hi(w.y);
    f[4] = bf16_lo(w.z); f[5] = bf16_hi(w.z);
    f[6] = bf16_lo(w.w); f[7] = bf16_hi(w.w);
}

// XCD-aware remap of a 1-D block id. The dispatcher hands consecutive block
// ids to the 8 XCDs round-robin; this returns a linear tile index such that
// each XCD works on a contiguous range of tiles (so a head's tiles share one
// L2). Identity when n is not a multiple of 8.
__device__ __forceinline__ uint32_t xcd_linear(uint32_t bid, uint32_t n) {
    if (n & 7u) return bid;
    return (bid & 7u) * (n >> 3) + (bid >> 3);
}

// Grids of per-head units placed by XCD: unit j (< n) of head h runs as block
// b = (h / 8) * 8n + 8j + h % 8, so with blocks handed to the 8 XCDs round-
// robin every unit of head h shares an XCD (and its L2) with block h of a
// one-block-per-head grid (the selection that wrote the head's indices).
// The grid has 8 ceil(H / 8) n blocks; blocks whose head is >= H have no
// work and must return before any barrier.
__host__ __device__ inline uint32_t xcd_head_grid(int H, int n) {
    return (uint32_t)((H + 7) / 8) * 8u * (uint32_t)n;
}
__device__ __forceinline__ void xcd_head_unit(uint32_t b, int n, int &h, int &j) {
    const uint32_t rest = b >> 3;
    j = (int)(rest % (uint32_t)n);
    h = (int)(rest / (uint32_t)n) * 8 + (int)(b & 7u);
}

// ---- wave- and block-wide scans (DPP, no LDS round trips inside a wave) --
// DPP controls of the gfx9 family: row_shr:n shifts within a row of 16 lanes;
// row_bcast:15 copies lane 15 of each row into the next row, row_bcast:31
// copies lane 31 into rows 2 and 3.
constexpr int kDppRowShr = 0x110, kDppBcast15 = 0x142, kDppBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active).
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 1, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 2, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 4, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr + 8, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppBcast15, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppBcast31, 0xc, 0xf, false);
    return x;
}

// Inclusive prefix maximum over the 64 lanes of a wave (all lanes active).
__device__ __forceinline__ int wave_incl_max(int x) {
    constexpr int lo = -2147483647 - 1;
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, kDppRowShr + 1, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, kDppRowShr + 2, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, kDppRowShr + 4, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, kDppRowShr + 8, 0xf, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, kDppBcast15, 0xa, 0xf, false));
    x = max(x, __builtin_amdgcn_update_dpp(lo, x, kDppBcast31, 0xc, 0xf, false));
    return x;
}

// Sum over the wave, the same value in every lane.
__device__ __forceinline__ int wave_sum(int x) {
    return __builtin_amdgcn_readlane(wave_incl_scan(x), 63);
}

// One DPP step on a double: lanes whose source is outside the row mask or
// the row read `id` instead.
template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_f64(double x, double id) {
    const uint64_t u = (uint64_t)__double_as_longlong(x), v = (uint64_t)__double_as_longlong(id);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)v, (int)(uint32_t)u,
                                                               CTRL, ROWS, 0xf, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp((int)(uint32_t)(v >> 32),
                                                               (int)(uint32_t)(u >> 32), CTRL,
                                                               ROWS, 0xf, false);
    return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Largest and smallest value over the wave (uniform results). Finite or
// infinite inputs; a NaN lane is ignored unless every lane is NaN.
__device__ __forceinline__ void wave_minmax_f64(double &mn, double &mx) {
    const double pinf = __longlong_as_double(0x7ff0000000000000ll), ninf = -pinf;
#define CKV_MM_STEP(CTRL, ROWS)                               \
    mn = fmin(mn, dpp_f64<CTRL, ROWS>(mn, pinf));            \
    mx = fmax(mx, dpp_f64<CTRL, ROWS>(mx, ninf));
    CKV_MM_STEP(kDppRowShr + 1, 0xf)
    CKV_MM_STEP(kDppRowShr + 2, 0xf)
    CKV_MM_STEP(kDppRowShr + 4, 0xf)
    CKV_MM_STEP(kDppRowShr + 8, 0xf)
    CKV_MM_STEP(kDppBcast15, 0xa)
    CKV_MM_STEP(kDppBcast31, 0xc)
#undef CKV_MM_STEP
    const uint64_t a = (uint64_t)__double_as_longlong(mn), b = (uint64_t)__double_as_longlong(mx);
    const uint32_t alo = __builtin_amdgcn_readlane((int)(uint32_t)a, 63);
    const uint32_t ahi = __builtin_amdgcn_readlane((int)(uint32_t)(a >> 32), 63);
    const uint32_t blo = __builtin_amdgcn_readlane((int)(uint32_t)b, 63);
    const uint32_t bhi = __builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), 63);
    mn = __longlong_as_double((long long)(((uint64_t)ahi << 32) | alo));
    mx = __longlong_as_double((long long)(((uint64_t)bhi << 32) | blo));
}

// Exclusive scan over a block of NW full waves with one barrier: wave scans,
// wave totals through LDS (wsum, NW ints), every thread adds the totals of
// the waves before its own. The caller places a barrier before wsum is
// written again.
template <int NW>
__device__ __forceinline__ int block_excl_scan_nw(int v, int *wsum, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int t = wsum[w];
        before += w < wave ? t : 0;
        tot += t;
    }
    total = tot;
    return before + x - v;
}

// Exclusive scan over a block of up to 1024 threads, a multiple of 64
// (every thread calls it); returns this thread's exclusive prefix; *total
// receives the block sum. wsum: 17 ints of LDS. Ends with a barrier, so wsum
// may be reused at once.
__device__ inline int block_excl_scan(int v, int *wsum, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = blockDim.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int before = 0, tot = 0;
    for (int w = 0; w < nw; ++w) {
        const int t = wsum[w];
        before += w < wave ? t : 0;
        tot += t;
    }
    *total = tot;
    __syncthreads();
    return before + x - v;
}

// Compute units of the current device (queried once per device, cached).
int device_cu_count();

// ---- launchers (defined in the .hip files) ------------------------------
// Largest idx row (budget B) a selection call accepts: the cut kernel runs
// one workgroup per 64 slots of every head.
constexpr int kMaxSelB = 1 << 20;
struct SelectPlan {
    int H, G, C, c_cap, n_sink, B, dtype;
    int64_t t_cap, pending_begin, n_pending;
    double *scores;           // workspace [H][C] fp64
};
hipError_t launch_sel_score(const SelectPlan &p, const void *q, const float *cent,
                            hipStream_t s);
hipError_t launch_select(const SelectPlan &p, const void *q, const float *cent,
                         const int32_t *offsets, const int32_t *tokens, int32_t *idx,
                         int32_t *n_sel, hipStream_t s);

struct AttnPlan {
    int H, G, B, dtype, S;    // S splits of idx rows
    int64_t kv_head_stride, kv_rows;
    double scale;
    void *partials;           // [H*G][S][2 + d] (float for bf16, double for f32)
    bool host_kv;             // K and V in pinned host memory (bf16: V gathered for the link)
};
hipError_t launch_attn(const AttnPlan &p, const void *q, const void *K, const void *V,
                       const int32_t *idx, const int32_t *n_sel, float *o, hipStream_t s);
hipError_t launch_attn_combine(const AttnPlan &p, float *o, hipStream_t s);

// One decode step, selection then attention (decode.hip); sp and ap describe
// the same heads, query heads per KV head, budget and element type.
hipError_t launch_select_attn(const SelectPlan &sp, const AttnPlan &ap, const void *q,
                              const float *cent, const int32_t *offsets, const int32_t *tokens,
                              const void *K, const void *V, int32_t *idx, int32_t *n_sel,
                              float *o, hipStream_t s);

}  // namespace ckv
