// ckv_dev.h -- internal declarations of libckv (device helpers + launchers).
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

// Exclusive scan over a block of up to 1024 threads (every thread calls it);
// returns this thread's exclusive prefix; *total receives the block sum.
// wsum: 17 ints of LDS.
__device__ inline int block_excl_scan(int v, int *wsum, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = (blockDim.x + 63) >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        int run = 0;
        for (int w = 0; w < nw; ++w) {
            const int t = wsum[w];
            wsum[w] = run;
            run += t;
        }
        wsum[16] = run;
    }
    __syncthreads();
    const int r = wsum[wave] + x - v;
    *total = wsum[16];
    __syncthreads();
    return r;
}

// ---- launchers (defined in the .hip files) ------------------------------
struct ClusterPlan {
    int H, C, Cpad, iters, n_sink, dtype, c_base, c_cap;
    int64_t L, Lp, k_head_stride, token_base, t_base, t_cap;
    int64_t ntiles;           // CSR tiles per head
    // workspace carve-up (device pointers)
    void *kt;                 // unit keys [H][Lp][d] (bf16 or f32)
    void *mt;                 // unit centroids [H][Cpad][d] (bf16 or f32)
    int32_t *tile_hist;       // [H][ntiles][C], then tile bases
    int32_t *tile_rank;       // [H][Lp]
    int32_t *counts;          // [H][C] cluster sizes
};

constexpr int kCsrTile = 512;          // tokens per CSR tile (one workgroup)

hipError_t launch_normalize_keys(const ClusterPlan &p, const void *K, int32_t *assign,
                                 hipStream_t s);
hipError_t launch_init_centroids(const ClusterPlan &p, const void *K, float *cent, hipStream_t s);
hipError_t launch_assign(const ClusterPlan &p, int32_t *assign, hipStream_t s);
hipError_t launch_csr(const ClusterPlan &p, const int32_t *assign, int32_t *offsets,
                      int32_t *tokens, hipStream_t s);
hipError_t launch_update(const ClusterPlan &p, const void *K, const int32_t *offsets,
                         const int32_t *tokens, float *cent, hipStream_t s);

struct SelectPlan {
    int H, G, C, c_cap, n_sink, B, dtype;
    int64_t t_cap, pending_begin, n_pending;
};
hipError_t launch_select(const SelectPlan &p, const void *q, const float *cent,
                         const int32_t *offsets, const int32_t *tokens, int32_t *idx,
                         int32_t *n_sel, hipStream_t s);

struct AttnPlan {
    int H, G, B, dtype, S;    // S splits of idx rows
    int64_t kv_head_stride, kv_rows;
    double scale;
    void *partials;           // [H*G][S][2 + d] (float for bf16, double for f32)
};
hipError_t launch_attn(const AttnPlan &p, const void *q, const void *K, const void *V,
                       const int32_t *idx, const int32_t *n_sel, float *o, hipStream_t s);

}  // namespace ckv
