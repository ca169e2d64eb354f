// cluster_dev.h -- plan and launchers of the clustering kernels (cluster.hip).
#pragma once
#include "ckv_dev.h"

namespace ckv {

// assignment distances (the values of ckv_metric)
constexpr int kCosine = 0, kInnerProduct = 1, kL2 = 2;

struct ClusterPlan {
    int H, C, Cpad, iters, n_sink, dtype, c_base, c_cap;
    int metric;               // kCosine, kInnerProduct or kL2
    int64_t L, Lp, k_head_stride, token_base, t_base, t_cap;
    int64_t ntiles;           // CSR tiles per head
    bool csr_wide;            // C <= kCsrWideMaxC: the two-launch CSR (else count, scan, scatter)
    int n_cu;                 // compute units of the device (persistent grids)
    // the rows the assignment reads: the first clustered row of head 0 (the
    // keys where they are, or their copy kt), heads ka_stride elements apart
    const void *ka;
    int64_t ka_stride;
    // the rows the update reads: token t of head h is row t - ku_base of
    // ku + h * ku_stride, rows [0, ku_rows) (the keys where they are, or kt)
    const void *ku;
    int64_t ku_stride, ku_rows, ku_base;
    // workspace carve-up (device pointers)
    void *kt;                 // copy of keys in pinned host memory [H][Lp][d]
    void *mt;                 // centroids as the assignment reads them [H][Cpad][d]
                              // (bf16 or f32; unit rows for the cosine)
    float *mb;                // per-cluster score bias [H][Cpad] (L2: -|mu|^2 / 2)
    int32_t *tile_hist;       // [H][ntiles][C], then tile bases
    int32_t *tile_rank;       // [H][Lp]
    int32_t *counts;          // [H][C] cluster sizes
};

constexpr int kCsrWideTile = 2048;     // tokens per CSR tile (one workgroup)
constexpr int kCsrWideMaxC = 512;      // clusters of the two-launch CSR (one per scatter thread)

hipError_t launch_copy_keys(const ClusterPlan &p, const void *K, hipStream_t s);
hipError_t launch_init_centroids(const ClusterPlan &p, const void *K, float *cent,
                                 int32_t *assign, hipStream_t s);
hipError_t launch_assign(const ClusterPlan &p, int32_t *assign, hipStream_t s);
hipError_t launch_csr(const ClusterPlan &p, const int32_t *assign, int32_t *offsets,
                      int32_t *tokens, hipStream_t s);
hipError_t launch_update(const ClusterPlan &p, const int32_t *offsets, const int32_t *tokens,
                         float *cent, hipStream_t s);

// Whole K-means of a small bf16 window in one launch (one workgroup per
// head), bitwise the general path's result.
constexpr int kSmallThreads = 1024;
constexpr int kSmallRows = kSmallThreads;   // window rows (one per thread)
constexpr int kSmallC = 16;                 // clusters (one MFMA M tile)
hipError_t launch_cluster_small(const ClusterPlan &p, const void *K, float *cent,
                                int32_t *assign, int32_t *offsets, int32_t *tokens,
                                hipStream_t s);

}  // namespace ckv
