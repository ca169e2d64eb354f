// cluster.hip -- semantic clustering of keys on gfx950.
//
// Method: "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
// Recallable Compression", section 核心方法细节 / 语义空间中的聚类 (clustering in
// semantic space, cosine distance D, K-means of Fig. 4) and section
// 选择与索引机制 (selection and indexing: cluster sizes, prefix sums and
// label-sorted token indices kept as metadata).
//
// One call runs, per independent KV head:
//   copy_keys                 only for keys in pinned host memory: one copy
//                             to device memory               (HBM-bound)
//   init_centroids            mu_c = k_{n_sink + s*c}
//   iters x {
//     assign                  cosine GEMM on bf16 MFMA (keys as stored,
//                             unit centroids) + fused row argmax
//     csr count/scan/scatter  atomic-free stable counting sort -> CSR
//     update                  per-cluster fp64 segmented sum of raw keys,
//                             mean -> fp32 centroid, unit centroid for the
//                             next assignment                (HBM-bound)
//   }
// The page's own update kernel (Fig. 7: shared-memory atomicAdd per cluster,
// threads strided along the sequence, channels split into P partitions) is
// replaced by the counting sort + segmented reduction: no atomics, so every
// result is bitwise reproducible.
#include <type_traits>

#include "cluster_dev.h"

namespace ckv {

// --------------------------------------------------------------------------
// Unit vector of a 128-element row held one element per thread (128 threads
// of the block participate; others pass active=false). |x|^2 is one fp64
// fused-multiply-add chain over j = 0..127 (evaluated by thread 0 in that
// order), |x| its fp64 square root, and element j becomes fp32(x_j / |x|)
// (one fp64 division), rounded once more to bf16 when BF16. A zero row
// stays zero.
template <bool BF16>
__device__ void block_unit_row(float x, bool active, int j, void *out_row,
                               float *sx, double *snrm) {
    if (active) sx[j] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        double ss = 0.0;
        for (int k = 0; k < kD; ++k) ss = __fma_rn((double)sx[k], (double)sx[k], ss);
        *snrm = sqrt(ss);
    }
    __syncthreads();
    if (active) {
        const double n = *snrm;
        float y = (n > 0.0) ? (float)((double)x / n) : 0.f;
        if (BF16)
            ((uint16_t *)out_row)[j] = (uint16_t)f32_to_bf16_rne(y);
        else
            ((float *)out_row)[j] = y;
    }
}

// The row as the inner-product and L2 assignments read it: element j
// rounded to the key type (bf16 when BF16). For L2 also the score bias
// -|x^|^2 / 2 of the rounded row x^: one fp64 fma chain over j = 0..127 by
// thread 0, halved, stored as fp32.
template <bool BF16, bool L2>
__device__ void block_store_row(float x, int j, void *out_row, float *sx, float *bias) {
    float y = x;
    if (BF16) {
        const uint32_t b = f32_to_bf16_rne(x);
        ((uint16_t *)out_row)[j] = (uint16_t)b;
        y = bf16_to_f32((uint16_t)b);
    } else {
        ((float *)out_row)[j] = x;
    }
    if (!L2) return;
    sx[j] = y;
    __syncthreads();
    if (threadIdx.x == 0) {
        double ss = 0.0;
        for (int k = 0; k < kD; ++k) ss = __fma_rn((double)sx[k], (double)sx[k], ss);
        *bias = (float)(-0.5 * ss);
    }
}

// --------------------------------------------------------------------------
// copy_keys: rows n_sink .. L-1 of every head copied into the workspace
// [H][Lp][d], for keys in pinned host memory only (device keys are read where
// they are). The assignment then reads them from device memory in every
// iteration instead of over the host link. Plain 16-byte chunks, four per
// thread in flight.
constexpr int kCkThreads = 256, kCkPer = 4;

__global__ __launch_bounds__(kCkThreads) void k_copy_keys(const u32x4 *__restrict__ K,
                                                          int64_t head_stride16,
                                                          int64_t row0_16, int64_t n16,
                                                          u32x4 *__restrict__ kt) {
    const int h = blockIdx.y;
    const int64_t e0 = (int64_t)blockIdx.x * (kCkThreads * kCkPer) + threadIdx.x;
    const u32x4 *src = K + h * head_stride16 + row0_16;
    u32x4 *dst = kt + h * n16;
    u32x4 v[kCkPer];
#pragma unroll
    for (int k = 0; k < kCkPer; ++k) {
        const int64_t e = e0 + kCkThreads * k;
        v[k] = src[e < n16 ? e : 0];
    }
#pragma unroll
    for (int k = 0; k < kCkPer; ++k) {
        const int64_t e = e0 + kCkThreads * k;
        if (e < n16) dst[e] = v[k];
    }
}

hipError_t launch_copy_keys(const ClusterPlan &p, const void *K, hipStream_t s) {
    const int64_t es = p.dtype == 1 ? 2 : 4;           // bytes per element
    const int64_t per_row = kD * es / 16;               // 16-byte chunks per row
    const int64_t n16 = p.Lp * per_row;
    const int64_t blk = kCkThreads * kCkPer;
    hipLaunchKernelGGL(k_copy_keys, dim3((unsigned)((n16 + blk - 1) / blk), p.H),
                       dim3(kCkThreads), 0, s, (const u32x4 *)K,
                       p.k_head_stride * es / 16, (int64_t)p.n_sink * per_row, n16,
                       (u32x4 *)p.kt);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// init_centroids: mu_c = raw key at window row n_sink + s*c, s = floor(Lp/C)
// (the page samples keys as initial centroids; evenly spaced tokens here).
// The first workgroup of a head also labels its sink rows -1.
template <bool BF16, int M>
__global__ __launch_bounds__(128) void k_init_centroids(
    const void *__restrict__ K, int64_t head_stride, int n_sink, int64_t Lp, int C,
    float *__restrict__ cent, int c_base, int c_cap, void *__restrict__ mt,
    float *__restrict__ mb, int Cpad, int32_t *__restrict__ assign, int64_t L) {
    __shared__ float sx[kD];
    __shared__ double snrm;
    const int c = blockIdx.x, h = blockIdx.y, j = threadIdx.x;
    if (c == 0)
        for (int i = j; i < n_sink; i += 128) assign[(int64_t)h * L + i] = -1;
    const int64_t row = n_sink + (Lp / C) * (int64_t)c;
    const int64_t e = h * head_stride + row * kD + j;
    const float x = BF16 ? bf16_to_f32(((const uint16_t *)K)[e]) : ((const float *)K)[e];
    cent[((int64_t)h * c_cap + c_base + c) * kD + j] = x;
    const int64_t mrow = ((int64_t)h * Cpad + c) * kD;
    void *out = BF16 ? (void *)((uint16_t *)mt + mrow) : (void *)((float *)mt + mrow);
    if (M == kCosine)
        block_unit_row<BF16>(x, true, j, out, sx, &snrm);
    else
        block_store_row<BF16, M == kL2>(x, j, out, sx, mb + (int64_t)h * Cpad + c);
}

template <int M>
static void launch_init_m(const ClusterPlan &p, const void *K, float *cent, int32_t *assign,
                          hipStream_t s) {
    dim3 grid(p.C, p.H);
    if (p.dtype == 1)
        hipLaunchKernelGGL((k_init_centroids<true, M>), grid, dim3(128), 0, s, K,
                           p.k_head_stride, p.n_sink, p.Lp, p.C, cent, p.c_base,
                           p.c_cap, p.mt, p.mb, p.Cpad, assign, p.L);
    else
        hipLaunchKernelGGL((k_init_centroids<false, M>), grid, dim3(128), 0, s, K,
                           p.k_head_stride, p.n_sink, p.Lp, p.C, cent, p.c_base,
                           p.c_cap, p.mt, p.mb, p.Cpad, assign, p.L);
}

hipError_t launch_init_centroids(const ClusterPlan &p, const void *K, float *cent,
                                 int32_t *assign, hipStream_t s) {
    if (p.metric == kCosine)
        launch_init_m<kCosine>(p, K, cent, assign, s);
    else if (p.metric == kInnerProduct)
        launch_init_m<kInnerProduct>(p, K, cent, assign, s);
    else
        launch_init_m<kL2>(p, K, cent, assign, s);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// assign (bf16): scores = K . Mt^T on v_mfma_f32_16x16x32_bf16 with fp32
// accumulation, fused with a per-token argmax (ties -> lower cluster id).
// For the cosine, Mt holds the unit centroids and K the keys as stored: a
// key's cosine with mu is <k, mu/|mu|> / |k|, and the positive factor 1/|k|
// is common to all its scores, so the largest <k, mu/|mu|> is the largest
// cosine and the keys are never normalised.
//
// Persistent workgroups of 8 waves (two per SIMD, 256 registers each), one
// per CU, each walking a contiguous range of 512-token tiles (head-major, so
// consecutive tiles share a head and the workgroups of one XCD share a head's
// centroids in L2). Tokens sit on the MFMA N dimension, clusters on M. Each
// wave owns 64 tokens of a tile: four 16-token N tiles whose B fragments stay
// in registers while the wave sweeps every cluster; the next tile's fragments
// are requested into a second register set as soon as the current tile
// starts, so the token rows arrive while the MFMAs run. The head's unit
// centroids sit in LDS, up to 512 clusters at a time (a round), XOR-swizzled
// so the 16 lanes reading one 16-byte column of 16 rows hit distinct banks;
// with a single round they are loaded once per head.
//
// Inside a wave the M tiles are software-pipelined: the 16 MFMAs of tile m
// are issued next to the argmax instructions of tile m - 1 (two sets of
// accumulators), and the A fragments of tile m + 1 are read from LDS
// meanwhile, so the matrix pipe, the vector ALU and LDS work at once.
//
// MFMA 16x16x32 fragment layout (wave64): lane l supplies row/column
// (l & 15) and the 8 consecutive k values 8*(l >> 4) .. +7 of a 32-wide k
// step, for A and B alike; the 16x16 fp32 result gives lane l column
// (l & 15) and rows 4*(l >> 4) + i, i = 0..3.
//
// The argmax is exact up to the fp32 accumulation of the scores:
//  * cosine: a token's accumulations start from beta = 2 |k| (its squared
//    norm summed from its own B fragments), so every score beta + s lies in
//    [0.99, 3.01] |k| and orders like its bit pattern. Within a group of
//    kAsGroup consecutive M tiles a lane's candidates carry a 5-bit key in
//    their low bits (larger for the lower id) and are reduced with float max;
//    the group's winner then replaces the running best only if its score with
//    the key bits cleared is strictly larger, and lanes merge on (truncated
//    score, id). Every decision therefore compares beta + s truncated to
//    2^-18 of its magnitude (1.2e-5 |k| at most, so 1.2e-5 in cosine units)
//    and resolves equal truncated scores -- exact ties included -- to the
//    lower id. A key whose squared norm is below 2^-100 takes beta = 2^-49:
//    a zero key then ties everywhere and joins cluster 0.
//  * inner product and L2: a plain compare-and-select per score (strict >
//    in ascending id order), then the same lane merge on (score, id).
constexpr int kAsWaves = 8;
constexpr int kAsThreads = 64 * kAsWaves;
constexpr int kAsTok = 64 * kAsWaves;   // tokens per tile
constexpr int kAsRound = 512;           // clusters resident in LDS at a time
constexpr int kAsGroup = 8;             // M tiles per packed-argmax group
constexpr uint32_t kAsKey = 4 * kAsGroup - 1;   // key bits of a group (5)
static_assert(kAsRound % (16 * kAsGroup) == 0, "groups never straddle a round");

// B fragments of the wave's 64 tokens from row tok0 of a head's rows K4
// (rows past the window read the last row; their results are not stored).
__device__ __forceinline__ void as_load_b(const u32x4 *K4, int64_t Lp, int64_t tok0, int col,
                                          int kq, bf16x8 (&b)[4][4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t row = tok0 + 16 * t + col;
        const int64_t rr = row < Lp ? row : Lp - 1;
#pragma unroll
        for (int s = 0; s < 4; ++s) b[t][s] = __builtin_bit_cast(bf16x8, K4[rr * 16 + 4 * s + kq]);
    }
}

// A fragments of M tile m (LDS rows 16m .. 16m + 15 of the round).
__device__ __forceinline__ void as_lds_a(const u32x4 *sA, int m, int col, int kq,
                                         bf16x8 (&a)[4]) {
    const int r = 16 * m + col;
#pragma unroll
    for (int s = 0; s < 4; ++s) a[s] = __builtin_bit_cast(bf16x8, sA[r * 16 + ((4 * s + kq) ^ col)]);
}

// Cosine offsets of the wave's tokens: beta[t] = 2 |k| for the token in
// column (l & 15) of N tile t. Each lane sums the squares of its 32 elements
// of the row (bf16 pairs on v_dot2), then the four lanes holding the row add
// their sums in a butterfly, so all four get the same value. Deterministic,
// so every path that clusters the same rows starts from the same offsets.
__device__ __forceinline__ float as_sq2(uint32_t u, float acc) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    bf16x2 v;
    __builtin_memcpy(&v, &u, 4);
    return __builtin_amdgcn_fdot2_f32_bf16(v, v, acc, false);
}

__device__ __forceinline__ void as_beta(const bf16x8 (&b)[4][4], float (&beta)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float n2 = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const u32x4 w = __builtin_bit_cast(u32x4, b[t][s]);
            n2 = as_sq2(w.x, n2);
            n2 = as_sq2(w.y, n2);
            n2 = as_sq2(w.z, n2);
            n2 = as_sq2(w.w, n2);
        }
        n2 += __shfl_xor(n2, 16);
        n2 += __shfl_xor(n2, 32);
        // a normal argument: the hardware square root needs no rescaling
        beta[t] = 2.f * __builtin_amdgcn_sqrtf(fmaxf(n2, 0x1p-100f));
    }
}

// The 16 MFMAs of one M tile against the wave's four N tiles, k steps in
// order for every N tile; the cosine's accumulation starts from beta.
template <bool COS>
__device__ __forceinline__ void as_mfma(const bf16x8 (&a)[4], const bf16x8 (&b)[4][4],
                                        const float (&beta)[4], f32x4 (&acc)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const float c0 = COS ? beta[t] : 0.f;
        acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[0], b[t][0], (f32x4){c0, c0, c0, c0},
                                                         0, 0, 0);
    }
#pragma unroll
    for (int s = 1; s < 4; ++s)
#pragma unroll
        for (int t = 0; t < 4; ++t)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[s], b[t][s], acc[t], 0, 0, 0);
}

// Cosine, one M tile at position mm of its group: the lane's rows c0 .. c0+3
// get keys kAsKey - (4 mm + i) in their low bits and join the group maxima
// gb[t]; MASK drops ids >= C (0 never wins against beta + s > 0).
// The insert (x & ~kAsKey) | key is one v_bitop3_b32 with kAsKey as an
// inline constant and the key (uniform) in a scalar register: truth table
// 0xBA, bit 4 a + 2 b + c of it being (a & ~b) | c for operand bits a, b, c.
template <bool MASK>
__device__ __forceinline__ void as_cos_tile(const f32x4 (&acc)[4], int mm, int c0, int C,
                                            float (&gb)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t key = kAsKey - (uint32_t)(4 * mm + i);
            p[i] = __uint_as_float(
                __builtin_amdgcn_bitop3_b32(__float_as_uint(acc[t][i]), kAsKey, key, 0xBA));
            if (MASK && c0 + i >= C) p[i] = 0.f;
        }
        gb[t] = fmaxf(fmaxf(gb[t], p[0]), p[1]);
        gb[t] = fmaxf(fmaxf(gb[t], p[2]), p[3]);
    }
}

// Cosine, end of group g: its winner replaces the running best (bv: the
// truncated score, bk: g << 5 | key) only if strictly larger; gb restarts.
__device__ __forceinline__ void as_cos_close(float (&gb)[4], int g, float (&bv)[4],
                                             uint32_t (&bk)[4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint32_t u = __float_as_uint(gb[t]);
        const float v = __uint_as_float(u & ~kAsKey);
        if (v > bv[t]) {
            bv[t] = v;
            bk[t] = ((uint32_t)g << 5) | (u & kAsKey);
        }
        gb[t] = 0.f;
    }
}

// The cluster id a lane's running best stands for.
__device__ __forceinline__ int as_cos_id(uint32_t bk, int kq) {
    const int j = (int)(kAsKey - (bk & kAsKey));       // 4 mm + i
    return 16 * (kAsGroup * (int)(bk >> 5) + (j >> 2)) + 4 * kq + (j & 3);
}

// Inner product and L2, one M tile: scores (plus the clusters' bias for L2,
// from LDS row 16m of the round) compared one by one in ascending id.
template <bool MASK, bool BIAS>
__device__ __forceinline__ void as_exact_tile(const f32x4 (&acc)[4], const float *sB, int m,
                                              int kq, int c0, int C, float (&bv)[4],
                                              int (&bc)[4]) {
    f32x4 bias = (f32x4){0.f, 0.f, 0.f, 0.f};
    if (BIAS) bias = *(const f32x4 *)(sB + 16 * m + 4 * kq);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float sc = BIAS ? acc[t][i] + bias[i] : acc[t][i];
            if ((!MASK || c0 + i < C) && sc > bv[t]) {
                bv[t] = sc;
                bc[t] = c0 + i;
            }
        }
}

// Merge the four row groups of a token (lanes l, l^16, l^32, l^48): larger
// score, then lower id.
__device__ __forceinline__ int as_merge(float v, int c) {
#pragma unroll
    for (int off = 16; off <= 32; off *= 2) {
        const float ov = __shfl_xor(v, off);
        const int oc = __shfl_xor(c, off);
        if (ov > v || (ov == v && oc < c)) {
            v = ov;
            c = oc;
        }
    }
    return c;
}

// LDS fill of one round: centroid rows rb .. rb + rows - 1 of the head at M4
// (and their score bias when BIAS), behind barriers on both sides. DEPTH
// 16-byte loads per thread are in flight at once (16 cover a whole round).
template <bool BIAS, int DEPTH>
__device__ __forceinline__ void as_fill(u32x4 *sA, float *sB, const u32x4 *M4,
                                        const float *mbh, int rb, int rows, int tid) {
    __syncthreads();                                      // the previous round is done
    for (int e0 = 0; e0 < rows * 16; e0 += kAsThreads * DEPTH) {
        u32x4 v[DEPTH];
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
            const int e = e0 + tid + kAsThreads * k;
            v[k] = M4[(int64_t)rb * 16 + (e < rows * 16 ? e : 0)];
        }
#pragma unroll
        for (int k = 0; k < DEPTH; ++k) {
            const int e = e0 + tid + kAsThreads * k;
            const int rr = e >> 4, q = e & 15;
            if (e < rows * 16) sA[rr * 16 + (q ^ (rr & 15))] = v[k];
        }
    }
    if (BIAS)
        for (int e = tid; e < rows; e += kAsThreads) sB[e] = mbh[rb + e];
    __syncthreads();
}

// ka: the first clustered row of head 0, heads ka_stride elements apart.
template <int M>
__global__ __launch_bounds__(kAsThreads) void k_assign_bf16(
    const uint16_t *__restrict__ ka, int64_t ka_stride, const uint16_t *__restrict__ mt,
    const float *__restrict__ mb, int64_t Lp, int C, int Cpad, int32_t *__restrict__ assign,
    int64_t L, int n_sink, int tiles_per_head, int n_tiles) {
    constexpr bool COS = M == kCosine, BIAS = M == kL2;
    __shared__ u32x4 sA[kAsRound * 16];
    __shared__ __align__(16) float sB[BIAS ? kAsRound : 4];
    const uint32_t w = xcd_linear(blockIdx.x, gridDim.x);
    const int t_begin = (int)((int64_t)w * n_tiles / gridDim.x);
    const int t_end = (int)((int64_t)(w + 1) * n_tiles / gridDim.x);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: keep it scalar
    const int col = lane & 15, kq = lane >> 4;
    const int crows = (C + 31) / 32 * 32;                 // even number of M tiles, <= Cpad
    const int nr = (crows + kAsRound - 1) / kAsRound;     // rounds per tile
    int h = t_begin / tiles_per_head;
    int tile = t_begin - h * tiles_per_head;
    // A single round stays resident while the head does not change: fill it
    // first, then request the first tile's rows (each wave starts as soon as
    // its own rows arrive). Fragments of tile t + 1 are requested while tile
    // t computes; no load is issued under a branch, so the compiler's waits
    // for b never include them.
    int loaded = -1;
    if (nr == 1) {
        as_fill<BIAS, kAsRound * 16 / kAsThreads>(sA, sB, (const u32x4 *)(mt + (int64_t)h * Cpad * kD),
                                                  mb + (int64_t)h * Cpad, 0, crows, tid);
        loaded = h;
    }
    bf16x8 b[4][4], bn[4][4];
    as_load_b((const u32x4 *)(ka + (int64_t)h * ka_stride), Lp, (int64_t)tile * kAsTok + wave * 64,
              col, kq, b);
    for (int t = t_begin; t < t_end; ++t) {
        const int64_t tok0 = (int64_t)tile * kAsTok + wave * 64;
        float beta[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (COS) as_beta(b, beta);
        const u32x4 *M4 = (const u32x4 *)(mt + (int64_t)h * Cpad * kD);
        // the next tile (the last one requests its own rows again: harmless)
        int hn = h, tilen = tile + 1;
        if (tilen == tiles_per_head) {
            tilen = 0;
            ++hn;
        }
        const bool more = t + 1 < t_end;
        const int hp = more ? hn : h, tp = more ? tilen : tile;
        float bv[4];
        uint32_t bk[4];
        int bc[4];
        float gb[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            bv[u] = COS ? 0.f : -INFINITY;
            bk[u] = kAsKey;
            bc[u] = 0x7fffffff;
            gb[u] = 0.f;
        }
        // one round: its LDS fill when needed, then its M tiles
        auto fill = [&](int r) {
            const int rb = r * kAsRound;
            const int rows = (crows - rb < kAsRound) ? crows - rb : kAsRound;
            if (nr > 1 || loaded != h) {
                as_fill<BIAS, 4>(sA, sB, M4, mb + (int64_t)h * Cpad, rb, rows, tid);
                loaded = h;
            }
        };
        // the next tile's fragments: requested halfway through round 0's M
        // tiles (earlier, the waves whose rows came first would delay the
        // others' first rows with their prefetch), or after them when round
        // 0 is too short to reach that point
        // (L2: no second register set -- its bias leaves no room -- so the
        // next tile's rows are requested only once this tile is done)
        auto prefetch = [&]() {
            if constexpr (!BIAS)
                as_load_b((const u32x4 *)(ka + (int64_t)hp * ka_stride), Lp,
                          (int64_t)tp * kAsTok + wave * 64, col, kq, bn);
        };
        auto run = [&](int r) {
            const int rb = r * kAsRound;
            const int rows = (crows - rb < kAsRound) ? crows - rb : kAsRound;
            const int nm = rows / 16;                     // even
            const int mg0 = rb / 16;                      // global index of the round's tile 0
            const int m_pf = (nm / 2) | 1;                // odd, like the loop's m
            bf16x8 aE[4], aO[4];
            f32x4 cE[4], cO[4];
            // argmax of tile m (global mg0 + m) held in acc
            auto amax = [&](const f32x4 (&acc)[4], int m, auto mask) {
                constexpr bool MK = decltype(mask)::value;
                const int mg = mg0 + m;
                if (COS)
                    as_cos_tile<MK>(acc, mg % kAsGroup, 16 * mg + 4 * kq, C, gb);
                else
                    as_exact_tile<MK, BIAS>(acc, sB, m, kq, 16 * mg + 4 * kq, C, bv, bc);
            };
            using NoMask = std::integral_constant<bool, false>;
            using Mask = std::integral_constant<bool, true>;
            as_lds_a(sA, 0, col, kq, aE);
            as_lds_a(sA, 1, col, kq, aO);
            as_mfma<COS>(aE, b, beta, cE);                // tile 0
            int m = 1;
            for (; m + 1 < nm; m += 2) {
                if (r == 0 && m == m_pf) prefetch();
                as_lds_a(sA, m + 1, col, kq, aE);
                as_mfma<COS>(aO, b, beta, cO);            // tile m
                amax(cE, m - 1, NoMask{});
                as_lds_a(sA, m + 2, col, kq, aO);
                as_mfma<COS>(aE, b, beta, cE);            // tile m + 1
                amax(cO, m, NoMask{});
                if (COS && (mg0 + m) % kAsGroup == kAsGroup - 1)
                    as_cos_close(gb, (mg0 + m) / kAsGroup, bv, bk);
            }
            if (r == 0 && m_pf + 1 >= nm) prefetch();
            as_mfma<COS>(aO, b, beta, cO);                // tile nm - 1
            amax(cE, nm - 2, Mask{});
            amax(cO, nm - 1, Mask{});
            if (COS) as_cos_close(gb, (mg0 + nm - 1) / kAsGroup, bv, bk);
        };
        fill(0);
        run(0);
        for (int r = 1; r < nr; ++r) {
            fill(r);
            run(r);
        }
        int res[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) res[u] = as_merge(bv[u], COS ? as_cos_id(bk[u], kq) : bc[u]);
        // the next tile's fragments become current (this waits for them),
        // then the labels are stored
        if constexpr (BIAS) {
            as_load_b((const u32x4 *)(ka + (int64_t)hp * ka_stride), Lp,
                      (int64_t)tp * kAsTok + wave * 64, col, kq, b);
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int s2 = 0; s2 < 4; ++s2) b[u][s2] = bn[u][s2];
        }
        const int64_t tok = tok0 + lane;
        const int v = (kq == 0) ? res[0] : (kq == 1) ? res[1] : (kq == 2) ? res[2] : res[3];
        if (tok < Lp) assign[(int64_t)h * L + n_sink + tok] = v;
        h = hn;
        tile = tilen;
    }
}

// assign (fp32): a workgroup takes 64 tokens; wave g scores them against the
// clusters c = g, g + 8, g + 16, ... (one token per lane, the cluster rows
// uniform across the wave, so they come through the scalar cache), each
// score the fp32 dot product over j = 0..127 in order of the key as stored
// and the row in mt (the unit centroid for the cosine, whose argmax needs no
// unit key, as in the bf16 kernel), plus the cluster's bias when mb is given
// (L2). Each wave keeps the strictly larger score in ascending id order;
// the eight candidates of a token then merge on (score, lower id), which is
// the argmax with ties to the lower id over all clusters (cluster 0 when no
// score exceeds -inf, as in one sequential scan). Used for fp32 keys.
constexpr int kAfTok = 64, kAfGroups = 8;

__global__ __launch_bounds__(64 * kAfGroups) void k_assign_f32(
    const float *__restrict__ ka, int64_t ka_stride, const float *__restrict__ mt,
    const float *__restrict__ mb, int64_t Lp, int C, int Cpad, int32_t *__restrict__ assign,
    int64_t L, int n_sink) {
    __shared__ float sbest[kAfGroups][kAfTok];
    __shared__ int sarg[kAfGroups][kAfTok];
    const int h = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t i = (int64_t)blockIdx.x * kAfTok + lane;
    const int64_t ii = i < Lp ? i : Lp - 1;
    float k[kD];
    const float *src = ka + (int64_t)h * ka_stride + ii * kD;
#pragma unroll
    for (int j = 0; j < kD; j += 4) {
        const float4 v = *(const float4 *)(src + j);
        k[j] = v.x;
        k[j + 1] = v.y;
        k[j + 2] = v.z;
        k[j + 3] = v.w;
    }
    float best = -INFINITY;
    int arg = 0x7fffffff;
    // two of the wave's clusters at a time: two independent chains, both
    // rows requested together
    for (int c = g; c < C; c += 2 * kAfGroups) {
        const int c2 = c + kAfGroups;
        const float *m1 = mt + ((int64_t)h * Cpad + c) * kD;
        const float *m2 = mt + ((int64_t)h * Cpad + (c2 < C ? c2 : c)) * kD;
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int j = 0; j < kD; ++j) {
            s1 = __fmaf_rn(k[j], m1[j], s1);
            s2 = __fmaf_rn(k[j], m2[j], s2);
        }
        if (mb) {
            s1 += mb[(int64_t)h * Cpad + c];
            s2 += mb[(int64_t)h * Cpad + (c2 < C ? c2 : c)];
        }
        if (s1 > best) {
            best = s1;
            arg = c;
        }
        if (c2 < C && s2 > best) {
            best = s2;
            arg = c2;
        }
    }
    sbest[g][lane] = best;
    sarg[g][lane] = arg;
    __syncthreads();
    if (g == 0 && i < Lp) {
        for (int q = 1; q < kAfGroups; ++q) {
            const float b2 = sbest[q][lane];
            const int a2 = sarg[q][lane];
            if (a2 != 0x7fffffff && (b2 > best || (b2 == best && a2 < arg))) {
                best = b2;
                arg = a2;
            }
        }
        // no score above -inf anywhere (as a sequential scan from cluster 0)
        assign[(int64_t)h * L + n_sink + i] = arg == 0x7fffffff ? 0 : arg;
    }
}

hipError_t launch_assign(const ClusterPlan &p, int32_t *assign, hipStream_t s) {
    if (p.dtype == 1) {
        const int tph = (int)((p.Lp + kAsTok - 1) / kAsTok);
        const int n_tiles = tph * p.H;
        const int grid = n_tiles < p.n_cu ? n_tiles : p.n_cu;
        auto kern = p.metric == kCosine ? k_assign_bf16<kCosine>
                  : p.metric == kL2     ? k_assign_bf16<kL2>
                                        : k_assign_bf16<kInnerProduct>;
        hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(kAsThreads), 0, s,
                           (const uint16_t *)p.ka, p.ka_stride, (const uint16_t *)p.mt,
                           (const float *)p.mb, p.Lp, p.C, p.Cpad, assign, p.L, p.n_sink, tph,
                           n_tiles);
    } else {
        dim3 grid((unsigned)((p.Lp + kAfTok - 1) / kAfTok), p.H);
        hipLaunchKernelGGL(k_assign_f32, grid, dim3(64 * kAfGroups), 0, s, (const float *)p.ka,
                           p.ka_stride, (const float *)p.mt,
                           p.metric == kL2 ? (const float *)p.mb : nullptr, p.Lp, p.C, p.Cpad,
                           assign, p.L, p.n_sink);
    }
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// CSR (cluster sizes, prefix sums, label-sorted token ids) by a stable
// counting sort over tiles of 2048 tokens, no atomics:
//  count:   per tile, each wave finds, for every lane, the lanes holding the
//           same label (one ballot per label bit), giving the lane's rank
//           among equal labels; per-wave label counts in LDS turn that into
//           a rank inside the tile, and their sums are the tile's histogram.
//  scan:    (C > 512) per head and cluster, exclusive prefix over tiles (tile
//           bases) and the cluster size.
//  scatter: offsets = exclusive prefix of the sizes over the clusters; token
//           i of tile T with label a goes to offsets[a] + base[T][a] + rank_i.
//           For C <= 512 the scatter also does the scan (one cluster per
//           thread), so that path is two launches.
// Ranks grow with the token position, so each cluster lists its tokens in
// ascending order.
// scan: per head, for every cluster, exclusive prefix of its tile counts over
// the tiles (in tile order) and its total count. Workgroup = 64 clusters x 16
// parts; part p owns the contiguous tiles [p*R, (p+1)*R), R = ceil(T/16);
// lanes of a wave are consecutive clusters, so the loads coalesce.
constexpr int kScanParts = 16;
constexpr int kScanBatch = 16;

__global__ __launch_bounds__(1024) void k_csr_scan(int32_t *__restrict__ tile_hist,
                                                   int64_t ntiles, int C,
                                                   int32_t *__restrict__ counts) {
    __shared__ int psum[kScanParts][64];
    const int h = blockIdx.y, tid = threadIdx.x;
    const int cl = tid & 63, part = tid >> 6;
    const int c = blockIdx.x * 64 + cl;
    const bool valid = c < C;
    const int cc = valid ? c : C - 1;
    const int64_t R = (ntiles + kScanParts - 1) / kScanParts;
    const int64_t t0 = part * R, t1 = (t0 + R < ntiles) ? t0 + R : ntiles;
    int32_t *col = tile_hist + (int64_t)h * ntiles * C + cc;
    // pass 1: the part's sum (batches of loads in flight, clamped, masked)
    int sum = 0;
    for (int64_t tb = t0; tb < t1; tb += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int k = 0; k < kScanBatch; ++k) {
            const int64_t t = tb + k;
            v[k] = col[(t < t1 ? t : t0) * C];
        }
#pragma unroll
        for (int k = 0; k < kScanBatch; ++k) sum += (tb + k < t1) ? v[k] : 0;
    }
    psum[part][cl] = sum;
    __syncthreads();
    int base = 0;
    for (int p = 0; p < part; ++p) base += psum[p][cl];
    if (part == kScanParts - 1 && valid) counts[(int64_t)h * C + c] = base + sum;
    // pass 2: rewrite the part's tiles with exclusive bases (values re-read:
    // they are still in L2)
    for (int64_t tb = t0; tb < t1; tb += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int k = 0; k < kScanBatch; ++k) {
            const int64_t t = tb + k;
            v[k] = col[(t < t1 ? t : t0) * C];
        }
#pragma unroll
        for (int k = 0; k < kScanBatch; ++k) {
            const int64_t t = tb + k;
            if (t < t1 && valid) col[t * C] = base;
            base += (t < t1) ? v[k] : 0;
        }
    }
}

// The kernels over 2048-token tiles (the scan above works on any tiling).
//  count_wide: wave w of the tile's 512 threads takes its tokens
//              [256 w, 256 w + 256) in 4 rounds of 64; a token's rank among
//              equal labels of its wave is its ballot rank in the round plus
//              the wave's running count of that label (LDS, updated by the
//              round's first lane of each label); after a barrier the counts
//              of the waves before it make that a rank in the tile, and the
//              waves' sums are the tile's histogram.
//  scatter_wide: thread c sums cluster c's histogram over all tiles of the
//              head (its size) and over the tiles before this one (its base
//              here); an exclusive scan over the sizes gives the offsets, and
//              token i of label a goes to offsets[a] + base[a] + rank_i.
// MAXC sizes the count's LDS: 512 clusters for the two-launch path, 2048 for
// the three-launch one.
constexpr int kCsrThreads = 512;
constexpr int kCsrRounds = kCsrWideTile / kCsrThreads;   // rounds of 64 per wave

template <int MAXC>
__global__ __launch_bounds__(kCsrThreads) void k_csr_count_wide(
    const int32_t *__restrict__ assign, int64_t L, int n_sink, int64_t Lp, int C, int nbits,
    int64_t ntiles, int32_t *__restrict__ tile_hist, int32_t *__restrict__ tile_rank) {
    static_assert(kCsrRounds * kCsrThreads == kCsrWideTile, "tile = waves x rounds x 64");
    __shared__ int32_t wcnt[kCsrThreads / 64][MAXC];
    const int h = blockIdx.y;
    const int64_t tile = blockIdx.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int64_t first = tile * kCsrWideTile + (int64_t)wave * (64 * kCsrRounds) + lane;
    int a[kCsrRounds];
    bool valid[kCsrRounds];
#pragma unroll
    for (int r = 0; r < kCsrRounds; ++r) {
        const int64_t i = first + 64 * r;
        valid[r] = i < Lp;
        const int v = valid[r] ? assign[(int64_t)h * L + n_sink + i] : 0;
        a[r] = v < 0 ? 0 : (v >= C ? C - 1 : v);
    }
    for (int e = tid; e < (kCsrThreads / 64) * MAXC; e += kCsrThreads) (&wcnt[0][0])[e] = 0;
    __syncthreads();
    int rk[kCsrRounds];
#pragma unroll
    for (int r = 0; r < kCsrRounds; ++r) {
        uint64_t eq = __ballot(valid[r]);
        for (int b = 0; b < nbits; ++b) {
            const int bit = (a[r] >> b) & 1;
            const uint64_t bb = __ballot(bit);
            eq &= bit ? bb : ~bb;
        }
        const int before = __popcll(eq & __lanemask_lt());
        // every lane reads the running count before the label's first lane
        // (one per label) writes it back: one wave, program order
        const int run = wcnt[wave][a[r]];
        rk[r] = run + before;
        if (valid[r] && before == 0) wcnt[wave][a[r]] = run + __popcll(eq);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kCsrRounds; ++r) {
        if (!valid[r]) continue;
        int base = 0;
        for (int w = 0; w < wave; ++w) base += wcnt[w][a[r]];
        tile_rank[(int64_t)h * Lp + first + 64 * r] = rk[r] + base;
    }
    int32_t *hist = tile_hist + ((int64_t)h * ntiles + tile) * C;
    for (int c = tid; c < C; c += kCsrThreads) {
        int sacc = 0;
#pragma unroll
        for (int w = 0; w < kCsrThreads / 64; ++w) sacc += wcnt[w][c];
        hist[c] = sacc;
    }
}

__global__ __launch_bounds__(kCsrThreads) void k_csr_scatter_wide(
    const int32_t *__restrict__ assign, int64_t L, int n_sink, int64_t Lp, int C,
    int64_t ntiles, const int32_t *__restrict__ tile_hist, const int32_t *__restrict__ tile_rank,
    int32_t *__restrict__ offsets, int c_base, int c_cap, int64_t t_base, int64_t t_cap,
    int64_t token_base, int32_t *__restrict__ tokens) {
    static_assert(kCsrWideMaxC <= kCsrThreads, "one cluster per thread");
    constexpr int NB = 16;                      // histogram loads in flight per batch
    __shared__ int start[kCsrWideMaxC];         // offsets[c] + base of this tile
    __shared__ int wsum[17];
    const int h = blockIdx.y, tid = threadIdx.x;
    const int64_t tile = blockIdx.x;
    // this thread's tokens: label and rank (loads in flight with the counts)
    int a[kCsrRounds], rk[kCsrRounds];
#pragma unroll
    for (int r = 0; r < kCsrRounds; ++r) {
        const int64_t i = tile * kCsrWideTile + (int64_t)kCsrThreads * r + tid;
        const int64_t ii = i < Lp ? i : Lp - 1;
        const int v = assign[(int64_t)h * L + n_sink + ii];
        a[r] = v < 0 ? 0 : (v >= C ? C - 1 : v);
        rk[r] = tile_rank[(int64_t)h * Lp + ii];
    }
    // cluster tid: its size over all tiles and its count in the tiles before this one
    int cnt = 0, base = 0;
    if (tid < C) {
        const int32_t *col = tile_hist + (int64_t)h * ntiles * C + tid;
        for (int64_t t0 = 0; t0 < ntiles; t0 += NB) {
            int v[NB];
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int64_t t = t0 + k;
                v[k] = col[(t < ntiles ? t : ntiles - 1) * C];
            }
#pragma unroll
            for (int k = 0; k < NB; ++k) {
                const int64_t t = t0 + k;
                cnt += t < ntiles ? v[k] : 0;
                base += t < tile ? v[k] : 0;
            }
        }
    }
    int total;
    const int run = block_excl_scan(tid < C ? cnt : 0, wsum, &total);
    if (tid < C) start[tid] = run + base;
    if (tile == 0) {
        int32_t *off = offsets + (int64_t)h * (c_cap + 1) + c_base;
        if (tid < C) off[tid] = (int32_t)(t_base + run);
        if (tid == 0) off[C] = (int32_t)(t_base + total);
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kCsrRounds; ++r) {
        const int64_t i = tile * kCsrWideTile + (int64_t)kCsrThreads * r + tid;
        const int64_t pos = (int64_t)start[a[r]] + rk[r];
        if (i < Lp && pos >= 0 && pos < Lp)
            tokens[(int64_t)h * t_cap + t_base + pos] = (int32_t)(token_base + n_sink + i);
    }
}

// Scatter over the same 2048-token tiles for C > 512, after k_csr_scan has
// turned the tile histograms into tile bases and cluster sizes: the offsets
// are an exclusive scan of the sizes (four per thread, in LDS; the tile-0
// workgroup writes them out), and token i of label a goes to
// offsets[a] + base[T][a] + rank_i, the tokens of a thread taken in the
// rounds of k_csr_scatter_wide.
__global__ __launch_bounds__(kCsrThreads) void k_csr_scatter_tiles(
    const int32_t *__restrict__ assign, int64_t L, int n_sink, int64_t Lp, int C,
    int64_t ntiles, const int32_t *__restrict__ counts, const int32_t *__restrict__ tile_base,
    const int32_t *__restrict__ tile_rank, int32_t *__restrict__ offsets, int c_base,
    int c_cap, int64_t t_base, int64_t t_cap, int64_t token_base, int32_t *__restrict__ tokens) {
    constexpr int PER = kMaxC / kCsrThreads;        // cluster sizes per thread
    __shared__ int start[kMaxC];                    // offsets[c] + base of this tile
    __shared__ int wsum[17];
    const int h = blockIdx.y, tid = threadIdx.x;
    const int64_t tile = blockIdx.x;
    int a[kCsrRounds], rk[kCsrRounds];
#pragma unroll
    for (int r = 0; r < kCsrRounds; ++r) {
        const int64_t i = tile * kCsrWideTile + (int64_t)kCsrThreads * r + tid;
        const int64_t ii = i < Lp ? i : Lp - 1;
        const int v = assign[(int64_t)h * L + n_sink + ii];
        a[r] = v < 0 ? 0 : (v >= C ? C - 1 : v);
        rk[r] = tile_rank[(int64_t)h * Lp + ii];
    }
    int cv[PER], bv[PER];
    const int32_t *tb = tile_base + ((int64_t)h * ntiles + tile) * C;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int c = tid * PER + k;
        const int cc = c < C ? c : C - 1;
        cv[k] = counts[(int64_t)h * C + cc];
        bv[k] = tb[cc];
    }
    int loc = 0;
#pragma unroll
    for (int k = 0; k < PER; ++k) loc += (tid * PER + k < C) ? cv[k] : 0;
    int total;
    int run = block_excl_scan(loc, wsum, &total);
    int32_t *off = offsets + (int64_t)h * (c_cap + 1) + c_base;
#pragma unroll
    for (int k = 0; k < PER; ++k) {
        const int c = tid * PER + k;
        if (c < C) {
            start[c] = run + bv[k];
            if (tile == 0) off[c] = (int32_t)(t_base + run);
        }
        run += (c < C) ? cv[k] : 0;
    }
    if (tile == 0 && tid == 0) off[C] = (int32_t)(t_base + total);
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kCsrRounds; ++r) {
        const int64_t i = tile * kCsrWideTile + (int64_t)kCsrThreads * r + tid;
        const int64_t pos = (int64_t)start[a[r]] + rk[r];
        if (i < Lp && pos >= 0 && pos < Lp)
            tokens[(int64_t)h * t_cap + t_base + pos] = (int32_t)(token_base + n_sink + i);
    }
}

hipError_t launch_csr(const ClusterPlan &p, const int32_t *assign, int32_t *offsets,
                      int32_t *tokens, hipStream_t s) {
    int nbits = 1;
    while ((1 << nbits) < p.C) ++nbits;
    dim3 grid((unsigned)p.ntiles, p.H);
    if (p.csr_wide) {
        hipLaunchKernelGGL(k_csr_count_wide<kCsrWideMaxC>, grid, dim3(kCsrThreads), 0, s, assign,
                           p.L, p.n_sink, p.Lp, p.C, nbits, p.ntiles, p.tile_hist, p.tile_rank);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(k_csr_scatter_wide, grid, dim3(kCsrThreads), 0, s, assign, p.L,
                           p.n_sink, p.Lp, p.C, p.ntiles, (const int32_t *)p.tile_hist,
                           (const int32_t *)p.tile_rank, offsets, p.c_base, p.c_cap, p.t_base,
                           p.t_cap, p.token_base, tokens);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_csr_count_wide<kMaxC>, grid, dim3(kCsrThreads), 0, s, assign, p.L,
                       p.n_sink, p.Lp, p.C, nbits, p.ntiles, p.tile_hist, p.tile_rank);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_csr_scan, dim3((p.C + 63) / 64, p.H), dim3(1024), 0, s, p.tile_hist,
                       p.ntiles, p.C, p.counts);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_csr_scatter_tiles, grid, dim3(kCsrThreads), 0, s, assign, p.L, p.n_sink,
                       p.Lp, p.C, p.ntiles, (const int32_t *)p.counts,
                       (const int32_t *)p.tile_hist, (const int32_t *)p.tile_rank, offsets,
                       p.c_base, p.c_cap, p.t_base, p.t_cap, p.token_base, tokens);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// update: one workgroup per cluster walks its CSR segment. 16 row slots x
// 16 lanes: lane (slot, q) adds channels 8q..8q+7 of rows slot, slot+16, ...
// into fp64 accumulators; slots are combined in a fixed order (lane
// butterflies, then the four waves in order), so the sum is reproducible.
// mean = sum / n in fp64, stored as fp32; an empty cluster keeps its
// centroid. The unit centroid for the next assignment is written too, by
// the first wave alone (no barrier after the reduction).
// First half: the partial sums of cluster c of head h by the 256 threads of
// a group (ltid = thread in the group) into red; returns the cluster size.
// off points at the cluster's offset pair and tok at its head's token list
// (global memory, or LDS copies of both), t_cap bounds the list.
// The pieces of the first half. upd_range: the cluster's CSR segment from
// its offset pair, clamped to [0, t_cap].
__device__ __forceinline__ void upd_range(const int32_t *off, int64_t t_cap, int64_t &beg,
                                          int64_t &end) {
    beg = off[0];
    end = off[1];
    beg = beg < 0 ? 0 : (beg > t_cap ? t_cap : beg);
    end = end < beg ? beg : (end > t_cap ? t_cap : end);
}

// rows beg + slot + 16k in batches of kUpdNB: a batch's token ids (clamped
// addresses; rows past the segment are masked when the keys are added)
constexpr int kUpdNB = 8;

__device__ __forceinline__ void upd_tokens(const int32_t *tok, int64_t r0, int64_t beg,
                                           int64_t end, int32_t (&tk)[kUpdNB]) {
    const int64_t last = end > beg ? end - 1 : beg;
#pragma unroll
    for (int k = 0; k < kUpdNB; ++k) {
        const int64_t r = r0 + 16 * k;
        tk[k] = tok[r < end ? r : last];
    }
}

// the 16 slots' sums combined in a fixed order (lane butterflies here, the
// waves in order in upd_final) into red[wave]
__device__ __forceinline__ void upd_reduce(double (&acc)[8], int lane, int wave,
                                           double (*red)[kD]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        acc[e] += __shfl_xor(acc[e], 16);
        acc[e] += __shfl_xor(acc[e], 32);
    }
    if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red[wave][8 * lane + e] = acc[e];
    }
}

template <bool BF16>
__device__ __forceinline__ int64_t upd_partial(
    const void *__restrict__ K, int64_t head_stride, int64_t L, int64_t token_base,
    const int32_t *off, const int32_t *tok, int64_t t_cap, int h, int ltid, double (*red)[kD]) {
    const int lane = ltid & 63, wave = ltid >> 6;
    const int slot = ltid >> 4, q = ltid & 15;
    int64_t beg, end;
    upd_range(off, t_cap, beg, end);
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    // a batch's token ids, then its key chunks, each set in flight at once
    constexpr int NB = kUpdNB;
    constexpr int NV = BF16 ? 1 : 2;              // 16-byte chunks per 8 channels
    for (int64_t r0 = beg + slot; r0 < end; r0 += 16 * NB) {
        int32_t tk[NB];
        upd_tokens(tok, r0, beg, end, tk);
        int64_t row[NB];
        bool ok[NB];
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            row[k] = (int64_t)tk[k] - token_base;
            ok[k] = r0 + 16 * k < end && row[k] >= 0 && row[k] < L;
            row[k] = ok[k] ? row[k] : 0;
        }
        u32x4 w[NB][NV];
#pragma unroll
        for (int k = 0; k < NB; ++k)
#pragma unroll
            for (int c = 0; c < NV; ++c)
                w[k][c] = BF16 ? *(const u32x4 *)((const uint16_t *)K + h * head_stride +
                                                  row[k] * kD + 8 * q)
                               : *(const u32x4 *)((const float *)K + h * head_stride +
                                                  row[k] * kD + 8 * q + 4 * c);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int k = 0; k < NB; ++k) {
            if (!ok[k]) continue;
            float f[8];
            if (BF16) {
                unpack8(w[k][0], f);
            } else {
                f[0] = __uint_as_float(w[k][0].x); f[1] = __uint_as_float(w[k][0].y);
                f[2] = __uint_as_float(w[k][0].z); f[3] = __uint_as_float(w[k][0].w);
                f[4] = __uint_as_float(w[k][NV - 1].x); f[5] = __uint_as_float(w[k][NV - 1].y);
                f[6] = __uint_as_float(w[k][NV - 1].z); f[7] = __uint_as_float(w[k][NV - 1].w);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (double)f[e];
        }
    }
    upd_reduce(acc, lane, wave, red);
    return end - beg;
}

// Second half, by the group's first wave once red is complete: lane l owns
// channels l and l + 64. mean = sum / n in fp64, stored as fp32 in the
// centroid row cp (an empty cluster keeps its centroid); then the row the
// next assignment reads: for the cosine the unit row (|mu|^2 as one fp64 fma
// chain over j = 0..127 in order, |mu| its fp64 square root, channel j ->
// fp32(mu_j / |mu|), then bf16 when BF16; a zero row stays zero), else the mean
// rounded to the key type and, for L2, the bias -|mu^|^2 / 2 of that rounded
// row. That row goes to mrow and the bias to *bias when they are given, and
// to row c of the swizzled LDS tile sA (and sB[c]) when those are given.
template <bool BF16, int M>
__device__ __forceinline__ void upd_final(int c, int lane, int64_t n, const double (*red)[kD],
                                          float *sx, float *cp, void *mrow, float *bias,
                                          u32x4 *sA = nullptr, float *sB = nullptr) {
    float mu[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int j = lane + 64 * k;
        if (n > 0) {
            const double ssum = ((red[0][j] + red[1][j]) + red[2][j]) + red[3][j];
            mu[k] = (float)(ssum / (double)n);
        } else {
            mu[k] = cp[j];
        }
        cp[j] = mu[k];
    }
    // channel j of row c in the swizzled tile: chunk j / 8, element j % 8
    auto put = [&](int j, uint16_t bits, float y) {
        if (BF16) {
            if (mrow) ((uint16_t *)mrow)[j] = bits;
            if (sA) ((uint16_t *)(sA + c * 16 + ((j >> 3) ^ (c & 15))))[j & 7] = bits;
        } else if (mrow) {
            ((float *)mrow)[j] = y;
        }
    };
    if (M != kCosine) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            float y = mu[k];
            uint16_t bits = 0;
            if (BF16) {
                bits = (uint16_t)f32_to_bf16_rne(mu[k]);
                y = bf16_to_f32(bits);
            }
            put(lane + 64 * k, bits, y);
            sx[lane + 64 * k] = y;
        }
        if (M == kL2) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            double ss = 0.0;
#pragma unroll 4
            for (int j4 = 0; j4 < kD / 4; ++j4) {
                const f32x4 x = *(const f32x4 *)(sx + 4 * j4);
                ss = __fma_rn((double)x[0], (double)x[0], ss);
                ss = __fma_rn((double)x[1], (double)x[1], ss);
                ss = __fma_rn((double)x[2], (double)x[2], ss);
                ss = __fma_rn((double)x[3], (double)x[3], ss);
            }
            if (lane == 0) {
                if (bias) *bias = (float)(-0.5 * ss);
                if (sB) sB[c] = (float)(-0.5 * ss);
            }
        }
        return;
    }
    // the row through LDS (one wave: its LDS accesses stay in order), then
    // every lane runs the chain on broadcast reads
    sx[lane] = mu[0];
    sx[lane + 64] = mu[1];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    double ss = 0.0;
#pragma unroll 4
    for (int j4 = 0; j4 < kD / 4; ++j4) {
        const f32x4 x = *(const f32x4 *)(sx + 4 * j4);
        ss = __fma_rn((double)x[0], (double)x[0], ss);
        ss = __fma_rn((double)x[1], (double)x[1], ss);
        ss = __fma_rn((double)x[2], (double)x[2], ss);
        ss = __fma_rn((double)x[3], (double)x[3], ss);
    }
    const double nrm = sqrt(ss);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const float y = (ss > 0.0) ? (float)((double)mu[k] / nrm) : 0.f;
        put(lane + 64 * k, BF16 ? (uint16_t)f32_to_bf16_rne(y) : (uint16_t)0, y);
    }
}

template <bool BF16, int M>
__global__ __launch_bounds__(256) void k_update(
    const void *__restrict__ K, int64_t head_stride, int64_t L, int64_t token_base,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ tokens, int c_base,
    int c_cap, int64_t t_cap, float *__restrict__ cent, void *__restrict__ mt,
    float *__restrict__ mb, int Cpad) {
    __shared__ double red[4][kD];
    __shared__ __align__(16) float sx[kD];
    const int c = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
    const int64_t n = upd_partial<BF16>(K, head_stride, L, token_base,
                                        offsets + (int64_t)h * (c_cap + 1) + c_base + c,
                                        tokens + (int64_t)h * t_cap, t_cap, h, tid, red);
    __syncthreads();
    if ((tid >> 6) == 0) {
        const int64_t mr = ((int64_t)h * Cpad + c) * kD;
        upd_final<BF16, M>(c, tid & 63, n, red, sx, cent + ((int64_t)h * c_cap + c_base + c) * kD,
                           BF16 ? (void *)((uint16_t *)mt + mr) : (void *)((float *)mt + mr),
                           mb + (int64_t)h * Cpad + c);
    }
}

template <int M>
static void launch_update_m(const ClusterPlan &p, const int32_t *offsets, const int32_t *tokens,
                            float *cent, hipStream_t s) {
    dim3 grid(p.C, p.H);
    if (p.dtype == 1)
        hipLaunchKernelGGL((k_update<true, M>), grid, dim3(256), 0, s, p.ku, p.ku_stride,
                           p.ku_rows, p.ku_base, offsets, tokens, p.c_base, p.c_cap, p.t_cap,
                           cent, p.mt, p.mb, p.Cpad);
    else
        hipLaunchKernelGGL((k_update<false, M>), grid, dim3(256), 0, s, p.ku, p.ku_stride,
                           p.ku_rows, p.ku_base, offsets, tokens, p.c_base, p.c_cap, p.t_cap,
                           cent, p.mt, p.mb, p.Cpad);
}

hipError_t launch_update(const ClusterPlan &p, const int32_t *offsets, const int32_t *tokens,
                         float *cent, hipStream_t s) {
    if (p.metric == kCosine)
        launch_update_m<kCosine>(p, offsets, tokens, cent, s);
    else if (p.metric == kInnerProduct)
        launch_update_m<kInnerProduct>(p, offsets, tokens, cent, s);
    else
        launch_update_m<kL2>(p, offsets, tokens, cent, s);
    return hipGetLastError();
}

// --------------------------------------------------------------------------
// Small windows (decode-time increments: 320 rows into 4 clusters) in one
// launch: one 1024-thread workgroup per head runs the whole K-means, with
// workgroup barriers where the general path has kernel boundaries. Every
// step is the general path's device code with the same thread-to-data
// mapping, so the results are bitwise those of the general path:
//  * the assignment and the update read the keys where the general ones do
//    (ka, ku), or, for windows of at most kSmallLdsRows rows, from an LDS
//    copy made once per call (the same values in the same order);
//  * initial centroids: the chain of block_unit_row / block_store_row, eight
//    128-thread groups at a time; centroids stay in LDS and the rows the
//    assignment reads go straight into its LDS tile;
//  * assignment: wave w takes tokens 64 w .. 64 w + 63 against the one
//    16-cluster M tile (as_load_b, as_beta, as_mfma and the general kernel's
//    argmax: the same comparisons in the same order);
//  * CSR: the stable counting sort (ballot ranks inside a wave, wave counts,
//    prefix over clusters), tokens in ascending order inside a cluster;
//  * update: four 256-thread groups run k_update's two halves for clusters
//    g, g + 4, ..., reading the CSR from LDS copies.
// Global memory gets only the results (the last iteration's labels and CSR,
// the final centroids): a barrier after a global store waits for it.
// Windows up to kSmallRows rows and kSmallC clusters, bf16 keys.

// Windows of at most kSmallLdsRows rows keep their key rows in LDS for the
// whole call (96 KB): row r's 16-byte chunk q at srow[16 r + (q ^ (r & 15))],
// so the 16 rows a wave reads at one chunk position fall in distinct banks.
constexpr int kSmallLdsRows = 384;

// as_load_b from those LDS rows
__device__ __forceinline__ void as_lds_b(const u32x4 *srow, int64_t Lp, int64_t tok0, int col,
                                         int kq, bf16x8 (&b)[4][4]) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const int64_t row = tok0 + 16 * t + col;
        const int rr = (int)(row < Lp ? row : Lp - 1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
            b[t][s] = __builtin_bit_cast(bf16x8, srow[rr * 16 + ((4 * s + kq) ^ (rr & 15))]);
    }
}

// upd_partial (bf16) with the rows from those LDS rows: the same rows added in
// the same order; token t is window row t - row0
__device__ __forceinline__ int64_t upd_partial_lds(const u32x4 *srow, int64_t Lp, int64_t row0,
                                                   const int32_t *off, const int32_t *tok,
                                                   int64_t t_cap, int ltid, double (*red)[kD]) {
    const int lane = ltid & 63, wave = ltid >> 6;
    const int slot = ltid >> 4, q = ltid & 15;
    int64_t beg, end;
    upd_range(off, t_cap, beg, end);
    double acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.0;
    for (int64_t r0 = beg + slot; r0 < end; r0 += 16 * kUpdNB) {
        int32_t tk[kUpdNB];
        upd_tokens(tok, r0, beg, end, tk);
        // every chunk of the batch read before the first is added (clamped
        // rows, masked values), as upd_partial keeps its loads in flight
        bool ok[kUpdNB];
        u32x4 w[kUpdNB];
#pragma unroll
        for (int k = 0; k < kUpdNB; ++k) {
            int64_t i = (int64_t)tk[k] - row0;
            ok[k] = r0 + 16 * k < end && i >= 0 && i < Lp;
            i = ok[k] ? i : 0;
            w[k] = srow[i * 16 + (q ^ (i & 15))];
        }
#pragma unroll
        for (int k = 0; k < kUpdNB; ++k) {
            if (!ok[k]) continue;
            float f[8];
            unpack8(w[k], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] += (double)f[e];
        }
    }
    upd_reduce(acc, lane, wave, red);
    return end - beg;
}

template <int M, bool LR>
__global__ __launch_bounds__(kSmallThreads) void k_cluster_small(
    const uint16_t *__restrict__ K, int64_t head_stride, int64_t L, int n_sink, int64_t Lp,
    int C, int iters, int64_t token_base, float *__restrict__ cent, int c_base, int c_cap,
    int32_t *__restrict__ assign, int32_t *__restrict__ offsets, int32_t *__restrict__ tokens,
    int64_t t_base, int64_t t_cap, const uint16_t *__restrict__ ka, int64_t ka_stride,
    const uint16_t *__restrict__ ku, int64_t ku_stride, int64_t ku_rows, int64_t ku_base) {
    constexpr bool BIAS = M == kL2;
    __shared__ u32x4 sA[16 * 16];
    __shared__ __align__(16) float sB[16];
    __shared__ int wcnt[16][kSmallC];
    __shared__ double red[4][4][kD];
    __shared__ __align__(16) float sx[8][kD];
    __shared__ double snrm[8];
    __shared__ float scent[kSmallC][kD];
    __shared__ int32_t stok[kSmallRows];
    __shared__ int32_t soff[kSmallC + 1];
    __shared__ u32x4 srow[LR ? kSmallLdsRows * 16 : 1];
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int32_t *as = assign + (int64_t)h * L;

    for (int i = tid; i < n_sink; i += kSmallThreads) as[i] = -1;   // sinks
    // initial centroids mu_c = row n_sink + s c, s = floor(Lp / C), eight at
    // a time (group g of 128 threads, channel j), as in k_init_centroids: the
    // centroid into LDS, the row the assignment reads into the LDS tile
    {
        const int g = tid >> 7, j = tid & 127;
        auto put = [&](int c, uint16_t bits) {
            ((uint16_t *)(sA + c * 16 + ((j >> 3) ^ (c & 15))))[j & 7] = bits;
        };
        for (int c0 = 0; c0 < C; c0 += 8) {
            const int c = c0 + g;
            const bool act = c < C;
            float x = 0.f;
            if (act) {
                const int64_t row = n_sink + (Lp / C) * (int64_t)c;
                x = bf16_to_f32(K[h * head_stride + row * kD + j]);
                scent[c][j] = x;
                if (M == kCosine) {
                    sx[g][j] = x;
                } else {
                    const uint32_t b = f32_to_bf16_rne(x);
                    put(c, (uint16_t)b);
                    sx[g][j] = bf16_to_f32((uint16_t)b);
                }
            }
            __syncthreads();
            if (act && j == 0 && (M == kCosine || M == kL2)) {
                double ss = 0.0;
                for (int k = 0; k < kD; ++k) ss = __fma_rn((double)sx[g][k], (double)sx[g][k], ss);
                if (M == kCosine)
                    snrm[g] = sqrt(ss);
                else
                    sB[c] = (float)(-0.5 * ss);
            }
            __syncthreads();
            if (M == kCosine && act)
                put(c, snrm[g] > 0.0 ? (uint16_t)f32_to_bf16_rne((float)((double)x / snrm[g]))
                                     : (uint16_t)0);
        }
    }
    __syncthreads();
    // LR (a window of at most kSmallLdsRows rows): its key rows into LDS once
    if constexpr (LR) {
        const u32x4 *src = (const u32x4 *)(ka + (int64_t)h * ka_stride);
        constexpr int PER = kSmallLdsRows * 16 / kSmallThreads;   // chunks per thread
        u32x4 v[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int e = tid + kSmallThreads * k;
            v[k] = src[e < Lp * 16 ? e : 0];
        }
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int e = tid + kSmallThreads * k, r = e >> 4;
            if (e < Lp * 16) srow[r * 16 + ((e & 15) ^ (r & 15))] = v[k];
        }
        __syncthreads();
    }

    const int col = lane & 15, kq = lane >> 4;
    const int64_t i = tid;                      // this thread's token
    const bool valid = i < Lp;
    int nbits = 1;
    while ((1 << nbits) < C) ++nbits;
    for (int it = 0; it < iters; ++it) {
        const bool last = it == iters - 1;       // only its labels and CSR are kept
        // assignment: wave w's 64 tokens against the one M tile
        {
            bf16x8 b[4][4], afr[4];
            // the rows are read again in every iteration: kept in registers
            // across the CSR and the update they would spill
            const uint16_t *kh = ka + (int64_t)h * ka_stride;
            asm volatile("" : "+s"(kh));
            // a wave whose 64 tokens all lie past the window loads nothing
            // (its labels are not kept): 11 of the 16 waves for a 320-row
            // window, whose clamped loads would triple the CU's row traffic
            if (wave * 64 < Lp) {
                if constexpr (LR)
                    as_lds_b(srow, Lp, (int64_t)wave * 64, col, kq, b);
                else
                    as_load_b((const u32x4 *)kh, Lp, (int64_t)wave * 64, col, kq, b);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int s2 = 0; s2 < 4; ++s2) b[t][s2] = bf16x8{};
            }
            float beta[4] = {0.f, 0.f, 0.f, 0.f};
            if (M == kCosine) as_beta(b, beta);
            as_lds_a(sA, 0, col, kq, afr);
            f32x4 acc[4];
            as_mfma<M == kCosine>(afr, b, beta, acc);
            int res[4];
            if (M == kCosine) {
                float gb[4] = {0.f, 0.f, 0.f, 0.f}, bv[4] = {0.f, 0.f, 0.f, 0.f};
                uint32_t bk[4] = {kAsKey, kAsKey, kAsKey, kAsKey};
                as_cos_tile<true>(acc, 0, 4 * kq, C, gb);
                as_cos_close(gb, 0, bv, bk);
#pragma unroll
                for (int u = 0; u < 4; ++u) res[u] = as_merge(bv[u], as_cos_id(bk[u], kq));
            } else {
                float bv[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
                int bc[4] = {0x7fffffff, 0x7fffffff, 0x7fffffff, 0x7fffffff};
                as_exact_tile<true, BIAS>(acc, sB, 0, kq, 4 * kq, C, bv, bc);
#pragma unroll
                for (int u = 0; u < 4; ++u) res[u] = as_merge(bv[u], bc[u]);
            }
            int a = (kq == 0) ? res[0] : (kq == 1) ? res[1] : (kq == 2) ? res[2] : res[3];
            if (last && valid) as[n_sink + i] = a;
            // CSR: rank among equal labels in the wave, then wave counts
            a = a < 0 ? 0 : (a >= C ? C - 1 : a);
            for (int e = tid; e < 16 * kSmallC; e += kSmallThreads) (&wcnt[0][0])[e] = 0;
            __syncthreads();
            uint64_t eq = __ballot(valid);
            for (int bt = 0; bt < nbits; ++bt) {
                const int bit = (a >> bt) & 1;
                const uint64_t bb = __ballot(bit);
                eq &= bit ? bb : ~bb;
            }
            const int rk = __popcll(eq & __lanemask_lt());
            if (valid && rk == 0) wcnt[wave][a] = __popcll(eq);
            __syncthreads();
            // the first wave turns the wave counts into the cluster offsets
            // (lane c: the size of cluster c, then an exclusive scan over the
            // lanes); the CSR offsets in LDS for the update, relative to the
            // window's first token slot, in global memory after the last
            // assignment
            if (wave == 0) {
                int sz = 0;
                if (lane < C)
#pragma unroll
                    for (int w = 0; w < 16; ++w) sz += wcnt[w][lane];
                const int ex = wave_incl_scan(sz) - sz;
                if (lane <= C) {
                    soff[lane] = ex;
                    if (last)
                        offsets[(int64_t)h * (c_cap + 1) + c_base + lane] = (int32_t)(t_base + ex);
                }
            }
            int base = 0;
#pragma unroll
            for (int w = 0; w < 16; ++w) base += w < wave ? wcnt[w][a] : 0;
            __syncthreads();
            if (valid) {
                const int pos = soff[a] + base + rk;
                if (pos >= 0 && pos < Lp) {
                    const int32_t t = (int32_t)(token_base + n_sink + i);
                    stok[pos] = t;
                    if (last) tokens[(int64_t)h * t_cap + t_base + pos] = t;
                }
            }
            __syncthreads();
        }
        // update: four groups of 256 threads, clusters g, g + 4, ...; the new
        // centroids stay in LDS, their assignment rows go to the LDS tile
        {
            const int g = tid >> 8, ltid = tid & 255;
            for (int c0 = 0; c0 < C; c0 += 4) {
                const int c = c0 + g;
                int64_t n = 0;
                if (c < C) {
                    if constexpr (LR)
                        n = upd_partial_lds(srow, Lp, token_base + n_sink, soff + c, stok, Lp,
                                            ltid, red[g]);
                    else
                        n = upd_partial<true>(ku, ku_stride, ku_rows, ku_base, soff + c, stok,
                                              Lp, h, ltid, red[g]);
                }
                __syncthreads();
                // wave g of group g finishes its cluster: waves 0, 5, 10 and
                // 15, one on each SIMD, so the four fp64 chains run side by side
                if (c < C && (ltid >> 6) == g)
                    upd_final<true, M>(c, lane, n, red[g], sx[g], scent[c], nullptr, nullptr, sA,
                                       BIAS ? sB : nullptr);
                __syncthreads();
            }
        }
    }
    // the final centroids
    for (int e = tid; e < C * kD; e += kSmallThreads)
        cent[((int64_t)h * c_cap + c_base + e / kD) * kD + e % kD] = scent[e / kD][e % kD];
}

template <int M, bool LR>
static void launch_small_m(const ClusterPlan &p, const void *K, float *cent, int32_t *assign,
                           int32_t *offsets, int32_t *tokens, hipStream_t s) {
    hipLaunchKernelGGL((k_cluster_small<M, LR>), dim3(p.H), dim3(kSmallThreads), 0, s,
                       (const uint16_t *)K, p.k_head_stride, p.L, p.n_sink, p.Lp, p.C, p.iters,
                       p.token_base, cent, p.c_base, p.c_cap, assign, offsets, tokens, p.t_base,
                       p.t_cap, (const uint16_t *)p.ka, p.ka_stride, (const uint16_t *)p.ku,
                       p.ku_stride, p.ku_rows, p.ku_base);
}

template <int M>
static void launch_small_lr(const ClusterPlan &p, const void *K, float *cent, int32_t *assign,
                            int32_t *offsets, int32_t *tokens, hipStream_t s) {
    if (p.Lp <= kSmallLdsRows)
        launch_small_m<M, true>(p, K, cent, assign, offsets, tokens, s);
    else
        launch_small_m<M, false>(p, K, cent, assign, offsets, tokens, s);
}

hipError_t launch_cluster_small(const ClusterPlan &p, const void *K, float *cent,
                                int32_t *assign, int32_t *offsets, int32_t *tokens,
                                hipStream_t s) {
    if (p.metric == kCosine)
        launch_small_lr<kCosine>(p, K, cent, assign, offsets, tokens, s);
    else if (p.metric == kInnerProduct)
        launch_small_lr<kInnerProduct>(p, K, cent, assign, offsets, tokens, s);
    else
        launch_small_lr<kL2>(p, K, cent, assign, offsets, tokens, s);
    return hipGetLastError();
}

}  // namespace ckv
