// cache.hip -- cluster-granular GPU cache of selected KV rows, on gfx950.
//
// Method: "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
// Recallable Compression", section 缓存选中Token的KV (the GPU keeps the KV of
// the tokens selected in the last R decode steps with their cluster labels;
// only clusters not in the cache are loaded from CPU memory) and the system
// overview of Fig. 5 (KV offloaded to CPU memory after prefill).
//
// The cache holds exactly the rows selected in the last R steps. Since a
// selection takes every admitted cluster's rows as a prefix of its CSR
// segment, that union is, per cluster c, the prefix of length N_c = the
// largest count c had in those steps; the state is a ring of per-cluster
// counts of the last R steps, and the layout is a function of it: sink rows
// 0 .. n_sink-1 in slots 0 .. n_sink-1, then the clusters in ascending id,
// cluster c's N_c rows in CSR order. The rows live in two buffers: step s
// writes buffer s & 1 from buffer (s - 1) & 1 (hits) and from the KV in
// host memory (misses), so nothing moves under a reader.
//
// Two launches per step:
//  * k_cache_plan, one 1024-thread workgroup per head: the step's row count
//    of every cluster (from the labels of its idx entries), the ring update,
//    old and new layouts (one paired block scan), the slot of every selected entry
//    (idx_cache), where every new slot comes from, its token id, and the
//    hit/load statistics;
//  * k_cache_fill: a gather of the new buffer, 16-byte chunks, every row's
//    K and V loads in flight together (the host rows cross the host link, so
//    many loads must be outstanding).
#include "cache_dev.h"

namespace ckv {

constexpr int kCacheThreads = 1024;
constexpr int kCacheEPT = kMaxCacheB / kCacheThreads;   // idx entries per thread
constexpr int kFillRows = 64;            // rows per fill workgroup

// label of selected token `tok` (cluster id, or -1 for a token outside the
// clustered rows: sinks, pending rows, -1 entries)
__device__ __forceinline__ int cache_label(int32_t tok, const int32_t *as, int64_t L,
                                           int64_t token_base, int C) {
    const int64_t row = (int64_t)tok - token_base;
    if (tok < 0 || row < 0 || row >= L) return -1;
    const int lab = as[row];
    return (lab >= 0 && lab < C) ? lab : -1;
}

// Exclusive scans of a[0 .. C) and b[0 .. C) together (C <= 2 * blockDim),
// each plus `base`, into oa and ob; one pair of barriers for both. Returns
// the total of b. wsum: 2 * 16 ints of LDS. Every thread calls it.
__device__ int cache_scan_pair(const int *a, const int *b, int *oa, int *ob, int C, int base,
                               int *wsum) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int c0 = 2 * threadIdx.x, c1 = c0 + 1;
    const int a0 = c0 < C ? a[c0] : 0, a1 = c1 < C ? a[c1] : 0;
    const int b0 = c0 < C ? b[c0] : 0, b1 = c1 < C ? b[c1] : 0;
    const int xa = wave_incl_scan(a0 + a1), xb = wave_incl_scan(b0 + b1);
    if (lane == 63) {
        wsum[wave] = xa;
        wsum[16 + wave] = xb;
    }
    __syncthreads();
    int pa = 0, pb = 0, tb = 0;
    for (int w = 0; w < nw; ++w) {
        const int ta = wsum[w], t2 = wsum[16 + w];
        pa += w < wave ? ta : 0;
        pb += w < wave ? t2 : 0;
        tb += t2;
    }
    const int ea = base + pa + xa - (a0 + a1), eb = base + pb + xb - (b0 + b1);
    if (c0 < C) {
        oa[c0] = ea;
        ob[c0] = eb;
    }
    if (c1 < C) {
        oa[c1] = ea + a0;
        ob[c1] = eb + b0;
    }
    __syncthreads();
    return tb;
}

__global__ __launch_bounds__(kCacheThreads) void k_cache_plan(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ n_sel, int B,
    const int32_t *__restrict__ assign, int64_t L, int64_t token_base,
    const int32_t *__restrict__ offsets, int c_cap, const int32_t *__restrict__ tokens,
    int64_t t_cap, int C, int n_sink, int R, int now, int first, int32_t *__restrict__ ring,
    int rows, int32_t *__restrict__ cache_tok, int32_t *__restrict__ idx_cache,
    int32_t *__restrict__ stats, int32_t *__restrict__ src, int32_t *__restrict__ tot) {
    __shared__ int sn[kMaxC], sm[kMaxC], sN[kMaxC], sfirst[kMaxC], sold[kMaxC], snew[kMaxC];
    __shared__ int soff[kMaxC];
    __shared__ int wsum[32];
    __shared__ int sstat[5];
    const int h = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
    constexpr int T = kCacheThreads;
    const int32_t *ix = idx + (int64_t)h * B;
    const int32_t *as = assign + (int64_t)h * L;
    const int32_t *off = offsets + (int64_t)h * (c_cap + 1);
    const int32_t *tk = tokens + (int64_t)h * t_cap;
    int32_t *ctok = cache_tok + (int64_t)h * rows;
    int32_t *srch = src + (int64_t)h * rows;
    int ns = n_sel[h];
    ns = ns < 0 ? 0 : (ns > B ? B : ns);

    // this thread's idx entries e = tid + T k: token and label, kept in
    // registers; the CSR offsets of every cluster into LDS meanwhile
    int32_t tok[kCacheEPT];
    int lab[kCacheEPT];
#pragma unroll
    for (int k = 0; k < kCacheEPT; ++k) {
        const int e = tid + T * k;
        tok[k] = e < ns ? ix[e] : -1;
    }
    for (int c = tid; c < C; c += T) {
        soff[c] = off[c];
        sn[c] = 0;
        sfirst[c] = INT32_MAX;
    }
    if (tid < 5) sstat[tid] = 0;
#pragma unroll
    for (int k = 0; k < kCacheEPT; ++k) lab[k] = cache_label(tok[k], as, L, token_base, C);
    __syncthreads();
    // this step's rows per cluster and the first idx entry of each cluster
#pragma unroll
    for (int k = 0; k < kCacheEPT; ++k)
        if (lab[k] >= 0) {
            atomicAdd(&sn[lab[k]], 1);
            atomicMin(&sfirst[lab[k]], tid + T * k);
        }
    __syncthreads();
    // cached rows before (m) and after (N) this step; the ring slot of the
    // step R ago becomes this step's
    int hit = 0, load = 0, chit = 0, csel = 0;
    for (int c = tid; c < C; c += T) {
        int32_t *rg = ring + ((int64_t)h * c_cap + c) * R;
        int m = 0, keep = 0;
        for (int k = 0; k < R; ++k) {
            const int v = rg[k];
            m = v > m ? v : m;
            if (k != now) keep = v > keep ? v : keep;
        }
        const int n = sn[c];
        rg[now] = n;
        sm[c] = m;
        sN[c] = n > keep ? n : keep;
        hit += n < m ? n : m;
        load += n > m ? n - m : 0;
        chit += (n > 0 && m >= n);
        csel += (n > 0);
    }
    __syncthreads();
    const int new_total = cache_scan_pair(sm, sN, sold, snew, C, n_sink, wsum);
    const int n_slots = n_sink + new_total < rows ? n_sink + new_total : rows;

    // the slot of every selected entry (-1: not in the cache)
    int unplaced = 0;
#pragma unroll
    for (int k = 0; k < kCacheEPT; ++k) {
        const int e = tid + T * k;
        if (e >= B) continue;
        int v = -1;
        if (e < ns) {
            if (lab[k] >= 0)
                v = snew[lab[k]] + (e - sfirst[lab[k]]);
            else if (tok[k] >= 0 && tok[k] < n_sink)
                v = tok[k];
            if (v >= n_slots) v = -1;
            unplaced += (v < 0);
        }
        idx_cache[(int64_t)h * B + e] = v;
    }
    // where every slot of the new buffer comes from: an old slot (>= 0) or a
    // host row (-1 - token id); and the token it holds
    for (int s = tid; s < rows; s += T) {
        int32_t t = -1, from = INT32_MIN;
        if (s < n_slots) {
            if (s < n_sink) {
                t = s;
                from = first ? -1 - s : s;
            } else {
                // last cluster whose first new slot is <= s (it is not empty)
                int lo = 0, hi = C - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if (snew[mid] <= s) lo = mid; else hi = mid - 1;
                }
                const int r = s - snew[lo];
                int64_t p = (int64_t)soff[lo] + r;
                p = p < 0 ? 0 : (p >= t_cap ? t_cap - 1 : p);
                t = tk[p];
                from = r < sm[lo] ? sold[lo] + r : -1 - t;
            }
        }
        ctok[s] = t;
        srch[s] = from;
    }
    // statistics: wave sums, then one LDS add per wave
    const int v0 = wave_sum(hit), v1 = wave_sum(load), v2 = wave_sum(chit),
              v3 = wave_sum(csel), v4 = wave_sum(unplaced);
    if (lane == 0) {
        atomicAdd(&sstat[0], v0);
        atomicAdd(&sstat[1], v1);
        atomicAdd(&sstat[2], v2);
        atomicAdd(&sstat[3], v3);
        atomicAdd(&sstat[4], v4);
    }
    __syncthreads();
    if (tid < 5) stats[(int64_t)h * 5 + tid] = sstat[tid];
    if (tid == 0) tot[h] = n_slots;
}

// New buffer rows [64 b, 64 b + 64) of head h from the old buffer or the
// KV in host memory. CH 16-byte chunks per row; a thread copies one chunk of
// K and of V for every row group, all loads issued before the stores.
template <int ES>
__global__ __launch_bounds__(256) void k_cache_fill(
    const int32_t *__restrict__ src, const int32_t *__restrict__ tot, int rows,
    const char *__restrict__ Kh, const char *__restrict__ Vh, int64_t kv_head_stride,
    int64_t kv_rows, const char *__restrict__ oldK, const char *__restrict__ oldV,
    char *__restrict__ newK, char *__restrict__ newV) {
    constexpr int RB = kD * ES;              // bytes per row
    constexpr int CH = RB / 16;              // chunks per row
    constexpr int RPI = 256 / CH;            // rows per pass
    constexpr int NP = kFillRows / RPI;      // passes
    const int h = blockIdx.y, tid = threadIdx.x, q = tid % CH;
    const int n = tot[h] < rows ? tot[h] : rows;
    const int64_t hb = (int64_t)h * rows;    // first row of this head in a buffer
    u32x4 k[NP], v[NP];
    bool ok[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        const int s = blockIdx.x * kFillRows + p * RPI + tid / CH;
        ok[p] = s < n;
        const int f = ok[p] ? src[hb + s] : 0;
        const char *pk, *pv;
        if (f >= 0) {
            const int64_t o = (hb + (f < rows ? f : 0)) * RB;
            pk = oldK + o;
            pv = oldV + o;
        } else {
            int64_t t = -1 - (int64_t)f;
            if (t >= kv_rows) {
                t = 0;
                ok[p] = false;
            }
            const int64_t o = ((int64_t)h * kv_head_stride + t * kD) * ES;
            pk = Kh + o;
            pv = Vh + o;
        }
        k[p] = ((const u32x4 *)pk)[q];
        v[p] = ((const u32x4 *)pv)[q];
    }
#pragma unroll
    for (int p = 0; p < NP; ++p) {
        if (!ok[p]) continue;
        const int s = blockIdx.x * kFillRows + p * RPI + tid / CH;
        const int64_t o = (hb + s) * RB;
        ((u32x4 *)(newK + o))[q] = k[p];
        ((u32x4 *)(newV + o))[q] = v[p];
    }
}

hipError_t launch_cache_step(const CachePlan &p, int64_t step, const int32_t *idx,
                             const int32_t *n_sel, const int32_t *assign,
                             const int32_t *offsets, const int32_t *tokens, const void *Kh,
                             const void *Vh, int32_t *ring, void *cache_K, void *cache_V,
                             int32_t *cache_tok, int32_t *idx_cache, int32_t *stats,
                             hipStream_t s) {
    const int cur = (int)(step & 1), prev = cur ^ 1;
    const int64_t es = p.dtype == 1 ? 2 : 4;
    const int64_t buf = (int64_t)p.H * p.rows * kD * es;     // bytes per buffer
    hipLaunchKernelGGL(k_cache_plan, dim3(p.H), dim3(kCacheThreads), 0, s, idx, n_sel, p.B,
                       assign, p.L, p.token_base, offsets, p.c_cap, tokens, p.t_cap, p.C,
                       p.n_sink, p.R, (int)(step % p.R), step == 0 ? 1 : 0, ring, p.rows,
                       cache_tok + (int64_t)cur * p.H * p.rows, idx_cache, stats, p.src,
                       p.tot);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((p.rows + kFillRows - 1) / kFillRows), p.H);
    const char *oK = (const char *)cache_K + prev * buf, *oV = (const char *)cache_V + prev * buf;
    char *nK = (char *)cache_K + cur * buf, *nV = (char *)cache_V + cur * buf;
    if (p.dtype == 1)
        hipLaunchKernelGGL(k_cache_fill<2>, grid, dim3(256), 0, s, p.src, p.tot, p.rows,
                           (const char *)Kh, (const char *)Vh, p.kv_head_stride, p.kv_rows, oK,
                           oV, nK, nV);
    else
        hipLaunchKernelGGL(k_cache_fill<4>, grid, dim3(256), 0, s, p.src, p.tot, p.rows,
                           (const char *)Kh, (const char *)Vh, p.kv_head_stride, p.kv_rows, oK,
                           oV, nK, nV);
    return hipGetLastError();
}

}  // namespace ckv
