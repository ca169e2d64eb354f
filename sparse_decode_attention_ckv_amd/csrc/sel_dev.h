// sel_dev.h -- device side of the decode-time selection, shared by the
// selection kernels (select.hip) and the fused selection + attention kernel
// (decode.hip). Internal; include/ckv.h is the public ABI.
//
// Method: "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
// Recallable Compression", section 核心方法细节 / 语义聚类粒度的选择
// (cluster-granular selection: score q.mu_i, take the clusters in descending
// score order until the budget B is reached) and section 选择与索引机制
// (selection and indexing, Fig. 8: cluster sizes, prefix sums, where the
// budget falls, trim of the last cluster, token indices).
//
// A decode step's selection runs as two launches:
//  1. k_sel_score: s_c = q_g . mu_c for every cluster, 32 clusters per
//     workgroup (8 lanes each), in fp64 with the fixed association of the
//     definition (32 fma chains of 4 channels, pairwise tree r + r+16, +8,
//     +4, +2, +1), to a [H][C] fp64 workspace. Spreading the 512 B centroid
//     rows over many compute units is what makes this step fast: one CU per
//     head pulls them at well under 100 GB/s.
//  2. a cut + emission kernel with one 256-thread workgroup per 64 output
//     slots of a head. Every workgroup of the head reads the same scores
//     and offsets (a few KB) and finds the same cut on its own, so no
//     workgroup waits for another; then it emits only its 64 slots.
//     The sizes' total and the score range are reduced from the registers
//     the loads land in, before the first barrier.
//     The cut is the cluster at which the running size total, in rank order
//     (score descending, then id ascending), first reaches the budget. It is
//     found without sorting, by a weighted select: one histogram of the
//     sizes over CMAX equal-width score buckets between the smallest and the
//     largest score (a monotone map, so bucket order is rank order); when the
//     bucket that reaches the budget holds one cluster, that is the cut;
//     otherwise exact radix passes over the rank key (64-bit score key, then
//     the cluster id) of that bucket's clusters finish the job.
//     Tokens are emitted by cluster id: an id-order prefix sum of the tokens
//     each cluster gives marks where every cluster's tokens start, and a
//     64-lane max-scan over the marks of a slot window gives every slot its
//     cluster.
#pragma once

#include "ckv_dev.h"

namespace ckv {

constexpr int kScoreThreads = 256;
constexpr int kScoreLanes = 8;                                  // lanes per cluster
constexpr int kScoreChunk = kScoreThreads / kScoreLanes;        // clusters per workgroup
constexpr int kCutThreads = 256;
constexpr int kSelSlice = 64;                                   // output slots per workgroup
constexpr int kCntBits = 12;       // histogram entry: weight << 12 | count (count <= 2048)

// Order-preserving 64-bit image of a finite double, inverted so that a larger
// score gives a smaller key; -0 and +0 map to the same key.
__device__ __forceinline__ uint64_t rank_key(double s) {
    s = s + 0.0;
    uint64_t u = (uint64_t)__double_as_longlong(s);
    u = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
    return ~u;
}

// q_g = sum of the G query rows of KV head h, fp64 in row order; thread
// tid < kD handles channel tid (loads first, the sum later).
template <bool BF16>
__device__ __forceinline__ void sel_q_load(const void *q, int G, int h, int tid, float (&qv)[8]) {
#pragma unroll
    for (int g = 0; g < 8; ++g) {
        const int64_t qi = ((int64_t)h * G + (g < G ? g : G - 1)) * kD + tid;
        qv[g] = BF16 ? bf16_to_f32(((const uint16_t *)q)[qi]) : ((const float *)q)[qi];
    }
}
__device__ __forceinline__ double sel_q_sum(const float (&qv)[8], int G) {
    double a = 0.0;
#pragma unroll
    for (int g = 0; g < 8; ++g)
        if (g < G) a += (double)qv[g];
    return a;
}

// LDS of the cut + emission, sized for up to CMAX clusters.
template <int CMAX>
struct SelLds {
    double sc[CMAX];                  // scores
    int off[CMAX + 1];                // clamped offsets
    int w[CMAX];                      // sizes clamped to the budget
    int pre[CMAX];                    // a bucket's last cluster; later the
                                      // id-order exclusive prefix of taken tokens
    unsigned long long hist[CMAX];    // weight << kCntBits | count per bucket
    int mark[kSelSlice];              // cluster whose tokens start at a slot
    int wsa[4], wsb[4], wsc[4], wsd[4];   // one per scan: no barrier needed between
    double wmn[4], wmx[4];
    int s_bucket, s_rem, s_cut, s_cnt;
    unsigned long long s_kmin, s_kmax;
};

// Result of the selection for one slot window of one head.
struct SelSlot {
    int32_t val;      // idx entry of this lane's slot (-1 past the selection)
    int n_sel;        // valid entries of the head's idx row
};

// The bucket (of this thread's NBK consecutive buckets) where the running
// weight first reaches R, if it lies in this thread's range; writes the
// bucket, what is left of R at its start, and its cluster count.
template <int NBK>
__device__ __forceinline__ void sel_find_bucket(const unsigned long long (&hv)[NBK], int ex,
                                                int bsum, int R, int tid, int &s_bucket,
                                                int &s_rem, int &s_cnt) {
    if (ex < R && ex + bsum >= R) {
        int before = ex, b = NBK - 1;
        bool found = false;
#pragma unroll
        for (int k = 0; k < NBK; ++k) {
            const int wk = (int)(hv[k] >> kCntBits);
            if (!found && before + wk >= R) {
                b = k;
                found = true;
            } else if (!found) {
                before += wk;
            }
        }
        s_bucket = NBK * tid + b;
        s_rem = R - before;
        s_cnt = (int)(hv[b] & ((1u << kCntBits) - 1));
    }
}

// Cut + emission for head h and the slot window [64 s, 64 s + 64) of its idx
// row, 256 threads. scores: this head's C fp64 scores; offh: its C + 1
// offsets; tok: its csr token row. Every thread returns the result for slot
// 64 s + (tid & 63) (each wave the same window). LDS is S.
template <int CMAX>
__device__ __forceinline__ SelSlot sel_cut_emit(SelLds<CMAX> &S, const double *__restrict__ scores,
                                                int C, const int32_t *__restrict__ offh,
                                                const int32_t *__restrict__ tok, int64_t t_cap,
                                                int n_sink, int64_t pending_begin,
                                                int64_t n_pending, int B, int s) {
    constexpr int T = kCutThreads, NW = T / 64, PER = CMAX / T, NB = CMAX, NBK = NB / T;
    constexpr int BITS = CMAX == 512 ? 9 : 11;
    static_assert(NB == (1 << BITS), "buckets = 2^BITS");
    static_assert(CMAX <= (1 << kCntBits) / 2, "count field");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    // ---- loads: scores and offsets of the head, all in flight at once
    // (cluster c = tid + T k, coalesced); the weights (sizes clamped to the
    // budget, which moves no cut), their total and the score range are
    // reduced from these registers before the first barrier
    const int64_t head = (int64_t)n_sink + n_pending;
    const int64_t beff64 = (int64_t)B - head;
    const int beff = (int)(beff64 > 0 ? beff64 : 0);
    const double pinf = __longlong_as_double(0x7ff0000000000000ll);
    double smin = pinf, smax = -pinf;
    int loc = 0;
    {
        double v[PER];
        int64_t o0[PER], o1[PER];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int c = tid + k * T;
            v[k] = scores[c < C ? c : C - 1];
            o0[k] = offh[c < C ? c : C];
            o1[k] = offh[c + 1 < C ? c + 1 : C];
        }
        const int64_t oC = offh[C];
#pragma unroll
        for (int k = 0; k < PER; ++k) {
            const int c = tid + k * T;
            const int64_t a = o0[k] < 0 ? 0 : (o0[k] > t_cap ? t_cap : o0[k]);
            const int64_t b = o1[k] < 0 ? 0 : (o1[k] > t_cap ? t_cap : o1[k]);
            const int64_t n = b - a;
            const int w = c < C ? (int)(n <= 0 ? 0 : (n < beff ? n : beff)) : 0;
            loc += w;
            smin = c < C ? fmin(smin, v[k]) : smin;
            smax = c < C ? fmax(smax, v[k]) : smax;
            if (c < C) {
                S.sc[c] = v[k];
                S.off[c] = (int)a;
                S.w[c] = w;
            }
        }
        if (tid == 0) S.off[C] = (int)(oC < 0 ? 0 : (oC > t_cap ? t_cap : oC));
    }
    loc = wave_sum(loc);
    wave_minmax_f64(smin, smax);
    if (lane == 0) {
        S.wsa[wave] = loc;
        S.wmn[wave] = smin;
        S.wmx[wave] = smax;
    }
    // the first histogram and the slot marks start cleared
#pragma unroll
    for (int k = 0; k < NBK; ++k) S.hist[tid + k * T] = 0;
    if (tid < kSelSlice) S.mark[tid] = -1;
    if (tid == 0) {
        S.s_kmin = ~0ull;
        S.s_kmax = 0ull;
        S.s_bucket = -1;     // stays so only if no bucket reaches the budget,
        S.s_rem = 0;         // which consistent offsets never allow
        S.s_cut = -1;
        S.s_cnt = 0;
    }
    __syncthreads();
    int total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        total += S.wsa[w];
        smin = fmin(smin, S.wmn[w]);
        smax = fmax(smax, S.wmx[w]);
    }
    // this thread's clusters PER tid .. PER tid + PER - 1 (id order)
    int wv[PER];
    double sv[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int c = PER * tid + u;
        wv[u] = c < C ? S.w[c] : 0;
        sv[u] = c < C ? S.sc[c] : 0.0;
    }

    // ---- the cut: first cluster (rank order) where the weights reach beff
    int cut = -1, rem = 0;               // -1: no cut, every cluster gives all
    if (beff == 0) {
        cut = -2;                        // nothing is taken
    } else if (total > beff) {
        // score pass: bucket = floor((smax - s) (NB - 1) / (smax - smin)), a
        // non-increasing function of s, so lower buckets rank first
        const double range = smax - smin;
        double scale = range > 0.0 ? (double)(NB - 1) / range : 0.0;
        if (!(scale < pinf)) scale = 0.0;    // range infinite or too small
        int bk[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int c = PER * tid + u;
            bk[u] = -1;
            if (c < C) {
                const double x = (smax - sv[u]) * scale;
                const int b = x >= (double)(NB - 1) ? NB - 1 : (x > 0.0 ? (int)x : 0);
                bk[u] = b;
                atomicAdd(&S.hist[b], ((unsigned long long)wv[u] << kCntBits) | 1ull);
                S.pre[b] = c;            // the bucket's cluster when it has one
            }
        }
        __syncthreads();
        int R = beff;
        {
            unsigned long long hv[NBK];
            int bsum = 0;
#pragma unroll
            for (int k = 0; k < NBK; ++k) {
                hv[k] = S.hist[NBK * tid + k];
                bsum += (int)(hv[k] >> kCntBits);
            }
            int tot;
            const int ex = block_excl_scan_nw<NW>(bsum, S.wsb, tot);
            int bb = -1, rr = 0, cn = 0;
            sel_find_bucket<NBK>(hv, ex, bsum, R, tid, bb, rr, cn);
            if (bb >= 0) {
                S.s_bucket = bb;
                S.s_rem = rr;
                S.s_cut = cn == 1 ? S.pre[bb] : -1;
            }
        }
        __syncthreads();
        const int bsel = S.s_bucket;
        R = S.s_rem;
        cut = S.s_cut;
        if (cut < 0) {
            // several clusters share that bucket: exact radix passes over their
            // rank keys, from the highest bit where those keys differ, then
            // the cluster id
            bool cand[PER];
            uint64_t key[PER];
#pragma unroll
            for (int u = 0; u < PER; ++u) {
                cand[u] = bk[u] == bsel;
                key[u] = rank_key(sv[u]);
                if (cand[u]) {
                    atomicMin(&S.s_kmin, (unsigned long long)key[u]);
                    atomicMax(&S.s_kmax, (unsigned long long)key[u]);
                }
            }
            __syncthreads();
            const uint64_t kdiff = S.s_kmin ^ S.s_kmax;
            const int hb = kdiff ? 63 - __clzll((long long)kdiff) : -1;
            const int nkey = hb < 0 ? 0 : (hb + BITS) / BITS;   // key passes
            for (int pos = 0; pos <= nkey; ++pos) {
                const bool in_id = pos == nkey;
                int sh = hb - (BITS - 1) - BITS * pos;
                sh = sh < 0 ? 0 : sh;
#pragma unroll
                for (int k = 0; k < NBK; ++k) S.hist[tid + k * T] = 0;
                __syncthreads();
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    const int c = PER * tid + u;
                    if (cand[u]) {
                        const int d = in_id ? c : (int)((key[u] >> sh) & (NB - 1));
                        atomicAdd(&S.hist[d], ((unsigned long long)wv[u] << kCntBits) | 1ull);
                    }
                }
                __syncthreads();
                unsigned long long hv[NBK];
                int bsum = 0;
#pragma unroll
                for (int k = 0; k < NBK; ++k) {
                    hv[k] = S.hist[NBK * tid + k];
                    bsum += (int)(hv[k] >> kCntBits);
                }
                int tot;
                const int ex = block_excl_scan_nw<NW>(bsum, pos & 1 ? S.wsc : S.wsb, tot);
                int bb = -1, rr = 0, cn = 0;
                sel_find_bucket<NBK>(hv, ex, bsum, R, tid, bb, rr, cn);
                if (bb >= 0) {
                    S.s_bucket = bb;
                    S.s_rem = rr;
                    S.s_cnt = cn;
                }
                __syncthreads();
                const int bs = S.s_bucket;
                R = S.s_rem;
#pragma unroll
                for (int u = 0; u < PER; ++u) {
                    const int c = PER * tid + u;
                    if (cand[u]) {
                        const int d = in_id ? c : (int)((key[u] >> sh) & (NB - 1));
                        cand[u] = d == bs;
                    }
                }
                const bool done = S.s_cnt == 1;   // uniform
                __syncthreads();
                if (done) break;
            }
#pragma unroll
            for (int u = 0; u < PER; ++u)
                if (cand[u]) S.s_cut = PER * tid + u;
            __syncthreads();
            cut = S.s_cut;
        }
        rem = R;
    }

    // ---- tokens each cluster gives and their id-order prefix; marks where the
    // taken clusters start inside this workgroup's slot window
    const double cs = cut >= 0 ? S.sc[cut] : 0.0;
    int tk[PER];
    loc = 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int c = PER * tid + u;
        int t = 0;
        if (c < C) {
            if (cut == -1) {
                t = wv[u];
            } else if (cut >= 0) {
                if (sv[u] > cs || (sv[u] == cs && c < cut)) t = wv[u];
                else if (c == cut) t = rem;
            }
        }
        tk[u] = t;
        loc += t;
    }
    int ntake;
    int run = block_excl_scan_nw<NW>(loc, S.wsd, ntake);
    const int64_t p0 = (int64_t)s * kSelSlice - head;    // token slot of the window start
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int c = PER * tid + u;
        if (c < C) S.pre[c] = run;
        if (tk[u] > 0) {
            const int64_t e = run - p0;                  // window slot of the first token
            if (e >= 0 && e < kSelSlice) S.mark[e] = c;
            else if (e < 0 && run + tk[u] > p0) S.mark[0] = c;   // covers the window start
        }
        run += tk[u];
    }
    __syncthreads();

    // ---- this lane's slot: the cluster is the largest mark at or before it
    const int64_t e = (int64_t)s * kSelSlice + lane;
    const int64_t p = e - head;
    const int mx = wave_incl_max(S.mark[lane]);
    SelSlot r;
    r.n_sel = (int)(head + ntake);
    r.val = -1;
    if (e < n_sink) {
        r.val = (int32_t)e;
    } else if (e < head) {
        r.val = (int32_t)(pending_begin + (e - n_sink));
    } else if (p < ntake && mx >= 0) {
        const int64_t src = (int64_t)S.off[mx] + (p - S.pre[mx]);
        if (src >= 0 && src < t_cap) r.val = tok[src];
    }
    return r;
}

}  // namespace ckv
