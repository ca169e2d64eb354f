// select.hip -- decode-time cluster-granular selection on gfx950.
//
// Method: "ClusterKV: Manipulating LLM KV Cache in Semantic Space for
// Recallable Compression", section 核心方法细节 / 语义聚类粒度的选择
// (cluster-granular selection: score q.mu_i, take the clusters in descending
// score order until the budget B is reached) and section 选择与索引机制
// (selection and indexing, Fig. 8: cluster sizes, prefix sums, where the
// budget falls, trim of the last cluster, token indices).
//
// Up to 512 clusters: one kernel per decode step, one 512-thread workgroup
// per KV head, no cross-workgroup handoff. Above 512 clusters the scores of
// step 1 come from a wider scoring-only kernel (several workgroups per head)
// through the workspace, and the same kernel then does steps 2 and 3.
//  1. score every cluster, s_c = q_g . mu_c in fp64 with the fixed
//     association of the definition (32 fma chains of 4 channels, pairwise
//     tree r + r+16, +8, +4, +2, +1). Four lanes share a cluster: lane l holds
//     the runs r = l (mod 4), so the first three tree levels stay inside the
//     lane and only the last two cross lanes. Every centroid load of a batch
//     is in flight at once. The total size and the score range are gathered
//     on the way.
//  2. the clusters admitted "in descending score until the budget" are found
//     without sorting, by a weighted select over the rank order (score
//     descending, then id ascending): the cut is the cluster at which the
//     running size total first reaches the budget. A first pass histograms
//     the sizes over 2048 equal-width score buckets between the smallest and
//     the largest score (a monotone map, so bucket order is rank order); when
//     the bucket that reaches the budget holds one cluster, that is the cut.
//     Otherwise exact radix passes over the 75-bit rank key (64-bit score
//     key, then the cluster id) of that bucket's clusters finish the job.
//  3. every cluster ranked before the cut gives all its tokens, the cut
//     cluster gives what still fits; tokens are emitted by cluster id: a
//     prefix sum in id order gives each taken cluster its first output slot,
//     marked in LDS, and a max-scan over the slots tells every slot its
//     cluster (a binary search over the prefix when more than 2048 tokens
//     are taken).
#include "ckv_dev.h"

namespace ckv {

constexpr int kSelThreads = 512;
constexpr int kSelLanes = 4;                        // lanes per cluster while scoring
constexpr int kSelPass = kSelThreads / kSelLanes;   // clusters per scoring pass
constexpr int kSelInFlight = 4;                     // passes whose loads fly together
constexpr int kSelPer = kMaxC / kSelThreads;        // clusters per thread later (4)
constexpr int kSelChunk = 2 * kSelPass;             // clusters per scoring-only workgroup
constexpr int kSelMarks = 2048;                     // token slots found by a max-scan
constexpr int kSelSlots = kSelMarks / kSelThreads;  // ... per thread (4)

// Buckets of the score pass and of each exact pass (11-bit digits; the last
// exact pass is the id itself, ids < kMaxC = 2^11).
constexpr int kRadixBuckets = 2048;
static_assert(kMaxC <= kRadixBuckets, "the id digit must fit one pass");
constexpr int kCntBits = 12;            // histogram entry: size << 12 | count

// Order-preserving 64-bit image of a finite double, inverted so that a larger
// score gives a smaller key; -0 and +0 map to the same key.
__device__ __forceinline__ uint64_t rank_key(double s) {
    s = s + 0.0;
    uint64_t u = (uint64_t)__double_as_longlong(s);
    u = (u >> 63) ? ~u : (u | 0x8000000000000000ull);
    return ~u;
}

// q_g = sum of the G query rows of KV head h, fp64 in row order; thread
// tid < kD handles channel tid (its loads first, the sum later).
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

// Centroid chunks of the NP scoring passes from cluster p0: pass pi holds
// cluster p0 + pi * kSelPass + slot (clamped to < c_hi), lane lam its
// channels 4 (lam + 4i) .. +3.
template <int NP>
__device__ __forceinline__ void sel_load_cent(const float *ch, int p0, int c_hi, int lam, int slot,
                                              u32x4 (&w)[NP][8]) {
#pragma unroll
    for (int pi = 0; pi < NP; ++pi) {
        const int c = p0 + pi * kSelPass + slot;
        const float *row = ch + (int64_t)(c < c_hi ? c : c_hi - 1) * kD;
#pragma unroll
        for (int i = 0; i < 8; ++i) w[pi][i] = *(const u32x4 *)(row + 4 * (lam + 4 * i));
    }
}

// s_c = q_g . mu_c for the clusters of those passes (c < c_hi), stored to
// out[c]: 32 fma runs of 4 channels (lane lam holds runs lam + 4i), then the
// pairwise tree r + r+16, +8, +4 inside the lane and +2, +1 across lanes.
template <int NP>
__device__ __forceinline__ void sel_score(const u32x4 (&w)[NP][8], const double *qg, int p0,
                                          int c_hi, int lam, int slot, double *out,
                                          double (&vals)[NP]) {
#pragma unroll
    for (int pi = 0; pi < NP; ++pi) {
        const int c = p0 + pi * kSelPass + slot;
        double run[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double *qr = qg + 4 * (lam + 4 * i);
            double a = 0.0;
            a = __fma_rn(qr[0], (double)__uint_as_float(w[pi][i].x), a);
            a = __fma_rn(qr[1], (double)__uint_as_float(w[pi][i].y), a);
            a = __fma_rn(qr[2], (double)__uint_as_float(w[pi][i].z), a);
            a = __fma_rn(qr[3], (double)__uint_as_float(w[pi][i].w), a);
            run[i] = a;
        }
        const double t0 = run[0] + run[4], t1 = run[1] + run[5];
        const double t2 = run[2] + run[6], t3 = run[3] + run[7];
        double v = (t0 + t2) + (t1 + t3);
        v = v + __shfl_xor(v, 2);
        v = v + __shfl_xor(v, 1);
        if (lam == 0 && c < c_hi) out[c] = v;
        vals[pi] = v;
    }
}

// Scores only, for many clusters: workgroup (h, s) of a per-head XCD grid
// scores clusters [s kSelChunk, (s + 1) kSelChunk) of KV head h into
// scores[h][c] (fp64), every load of the workgroup in flight at once.
template <bool BF16>
__global__ __launch_bounds__(kSelThreads) void k_sel_score(
    const void *__restrict__ q, int G, const float *__restrict__ cent, int C, int c_cap, int H,
    int S, double *__restrict__ scores) {
    __shared__ double qg[kD];
    int h, s;
    xcd_head_unit(blockIdx.x, S, h, s);
    if (h >= H) return;
    const int tid = threadIdx.x, lam = tid & (kSelLanes - 1), slot = tid >> 2;
    const int p0 = s * kSelChunk, c_hi = (p0 + kSelChunk < C) ? p0 + kSelChunk : C;
    u32x4 w[kSelChunk / kSelPass][8];
    sel_load_cent<kSelChunk / kSelPass>(cent + (int64_t)h * c_cap * kD, p0, c_hi, lam, slot, w);
    float qv[8];
    if (tid < kD) sel_q_load<BF16>(q, G, h, tid, qv);
    if (tid < kD) qg[tid] = sel_q_sum(qv, G);
    __syncthreads();
    double vals[kSelChunk / kSelPass];
    sel_score<kSelChunk / kSelPass>(w, qg, p0, c_hi, lam, slot, scores + (int64_t)h * C, vals);
}

// PRE: the scores come from k_sel_score (scores[h][c]) instead of being
// computed here.
template <bool BF16, bool PRE>
__global__ __launch_bounds__(kSelThreads) void k_select(
    const void *__restrict__ q, int G, const float *__restrict__ cent, int C, int c_cap,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ tokens, int64_t t_cap,
    int n_sink, int64_t pending_begin, int64_t n_pending, int B, int32_t *__restrict__ idx,
    int32_t *__restrict__ n_sel, const double *__restrict__ scores) {
    constexpr int NW = kSelThreads / 64;
    __shared__ double qg[kD];
    __shared__ double sc[kMaxC];           // scores
    __shared__ int wt[kMaxC];              // tokens each cluster gives
    __shared__ int off[kMaxC + 1];         // clamped offsets
    __shared__ int inc[kMaxC];             // inclusive prefix of wt in id order;
                                           // before that, a bucket's last cluster
    __shared__ uint64_t hist[kRadixBuckets];
    __shared__ int mark[kSelMarks];        // first token slot of each taken cluster
    __shared__ int ws_a[NW], ws_b[NW], ws_c[NW];
    __shared__ double s_mn[NW], s_mx[NW];
    __shared__ int s_bucket, s_rem, s_cnt, s_cut;
    __shared__ unsigned long long s_kmin, s_kmax;
    const int T = kSelThreads, tid = threadIdx.x;
    const int h = blockIdx.x;

    // ---- loads: the first batch of centroid chunks (or the scores), the
    // offsets and q, all in flight together (the centroids do not wait for q)
    const int lam = tid & (kSelLanes - 1), slot = tid >> 2;
    const float *ch = cent + (int64_t)h * c_cap * kD;
    u32x4 w[kSelInFlight][8];
    constexpr int NS = kMaxC / kSelThreads;
    double pv[NS];
    if (PRE) {
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int c = tid + k * T;
            pv[k] = scores[(int64_t)h * C + (c < C ? c : C - 1)];
        }
    } else {
        sel_load_cent<kSelInFlight>(ch, 0, C, lam, slot, w);
    }
    const int32_t *offh = offsets + (int64_t)h * (c_cap + 1);
    {
        constexpr int NO = (kMaxC + kSelThreads) / kSelThreads;
        int64_t v[NO];
#pragma unroll
        for (int k = 0; k < NO; ++k) {
            const int c = tid + k * T;
            v[k] = offh[c <= C ? c : C];
        }
        float qv[8];
        if (!PRE && tid < kD) sel_q_load<BF16>(q, G, h, tid, qv);
#pragma unroll
        for (int k = 0; k < NO; ++k) {
            const int c = tid + k * T;
            if (c <= C) off[c] = (int)(v[k] < 0 ? 0 : (v[k] > t_cap ? t_cap : v[k]));
        }
        if (!PRE && tid < kD) qg[tid] = sel_q_sum(qv, G);
    }
    // the total size and the score range, gathered while the scores are made
    // (each cluster counted once) and reduced before the barrier that ends
    // this phase
    const double pinf = __longlong_as_double(0x7ff0000000000000ll);
    int loc = 0;
    double smin = pinf, smax = -pinf;
    auto take = [&](int c, double v) {
        const int n = off[c + 1] - off[c];
        loc += n > 0 ? n : 0;
        smin = fmin(smin, v);
        smax = fmax(smax, v);
    };
    if (PRE) {
        __syncthreads();                   // off[] complete
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const int c = tid + k * T;
            if (c < C) {
                sc[c] = pv[k];
                take(c, pv[k]);
            }
        }
    } else {
        __syncthreads();
        // ---- 1. scores ----------------------------------------------------
        for (int p0 = 0; p0 < C; p0 += kSelPass * kSelInFlight) {
            if (p0 > 0) sel_load_cent<kSelInFlight>(ch, p0, C, lam, slot, w);
            double vals[kSelInFlight];
            sel_score<kSelInFlight>(w, qg, p0, C, lam, slot, sc, vals);
#pragma unroll
            for (int pi = 0; pi < kSelInFlight; ++pi) {
                const int c = p0 + pi * kSelPass + slot;
                if (lam == 0 && c < C) take(c, vals[pi]);
            }
        }
    }
    loc = wave_sum(loc);
    wave_minmax_f64(smin, smax);
    if ((tid & 63) == 0) {
        ws_a[tid >> 6] = loc;
        s_mn[tid >> 6] = smin;
        s_mx[tid >> 6] = smax;
    }
    // the first histogram and the slot marks start cleared
#pragma unroll
    for (int u = 0; u < kRadixBuckets / kSelThreads; ++u) hist[tid + u * kSelThreads] = 0;
#pragma unroll
    for (int u = 0; u < kSelSlots; ++u) mark[tid + u * kSelThreads] = -1;
    if (tid == 0) {
        s_kmin = ~0ull;
        s_kmax = 0ull;
    }
    __syncthreads();

    // ---- 2. the cut: first cluster (rank order) where the sizes reach B_eff
    const int64_t beff64 = (int64_t)B - n_sink - n_pending;
    const int beff = (int)(beff64 > 0 ? beff64 : 0);
    // this thread's clusters 4 tid .. 4 tid + 3: sizes, scores
    int wv[kSelPer];
    double sv[kSelPer];
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int c = kSelPer * tid + u;
        wv[u] = 0;
        sv[u] = 0.0;
        if (c < C) {
            const int n = off[c + 1] - off[c];
            wv[u] = n > 0 ? n : 0;
            sv[u] = sc[c];
        }
    }
    int total = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        total += ws_a[w];
        smin = fmin(smin, s_mn[w]);
        smax = fmax(smax, s_mx[w]);
    }
    int cut = -1, rem = 0;                 // no cut: every cluster gives all
    if (beff == 0) {
        cut = -2;                          // nothing is taken
    } else if (total > beff) {
        // score pass: bucket = floor((smax - s) * 2047 / (smax - smin)), a
        // non-increasing function of s, so lower buckets rank first
        const double range = smax - smin;
        double scale = range > 0.0 ? (double)(kRadixBuckets - 1) / range : 0.0;
        if (!(scale < pinf)) scale = 0.0;  // range infinite or too small
        int bk[kSelPer];
#pragma unroll
        for (int u = 0; u < kSelPer; ++u) {
            const int c = kSelPer * tid + u;
            bk[u] = -1;
            if (c < C) {
                const double x = (smax - sv[u]) * scale;
                const int b = x >= (double)(kRadixBuckets - 1) ? kRadixBuckets - 1
                                                               : (x > 0.0 ? (int)x : 0);
                bk[u] = b;
                atomicAdd((unsigned long long *)&hist[b],
                          ((unsigned long long)wv[u] << kCntBits) | 1ull);
                inc[b] = c;                // the bucket's cluster when it has one
            }
        }
        __syncthreads();
        // buckets 4 tid .. 4 tid + 3 in rank order; the thread whose range of
        // the running size reaches R names the bucket
        constexpr int NBK = kRadixBuckets / kSelThreads;
        int R = beff;
        {
            uint64_t hv[NBK];
            int bsum = 0;
#pragma unroll
            for (int k = 0; k < NBK; ++k) {
                hv[k] = hist[NBK * tid + k];
                bsum += (int)(hv[k] >> kCntBits);
            }
            int tot;
            const int ex = block_excl_scan_nw<NW>(bsum, ws_b, tot);
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
                const int bb = NBK * tid + b;
                const int cnt = (int)(hv[b] & ((1u << kCntBits) - 1));
                s_bucket = bb;
                s_rem = R - before;
                s_cut = cnt == 1 ? inc[bb] : -1;
            }
        }
        __syncthreads();
        const int bsel = s_bucket;
        R = s_rem;
        cut = s_cut;
        if (cut < 0) {
            // several clusters share that bucket: exact radix passes over their
            // rank keys, from the highest bit where those keys differ
            bool cand[kSelPer];
            uint64_t key[kSelPer];
#pragma unroll
            for (int u = 0; u < kSelPer; ++u) {
                cand[u] = bk[u] == bsel;
                key[u] = rank_key(sv[u]);
                if (cand[u]) {
                    atomicMin(&s_kmin, (unsigned long long)key[u]);
                    atomicMax(&s_kmax, (unsigned long long)key[u]);
                }
            }
            __syncthreads();
            const uint64_t kdiff = s_kmin ^ s_kmax;
            const int hb = kdiff ? 63 - __clzll((long long)kdiff) : -1;
            const int nkey = hb < 0 ? 0 : (hb + 11) / 11;       // key passes
            for (int pos = 0; pos <= nkey; ++pos) {
                const bool in_id = pos == nkey;
                int sh = hb - 10 - 11 * pos;
                sh = sh < 0 ? 0 : sh;
#pragma unroll
                for (int u = 0; u < NBK; ++u) hist[tid + u * kSelThreads] = 0;
                __syncthreads();
#pragma unroll
                for (int u = 0; u < kSelPer; ++u) {
                    const int c = kSelPer * tid + u;
                    if (cand[u]) {
                        const int d = in_id ? c : (int)((key[u] >> sh) & (kRadixBuckets - 1));
                        atomicAdd((unsigned long long *)&hist[d],
                                  ((unsigned long long)wv[u] << kCntBits) | 1ull);
                    }
                }
                __syncthreads();
                uint64_t hv[NBK];
                int bsum = 0;
#pragma unroll
                for (int k = 0; k < NBK; ++k) {
                    hv[k] = hist[NBK * tid + k];
                    bsum += (int)(hv[k] >> kCntBits);
                }
                int tot;
                const int ex = block_excl_scan_nw<NW>(bsum, pos & 1 ? ws_c : ws_b, tot);
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
                __syncthreads();
                const int bs = s_bucket;
                R = s_rem;
#pragma unroll
                for (int u = 0; u < kSelPer; ++u) {
                    const int c = kSelPer * tid + u;
                    if (cand[u]) {
                        const int d = in_id ? c : (int)((key[u] >> sh) & (kRadixBuckets - 1));
                        cand[u] = d == bs;
                    }
                }
                const bool done = s_cnt == 1;  // uniform
                __syncthreads();
                if (done) break;
            }
#pragma unroll
            for (int u = 0; u < kSelPer; ++u)
                if (cand[u]) s_cut = kSelPer * tid + u;
            __syncthreads();
            cut = s_cut;
        }
        rem = R;
    }
    // ---- 3. tokens each cluster gives, prefix in id order, emission --------
    const double cs = cut >= 0 ? sc[cut] : 0.0;
    int tk[kSelPer];
    loc = 0;
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int c = kSelPer * tid + u;
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
    int run = block_excl_scan_nw<NW>(loc, ws_c, ntake);
#pragma unroll
    for (int u = 0; u < kSelPer; ++u) {
        const int c = kSelPer * tid + u;
        if (tk[u] > 0 && run < kSelMarks) mark[run] = c;
        run += tk[u];
        if (c < C) {
            inc[c] = run;
            wt[c] = tk[u];
        }
    }
    __syncthreads();

    const int64_t head = (int64_t)n_sink + n_pending;
    const int32_t *tok = tokens + (int64_t)h * t_cap;
    int32_t *out = idx + (int64_t)h * B;
    if (ntake <= kSelMarks) {              // uniform
        // sinks, pending tokens and the unused tail
        for (int64_t e = tid; e < B; e += T) {
            if (e < n_sink) out[e] = (int32_t)e;
            else if (e < head) out[e] = (int32_t)(pending_begin + (e - n_sink));
            else if (e - head >= ntake) out[e] = -1;
        }
        // token slots p = 4 tid .. 4 tid + 3: the cluster of slot p is the
        // largest marked id at or before p (ids rise with the slots), found by
        // a running max inside the thread, then an exclusive max-scan over
        // the threads before it
        int cm[kSelSlots];
        int mx = -1;
#pragma unroll
        for (int k = 0; k < kSelSlots; ++k) {
            const int p = kSelSlots * tid + k;
            const int v = p < ntake ? mark[p] : -1;
            mx = v > mx ? v : mx;
            cm[k] = mx;
        }
        const int lane = tid & 63, wave = tid >> 6;
        const int incl = wave_incl_max(mx);
        int prev = __shfl_up(incl, 1);
        prev = lane == 0 ? -1 : prev;
        if (lane == 63) ws_b[wave] = incl;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w)
            if (w < wave) prev = ws_b[w] > prev ? ws_b[w] : prev;
        int src[kSelSlots];
#pragma unroll
        for (int k = 0; k < kSelSlots; ++k) {
            const int p = kSelSlots * tid + k;
            const int c = cm[k] > prev ? cm[k] : prev;
            src[k] = (p < ntake && c >= 0) ? off[c] + (p - (inc[c] - wt[c])) : -1;
        }
        int32_t t[kSelSlots];
#pragma unroll
        for (int k = 0; k < kSelSlots; ++k) t[k] = tok[src[k] >= 0 ? src[k] : 0];
#pragma unroll
        for (int k = 0; k < kSelSlots; ++k)
            if (src[k] >= 0) out[head + kSelSlots * tid + k] = t[k];
    } else {
        // many taken tokens: output slots in batches, each token slot's
        // cluster by binary search over the id-order prefix, then every token
        // load of the batch in flight, then the stores
        constexpr int NE = 8;
        for (int e0 = tid; e0 < B; e0 += NE * T) {
            int src[NE];
            int32_t val[NE];
#pragma unroll
            for (int k = 0; k < NE; ++k) {
                const int64_t e = e0 + (int64_t)k * T;
                src[k] = -1;
                val[k] = -1;
                if (e < n_sink) {
                    val[k] = (int32_t)e;
                } else if (e < head) {
                    val[k] = (int32_t)(pending_begin + (e - n_sink));
                } else if (e - head < ntake) {
                    const int p = (int)(e - head);
                    int lo = 0, hi = C - 1;    // first cluster whose inclusive prefix exceeds p
                    while (lo < hi) {
                        const int mid = (lo + hi) >> 1;
                        if (inc[mid] > p) hi = mid; else lo = mid + 1;
                    }
                    src[k] = off[lo] + (p - (inc[lo] - wt[lo]));
                }
            }
            int32_t t[NE];
#pragma unroll
            for (int k = 0; k < NE; ++k) t[k] = tok[src[k] >= 0 ? src[k] : 0];
#pragma unroll
            for (int k = 0; k < NE; ++k) {
                const int64_t e = e0 + (int64_t)k * T;
                if (e < B) out[e] = src[k] >= 0 ? t[k] : val[k];
            }
        }
    }
    if (tid == 0) n_sel[h] = (int32_t)(head + ntake);
}

hipError_t launch_select(const SelectPlan &p, const void *q, const float *cent,
                         const int32_t *offsets, const int32_t *tokens, int32_t *idx,
                         int32_t *n_sel, hipStream_t s) {
    const bool pre = p.C > kSelOneKernelMaxC;
    if (pre) {
        const int S = (p.C + kSelChunk - 1) / kSelChunk;
        if (p.dtype == 1)
            hipLaunchKernelGGL(k_sel_score<true>, dim3(xcd_head_grid(p.H, S)), dim3(kSelThreads),
                               0, s, q, p.G, cent, p.C, p.c_cap, p.H, S, p.scores);
        else
            hipLaunchKernelGGL(k_sel_score<false>, dim3(xcd_head_grid(p.H, S)),
                               dim3(kSelThreads), 0, s, q, p.G, cent, p.C, p.c_cap, p.H, S,
                               p.scores);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
#define CKV_SEL(BF, PR)                                                                      \
    hipLaunchKernelGGL((k_select<BF, PR>), dim3(p.H), dim3(kSelThreads), 0, s, q, p.G, cent,  \
                       p.C, p.c_cap, offsets, tokens, p.t_cap, p.n_sink, p.pending_begin,    \
                       p.n_pending, p.B, idx, n_sel, (const double *)p.scores)
    if (p.dtype == 1) {
        if (pre) CKV_SEL(true, true); else CKV_SEL(true, false);
    } else {
        if (pre) CKV_SEL(false, true); else CKV_SEL(false, false);
    }
#undef CKV_SEL
    return hipGetLastError();
}

}  // namespace ckv
