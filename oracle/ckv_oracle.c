/*
 * ckv_oracle.c -- plain, slow, single-threaded CPU oracle for ClusterKV's
 * cluster-granular recallable KV selection.
 *
 * TEST INFRASTRUCTURE. Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library. It shares no code,
 * header, table or helper with the GPU library; it is built with gcc from
 * this file alone.
 *
 * Source of every definition: the page "ClusterKV: Manipulating LLM KV Cache
 * in Semantic Space for Recallable Compression" (a summary of arXiv
 * 2412.03213). Section names below are that page's headings, glossed:
 *   [LLM inference & KV cache]        背景知识与设计原则 / LLM推理与KV缓存
 *   [Long context & KV compression]   背景知识与设计原则 / 长上下文推理与KV缓存压缩
 *   [Problem formulation]             核心方法细节 / 问题建模与设计原则
 *   [Clustering in semantic space]    核心方法细节 / 语义空间中的聚类  (distance D, Fig. 4)
 *   [Cluster-granular selection]      核心方法细节 / 语义聚类粒度的选择
 *   [Selection and indexing]          核心方法细节 / 选择与索引机制     (Fig. 8)
 *
 * Arithmetic is fp64 throughout. Two modes:
 *   ORC_EXACT  -- no intermediate rounding beyond fp64: cosine scores from
 *                 fp64 unit vectors, centroids kept in fp64.
 *   ORC_MIRROR -- identical steps, but the operands of the scores are the
 *                 ones the GPU stores: the key as stored (bf16), and for
 *                 the cosine the unit centroid rounded fp64 -> fp32 -> bf16
 *                 (nearest-even each time); centroids are stored as fp32.
 *                 The scores themselves are still fp64 dot products of those
 *                 operands.
 *
 * Readings taken where the page is silent (each one is listed with its
 * reason in the design notes of the repository):
 *   - a centroid is the mean of the RAW keys assigned to it;
 *   - K-means starts from the keys at positions n_sink + s*c, s = floor(L'/C);
 *   - argmax and sort ties go to the lower cluster id;
 *   - an empty cluster keeps its previous centroid;
 *   - the returned partition is the last iteration's, the returned centroids
 *     are that partition's means;
 *   - a KV head shared by G query heads is selected once, scored with the
 *     sum of the G queries;
 *   - sinks (and, for incremental decode, not-yet-clustered tokens) are always
 *     selected and count toward the budget B;
 *   - the last admitted cluster is trimmed to its lowest positions;
 *   - idx order: sinks, pending, then the admitted clusters in ascending
 *     cluster id, each ascending (the page fixes which tokens are selected,
 *     not the order in which they are handed to attention).
 *   - fixed association of the selection score (see orc_score).
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -shared -fPIC ckv_oracle.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXACT 0
#define ORC_MIRROR 1

/* Assignment distances. The page argues for the cosine distance over L2 and
 * inner-product distance (outlier channels of large magnitude make the
 * latter two swing) and ablates the three [Clustering in semantic space;
 * recall experiment, Fig. 11b]. */
#define ORC_COSINE 0
#define ORC_INNER_PRODUCT 1
#define ORC_L2 2

/* ------------------------------------------------------------ rounding -- */

/* Round a float to bfloat16 (nearest, ties to even) and return it as float.
 * Finite inputs only. */
static float orc_round_bf16(float x)
{
    uint32_t u;
    memcpy(&u, &x, 4);
    u = u + 0x7FFFu + ((u >> 16) & 1u);
    u &= 0xFFFF0000u;
    float r;
    memcpy(&r, &u, 4);
    return r;
}

double orc_bf16_round_value(double x) { return (double)orc_round_bf16((float)x); }

/* Sum of squares as one fp64 fused-multiply-add chain over j = 0..d-1. */
static double orc_sumsq(const double *x, int d)
{
    double s = 0.0;
    for (int j = 0; j < d; ++j) s = fma(x[j], x[j], s);
    return s;
}

/* Unit vector of x, for the cosine distance D(i,j) = 1 - <k_i,k_j>/(|k_i||k_j|)
 * [Clustering in semantic space]. A zero vector maps to zero (its cosine
 * with anything is taken as 0). |x| = sqrt of the fp64 chain above, and
 * the quotient x_j / |x| is one fp64 division.
 *   EXACT : the fp64 quotient.
 *   MIRROR: bf16(fp32(quotient)), nearest-even both times. */
static void orc_unit(const double *x, int d, int mode, double *out)
{
    double ss = orc_sumsq(x, d);
    if (!(ss > 0.0)) {
        for (int j = 0; j < d; ++j) out[j] = 0.0;
        return;
    }
    double n = sqrt(ss);
    for (int j = 0; j < d; ++j) {
        double u = x[j] / n;
        out[j] = (mode == ORC_EXACT) ? u : (double)orc_round_bf16((float)u);
    }
}

void orc_unit_rows(int64_t n, int d, const double *x, int mode, double *out)
{
    for (int64_t i = 0; i < n; ++i) orc_unit(x + i * d, d, mode, out + i * d);
}

static double orc_dot(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int j = 0; j < d; ++j) s += a[j] * b[j];
    return s;
}

/* ----------------------------------------------------- K-means pieces -- */

/* Initial centroids: mu_c = k_{n_sink + s*c}, s = floor(L'/C)
 * [Clustering in semantic space: the initial centroids are keys sampled at
 * random; read here as evenly spaced tokens]. K is one head [L][d]. */
void orc_init_centroids(int64_t L, int d, const double *K, int n_sink, int C,
                        double *mu)
{
    int64_t Lp = L - n_sink;
    int64_t s = Lp / C;
    for (int c = 0; c < C; ++c)
        memcpy(mu + (int64_t)c * d, K + (n_sink + s * c) * d, sizeof(double) * d);
}

/* A key or centroid as the inner-product and L2 comparisons see it:
 *   EXACT : x itself.
 *   MIRROR: bf16(fp32(x_j)), the way the GPU stores its operands. */
static void orc_store(const double *x, int d, int mode, double *out)
{
    for (int j = 0; j < d; ++j)
        out[j] = (mode == ORC_EXACT) ? x[j] : (double)orc_round_bf16((float)x[j]);
}

/* Squared Euclidean distance sum_j (a_j - b_j)^2, summed in channel order. */
static double orc_dist2(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int j = 0; j < d; ++j) s += (a[j] - b[j]) * (a[j] - b[j]);
    return s;
}

/* Assignment step under one of the three distances [Clustering in semantic
 * space, Fig. 4, and its ablation]. Each non-sink key joins
 *   ORC_COSINE       : the centroid of largest cosine similarity (smallest D);
 *   ORC_INNER_PRODUCT: the centroid of largest <k, mu>;
 *   ORC_L2           : the centroid of smallest sum_j (k_j - mu_j)^2.
 * Ties go to the lower cluster id. Writes assign[0..L) (-1 for sinks) and,
 * if margin is not NULL, margin[i] = the gap between the best and the
 * second-best candidate (cosine gap for the cosine, score gap for the inner
 * product, squared distance gap for L2; +inf when C == 1, and for sinks).
 * K is one head [L][d]; mu is [C][d].
 * Cosine: EXACT compares the cosines themselves, dot products of the two
 * fp64 unit vectors. cos(k, mu) = <k, mu/|mu|> / |k|, and |k| > 0 is the
 * same for every centroid, so the largest cosine is also the largest
 * <k, mu/|mu|>: MIRROR compares those, with the key as stored and the
 * rounded unit centroid, and divides the gap by |k| to give it in cosine
 * units (a zero key has gap 0: all its scores are 0). */
void orc_assign_metric(int64_t L, int d, const double *K, int n_sink, int C,
                       const double *mu, int metric, int mode, int32_t *assign,
                       double *margin)
{
    double *mt = malloc(sizeof(double) * (size_t)C * d);
    double *kt = malloc(sizeof(double) * d);
    for (int c = 0; c < C; ++c) {
        if (metric == ORC_COSINE)
            orc_unit(mu + (int64_t)c * d, d, mode, mt + (int64_t)c * d);
        else
            orc_store(mu + (int64_t)c * d, d, mode, mt + (int64_t)c * d);
    }
    for (int64_t i = 0; i < L; ++i) {
        if (i < n_sink) {
            assign[i] = -1;
            if (margin) margin[i] = INFINITY;
            continue;
        }
        if (metric == ORC_COSINE && mode == ORC_EXACT)
            orc_unit(K + i * d, d, mode, kt);
        else
            orc_store(K + i * d, d, mode, kt);
        double best = -INFINITY, second = -INFINITY;
        int arg = 0;
        for (int c = 0; c < C; ++c) {
            /* larger is better: similarity, or the negated distance */
            double s = (metric == ORC_L2) ? -orc_dist2(kt, mt + (int64_t)c * d, d)
                                          : orc_dot(kt, mt + (int64_t)c * d, d);
            if (s > best) {
                second = best;
                best = s;
                arg = c;
            } else if (s > second) {
                second = s;
            }
        }
        assign[i] = arg;
        if (margin) {
            double gap = best - second;
            if (metric == ORC_COSINE && mode == ORC_MIRROR) {
                double nk = sqrt(orc_sumsq(kt, d));
                gap = nk > 0.0 ? gap / nk : 0.0;
            }
            margin[i] = (C == 1) ? INFINITY : gap;
        }
    }
    free(kt);
    free(mt);
}

/* The page's assignment: cosine distance. */
void orc_assign(int64_t L, int d, const double *K, int n_sink, int C,
                const double *mu, int mode, int32_t *assign, double *margin)
{
    orc_assign_metric(L, d, K, n_sink, C, mu, ORC_COSINE, mode, assign, margin);
}

/* Cluster metadata [Selection and indexing, Fig. 8]: cluster sizes, their
 * exclusive prefix sums (offsets, C+1 entries) and the token indices sorted
 * by label (stable, so ascending within a cluster). Tokens are written as
 * absolute ids i + token_base. */
void orc_csr(int64_t L, int n_sink, int C, const int32_t *assign,
             int64_t token_base, int32_t *offsets, int32_t *tokens)
{
    int64_t *cnt = calloc((size_t)C + 1, sizeof(int64_t));
    for (int64_t i = n_sink; i < L; ++i) cnt[assign[i] + 1] += 1;
    for (int c = 0; c < C; ++c) cnt[c + 1] += cnt[c];
    for (int c = 0; c <= C; ++c) offsets[c] = (int32_t)cnt[c];
    for (int64_t i = n_sink; i < L; ++i) {
        int a = assign[i];
        tokens[cnt[a]] = (int32_t)(i + token_base);
        cnt[a] += 1;
    }
    free(cnt);
}

/* Update step: each centroid becomes the mean of the keys assigned to it
 * [Clustering in semantic space: a centroid is replaced by the average of
 * its cluster's keys]. Raw keys, fp64 sum in ascending token order, then one
 * division. MIRROR stores the mean rounded to fp32. A cluster with no keys
 * keeps mu_old. */
void orc_update(int64_t L, int d, const double *K, int n_sink, int C,
                const int32_t *assign, const double *mu_old, int mode,
                double *mu_new)
{
    double *acc = calloc((size_t)C * d, sizeof(double));
    int64_t *n = calloc((size_t)C, sizeof(int64_t));
    for (int64_t i = n_sink; i < L; ++i) {
        int a = assign[i];
        n[a] += 1;
        for (int j = 0; j < d; ++j) acc[(int64_t)a * d + j] += K[i * d + j];
    }
    for (int c = 0; c < C; ++c) {
        for (int j = 0; j < d; ++j) {
            int64_t e = (int64_t)c * d + j;
            if (n[c] == 0) {
                mu_new[e] = mu_old[e];
            } else {
                double m = acc[e] / (double)n[c];
                mu_new[e] = (mode == ORC_MIRROR) ? (double)(float)m : m;
            }
        }
    }
    free(n);
    free(acc);
}

/* K-means objective that the page's alternation decreases: the norm-weighted
 * cosine distance J_w = sum_i |k_i| * D(k_i, mu_{a_i})
 *                     = sum_i (|k_i| - <k_i, mu_a> / |mu_a|).
 * Cosine assignment minimises every term for fixed centroids; the raw-key
 * mean points along the direction that maximises sum <k_i, u> over unit u for
 * a fixed partition. fp64, EXACT. A zero centroid contributes |k_i|. */
double orc_objective(int64_t L, int d, const double *K, int n_sink,
                     const int32_t *assign, const double *mu)
{
    double J = 0.0;
    for (int64_t i = n_sink; i < L; ++i) {
        const double *k = K + i * d;
        const double *m = mu + (int64_t)assign[i] * d;
        double nk = sqrt(orc_sumsq(k, d));
        double nm = sqrt(orc_sumsq(m, d));
        double ip = orc_dot(k, m, d);
        J += nk - (nm > 0.0 ? ip / nm : 0.0);
    }
    return J;
}

/* Whole K-means for H independent heads [Clustering in semantic space]:
 * centroids from orc_init_centroids, then `iters` rounds of
 * (assign, update). K is [H][L][d]; outputs mu [H][C][d], assign [H][L],
 * offsets [H][C+1], tokens [H][L - n_sink] (absolute ids, + token_base).
 * If trace is not NULL it receives, per head, 2*iters objective values:
 * J after each assignment and after each update (EXACT meaning). If
 * changed is not NULL it receives per head and iteration the number of
 * tokens whose label differs from the previous iteration (first iteration:
 * all tokens). */
void orc_cluster_metric(int metric, int mode, int H, int64_t L, int d, const double *K,
                        int n_sink, int C, int iters, int64_t token_base, double *mu,
                        int32_t *assign, int32_t *offsets, int32_t *tokens,
                        double *trace, int64_t *changed);

void orc_cluster(int mode, int H, int64_t L, int d, const double *K, int n_sink,
                 int C, int iters, int64_t token_base, double *mu,
                 int32_t *assign, int32_t *offsets, int32_t *tokens,
                 double *trace, int64_t *changed)
{
    orc_cluster_metric(ORC_COSINE, mode, H, L, d, K, n_sink, C, iters, token_base, mu,
                       assign, offsets, tokens, trace, changed);
}

/* The same loop with the assignment under `metric` (the update is the mean
 * of the raw keys for every metric); trace must be NULL unless the metric
 * is the cosine, whose objective it records. */
void orc_cluster_metric(int metric, int mode, int H, int64_t L, int d, const double *K,
                        int n_sink, int C, int iters, int64_t token_base, double *mu,
                        int32_t *assign, int32_t *offsets, int32_t *tokens,
                        double *trace, int64_t *changed)
{
    if (metric != ORC_COSINE) trace = NULL;
    int64_t Lp = L - n_sink;
    double *mu_next = malloc(sizeof(double) * (size_t)C * d);
    int32_t *prev = malloc(sizeof(int32_t) * (size_t)L);
    for (int h = 0; h < H; ++h) {
        const double *Kh = K + (int64_t)h * L * d;
        double *muh = mu + (int64_t)h * C * d;
        int32_t *ah = assign + (int64_t)h * L;
        orc_init_centroids(L, d, Kh, n_sink, C, muh);
        for (int64_t i = 0; i < L; ++i) prev[i] = -2;
        for (int t = 0; t < iters; ++t) {
            orc_assign_metric(L, d, Kh, n_sink, C, muh, metric, mode, ah, NULL);
            if (trace) trace[(int64_t)h * 2 * iters + 2 * t] =
                orc_objective(L, d, Kh, n_sink, ah, muh);
            if (changed) {
                int64_t ch = 0;
                for (int64_t i = n_sink; i < L; ++i) ch += (ah[i] != prev[i]);
                changed[(int64_t)h * iters + t] = ch;
            }
            memcpy(prev, ah, sizeof(int32_t) * (size_t)L);
            orc_update(L, d, Kh, n_sink, C, ah, muh, mode, mu_next);
            memcpy(muh, mu_next, sizeof(double) * (size_t)C * d);
            if (trace) trace[(int64_t)h * 2 * iters + 2 * t + 1] =
                orc_objective(L, d, Kh, n_sink, ah, muh);
        }
        orc_csr(L, n_sink, C, ah, token_base, offsets + (int64_t)h * (C + 1),
                tokens + (int64_t)h * Lp);
    }
    free(prev);
    free(mu_next);
}

/* ---------------------------------------------------------- selection -- */

/* Selection score s_c = q_g . mu_c, the inner product (not the cosine) of
 * the query with the centroid [Cluster-granular selection]. The page fixes
 * no precision; here it is fp64 with this fixed association so that a
 * parallel evaluation can reproduce it bit for bit: the d channels form
 * d/4 runs of 4 consecutive channels, each run is a fused-multiply-add chain
 * starting from 0, and the d/4 run sums are added pairwise, run r with run
 * r + d/8, then r with r + d/16, ..., down to one value. d/4 must be a power
 * of two. */
static double orc_score(const double *q, const double *mu, int d)
{
    int nr = d / 4;
    double part[1024];
    for (int r = 0; r < nr; ++r) {
        double a = 0.0;
        for (int j = 4 * r; j < 4 * r + 4; ++j) a = fma(q[j], mu[j], a);
        part[r] = a;
    }
    for (int w = nr / 2; w >= 1; w /= 2)
        for (int r = 0; r < w; ++r) part[r] = part[r] + part[r + w];
    return part[0];
}

typedef struct {
    double s;
    int c;
} orc_rank_t;

/* Descending score, then ascending cluster id. */
static int orc_rank_cmp(const void *pa, const void *pb)
{
    const orc_rank_t *a = pa, *b = pb;
    if (a->s > b->s) return -1;
    if (a->s < b->s) return 1;
    return (a->c < b->c) ? -1 : (a->c > b->c);
}

/* Decode-time selection for H KV heads [Cluster-granular selection;
 * Selection and indexing, Fig. 8]:
 *   q_g   = sum of the G query rows of KV head g (fp64, in row order);
 *   s_c   = orc_score(q_g, mu_c);
 *   order = clusters by (s desc, c asc);
 *   walk the order, taking each cluster's tokens until B_eff = B - n_sink -
 *   n_pending tokens are taken; the last cluster taken is cut to the tokens
 *   that still fit (the first ones of its CSR segment, its lowest positions);
 *   idx   = [0 .. n_sink) ++ [pending_begin .. pending_begin + n_pending)
 *           ++ the taken tokens of each cluster, clusters in ascending id,
 *           then -1 up to B; n_sel = number written.
 * q: [H*G][d]; mu: [H][c_stride][d]; offsets: [H][c_stride+1] (absolute
 * positions into the head's token row); tokens: [H][t_stride]; idx [H][B].
 * If scores is not NULL it receives [H][C] scores. Returns 0, or -1 if
 * B < n_sink + n_pending. */
int orc_select(int H, int G, int d, const double *q, int C, int c_stride,
               const double *mu, const int32_t *offsets, const int32_t *tokens,
               int64_t t_stride, int n_sink, int64_t pending_begin,
               int64_t n_pending, int B, int32_t *idx, int32_t *n_sel,
               double *scores)
{
    if ((int64_t)B < n_sink + n_pending) return -1;
    double *qg = malloc(sizeof(double) * d);
    orc_rank_t *rk = malloc(sizeof(orc_rank_t) * (size_t)(C > 0 ? C : 1));
    int64_t *take = malloc(sizeof(int64_t) * (size_t)(C > 0 ? C : 1));
    for (int g = 0; g < H; ++g) {
        for (int j = 0; j < d; ++j) {
            double a = 0.0;
            for (int h = 0; h < G; ++h) a += q[((int64_t)g * G + h) * d + j];
            qg[j] = a;
        }
        const double *mug = mu + (int64_t)g * c_stride * d;
        const int32_t *off = offsets + (int64_t)g * (c_stride + 1);
        const int32_t *tok = tokens + (int64_t)g * t_stride;
        for (int c = 0; c < C; ++c) {
            rk[c].s = orc_score(qg, mug + (int64_t)c * d, d);
            rk[c].c = c;
            if (scores) scores[(int64_t)g * C + c] = rk[c].s;
        }
        qsort(rk, (size_t)C, sizeof(orc_rank_t), orc_rank_cmp);

        /* walk the rank order: how many tokens each cluster gives */
        int64_t budget = (int64_t)B - n_sink - n_pending;
        int64_t filled = 0;
        for (int c = 0; c < C; ++c) take[c] = 0;
        for (int r = 0; r < C && filled < budget; ++r) {
            int c = rk[r].c;
            int64_t n = off[c + 1] - off[c];
            take[c] = n < budget - filled ? n : budget - filled;
            filled += take[c];
        }
        /* emit: sinks, pending, then clusters in ascending id */
        int32_t *out = idx + (int64_t)g * B;
        int64_t w = 0;
        for (int i = 0; i < n_sink; ++i) out[w++] = i;
        for (int64_t i = 0; i < n_pending; ++i) out[w++] = (int32_t)(pending_begin + i);
        for (int c = 0; c < C; ++c)
            for (int64_t t = 0; t < take[c]; ++t) out[w++] = tok[off[c] + t];
        n_sel[g] = (int32_t)w;
        while (w < B) out[w++] = -1;
    }
    free(take);
    free(rk);
    free(qg);
    return 0;
}

/* ---------------------------------------------------------- attention -- */

/* Decode attention over a token subset, softmax(q K_S^T / sqrt(d)) V_S
 * [Long context & KV compression], for each query head h of KV head
 * g = h / G, with K_S, V_S the rows idx[g][0 .. n_sel[g]). fp64:
 * z_t = scale * (q_h . k_t), p_t = exp(z_t - max z), o = sum p_t v_t / sum p_t.
 * K, V: [H][kv_stride][d] (row r of head g at (g*kv_stride + r)*d).
 * scale <= 0 means 1/sqrt(d). o: [H*G][d]. */
void orc_attn(int H, int G, int d, const double *q, const double *K,
              const double *V, int64_t kv_stride, const int32_t *idx,
              const int32_t *n_sel, int B, double scale, double *o)
{
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)d);
    double *z = malloc(sizeof(double) * (size_t)(B > 0 ? B : 1));
    for (int g = 0; g < H; ++g) {
        int n = n_sel[g];
        const int32_t *ix = idx + (int64_t)g * B;
        const double *Kg = K + (int64_t)g * kv_stride * d;
        const double *Vg = V + (int64_t)g * kv_stride * d;
        for (int hh = 0; hh < G; ++hh) {
            int64_t h = (int64_t)g * G + hh;
            const double *qh = q + h * d;
            double *oh = o + h * d;
            double m = -INFINITY;
            for (int t = 0; t < n; ++t) {
                z[t] = scale * orc_dot(qh, Kg + (int64_t)ix[t] * d, d);
                if (z[t] > m) m = z[t];
            }
            double l = 0.0;
            for (int j = 0; j < d; ++j) oh[j] = 0.0;
            for (int t = 0; t < n; ++t) {
                double p = exp(z[t] - m);
                l += p;
                const double *v = Vg + (int64_t)ix[t] * d;
                for (int j = 0; j < d; ++j) oh[j] += p * v[j];
            }
            for (int j = 0; j < d; ++j) oh[j] = (n > 0) ? oh[j] / l : 0.0;
        }
    }
    free(z);
}

/* Dense decode attention softmax(q K^T / sqrt(d)) V over rows 0..L-1
 * [LLM inference & KV cache]; written without an index set. */
void orc_dense_attn(int H, int G, int d, const double *q, const double *K,
                    const double *V, int64_t kv_stride, int64_t L, double scale,
                    double *o)
{
    if (!(scale > 0.0)) scale = 1.0 / sqrt((double)d);
    double *z = malloc(sizeof(double) * (size_t)(L > 0 ? L : 1));
    for (int g = 0; g < H; ++g) {
        const double *Kg = K + (int64_t)g * kv_stride * d;
        const double *Vg = V + (int64_t)g * kv_stride * d;
        for (int hh = 0; hh < G; ++hh) {
            int64_t h = (int64_t)g * G + hh;
            double m = -INFINITY;
            for (int64_t t = 0; t < L; ++t) {
                z[t] = scale * orc_dot(q + h * d, Kg + t * d, d);
                if (z[t] > m) m = z[t];
            }
            double l = 0.0;
            for (int j = 0; j < d; ++j) o[h * d + j] = 0.0;
            for (int64_t t = 0; t < L; ++t) {
                double p = exp(z[t] - m);
                l += p;
                for (int j = 0; j < d; ++j) o[h * d + j] += p * Vg[t * d + j];
            }
            for (int j = 0; j < d; ++j) o[h * d + j] /= l;
        }
    }
    free(z);
}
