/* Exercises every function of the CPU oracle (oracle/ckv_oracle.c) on small
 * seeded inputs, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py). Prints one
 * checksum line; any sanitizer report makes the process fail. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void orc_unit_rows(int64_t n, int d, const double *x, int mode, double *out);
void orc_init_centroids(int64_t L, int d, const double *K, int n_sink, int C, double *mu);
void orc_assign_metric(int64_t L, int d, const double *K, int n_sink, int C, const double *mu,
                       int metric, int mode, int32_t *assign, double *margin);
void orc_csr(int64_t L, int n_sink, int C, const int32_t *assign, int64_t token_base,
             int32_t *offsets, int32_t *tokens);
void orc_update(int64_t L, int d, const double *K, int n_sink, int C, const int32_t *assign,
                const double *mu_old, int mode, double *mu_new);
double orc_objective(int64_t L, int d, const double *K, int n_sink, const int32_t *assign,
                     const double *mu);
void orc_cluster_metric(int metric, int mode, int H, int64_t L, int d, const double *K,
                        int n_sink, int C, int iters, int64_t token_base, double *mu,
                        int32_t *assign, int32_t *offsets, int32_t *tokens, double *trace,
                        int64_t *changed);
int orc_select(int H, int G, int d, const double *q, int C, int c_stride, const double *mu,
               const int32_t *offsets, const int32_t *tokens, int64_t t_stride, int n_sink,
               int64_t pending_begin, int64_t n_pending, int B, int32_t *idx, int32_t *n_sel,
               double *scores);
void orc_attn(int H, int G, int d, const double *q, const double *K, const double *V,
              int64_t kv_stride, const int32_t *idx, const int32_t *n_sel, int B, double scale,
              double *o);
void orc_dense_attn(int H, int G, int d, const double *q, const double *K, const double *V,
                    int64_t kv_stride, int64_t L, double scale, double *o);
double orc_bf16_round_value(double x);

static uint64_t st = 0x9E3779B97F4A7C15ull;
static double rnd(void)   /* uniform in [-1, 1) from a 64-bit LCG */
{
    st = st * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(st >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}

int main(void)
{
    enum { H = 2, G = 2, D = 128, L = 300, NS = 16, C = 7, IT = 4, B = 64 };
    const int Lp = L - NS;
    double *K = malloc(sizeof(double) * H * L * D), *V = malloc(sizeof(double) * H * L * D);
    double *q = malloc(sizeof(double) * H * G * D);
    for (int i = 0; i < H * L * D; ++i) K[i] = 3.0 * rnd(), V[i] = rnd();
    for (int i = 0; i < H * G * D; ++i) q[i] = rnd();
    for (int i = 0; i < D; ++i) K[(NS + 5) * D + i] = 0.0;        /* a zero key */
    double sum = 0.0;

    double *u = malloc(sizeof(double) * L * D);
    for (int mode = 0; mode < 2; ++mode) {
        orc_unit_rows(L, D, K, mode, u);
        for (int i = 0; i < L * D; ++i) sum += u[i];
    }
    double *mu = malloc(sizeof(double) * H * C * D), *mu2 = malloc(sizeof(double) * C * D);
    int32_t *as = malloc(sizeof(int32_t) * H * L), *off = malloc(sizeof(int32_t) * H * (C + 1));
    int32_t *tok = malloc(sizeof(int32_t) * H * Lp);
    double *mg = malloc(sizeof(double) * L), *tr = malloc(sizeof(double) * H * 2 * IT);
    int64_t *ch = malloc(sizeof(int64_t) * H * IT);
    orc_init_centroids(L, D, K, NS, C, mu);
    for (int metric = 0; metric < 3; ++metric)
        for (int mode = 0; mode < 2; ++mode) {
            orc_assign_metric(L, D, K, NS, C, mu, metric, mode, as, mg);
            orc_csr(L, NS, C, as, 1000, off, tok);
            orc_update(L, D, K, NS, C, as, mu, mode, mu2);
            sum += orc_objective(L, D, K, NS, as, mu2) + off[C] + tok[Lp - 1];
            orc_cluster_metric(metric, mode, H, L, D, K, NS, C, IT, 0, mu, as, off, tok,
                               metric == 0 ? tr : NULL, ch);
            sum += mu[H * C * D - 1] + (double)ch[H * IT - 1];
        }
    int32_t *idx = malloc(sizeof(int32_t) * H * B), ns[H];
    double *sc = malloc(sizeof(double) * H * C), *o = malloc(sizeof(double) * H * G * D);
    for (int np = 0; np < 3; ++np) {
        if (orc_select(H, G, D, q, C, C, mu, off, tok, Lp, NS, L - np, np, B, idx, ns, sc) != 0)
            return 2;
        orc_attn(H, G, D, q, K, V, L, idx, ns, B, 0.0, o);
        for (int i = 0; i < H * G * D; ++i) sum += o[i];
    }
    if (orc_select(H, G, D, q, C, C, mu, off, tok, Lp, NS, 0, 0, NS - 1, idx, ns, sc) != -1)
        return 3;
    orc_dense_attn(H, G, D, q, K, V, L, L, 0.0, o);
    for (int i = 0; i < H * G * D; ++i) sum += o[i];
    sum += orc_bf16_round_value(1.0 / 3.0);
    printf("checksum %.17g\n", sum);
    free(K); free(V); free(q); free(u); free(mu); free(mu2); free(as); free(off); free(tok);
    free(mg); free(tr); free(ch); free(idx); free(sc); free(o);
    return isfinite(sum) ? 0 : 4;
}
