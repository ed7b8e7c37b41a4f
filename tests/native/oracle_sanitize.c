/* Drives every routine of oracle/oracle.c once on small inputs, for a build
 * with AddressSanitizer and UndefinedBehaviorSanitizer (any report aborts).
 * Also checks the printed anchor row of flash_attention_numpy.py (scale 1:
 * row 0 of O is [0.910, 0.755] to three decimals). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_dense_fwd(const double *, const double *, const double *, double *, double *, int64_t,
                     int64_t, int64_t, int64_t, int64_t, int64_t, double, int, int64_t,
                     const int64_t *, int64_t, int);
int oracle_online_fwd(const double *, const double *, const double *, double *, double *,
                      int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, double, int, int64_t,
                      int64_t, const int64_t *, int64_t, int);
int oracle_dense_bwd(const double *, const double *, const double *, const double *, double *,
                     double *, double *, double *, double *, double *, int64_t, int64_t, int64_t,
                     int64_t, int64_t, int64_t, double, int, int64_t, const int64_t *, int64_t,
                     int);
int oracle_bwd_query_rows(const double *, const double *, const double *, const double *,
                          double *, double *, double *, double *, int64_t, int64_t, int64_t,
                          int64_t, int64_t, int64_t, double, int, int64_t, const int64_t *,
                          int64_t, int);
int oracle_bwd_key_rows(const double *, const double *, const double *, const double *,
                        const double *, const double *, double *, double *, int64_t, int64_t,
                        int64_t, int64_t, int64_t, int64_t, double, int, int64_t,
                        const int64_t *, int64_t, int);
void oracle_state(const double *, const double *, int64_t, int64_t, double *, double *, double *);
void oracle_merge(double, double, const double *, double, double, const double *, int64_t,
                  double *, double *, double *);
int oracle_split_decode(const double *, const double *, const double *, double *, double *,
                        double *, double *, double *, int64_t, int64_t, int64_t, int64_t, int64_t,
                        int64_t, int64_t, double, const int64_t *, int64_t, int);

static double *randn(int64_t n, unsigned *seed)
{
    double *a = (double *)malloc((size_t)n * sizeof(double));
    for (int64_t i = 0; i < n; ++i) a[i] = (double)rand_r(seed) / RAND_MAX - 0.5;
    return a;
}

int main(void)
{
    int bad = 0;
    /* the 3 x 2 anchor, unscaled */
    const double Q[] = {1, 0, 0, 2, 1, 1}, K[] = {1, 1, 0, 1, 2, 0}, V[] = {1, 0, 0, 1, 1, 1};
    double O[6], L[3];
    bad |= oracle_dense_fwd(Q, K, V, O, L, 1, 1, 3, 3, 2, 2, 1.0, 0, 0, NULL, 0, 2);
    if (fabs(O[0] - 0.910) > 5e-4 || fabs(O[1] - 0.755) > 5e-4) bad |= 1;
    for (int64_t b = 1; b <= 4; ++b) {
        double O2[6], L2[3];
        bad |= oracle_online_fwd(Q, K, V, O2, L2, 1, 1, 3, 3, 2, 2, 1.0, (int)(b & 1), 0, b,
                                 NULL, 0, 3);
    }
    /* random shapes with causal offsets, rows subsets and every backward */
    unsigned seed = 7;
    const int64_t B = 2, H = 3, Nq = 9, Nk = 13, d = 5, dv = 4, n = 5;
    double *q = randn(B * H * Nq * d, &seed), *k = randn(B * H * Nk * d, &seed);
    double *v = randn(B * H * Nk * dv, &seed), *g = randn(B * H * Nq * dv, &seed);
    double *o = malloc(sizeof(double) * B * H * Nq * dv), *l = malloc(sizeof(double) * B * H * Nq);
    double *dq = malloc(sizeof(double) * B * H * Nq * d), *dk = malloc(sizeof(double) * B * H * Nk * d);
    double *dvv = malloc(sizeof(double) * B * H * Nk * dv), *D = malloc(sizeof(double) * B * H * Nq);
    for (int causal = 0; causal < 2; ++causal) {
        int64_t qs = causal ? 4 : 0;
        const int64_t rows[] = {0, 17, 53, 8};
        bad |= oracle_dense_fwd(q, k, v, o, l, B, H, Nq, Nk, d, dv, 0.4, causal, qs, NULL, 0, 3);
        bad |= oracle_dense_fwd(q, k, v, o, l, B, H, Nq, Nk, d, dv, 0.4, causal, qs, rows, 4, 2);
        bad |= oracle_online_fwd(q, k, v, o, l, B, H, Nq, Nk, d, dv, 0.4, causal, qs, 3, NULL, 0,
                                 4);
        bad |= oracle_online_fwd(q, k, v, o, l, B, H, Nq, Nk, d, dv, 0.4, causal, qs, 5, rows, 4,
                                 1);
        bad |= oracle_dense_bwd(q, k, v, g, dq, dk, dvv, o, l, D, B, H, Nq, Nk, d, dv, 0.4,
                                causal, qs, NULL, 0, 3);
        const int64_t heads[] = {5, 0};
        bad |= oracle_dense_bwd(q, k, v, g, dq, dk, dvv, o, l, D, B, H, Nq, Nk, d, dv, 0.4,
                                causal, qs, heads, 2, 2);
        bad |= oracle_bwd_query_rows(q, k, v, g, dq, o, l, D, B, H, Nq, Nk, d, dv, 0.4, causal,
                                     qs, rows, 4, 2);
        /* L and D of every row for the key-row routine */
        double *Lall = malloc(sizeof(double) * B * H * Nq), *Dall = malloc(sizeof(double) * B * H * Nq);
        int64_t *all = malloc(sizeof(int64_t) * B * H * Nq);
        for (int64_t r = 0; r < B * H * Nq; ++r) all[r] = r;
        double *dq2 = malloc(sizeof(double) * B * H * Nq * d), *o2 = malloc(sizeof(double) * B * H * Nq * dv);
        bad |= oracle_bwd_query_rows(q, k, v, g, dq2, o2, Lall, Dall, B, H, Nq, Nk, d, dv, 0.4,
                                     causal, qs, all, B * H * Nq, 4);
        const int64_t keys[] = {0, 12, 77, 40};
        bad |= oracle_bwd_key_rows(q, k, v, g, Lall, Dall, dk, dvv, B, H, Nq, Nk, d, dv, 0.4,
                                   causal, qs, keys, 4, 2);
        free(Lall), free(Dall), free(all), free(dq2), free(o2);
    }
    /* states, merges and split decoding, empty splits included */
    double m1, l1, o1[4], m2, l2, o2[4], m3, l3, o3[4];
    const double s[] = {0.3, -1.0, 2.0};
    oracle_state(s, v, 3, dv, &m1, &l1, o1);
    oracle_state(s, v, 0, dv, &m2, &l2, o2);
    oracle_merge(m1, l1, o1, m2, l2, o2, dv, &m3, &l3, o3);
    oracle_merge(m2, l2, o2, m2, l2, o2, dv, &m3, &l3, o3);
    if (!isinf(m3) || l3 != 0.0) bad |= 1;
    double *pm = malloc(sizeof(double) * B * H * Nq * 20), *pl = malloc(sizeof(double) * B * H * Nq * 20);
    double *po = malloc(sizeof(double) * B * H * Nq * 20 * dv);
    for (int64_t ns = 1; ns <= 20; ns += 19)
        bad |= oracle_split_decode(q, k, v, o, l, pm, pl, po, B, H, Nq, Nk, d, dv, ns, 0.4, NULL,
                                   0, 3);
    free(q), free(k), free(v), free(g), free(o), free(l), free(dq), free(dk), free(dvv), free(D);
    free(pm), free(pl), free(po);
    if (bad) {
        printf("oracle routines reported an error\n");
        return 1;
    }
    printf("ok\n");
    return 0;
}
