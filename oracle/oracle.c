/*
 * oracle.c -- plain, slow fp64 CPU reference for exact softmax attention.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker that the GPU library is
 * compared against.  Only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg load it.  It shares no code, header, table or constant with
 * the HIP library, and the HIP library never loads it.
 *
 * Every array is fp64, contiguous, laid out [B][H][N][d] with d fastest.
 * Scores are S_ij = scale * sum_c Q_ic K_jc.  With `causal` set, key j is
 * visible to query i iff j <= q_start + i (absolute positions; q_start = 0 is
 * the top-left alignment).  The log-sum-exp L is the natural logarithm.
 *
 * Sources (the pages):
 *   attention_kernels.py (CMU 15-779 lecture 5): SoftmaxState, merge_states,
 *     state_of_scores, standard_attention, flash_backward, flash_decode.
 *   lab.py (hs-black FlashAttention post): dense, tiled, backward.
 *   model.py (tensorviz flash-attention): TiledAttention.
 *
 * Planted mistakes: building with -DORACLE_PLANT_<NAME> swaps one step for a
 * plausible error (NO_RESCALE, NO_MASK, NO_SCALE, BWD_SIGN, BWD_OPERAND,
 * MERGE_NO_REBASE, SPLIT_OVERLAP).  The CPU self-tests build these variants to
 * show that the pins fail on them; the normal build defines none of them.
 *
 * Routines:
 *   oracle_dense_fwd   -- the definition: whole score row, max, exp, sum.
 *   oracle_online_fwd  -- the per-row online softmax over key blocks.
 *   oracle_dense_bwd   -- dQ, dK, dV of <O, dO> by the softmax Jacobian.
 *   oracle_bwd_query_rows / oracle_bwd_key_rows -- the same for chosen rows.
 *   oracle_state / oracle_merge -- (m, l, o) segment summaries and their merge.
 *   oracle_split_decode -- split the keys, summarise each split, fold merges.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* A minimal thread pool over an index range [0, n).                         */
/* ------------------------------------------------------------------------ */
typedef void (*work_fn)(void *ctx, int64_t item);

struct pool {
    work_fn fn;
    void *ctx;
    int64_t n;
    int64_t next; /* shared counter, advanced atomically */
};

static void *pool_worker(void *arg)
{
    struct pool *p = (struct pool *)arg;
    for (;;) {
        int64_t item = __atomic_fetch_add(&p->next, 1, __ATOMIC_RELAXED);
        if (item >= p->n) break;
        p->fn(p->ctx, item);
    }
    return NULL;
}

static void parallel_for(int64_t n, int nthreads, work_fn fn, void *ctx)
{
    struct pool p = {fn, ctx, n, 0};
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads == 1 || n <= 1) {
        pool_worker(&p);
        return;
    }
    pthread_t tid[256];
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        if (pthread_create(&tid[t], NULL, pool_worker, &p) != 0) break;
        ++started;
    }
    if (started == 0) pool_worker(&p);
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
}

/* Number of keys visible to query i (keys 0 .. nvis-1). */
static int64_t visible_keys(int64_t i, int64_t Nk, int causal, int64_t q_start)
{
#ifdef ORACLE_PLANT_NO_MASK
    causal = 0;
#endif
    if (!causal) return Nk;
    int64_t last = q_start + i; /* the last visible key position */
    if (last < 0) return 0;
    return last + 1 < Nk ? last + 1 : Nk;
}

static double dot(const double *a, const double *b, int64_t n)
{
    double s = 0.0;
    for (int64_t c = 0; c < n; ++c) s += a[c] * b[c];
    return s;
}

/* ------------------------------------------------------------------------ */
/* R1: the definition.  For one query row, build the whole visible score     */
/* row, take its maximum, exponentiate, sum, and divide once.                */
/* standard_attention (attention_kernels.py) and dense (lab.py).            */
/* ------------------------------------------------------------------------ */
struct fwd_args {
    const double *Q, *K, *V;
    double *O, *L;
    int64_t H, Nq, Nk, d, dv;
    double scale;
    int causal;
    int64_t q_start;
    const int64_t *rows; /* NULL: all rows; else flat row ids (bh * Nq + i) */
    int64_t block;       /* online routine only */
    int status;          /* set to 1 if a row sees no key */
};

static void dense_row(void *vctx, int64_t item)
{
    struct fwd_args *a = (struct fwd_args *)vctx;
    int64_t row = a->rows ? a->rows[item] : item;
    int64_t bh = row / a->Nq, i = row % a->Nq;
    const double *q = a->Q + row * a->d;
    const double *K = a->K + bh * a->Nk * a->d;
    const double *V = a->V + bh * a->Nk * a->dv;
    double *o = a->O + item * a->dv;
    int64_t nvis = visible_keys(i, a->Nk, a->causal, a->q_start);
    if (nvis == 0) {
        a->status = 1;
        for (int64_t c = 0; c < a->dv; ++c) o[c] = NAN;
        a->L[item] = NAN;
        return;
    }
    double *s = (double *)malloc((size_t)nvis * sizeof(double));
    for (int64_t j = 0; j < nvis; ++j) s[j] = a->scale * dot(q, K + j * a->d, a->d);
#ifdef ORACLE_PLANT_NO_SCALE
    for (int64_t j = 0; j < nvis; ++j) s[j] = dot(q, K + j * a->d, a->d);
#endif
    double m = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j) m = s[j] > m ? s[j] : m;
    double l = 0.0;
    for (int64_t j = 0; j < nvis; ++j) l += exp(s[j] - m);
    for (int64_t c = 0; c < a->dv; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        double p = exp(s[j] - m) / l;
        for (int64_t c = 0; c < a->dv; ++c) o[c] += p * V[j * a->dv + c];
    }
    a->L[item] = m + log(l);
    free(s);
}

/* Full forward when rows == NULL (O, L sized [B*H*Nq][dv], [B*H*Nq]); else
 * only the listed flat rows, packed in list order.  Returns 0, or 1 when a
 * row sees no key (its outputs are NaN). */
int oracle_dense_fwd(const double *Q, const double *K, const double *V, double *O, double *L,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                     double scale, int causal, int64_t q_start, const int64_t *rows,
                     int64_t nrows, int nthreads)
{
    struct fwd_args a = {Q, K, V, O, L, H, Nq, Nk, d, dv, scale, causal, q_start, rows, 0, 0};
    int64_t n = rows ? nrows : B * H * Nq;
    parallel_for(n, nthreads, dense_row, &a);
    return a.status;
}

/* ------------------------------------------------------------------------ */
/* R2: the per-row online softmax.  Keys are visited `block` at a time; the  */
/* running maximum m, denominator l and unnormalised numerator are rescaled  */
/* by exp(m_old - m_new) whenever a block raises the maximum; the first      */
/* block (l == 0) takes no rescale.  One division at the end.                */
/* tiled (lab.py); the same recurrence as TiledAttention (model.py) and      */
/* flash_forward (attention_kernels.py).                                     */
/* ------------------------------------------------------------------------ */
static void online_row(void *vctx, int64_t item)
{
    struct fwd_args *a = (struct fwd_args *)vctx;
    int64_t row = a->rows ? a->rows[item] : item;
    int64_t bh = row / a->Nq, i = row % a->Nq;
    const double *q = a->Q + row * a->d;
    const double *K = a->K + bh * a->Nk * a->d;
    const double *V = a->V + bh * a->Nk * a->dv;
    double *o = a->O + item * a->dv;
    /* The visible keys are the prefix 0 .. nvis-1; it is cut into blocks of
     * `block` keys (the last one shorter), visited in order. */
    int64_t nvis = visible_keys(i, a->Nk, a->causal, a->q_start);
    if (nvis == 0) {
        a->status = 1;
        for (int64_t c = 0; c < a->dv; ++c) o[c] = NAN;
        a->L[item] = NAN;
        return;
    }
    double *num = (double *)calloc((size_t)a->dv, sizeof(double));
    double *s = (double *)malloc((size_t)a->block * sizeof(double));
    /* running state after the blocks seen so far: maximum m, denominator l,
     * unnormalised numerator num (all three relative to m) */
    double m = -INFINITY, l = 0.0;
    for (int64_t j0 = 0; j0 < nvis; j0 += a->block) {
        int64_t nb = nvis - j0 < a->block ? nvis - j0 : a->block;
        double bmax = -INFINITY;
        for (int64_t t = 0; t < nb; ++t) {
            s[t] = a->scale * dot(q, K + (j0 + t) * a->d, a->d);
            if (s[t] > bmax) bmax = s[t];
        }
        double m_new = bmax > m ? bmax : m;
        /* old state rebased onto the new maximum; there is none before the
         * first block, so nothing is carried (and -inf - -inf never formed) */
        double alpha = j0 == 0 ? 0.0 : exp(m - m_new);
#ifdef ORACLE_PLANT_NO_RESCALE
        alpha = 1.0;
#endif
        l *= alpha;
        for (int64_t c = 0; c < a->dv; ++c) num[c] *= alpha;
        for (int64_t t = 0; t < nb; ++t) {
            double e = exp(s[t] - m_new);
            l += e;
            for (int64_t c = 0; c < a->dv; ++c) num[c] += e * V[(j0 + t) * a->dv + c];
        }
        m = m_new;
    }
    for (int64_t c = 0; c < a->dv; ++c) o[c] = num[c] / l;
    a->L[item] = m + log(l);
    free(num);
    free(s);
}

/* All rows when rows == NULL, else the listed flat rows packed in list order
 * (as oracle_dense_fwd). */
int oracle_online_fwd(const double *Q, const double *K, const double *V, double *O, double *L,
                      int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                      double scale, int causal, int64_t q_start, int64_t block,
                      const int64_t *rows, int64_t nrows, int nthreads)
{
    if (block < 1) return 2;
    struct fwd_args a = {Q, K, V, O, L, H, Nq, Nk, d, dv, scale, causal, q_start, rows, block, 0};
    parallel_for(rows ? nrows : B * H * Nq, nthreads, online_row, &a);
    return a.status;
}

/* ------------------------------------------------------------------------ */
/* R3: backward of the scalar <O, dO>.  Per head: P_ij = exp(S_ij - L_i) on   */
/* the visible keys, D_i = sum_c dO_ic O_ic, dP_ij = dO_i . V_j,             */
/* dS_ij = P_ij (dP_ij - D_i), dQ_i = scale sum_j dS_ij K_j,                 */
/* dK_j = scale sum_i dS_ij Q_i, dV_j = sum_i P_ij dO_i.                     */
/* flash_backward docstring (attention_kernels.py) gives the Jacobian step;  */
/* backward (lab.py) the same formulas row by row.  O and L are this         */
/* oracle's own fp64 forward, computed here from the definition.             */
/* ------------------------------------------------------------------------ */
struct bwd_args {
    const double *Q, *K, *V, *dO;
    double *dQ, *dK, *dV, *O, *L, *Dv;
    int64_t H, Nq, Nk, d, dv;
    double scale;
    int causal;
    int64_t q_start;
    const int64_t *heads; /* NULL: all heads; else flat head ids (b * H + h) */
    int status;
};

static void bwd_head(void *vctx, int64_t item)
{
    struct bwd_args *a = (struct bwd_args *)vctx;
    int64_t bh = a->heads ? a->heads[item] : item;
    int64_t Nq = a->Nq, Nk = a->Nk, d = a->d, dv = a->dv;
    const double *Q = a->Q + bh * Nq * d;
    const double *K = a->K + bh * Nk * d;
    const double *V = a->V + bh * Nk * dv;
    const double *dO = a->dO + bh * Nq * dv;
    double *dQ = a->dQ + item * Nq * d;
    double *dK = a->dK + item * Nk * d;
    double *dV = a->dV + item * Nk * dv;
    double *O = a->O + item * Nq * dv;
    double *L = a->L + item * Nq;
    double *Dv = a->Dv + item * Nq;
    double *s = (double *)malloc((size_t)Nk * sizeof(double));
    memset(dK, 0, (size_t)(Nk * d) * sizeof(double));
    memset(dV, 0, (size_t)(Nk * dv) * sizeof(double));
    for (int64_t i = 0; i < Nq; ++i) {
        const double *q = Q + i * d;
        const double *g = dO + i * dv;
        double *o = O + i * dv;
        double *dq = dQ + i * d;
        int64_t nvis = visible_keys(i, Nk, a->causal, a->q_start);
        for (int64_t c = 0; c < d; ++c) dq[c] = 0.0;
        if (nvis == 0) {
            a->status = 1;
            for (int64_t c = 0; c < dv; ++c) o[c] = NAN;
            L[i] = NAN;
            Dv[i] = NAN;
            continue;
        }
        /* forward row from the definition */
        double m = -INFINITY;
        for (int64_t j = 0; j < nvis; ++j) {
            s[j] = a->scale * dot(q, K + j * d, d);
            m = s[j] > m ? s[j] : m;
        }
        double l = 0.0;
        for (int64_t j = 0; j < nvis; ++j) l += exp(s[j] - m);
        double lse = m + log(l);
        for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
        for (int64_t j = 0; j < nvis; ++j) {
            double p = exp(s[j] - lse);
            for (int64_t c = 0; c < dv; ++c) o[c] += p * V[j * dv + c];
        }
        L[i] = lse;
        double D = dot(g, o, dv);
        Dv[i] = D;
        /* gradient row */
        for (int64_t j = 0; j < nvis; ++j) {
            double p = exp(s[j] - lse);
            double dp = dot(g, V + j * dv, dv);
            double ds = p * (dp - D);
#ifdef ORACLE_PLANT_BWD_SIGN
            ds = p * (dp + D);
#endif
            for (int64_t c = 0; c < d; ++c) {
#ifdef ORACLE_PLANT_BWD_OPERAND
                dq[c] += a->scale * ds * q[c];
#else
                dq[c] += a->scale * ds * K[j * d + c];
#endif
                dK[j * d + c] += a->scale * ds * q[c];
            }
            for (int64_t c = 0; c < dv; ++c) dV[j * dv + c] += p * g[c];
        }
    }
    free(s);
}

/* Gradients for all heads (heads == NULL) or for the listed heads, packed in
 * list order.  O, L, Dv receive the oracle's own forward and D = rowsum(dO*O). */
int oracle_dense_bwd(const double *Q, const double *K, const double *V, const double *dO,
                     double *dQ, double *dK, double *dV, double *O, double *L, double *Dv,
                     int64_t B, int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv,
                     double scale, int causal, int64_t q_start, const int64_t *heads,
                     int64_t nheads, int nthreads)
{
    struct bwd_args a = {Q, K, V, dO, dQ, dK, dV, O, L, Dv, H, Nq, Nk, d, dv,
                         scale, causal, q_start, heads, 0};
    parallel_for(heads ? nheads : B * H, nthreads, bwd_head, &a);
    return a.status;
}

/* ------------------------------------------------------------------------ */
/* R3 restricted to chosen rows, for checks at sizes where the whole         */
/* backward is too slow.  The same formulas as bwd_head:                     */
/*   query row i:  O_i, L_i from the definition, D_i = dO_i . O_i,           */
/*                 dQ_i = scale sum_j P_ij (dO_i . V_j - D_i) K_j;           */
/*   key row j:    dV_j = sum_i P_ij dO_i,                                    */
/*                 dK_j = scale sum_i P_ij (dO_i . V_j - D_i) Q_i,            */
/*                 over the queries i that see key j, with P_ij =             */
/*                 exp(S_ij - L_i) and L_i, D_i given by the caller (this     */
/*                 oracle's own forward of those queries).                    */
/* flash_backward (attention_kernels.py); backward (lab.py).                 */
/* ------------------------------------------------------------------------ */
struct rows_args {
    const double *Q, *K, *V, *dO, *Lin, *Din;
    double *out1, *out2, *out3, *out4;
    int64_t H, Nq, Nk, d, dv;
    double scale;
    int causal;
    int64_t q_start;
    const int64_t *rows;
    int status;
};

static void bwd_query_row(void *vctx, int64_t item)
{
    struct rows_args *a = (struct rows_args *)vctx;
    int64_t row = a->rows[item];
    int64_t bh = row / a->Nq, i = row % a->Nq;
    int64_t Nk = a->Nk, d = a->d, dv = a->dv;
    const double *q = a->Q + row * d;
    const double *g = a->dO + row * dv;
    const double *K = a->K + bh * Nk * d;
    const double *V = a->V + bh * Nk * dv;
    double *dq = a->out1 + item * d, *o = a->out2 + item * dv;
    int64_t nvis = visible_keys(i, Nk, a->causal, a->q_start);
    if (nvis == 0) {
        a->status = 1;
        for (int64_t c = 0; c < d; ++c) dq[c] = NAN;
        for (int64_t c = 0; c < dv; ++c) o[c] = NAN;
        a->out3[item] = NAN;
        a->out4[item] = NAN;
        return;
    }
    double *s = (double *)malloc((size_t)nvis * sizeof(double));
    double m = -INFINITY;
    for (int64_t j = 0; j < nvis; ++j) {
        s[j] = a->scale * dot(q, K + j * d, d);
        if (s[j] > m) m = s[j];
    }
    double l = 0.0;
    for (int64_t j = 0; j < nvis; ++j) l += exp(s[j] - m);
    double lse = m + log(l);
    for (int64_t c = 0; c < dv; ++c) o[c] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        double p = exp(s[j] - lse);
        for (int64_t c = 0; c < dv; ++c) o[c] += p * V[j * dv + c];
    }
    double D = dot(g, o, dv);
    for (int64_t c = 0; c < d; ++c) dq[c] = 0.0;
    for (int64_t j = 0; j < nvis; ++j) {
        double p = exp(s[j] - lse);
        double ds = p * (dot(g, V + j * dv, dv) - D);
        for (int64_t c = 0; c < d; ++c) dq[c] += a->scale * ds * K[j * d + c];
    }
    a->out3[item] = lse;
    a->out4[item] = D;
    free(s);
}

static void bwd_key_row(void *vctx, int64_t item)
{
    struct rows_args *a = (struct rows_args *)vctx;
    int64_t key = a->rows[item];
    int64_t bh = key / a->Nk, j = key % a->Nk;
    int64_t Nq = a->Nq, d = a->d, dv = a->dv;
    const double *k = a->K + key * d;
    const double *v = a->V + key * dv;
    const double *Q = a->Q + bh * Nq * d;
    const double *dO = a->dO + bh * Nq * dv;
    const double *L = a->Lin + bh * Nq, *Dv = a->Din + bh * Nq;
    double *dk = a->out1 + item * d, *dvr = a->out2 + item * dv;
    for (int64_t c = 0; c < d; ++c) dk[c] = 0.0;
    for (int64_t c = 0; c < dv; ++c) dvr[c] = 0.0;
    for (int64_t i = 0; i < Nq; ++i) {
        if (j >= visible_keys(i, a->Nk, a->causal, a->q_start)) continue;
        const double *g = dO + i * dv;
        double p = exp(a->scale * dot(Q + i * d, k, d) - L[i]);
        double ds = p * (dot(g, v, dv) - Dv[i]);
        for (int64_t c = 0; c < d; ++c) dk[c] += a->scale * ds * Q[i * d + c];
        for (int64_t c = 0; c < dv; ++c) dvr[c] += p * g[c];
    }
}

/* dQ, O, L, D of the listed query rows (flat ids bh * Nq + i), packed in list
 * order: dQ [n][d], O [n][dv], L [n], D [n].  Returns 1 if a row sees no key. */
int oracle_bwd_query_rows(const double *Q, const double *K, const double *V, const double *dO,
                          double *dQ, double *O, double *L, double *Dv, int64_t B, int64_t H,
                          int64_t Nq, int64_t Nk, int64_t d, int64_t dv, double scale,
                          int causal, int64_t q_start, const int64_t *rows, int64_t nrows,
                          int nthreads)
{
    (void)B;
    struct rows_args a = {Q, K, V, dO, NULL, NULL, dQ, O, L, Dv, H, Nq, Nk, d, dv,
                          scale, causal, q_start, rows, 0};
    parallel_for(nrows, nthreads, bwd_query_row, &a);
    return a.status;
}

/* dK [n][d] and dV [n][dv] of the listed key rows (flat ids bh * Nk + j),
 * packed in list order, from the caller's L and D ([B*H*Nq] each: this
 * oracle's forward of every query of the heads involved). */
int oracle_bwd_key_rows(const double *Q, const double *K, const double *V, const double *dO,
                        const double *L, const double *Dv, double *dK, double *dV, int64_t B,
                        int64_t H, int64_t Nq, int64_t Nk, int64_t d, int64_t dv, double scale,
                        int causal, int64_t q_start, const int64_t *keys, int64_t nkeys,
                        int nthreads)
{
    (void)B;
    struct rows_args a = {Q, K, V, dO, L, Dv, dK, dV, NULL, NULL, H, Nq, Nk, d, dv,
                          scale, causal, q_start, keys, 0};
    parallel_for(nkeys, nthreads, bwd_key_row, &a);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* R5: segment summaries.  state(s, v) = (m, l, o) with m = max s,           */
/* l = sum exp(s - m), o = sum exp(s - m) v (unnormalised); an all -inf or   */
/* empty segment is the identity (-inf, 0, 0).  merge takes the larger m and */
/* rebases both sides onto it; when both m are -inf the base is 0, so no     */
/* -inf - (-inf) is ever formed.                                             */
/* SoftmaxState, merge_states, state_of_scores (attention_kernels.py).       */
/* ------------------------------------------------------------------------ */
void oracle_state(const double *s, const double *v, int64_t n, int64_t dv, double *m_out,
                  double *l_out, double *o_out)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) m = s[j] > m ? s[j] : m;
    double base = isinf(m) ? 0.0 : m;
    double l = 0.0;
    for (int64_t c = 0; c < dv; ++c) o_out[c] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        double e = exp(s[j] - base);
        l += e;
        for (int64_t c = 0; c < dv; ++c) o_out[c] += e * v[j * dv + c];
    }
    *m_out = m;
    *l_out = l;
}

void oracle_merge(double ma, double la, const double *oa, double mb, double lb, const double *ob,
                  int64_t dv, double *m_out, double *l_out, double *o_out)
{
    double m = ma > mb ? ma : mb;
    double base = isinf(m) ? 0.0 : m;
    double ca = exp(ma - base), cb = exp(mb - base);
#ifdef ORACLE_PLANT_MERGE_NO_REBASE
    ca = 1.0;
    cb = 1.0;
#endif
    *m_out = m;
    *l_out = la * ca + lb * cb;
    for (int64_t c = 0; c < dv; ++c) o_out[c] = oa[c] * ca + ob[c] * cb;
}

/* ------------------------------------------------------------------------ */
/* R6: split-KV decoding.  Split s covers keys [floor(Nk*s/n), floor(Nk*(s+1)/n)); */
/* each split is summarised with oracle_state (an empty split is the         */
/* identity), the summaries are folded left to right with oracle_merge, and  */
/* the result is O = o / l, L = m + log l.  No causal mask.                  */
/* flash_decode (attention_kernels.py).                                      */
/* ------------------------------------------------------------------------ */
struct dec_args {
    const double *Q, *K, *V;
    double *O, *L, *pm, *pl, *po;
    int64_t H, Nq, Nk, d, dv, n_split;
    double scale;
    const int64_t *heads;
};

static void decode_row(void *vctx, int64_t item)
{
    struct dec_args *a = (struct dec_args *)vctx;
    int64_t Nq = a->Nq, Nk = a->Nk, d = a->d, dv = a->dv, n = a->n_split;
    int64_t hi = item / Nq, i = item % Nq;
    int64_t bh = a->heads ? a->heads[hi] : hi;
    const double *q = a->Q + (bh * Nq + i) * d;
    const double *K = a->K + bh * Nk * d;
    const double *V = a->V + bh * Nk * dv;
    double *pm = a->pm + item * n, *pl = a->pl + item * n, *po = a->po + item * n * dv;
    double *s = (double *)malloc((size_t)(Nk > 0 ? Nk : 1) * sizeof(double));
    for (int64_t sp = 0; sp < n; ++sp) {
        int64_t j0 = Nk * sp / n, j1 = Nk * (sp + 1) / n;
#ifdef ORACLE_PLANT_SPLIT_OVERLAP
        if (j0 > 0) j0 -= 1;
#endif
        for (int64_t j = j0; j < j1; ++j) s[j - j0] = a->scale * dot(q, K + j * d, d);
        oracle_state(s, V + j0 * dv, j1 - j0, dv, &pm[sp], &pl[sp], po + sp * dv);
    }
    double m = pm[0], l = pl[0];
    double *o = (double *)malloc((size_t)dv * sizeof(double));
    double *t = (double *)malloc((size_t)dv * sizeof(double));
    memcpy(o, po, (size_t)dv * sizeof(double));
    for (int64_t sp = 1; sp < n; ++sp) {
        double m2, l2;
        oracle_merge(m, l, o, pm[sp], pl[sp], po + sp * dv, dv, &m2, &l2, t);
        m = m2;
        l = l2;
        memcpy(o, t, (size_t)dv * sizeof(double));
    }
    for (int64_t c = 0; c < dv; ++c) a->O[item * dv + c] = o[c] / l;
    a->L[item] = m + log(l);
    free(s);
    free(o);
    free(t);
}

/* O [nh*Nq][dv], L [nh*Nq], pm/pl [nh*Nq][n_split], po [nh*Nq][n_split][dv],
 * where nh = B*H (heads == NULL) or nheads (listed flat heads b*H + h). */
int oracle_split_decode(const double *Q, const double *K, const double *V, double *O, double *L,
                        double *pm, double *pl, double *po, int64_t B, int64_t H, int64_t Nq,
                        int64_t Nk, int64_t d, int64_t dv, int64_t n_split, double scale,
                        const int64_t *heads, int64_t nheads, int nthreads)
{
    if (n_split < 1) return 2;
    struct dec_args a = {Q, K, V, O, L, pm, pl, po, H, Nq, Nk, d, dv, n_split, scale, heads};
    parallel_for((heads ? nheads : B * H) * Nq, nthreads, decode_row, &a);
    return 0;
}
