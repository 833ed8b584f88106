/*
 * attn_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow CPU reference of exact scaled-dot-product attention in fp64.
 * Only the tests, the smoke check and the benchmark's CPU-baseline leg use
 * it; the library under exact_attention_39_amd/ never links or calls it and
 * shares no code with it.
 *
 * What it computes.  The FlashAttention-4 pages (hyper.ai news story, single
 * paragraph; gist.science explainer "FlashAttention-4: Algorithm and Kernel
 * Pipelining Co-Design for Asymmetric Hardware Scaling", technical summary,
 * "Probleemstelling") describe a faster implementation of the standard
 * attention of a Transformer that leaves the mathematical result unchanged.
 * The pages never print the formula, so this file writes out the standard
 * definition (the plainest reading of pages that state the method in words):
 *
 *   s_ij   = scale * sum_k q_ik k_jk
 *   A_i    = { j : j <= i } when causal (top-left aligned), else all j
 *   m_i    = max_{j in A_i} s_ij
 *   Z_i    = sum_{j in A_i} exp(s_ij - m_i)
 *   p_ij   = exp(s_ij - m_i) / Z_i  for j in A_i, 0 otherwise
 *   o_i    = sum_j p_ij v_j
 *   lse_i  = m_i + ln Z_i                      (natural log)
 *
 * and its gradient for L = sum(dO * O) by the chain rule:
 *
 *   D_i    = sum_k dO_ik o_ik
 *   dP_ij  = sum_k dO_ik v_jk
 *   dS_ij  = p_ij (dP_ij - D_i)
 *   dV_j   = sum_i p_ij dO_i
 *   dQ_i   = scale * sum_j dS_ij k_j
 *   dK_j   = scale * sum_i dS_ij q_i
 *
 * Every array is row-major double.  A "head" is [S][d]; full tensors are
 * [BH][S][d] with BH = batch * heads.  No tiling, no online softmax, no
 * polynomial exp: rows are processed one at a time with two passes (max,
 * then sum).  Threads split independent heads or independent rows; partial
 * column sums from row-split threads are added in thread order, so results
 * do not depend on timing.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

static double dot(const double *a, const double *b, int64_t d) {
    double acc = 0.0;
    for (int64_t k = 0; k < d; ++k) acc += a[k] * b[k];
    return acc;
}

/* Number of keys row i may attend to: A_i is the prefix [0, n). */
static int64_t row_extent(int64_t i, int64_t S, int causal) {
    return causal ? i + 1 : S;
}

/*
 * Softmax row of query i against keys K[0..n).  On return p[0..n) holds
 * p_ij, and *m, *z hold m_i and Z_i.
 */
static void softmax_row(const double *qi, const double *K, int64_t n, int64_t d,
                        double scale, double *p, double *m, double *z) {
    double mx = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        p[j] = scale * dot(qi, K + j * d, d);
        if (p[j] > mx) mx = p[j];
    }
    double sum = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        p[j] = exp(p[j] - mx);
        sum += p[j];
    }
    for (int64_t j = 0; j < n; ++j) p[j] /= sum;
    *m = mx;
    *z = sum;
}

/* o_i = sum_j p_ij v_j over j < n. */
static void weighted_rows(const double *p, const double *V, int64_t n, int64_t d, double *o) {
    for (int64_t k = 0; k < d; ++k) o[k] = 0.0;
    for (int64_t j = 0; j < n; ++j) {
        const double *vj = V + j * d;
        for (int64_t k = 0; k < d; ++k) o[k] += p[j] * vj[k];
    }
}

static int resolve_threads(int nthreads) {
    if (nthreads > 0) return nthreads;
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    return n > 0 ? (int)n : 1;
}

/* ------------------------------------------------------------------ */
/* Forward over full tensors, threads split heads.                     */

typedef struct {
    const double *q, *k, *v;
    int64_t BH, S, d;
    double scale;
    int causal;
    double *o, *lse;
    int tid, nthreads;
    int err;
} fwd_job;

static void *fwd_worker(void *arg) {
    fwd_job *J = (fwd_job *)arg;
    double *p = (double *)malloc(sizeof(double) * (size_t)(J->S > 0 ? J->S : 1));
    if (!p) { J->err = 1; return NULL; }
    for (int64_t bh = J->tid; bh < J->BH; bh += J->nthreads) {
        const double *Q = J->q + bh * J->S * J->d;
        const double *K = J->k + bh * J->S * J->d;
        const double *V = J->v + bh * J->S * J->d;
        for (int64_t i = 0; i < J->S; ++i) {
            int64_t n = row_extent(i, J->S, J->causal);
            double m, z;
            softmax_row(Q + i * J->d, K, n, J->d, J->scale, p, &m, &z);
            weighted_rows(p, V, n, J->d, J->o + (bh * J->S + i) * J->d);
            J->lse[bh * J->S + i] = m + log(z);
        }
    }
    free(p);
    return NULL;
}

int oracle_attention_forward(const double *q, const double *k, const double *v,
                             int64_t BH, int64_t S, int64_t d, double scale, int causal,
                             double *o, double *lse, int nthreads) {
    int T = resolve_threads(nthreads);
    if (T > BH) T = BH > 0 ? (int)BH : 1;
    fwd_job *jobs = (fwd_job *)calloc((size_t)T, sizeof(fwd_job));
    pthread_t *th = (pthread_t *)calloc((size_t)T, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return 1; }
    for (int t = 0; t < T; ++t) {
        fwd_job j = {q, k, v, BH, S, d, scale, causal, o, lse, t, T, 0};
        jobs[t] = j;
        pthread_create(&th[t], NULL, fwd_worker, &jobs[t]);
    }
    int err = 0;
    for (int t = 0; t < T; ++t) { pthread_join(th[t], NULL); err |= jobs[t].err; }
    free(jobs); free(th);
    return err;
}

/* ------------------------------------------------------------------ */
/* Backward over full tensors, threads split heads.                    */

typedef struct {
    const double *q, *k, *v, *dO;
    int64_t BH, S, d;
    double scale;
    int causal;
    double *dq, *dk, *dv;
    int tid, nthreads;
    int err;
} bwd_job;

static void *bwd_worker(void *arg) {
    bwd_job *J = (bwd_job *)arg;
    const int64_t S = J->S, d = J->d;
    double *p = (double *)malloc(sizeof(double) * (size_t)(S > 0 ? S : 1));
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    if (!p || !o) { free(p); free(o); J->err = 1; return NULL; }
    for (int64_t bh = J->tid; bh < J->BH; bh += J->nthreads) {
        const double *Q = J->q + bh * S * d, *K = J->k + bh * S * d;
        const double *V = J->v + bh * S * d, *dO = J->dO + bh * S * d;
        double *dQ = J->dq + bh * S * d, *dK = J->dk + bh * S * d, *dV = J->dv + bh * S * d;
        memset(dQ, 0, sizeof(double) * (size_t)(S * d));
        memset(dK, 0, sizeof(double) * (size_t)(S * d));
        memset(dV, 0, sizeof(double) * (size_t)(S * d));
        for (int64_t i = 0; i < S; ++i) {
            int64_t n = row_extent(i, S, J->causal);
            double m, z;
            const double *qi = Q + i * d, *doi = dO + i * d;
            softmax_row(qi, K, n, d, J->scale, p, &m, &z);
            weighted_rows(p, V, n, d, o);
            double Di = dot(doi, o, d);
            for (int64_t j = 0; j < n; ++j) {
                double dP = dot(doi, V + j * d, d);
                double dS = p[j] * (dP - Di);
                for (int64_t c = 0; c < d; ++c) {
                    dV[j * d + c] += p[j] * doi[c];
                    dK[j * d + c] += J->scale * dS * qi[c];
                    dQ[i * d + c] += J->scale * dS * K[j * d + c];
                }
            }
        }
    }
    free(p); free(o);
    return NULL;
}

int oracle_attention_backward(const double *q, const double *k, const double *v, const double *dO,
                              int64_t BH, int64_t S, int64_t d, double scale, int causal,
                              double *dq, double *dk, double *dv, int nthreads) {
    int T = resolve_threads(nthreads);
    if (T > BH) T = BH > 0 ? (int)BH : 1;
    bwd_job *jobs = (bwd_job *)calloc((size_t)T, sizeof(bwd_job));
    pthread_t *th = (pthread_t *)calloc((size_t)T, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return 1; }
    for (int t = 0; t < T; ++t) {
        bwd_job j = {q, k, v, dO, BH, S, d, scale, causal, dq, dk, dv, t, T, 0};
        jobs[t] = j;
        pthread_create(&th[t], NULL, bwd_worker, &jobs[t]);
    }
    int err = 0;
    for (int t = 0; t < T; ++t) { pthread_join(th[t], NULL); err |= jobs[t].err; }
    free(jobs); free(th);
    return err;
}

/* ------------------------------------------------------------------ */
/* Selected rows / columns of one head (large S).  Threads split rows. */

typedef struct {
    const double *q, *k, *v, *dO;
    int64_t S, d;
    double scale;
    int causal;
    const int64_t *idx;     /* selected rows (fwd, dq) or columns (dk/dv) */
    int64_t nidx;
    double *out_a, *out_b;  /* fwd: o, lse | dq: dq | cols: dk, dv partials */
    int64_t row_lo, row_hi; /* cols mode: rows handled by this thread */
    int tid, nthreads;
    int err;
} sel_job;

static void *fwd_rows_worker(void *arg) {
    sel_job *J = (sel_job *)arg;
    double *p = (double *)malloc(sizeof(double) * (size_t)(J->S > 0 ? J->S : 1));
    if (!p) { J->err = 1; return NULL; }
    for (int64_t r = J->tid; r < J->nidx; r += J->nthreads) {
        int64_t i = J->idx[r];
        int64_t n = row_extent(i, J->S, J->causal);
        double m, z;
        softmax_row(J->q + i * J->d, J->k, n, J->d, J->scale, p, &m, &z);
        weighted_rows(p, J->v, n, J->d, J->out_a + r * J->d);
        J->out_b[r] = m + log(z);
    }
    free(p);
    return NULL;
}

static void *dq_rows_worker(void *arg) {
    sel_job *J = (sel_job *)arg;
    const int64_t d = J->d;
    double *p = (double *)malloc(sizeof(double) * (size_t)(J->S > 0 ? J->S : 1));
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    if (!p || !o) { free(p); free(o); J->err = 1; return NULL; }
    for (int64_t r = J->tid; r < J->nidx; r += J->nthreads) {
        int64_t i = J->idx[r];
        int64_t n = row_extent(i, J->S, J->causal);
        const double *qi = J->q + i * d, *doi = J->dO + i * d;
        double m, z;
        softmax_row(qi, J->k, n, d, J->scale, p, &m, &z);
        weighted_rows(p, J->v, n, d, o);
        double Di = dot(doi, o, d);
        double *dqi = J->out_a + r * d;
        for (int64_t c = 0; c < d; ++c) dqi[c] = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            double dS = p[j] * (dot(doi, J->v + j * d, d) - Di);
            for (int64_t c = 0; c < d; ++c) dqi[c] += J->scale * dS * J->k[j * d + c];
        }
    }
    free(p); free(o);
    return NULL;
}

static void *cols_worker(void *arg) {
    sel_job *J = (sel_job *)arg;
    const int64_t d = J->d;
    double *p = (double *)malloc(sizeof(double) * (size_t)(J->S > 0 ? J->S : 1));
    double *o = (double *)malloc(sizeof(double) * (size_t)d);
    if (!p || !o) { free(p); free(o); J->err = 1; return NULL; }
    for (int64_t i = J->row_lo; i < J->row_hi; ++i) {
        int64_t n = row_extent(i, J->S, J->causal);
        int any = 0;
        for (int64_t c = 0; c < J->nidx; ++c) any |= (J->idx[c] < n);
        if (!any) continue;
        const double *qi = J->q + i * d, *doi = J->dO + i * d;
        double m, z;
        softmax_row(qi, J->k, n, d, J->scale, p, &m, &z);
        weighted_rows(p, J->v, n, d, o);
        double Di = dot(doi, o, d);
        for (int64_t c = 0; c < J->nidx; ++c) {
            int64_t j = J->idx[c];
            if (j >= n) continue;
            double dS = p[j] * (dot(doi, J->v + j * d, d) - Di);
            double *dkj = J->out_a + c * d, *dvj = J->out_b + c * d;
            for (int64_t e = 0; e < d; ++e) {
                dvj[e] += p[j] * doi[e];
                dkj[e] += J->scale * dS * qi[e];
            }
        }
    }
    free(p); free(o);
    return NULL;
}

int oracle_forward_rows(const double *q, const double *k, const double *v, int64_t S, int64_t d,
                        double scale, int causal, const int64_t *rows, int64_t nrows,
                        double *o_rows, double *lse_rows, int nthreads) {
    int T = resolve_threads(nthreads);
    if (T > nrows) T = nrows > 0 ? (int)nrows : 1;
    sel_job *jobs = (sel_job *)calloc((size_t)T, sizeof(sel_job));
    pthread_t *th = (pthread_t *)calloc((size_t)T, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return 1; }
    for (int t = 0; t < T; ++t) {
        sel_job j = {q, k, v, NULL, S, d, scale, causal, rows, nrows, o_rows, lse_rows, 0, 0, t, T, 0};
        jobs[t] = j;
        pthread_create(&th[t], NULL, fwd_rows_worker, &jobs[t]);
    }
    int err = 0;
    for (int t = 0; t < T; ++t) { pthread_join(th[t], NULL); err |= jobs[t].err; }
    free(jobs); free(th);
    return err;
}

int oracle_backward_dq_rows(const double *q, const double *k, const double *v, const double *dO,
                            int64_t S, int64_t d, double scale, int causal,
                            const int64_t *rows, int64_t nrows, double *dq_rows, int nthreads) {
    int T = resolve_threads(nthreads);
    if (T > nrows) T = nrows > 0 ? (int)nrows : 1;
    sel_job *jobs = (sel_job *)calloc((size_t)T, sizeof(sel_job));
    pthread_t *th = (pthread_t *)calloc((size_t)T, sizeof(pthread_t));
    if (!jobs || !th) { free(jobs); free(th); return 1; }
    for (int t = 0; t < T; ++t) {
        sel_job j = {q, k, v, dO, S, d, scale, causal, rows, nrows, dq_rows, NULL, 0, 0, t, T, 0};
        jobs[t] = j;
        pthread_create(&th[t], NULL, dq_rows_worker, &jobs[t]);
    }
    int err = 0;
    for (int t = 0; t < T; ++t) { pthread_join(th[t], NULL); err |= jobs[t].err; }
    free(jobs); free(th);
    return err;
}

int oracle_backward_dkdv_cols(const double *q, const double *k, const double *v, const double *dO,
                              int64_t S, int64_t d, double scale, int causal,
                              const int64_t *cols, int64_t ncols,
                              double *dk_cols, double *dv_cols, int nthreads) {
    int T = resolve_threads(nthreads);
    if (T > S) T = S > 0 ? (int)S : 1;
    sel_job *jobs = (sel_job *)calloc((size_t)T, sizeof(sel_job));
    pthread_t *th = (pthread_t *)calloc((size_t)T, sizeof(pthread_t));
    double *part = (double *)calloc((size_t)T * 2 * (size_t)(ncols * d) + 1, sizeof(double));
    if (!jobs || !th || !part) { free(jobs); free(th); free(part); return 1; }
    /* Rows are dealt out in contiguous ranges; under a causal mask later rows
       see more keys, so the ranges shrink towards the end. */
    int64_t lo = 0;
    for (int t = 0; t < T; ++t) {
        int64_t hi;
        if (causal) {
            double frac = sqrt((double)(t + 1) / (double)T);
            hi = (t == T - 1) ? S : (int64_t)(frac * (double)S);
        } else {
            hi = (t == T - 1) ? S : (S * (t + 1)) / T;
        }
        if (hi < lo) hi = lo;
        double *pa = part + (size_t)t * 2 * (size_t)(ncols * d);
        sel_job j = {q, k, v, dO, S, d, scale, causal, cols, ncols, pa, pa + ncols * d, lo, hi, t, T, 0};
        jobs[t] = j;
        pthread_create(&th[t], NULL, cols_worker, &jobs[t]);
        lo = hi;
    }
    int err = 0;
    for (int t = 0; t < T; ++t) { pthread_join(th[t], NULL); err |= jobs[t].err; }
    for (int64_t e = 0; e < ncols * d; ++e) { dk_cols[e] = 0.0; dv_cols[e] = 0.0; }
    for (int t = 0; t < T; ++t) {
        const double *pa = part + (size_t)t * 2 * (size_t)(ncols * d);
        for (int64_t e = 0; e < ncols * d; ++e) {
            dk_cols[e] += pa[e];
            dv_cols[e] += pa[ncols * d + e];
        }
    }
    free(jobs); free(th); free(part);
    return err;
}
