/*
 * oracle_sanitize_driver.c -- runs every entry point of oracle/attn_oracle.c
 * on small inputs so that a build with -fsanitize=address,undefined can check
 * the oracle's memory accesses and arithmetic for undefined behaviour (the
 * race/memory checks planned for the CPU side of the test suite).  It also
 * checks that the sampled entry points agree with the full ones and that
 * the results do not depend on the thread count.  Exit status 0 = all good.
 * Test infrastructure only.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_attention_forward(const double *q, const double *k, const double *v, int64_t BH, int64_t S,
                             int64_t d, double scale, int causal, double *o, double *lse, int nthreads);
int oracle_attention_backward(const double *q, const double *k, const double *v, const double *dO,
                              int64_t BH, int64_t S, int64_t d, double scale, int causal, double *dq,
                              double *dk, double *dv, int nthreads);
int oracle_forward_rows(const double *q, const double *k, const double *v, int64_t S, int64_t d,
                        double scale, int causal, const int64_t *rows, int64_t nrows, double *o_rows,
                        double *lse_rows, int nthreads);
int oracle_backward_dq_rows(const double *q, const double *k, const double *v, const double *dO,
                            int64_t S, int64_t d, double scale, int causal, const int64_t *rows,
                            int64_t nrows, double *dq_rows, int nthreads);
int oracle_backward_dkdv_cols(const double *q, const double *k, const double *v, const double *dO,
                              int64_t S, int64_t d, double scale, int causal, const int64_t *cols,
                              int64_t ncols, double *dk_cols, double *dv_cols, int nthreads);

static uint64_t state = 0x9E3779B97F4A7C15ull;
static double uniform_pm1(void) {   /* xorshift64*, only for test data */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 2685821657736338717ull) >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}

static double maxdiff(const double *a, const double *b, int64_t n) {
    double m = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        const double e = fabs(a[i] - b[i]);
        if (!(e <= m)) m = e;   /* NaN propagates */
    }
    return m;
}

static int run_case(int64_t BH, int64_t S, int64_t d, int causal) {
    const int64_t n = BH * S * d;
    double *q = malloc(sizeof(double) * n), *k = malloc(sizeof(double) * n), *v = malloc(sizeof(double) * n);
    double *g = malloc(sizeof(double) * n);
    double *o1 = malloc(sizeof(double) * n), *o3 = malloc(sizeof(double) * n);
    double *l1 = malloc(sizeof(double) * BH * S), *l3 = malloc(sizeof(double) * BH * S);
    double *dq1 = malloc(sizeof(double) * n), *dk1 = malloc(sizeof(double) * n), *dv1 = malloc(sizeof(double) * n);
    double *dq3 = malloc(sizeof(double) * n), *dk3 = malloc(sizeof(double) * n), *dv3 = malloc(sizeof(double) * n);
    for (int64_t i = 0; i < n; ++i) {
        q[i] = uniform_pm1();
        k[i] = uniform_pm1();
        v[i] = uniform_pm1();
        g[i] = uniform_pm1();
    }
    const double scale = 1.0 / sqrt((double)d);
    int bad = 0;
    bad |= oracle_attention_forward(q, k, v, BH, S, d, scale, causal, o1, l1, 1);
    bad |= oracle_attention_forward(q, k, v, BH, S, d, scale, causal, o3, l3, 3);
    bad |= oracle_attention_backward(q, k, v, g, BH, S, d, scale, causal, dq1, dk1, dv1, 1);
    bad |= oracle_attention_backward(q, k, v, g, BH, S, d, scale, causal, dq3, dk3, dv3, 3);
    if (bad) { fprintf(stderr, "entry point failed\n"); return 1; }
    if (maxdiff(o1, o3, n) != 0.0 || maxdiff(l1, l3, BH * S) != 0.0 || maxdiff(dq1, dq3, n) > 1e-12 ||
        maxdiff(dk1, dk3, n) > 1e-12 || maxdiff(dv1, dv3, n) > 1e-12) {
        fprintf(stderr, "thread count changed the result (S=%lld causal=%d)\n", (long long)S, causal);
        return 1;
    }
    /* sampled entry points on the last head against the full ones */
    const int64_t h = BH - 1, off = h * S * d;
    int64_t idx[4] = {0, S / 2, S - 1, S > 2 ? 1 : 0};
    double orow[4 * 64], lrow[4], dqrow[4 * 64], dkc[4 * 64], dvc[4 * 64];
    if (d > 64) return 1;
    bad |= oracle_forward_rows(q + off, k + off, v + off, S, d, scale, causal, idx, 4, orow, lrow, 2);
    bad |= oracle_backward_dq_rows(q + off, k + off, v + off, g + off, S, d, scale, causal, idx, 4, dqrow, 2);
    for (int i = 0; i < 4 * 64; ++i) dkc[i] = dvc[i] = 0.0;
    bad |= oracle_backward_dkdv_cols(q + off, k + off, v + off, g + off, S, d, scale, causal, idx, 4, dkc, dvc, 2);
    if (bad) { fprintf(stderr, "sampled entry point failed\n"); return 1; }
    for (int c = 0; c < 4; ++c) {
        const int64_t r = idx[c];
        if (maxdiff(orow + c * d, o1 + off + r * d, d) > 1e-12 || fabs(lrow[c] - l1[h * S + r]) > 1e-12 ||
            maxdiff(dqrow + c * d, dq1 + off + r * d, d) > 1e-12 || maxdiff(dkc + c * d, dk1 + off + r * d, d) > 1e-12 ||
            maxdiff(dvc + c * d, dv1 + off + r * d, d) > 1e-12) {
            fprintf(stderr, "sampled entry point differs at row %lld (S=%lld causal=%d)\n", (long long)r,
                    (long long)S, causal);
            return 1;
        }
    }
    free(q); free(k); free(v); free(g); free(o1); free(o3); free(l1); free(l3);
    free(dq1); free(dk1); free(dv1); free(dq3); free(dk3); free(dv3);
    return 0;
}

int main(void) {
    const int64_t shapes[][3] = {{1, 1, 4}, {2, 7, 8}, {3, 33, 16}, {1, 64, 64}, {2, 5, 1}};
    for (int s = 0; s < 5; ++s)
        for (int causal = 0; causal < 2; ++causal)
            if (run_case(shapes[s][0], shapes[s][1], shapes[s][2], causal)) return 1;
    /* an empty head set and S = 0 rows are valid no-ops */
    if (oracle_attention_forward(NULL, NULL, NULL, 0, 0, 8, 1.0, 0, NULL, NULL, 1)) return 1;
    printf("oracle sanitizer driver: ok\n");
    return 0;
}
