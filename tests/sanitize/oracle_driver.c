/*
 * Runs every entry point of the CPU oracle on small inputs under
 * AddressSanitizer and UndefinedBehaviorSanitizer (built by
 * tests/test_sanitizers.py): full and partial selections, a short last block,
 * top-k 1 and top-k >= the block count, bf16 and fp32 storage, GQA, and the
 * argument errors.  Prints "ok" and exits 0 when every call returns what it
 * should; any sanitizer report aborts the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_pool(const void *k, int code, int batch, int S, int hkv, int d, int block, double *kbar);
int oracle_gate(const void *q, int code, const double *kbar, int batch, int S, int hq, int hkv, int d,
                int block, int topk, long long R, const long long *rows, int *idx_out,
                double *margin_out, double *scores_out);
int oracle_attend(const void *q, const void *k, const void *v, int code, int batch, int S, int hq,
                  int hkv, int d, int block, int topk, long long R, const long long *rows,
                  const int *idx, double *out, double *lse);
int oracle_attend_merged(const void *q, const void *k, const void *v, int code, int batch, int S,
                         int hq, int hkv, int d, int block, int topk, long long R,
                         const long long *rows, const int *idx, double *out, double *lse);
int oracle_selection_gap(const void *q, int code, const double *kbar, int batch, int S, int hq,
                         int hkv, int d, int block, int topk, long long R, const long long *rows,
                         const int *idx, int *valid_out, double *gap_out);
int oracle_backward(const void *q, const void *k, const void *v, int code, const double *dout,
                    int batch, int S, int hq, int hkv, int d, int block, int topk, const int *idx,
                    int t_lo, double *dq, double *dk, double *dv);

static uint64_t state = 0x9e3779b97f4a7c15ull;
static double uniform(void) {            /* xorshift64*, in (-1, 1) */
    state ^= state >> 12;
    state ^= state << 25;
    state ^= state >> 27;
    return (double)((state * 0x2545f4914f6cdd1dull) >> 11) / 4503599627370496.0 - 1.0;
}
static void fill(void *p, int code, size_t n) {
    for (size_t i = 0; i < n; ++i) {
        const float x = (float)(0.5 * uniform());
        if (code == 1) {
            ((float *)p)[i] = x;
        } else {
            uint32_t u;
            memcpy(&u, &x, 4);
            ((uint16_t *)p)[i] = (uint16_t)(u >> 16);   /* truncation is fine for test data */
        }
    }
}

static int failures = 0;
#define EXPECT(cond)                                                       \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "FAILED line %d: %s\n", __LINE__, #cond);      \
            ++failures;                                                    \
        }                                                                  \
    } while (0)

static void run_case(int code, int batch, int S, int hq, int hkv, int d, int block, int topk) {
    const int n = (S + block - 1) / block;
    const size_t es = code == 1 ? 4 : 2;
    const size_t nq = (size_t)batch * S * hq * d, nk = (size_t)batch * S * hkv * d;
    void *q = malloc(nq * es), *k = malloc(nk * es), *v = malloc(nk * es);
    fill(q, code, nq);
    fill(k, code, nk);
    fill(v, code, nk);
    double *kbar = malloc(sizeof(double) * (size_t)batch * hkv * n * d);
    EXPECT(oracle_pool(k, code, batch, S, hkv, d, block, kbar) == 0);
    const long long R = (long long)batch * hq * S;
    long long *rows = malloc(sizeof(long long) * 3 * (size_t)R);
    long long r = 0;
    for (int b = 0; b < batch; ++b)
        for (int h = 0; h < hq; ++h)
            for (int t = 0; t < S; ++t, ++r) {
                rows[3 * r] = b;
                rows[3 * r + 1] = h;
                rows[3 * r + 2] = t;
            }
    int *idx = malloc(sizeof(int) * (size_t)R * topk);
    double *margin = malloc(sizeof(double) * (size_t)R);
    double *scores = malloc(sizeof(double) * (size_t)R * n);
    EXPECT(oracle_gate(q, code, kbar, batch, S, hq, hkv, d, block, topk, R, rows, idx, margin, scores) == 0);
    double *o1 = malloc(sizeof(double) * (size_t)R * d), *o2 = malloc(sizeof(double) * (size_t)R * d);
    double *l1 = malloc(sizeof(double) * (size_t)R), *l2 = malloc(sizeof(double) * (size_t)R);
    EXPECT(oracle_attend(q, k, v, code, batch, S, hq, hkv, d, block, topk, R, rows, idx, o1, l1) == 0);
    EXPECT(oracle_attend_merged(q, k, v, code, batch, S, hq, hkv, d, block, topk, R, rows, idx, o2, l2) == 0);
    double worst = 0.0;
    for (size_t i = 0; i < (size_t)R * d; ++i) worst = fmax(worst, fabs(o1[i] - o2[i]));
    EXPECT(worst < 1e-12);
    int *valid = malloc(sizeof(int) * (size_t)R);
    double *gap = malloc(sizeof(double) * (size_t)R);
    EXPECT(oracle_selection_gap(q, code, kbar, batch, S, hq, hkv, d, block, topk, R, rows, idx, valid, gap) == 0);
    int all_valid = 1;
    for (long long i = 0; i < R; ++i) all_valid &= valid[i] == 1 && gap[i] >= 0.0;
    EXPECT(all_valid);
    /* the backward takes the selection in the [batch][hq][S][topk] layout the rows above follow */
    {
        double *dout = malloc(sizeof(double) * nq), *dq = malloc(sizeof(double) * nq);
        double *dk = malloc(sizeof(double) * nk), *dv = malloc(sizeof(double) * nk);
        for (size_t i = 0; i < nq; ++i) dout[i] = 0.1 * uniform();
        EXPECT(oracle_backward(q, k, v, code, dout, batch, S, hq, hkv, d, block, topk, idx, 0, dq, dk, dv) == 0);
        EXPECT(oracle_backward(q, k, v, code, dout, batch, S, hq, hkv, d, block, topk, idx, S / 2, dq, dk, dv) == 0);
        free(dout); free(dq); free(dk); free(dv);
    }
    /* a selection entry naming a future block is refused, not read past */
    if (n > 1 && topk > 1) {
        const int keep = idx[0 * topk + topk - 1];
        idx[0 * topk + topk - 1] = n + 5;                 /* row (0, 0, 0): out of range */
        EXPECT(oracle_attend(q, k, v, code, batch, S, hq, hkv, d, block, topk, 1, rows, idx, o1, l1) == 2);
        idx[0 * topk + topk - 1] = keep;
    }
    free(q); free(k); free(v); free(kbar); free(rows); free(idx); free(margin); free(scores);
    free(o1); free(o2); free(l1); free(l2); free(valid); free(gap);
}

int main(void) {
    run_case(0, 1, 512, 2, 1, 64, 64, 3);        /* bf16, GQA 2 */
    run_case(1, 2, 448, 2, 2, 64, 128, 2);       /* fp32, two sequences, short last block */
    run_case(0, 1, 320, 4, 2, 128, 64, 1);       /* own block only */
    run_case(1, 1, 256, 2, 1, 64, 64, 9);        /* top-k above the block count: dense */
    run_case(0, 1, 640, 2, 1, 64, 64, 5);        /* ten blocks, four past selected */
    /* argument errors */
    double kb[64];
    long long row[3] = {0, 0, 0};
    int id[3] = {0, -1, -1};
    double out[64], lse[1], margin[1];
    uint16_t q[64 * 64];
    memset(q, 0, sizeof q);
    EXPECT(oracle_pool(NULL, 0, 1, 64, 1, 64, 64, kb) == 1);
    EXPECT(oracle_pool(q, 0, 1, 64, 1, 64, 0, kb) == 1);
    EXPECT(oracle_gate(q, 0, kb, 1, 64, 3, 2, 64, 64, 3, 1, row, id, margin, NULL) == 1);   /* Hq % Hkv */
    EXPECT(oracle_attend(q, q, q, 0, 1, 64, 1, 1, 64, 64, 0, 1, row, id, out, lse) == 1);   /* topk 0 */
    EXPECT(oracle_attend(q, q, NULL, 0, 1, 64, 1, 1, 64, 64, 3, 1, row, id, out, lse) == 1);
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
