/*
 * CPU oracle for C = A * B, A sparse (COO triplets), B dense row-major.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code with the GPU library.
 *
 * What it computes is the plain definition of the product the AsyncSparse
 * paper sets up in its sparse-format background section (II-C: C = A x B with
 * A in R^{m x k} sparse and B in R^{k x n} dense):
 *
 *     C[i][n]     = sum over triplets t with row_t == i of  a_t * B[col_t][n]
 *     Bound[i][n] = sum over the same triplets of           |a_t| * |B[col_t][n]|
 *
 * accumulated in IEEE double, triplets of one row taken in input order.
 * Bound is the scale of the acceptance test |C_gpu - C| <= tol * Bound.
 * Inputs are 16-bit codes (binary16 or bfloat16) decoded exactly by
 * oracle_decode16 below (every such value is exact in double).
 *
 * Rows are independent, so they are split across POSIX threads; the order of
 * the additions inside a row never depends on the thread count.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { ORACLE_FP16 = 0, ORACLE_BF16 = 1, ORACLE_FP8_E4M3 = 3 };

/* Exact value of an OCP FP8 E4M3 code (the low byte): 1 sign, 4 exponent bits
 * (bias 7), 3 fraction bits; exponent field 0 = zero/subnormal; no infinities,
 * exponent and fraction all ones = NaN. */
static double decode_fp8_e4m3(uint16_t code)
{
    int sign = (code >> 7) & 1;
    int e = (code >> 3) & 15;
    int f = code & 7;
    double v;
    if (e == 15 && f == 7)
        v = NAN;
    else if (e == 0)
        v = ldexp((double)f, 1 - 7 - 3);          /* 0.f * 2^(1 - bias) */
    else
        v = ldexp((double)(8 + f), e - 7 - 3);    /* 1.f * 2^(e - bias) */
    return sign ? -v : v;
}

/* Exact value of a 16-bit floating-point code (or, for ORACLE_FP8_E4M3, of the
 * FP8 code in its low byte).
 * binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.
 * bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits (the upper half of
 * an IEEE single). Exponent field 0 = zero/subnormal, all ones = inf/NaN. */
double oracle_decode16(uint16_t code, int dtype)
{
    if (dtype == ORACLE_FP8_E4M3)
        return decode_fp8_e4m3(code);
    int ebits = (dtype == ORACLE_BF16) ? 8 : 5;
    int fbits = (dtype == ORACLE_BF16) ? 7 : 10;
    int bias = (1 << (ebits - 1)) - 1;
    int sign = (code >> 15) & 1;
    int e = (code >> fbits) & ((1 << ebits) - 1);
    int f = code & ((1 << fbits) - 1);
    double v;
    if (e == (1 << ebits) - 1) {
        v = (f == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        /* subnormal: 0.f * 2^(1 - bias) = f * 2^(1 - bias - fbits) */
        v = ldexp((double)f, 1 - bias - fbits);
    } else {
        /* normal: 1.f * 2^(e - bias) = (2^fbits + f) * 2^(e - bias - fbits) */
        v = ldexp((double)((1 << fbits) + f), e - bias - fbits);
    }
    return sign ? -v : v;
}

void oracle_decode16_array(const uint16_t *codes, int64_t n, int dtype, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = oracle_decode16(codes[i], dtype);
}

typedef struct {
    int64_t N;
    const int64_t *row_start;   /* [m+1] into order[] */
    const int64_t *order;       /* triplet ids grouped by row, input order kept */
    const int32_t *cols;
    const uint16_t *a_codes;
    const uint16_t *b_codes;
    int dtype;
    const int64_t *out_rows;    /* which rows to produce */
    int64_t n_out;
    double *C;
    double *bound;
    int64_t first, last;        /* slice of out_rows this thread owns */
} job_t;

static void *run_rows(void *arg)
{
    job_t *j = (job_t *)arg;
    const int64_t N = j->N;
    for (int64_t o = j->first; o < j->last; ++o) {
        int64_t i = j->out_rows[o];
        double *c = j->C + o * N;
        double *b = j->bound + o * N;
        for (int64_t n = 0; n < N; ++n) {
            c[n] = 0.0;
            b[n] = 0.0;
        }
        for (int64_t s = j->row_start[i]; s < j->row_start[i + 1]; ++s) {
            int64_t t = j->order[s];
            double a = oracle_decode16(j->a_codes[t], j->dtype);
            const uint16_t *brow = j->b_codes + (int64_t)j->cols[t] * N;
            for (int64_t n = 0; n < N; ++n) {
                double x = oracle_decode16(brow[n], j->dtype);
                c[n] += a * x;
                b[n] += fabs(a) * fabs(x);
            }
        }
    }
    return NULL;
}

/*
 * Output rows out_rows[0..n_out) (all rows 0..m-1 in order when out_rows is
 * NULL, then n_out must be m) of C and Bound, each written row-major into
 * n_out x N doubles.  B is k x N row-major (leading dimension N).
 * Returns 0 on success, -1 on a bad argument (index out of range),
 * -2 when memory runs out.
 */
int oracle_spmm(int64_t m, int64_t k, int64_t N, int64_t nnz,
                const int32_t *rows, const int32_t *cols, const uint16_t *a_codes,
                const uint16_t *b_codes, int dtype,
                const int64_t *out_rows, int64_t n_out,
                double *C, double *bound, int nthreads)
{
    if (m < 0 || k < 0 || N < 0 || nnz < 0 || n_out < 0)
        return -1;
    if (!out_rows && n_out != m)
        return -1;
    for (int64_t t = 0; t < nnz; ++t)
        if (rows[t] < 0 || rows[t] >= m || cols[t] < 0 || cols[t] >= k)
            return -1;
    for (int64_t o = 0; out_rows && o < n_out; ++o)
        if (out_rows[o] < 0 || out_rows[o] >= m)
            return -1;

    /* counting sort of the triplets by row (stable) */
    int64_t *row_start = (int64_t *)calloc((size_t)m + 1, sizeof(int64_t));
    int64_t *order = (int64_t *)malloc((size_t)(nnz > 0 ? nnz : 1) * sizeof(int64_t));
    int64_t *fill = (int64_t *)malloc((size_t)(m > 0 ? m : 1) * sizeof(int64_t));
    int64_t *all_rows = NULL;
    if (!row_start || !order || !fill) {
        free(row_start); free(order); free(fill);
        return -2;
    }
    for (int64_t t = 0; t < nnz; ++t)
        row_start[rows[t] + 1] += 1;
    for (int64_t i = 0; i < m; ++i)
        row_start[i + 1] += row_start[i];
    memcpy(fill, row_start, (size_t)m * sizeof(int64_t));
    for (int64_t t = 0; t < nnz; ++t)
        order[fill[rows[t]]++] = t;
    free(fill);

    if (!out_rows) {
        all_rows = (int64_t *)malloc((size_t)(m > 0 ? m : 1) * sizeof(int64_t));
        if (!all_rows) {
            free(row_start); free(order);
            return -2;
        }
        for (int64_t i = 0; i < m; ++i)
            all_rows[i] = i;
        out_rows = all_rows;
    }

    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 512)
        nthreads = 512;
    job_t jobs[512];
    pthread_t tids[512];
    int started = 0;
    for (int w = 0; w < nthreads; ++w) {
        jobs[w] = (job_t){N, row_start, order, cols, a_codes, b_codes, dtype, out_rows, n_out,
                          C, bound, n_out * w / nthreads, n_out * (w + 1) / nthreads};
    }
    for (int w = 1; w < nthreads; ++w) {
        if (pthread_create(&tids[w], NULL, run_rows, &jobs[w]) != 0)
            break;
        started = w;
    }
    /* this thread takes slice 0 and every slice whose thread did not start */
    run_rows(&jobs[0]);
    for (int w = started + 1; w < nthreads; ++w)
        run_rows(&jobs[w]);
    for (int w = 1; w <= started; ++w)
        pthread_join(tids[w], NULL);
    free(all_rows);
    free(row_start);
    free(order);
    return 0;
}
