/*
 * Driver for the sanitizer build of the C oracle (test infrastructure only).
 * Built with -fsanitize=address,undefined together with oracle/spmm_oracle.c
 * and run by tests/test_sanitizers.py: random COO triplets (duplicates and
 * empty rows included) go through oracle_spmm with 1..7 threads, all rows and
 * row subsets, and each result is compared with a plain loop written here;
 * every 16-bit code of both formats and every byte code of FP8 is decoded.
 * Any out-of-bounds access, leak or undefined behaviour aborts the run.
 * Prints "ok" at the end.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double oracle_decode16(uint16_t code, int dtype);
void oracle_decode16_array(const uint16_t *codes, int64_t n, int dtype, double *out);
int oracle_spmm(int64_t m, int64_t k, int64_t N, int64_t nnz, const int32_t *rows,
                const int32_t *cols, const uint16_t *a_codes, const uint16_t *b_codes, int dtype,
                const int64_t *out_rows, int64_t n_out, double *C, double *bound, int nthreads);

static uint64_t s = 88172645463325252ull;
static uint64_t next(void)
{
    s ^= s << 13;
    s ^= s >> 7;
    s ^= s << 17;
    return s;
}

int main(void)
{
    int fails = 0;
    static uint16_t codes[65536];
    static double vals[65536];
    for (int c = 0; c < 65536; ++c)
        codes[c] = (uint16_t)c;
    for (int dt = 0; dt < 4; dt += (dt == 1 ? 2 : 1)) {
        oracle_decode16_array(codes, dt == 3 ? 256 : 65536, dt, vals);
        for (int c = 0; c < (dt == 3 ? 256 : 65536); c += 997)
            if (!(vals[c] == oracle_decode16((uint16_t)c, dt) || (isnan(vals[c]) && isnan(oracle_decode16((uint16_t)c, dt)))))
                ++fails;
    }
    for (int rep = 0; rep < 60; ++rep) {
        const int64_t m = (int64_t)(next() % 70), k = 1 + (int64_t)(next() % 50), N = (int64_t)(next() % 20);
        const int64_t nnz = m ? (int64_t)(next() % (3 * m + 1)) : 0;
        int32_t *r = malloc((size_t)(nnz + 1) * sizeof(int32_t)), *cl = malloc((size_t)(nnz + 1) * sizeof(int32_t));
        uint16_t *a = malloc((size_t)(nnz + 1) * sizeof(uint16_t)), *b = malloc((size_t)(k * N + 1) * sizeof(uint16_t));
        for (int64_t t = 0; t < nnz; ++t) {
            r[t] = (int32_t)(next() % (uint64_t)m);
            cl[t] = (int32_t)(next() % (uint64_t)k);
            a[t] = (uint16_t)(0x3C00 + next() % 0x400); /* fp16 values in [1, 2) */
        }
        for (int64_t q = 0; q < k * N; ++q)
            b[q] = (uint16_t)((next() & 0x8000) | (0x3800 + next() % 0x800));
        double *C = malloc((size_t)(m * N + 1) * sizeof(double)), *B = malloc((size_t)(m * N + 1) * sizeof(double));
        const int th = 1 + (int)(next() % 7);
        if (oracle_spmm(m, k, N, nnz, r, cl, a, b, 0, NULL, m, C, B, th) != 0)
            ++fails;
        for (int64_t i = 0; i < m; ++i)
            for (int64_t n = 0; n < N; ++n) {
                double ref = 0.0;
                for (int64_t t = 0; t < nnz; ++t)
                    if (r[t] == i)
                        ref += oracle_decode16(a[t], 0) * oracle_decode16(b[cl[t] * N + n], 0);
                if (fabs(ref - C[i * N + n]) > 1e-12 * (1.0 + fabs(ref)))
                    ++fails;
            }
        /* a subset of rows, in reverse order */
        if (m > 0) {
            int64_t sub[3] = {m - 1, m / 2, 0};
            double C2[3 * 20], B2[3 * 20];
            if (oracle_spmm(m, k, N, nnz, r, cl, a, b, 0, sub, 3, C2, B2, 2) != 0)
                ++fails;
            for (int o = 0; o < 3; ++o)
                for (int64_t n = 0; n < N; ++n)
                    if (C2[o * N + n] != C[sub[o] * N + n])
                        ++fails;
        }
        /* an index out of range is refused */
        if (nnz > 0) {
            cl[0] = (int32_t)k;
            if (oracle_spmm(m, k, N, nnz, r, cl, a, b, 0, NULL, m, C, B, 1) != -1)
                ++fails;
        }
        free(r); free(cl); free(a); free(b); free(C); free(B);
    }
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("ok\n");
    return 0;
}
