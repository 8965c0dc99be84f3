/*
 * CPU oracle for the dense fp16 GEMM C = A * B^T (fp16 in, fp16 out).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file: only the tests, the package's smoke check and the CPU
 * baseline leg of the benchmark use it.  It shares no code, header, table or
 * helper with the HIP library.
 *
 * What it computes (written out from the definition, not tuned):
 *
 *   C[m][n] = RNE_fp16( sum_{k=0}^{K-1} double(A[m][k]) * double(B[n][k]) )
 *
 *   - A is [M,K] row-major and B is [N,K] with K contiguous: the tutorial
 *     "1. WGMMA: Hopper's Asynchronous Tensor Core" (Tilus), section "The
 *     Full Kernel", views A as [m_size, k_size] and B as [n_size, k_size] and
 *     multiplies by the transposed B tile.
 *   - The accumulator starts at zero and the sum is taken in increasing k in
 *     one fp64 accumulator per output, as in the plain triple loop in double
 *     that "wgmma_gemm.cu" (day 78) uses as its CPU reference (gemmCpu).
 *   - Every product of two fp16 values is exact in fp64 (11 + 11 significant
 *     bits), so the only roundings are the fp64 additions and the single
 *     final rounding.
 *   - The tutorial casts the accumulator to float16 before the store (same
 *     section).  The cast is read as IEEE 754 round-to-nearest, ties to even,
 *     applied once, directly from fp64 (never via fp32, which would round
 *     twice).  |x| >= 65520 becomes +-inf; NaN stays NaN.
 *
 * A second function, oracle_gemm_f16_nn_f64 (end of this file), is the
 * day-78 listing's reference as printed: D = A * B with B [K,N], fp64 sums
 * left unrounded.
 *
 * Parity pins (tests/test_oracle_*.py): exact rational brute force on tiny
 * shapes, the identity / all-ones / one-hot / rank-1 closed forms, an exact
 * integer GEMM on {-8..8}/8 inputs, and the binary16 converter against exact
 * rational rounding over all ties, subnormals and the overflow edge.
 *
 * Build: gcc -O2 -fPIC -shared -pthread gemm_ref.c -o libgemm_ref.so -lm
 * (no -ffast-math: it would allow the compiler to reassociate the k-sum).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>

/* ---- IEEE 754 binary16 <-> binary64, from the format's definition ------ */
/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * exponent 0 = zero / subnormal (value = frac * 2^-24),
 * exponent 31 = inf (frac 0) or NaN (frac != 0),
 * otherwise value = (1024 + frac) * 2^(exponent - 25). */
double oracle_f16_to_f64(uint16_t h)
{
    const int sign = (h >> 15) & 1;
    const int e = (h >> 10) & 0x1f;
    const int f = h & 0x3ff;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);
    } else if (e == 31) {
        v = (f == 0) ? INFINITY : NAN;
    } else {
        v = ldexp((double)(1024 + f), e - 25);
    }
    return sign ? -v : v;
}

/* Round a non-negative integer-valued-or-not double q to the nearest
 * integer, ties to the even integer.  Written with floor and an explicit
 * comparison so that it does not depend on the floating-point environment. */
static double round_half_even(double q)
{
    const double fl = floor(q);
    const double rem = q - fl; /* exact: q and fl share an exponent range */
    if (rem > 0.5) return fl + 1.0;
    if (rem < 0.5) return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

uint16_t oracle_f64_to_f16(double x)
{
    if (isnan(x)) return 0x7e00;
    const uint16_t sign = signbit(x) ? 0x8000 : 0;
    const double ax = fabs(x);
    /* Largest finite binary16 is 65504; the midpoint to the next binade
     * step (65536) is 65520, which ties to the even neighbour, i.e. inf. */
    if (ax >= 65520.0) return sign | 0x7c00;
    if (ax == 0.0) return sign;

    int e2;
    frexp(ax, &e2);          /* ax = f * 2^e2, f in [0.5, 1) */
    int e = e2 - 1;          /* ax in [2^e, 2^(e+1)) */
    if (e < -14) {
        /* Subnormal range: spacing 2^-24. */
        const double q = round_half_even(ldexp(ax, 24));
        /* q == 1024 is exactly the smallest normal, whose bits are 0x0400. */
        return sign | (uint16_t)q;
    }
    /* Normal range: spacing 2^(e-10); q in [1024, 2048]. */
    double q = round_half_even(ldexp(ax, 10 - e));
    if (q == 2048.0) { /* rounded up into the next binade */
        q = 1024.0;
        e += 1;
    }
    if (e + 15 >= 31) return sign | 0x7c00;
    return sign | (uint16_t)(((e + 15) << 10) | ((int)q - 1024));
}

/* ---- the GEMM ------------------------------------------------------------ */

typedef struct {
    int64_t m, n, k;
    const uint16_t *a, *b;
    uint16_t *c;               /* full C, or the rows listed in rows[] */
    double *c64;               /* optional unrounded output */
    const int64_t *rows;       /* NULL = all rows in order */
    int64_t row_begin, row_end;
    const double *table;       /* binary16 bit pattern -> value */
} job_t;

static void *run_rows(void *p)
{
    const job_t *j = (const job_t *)p;
    for (int64_t r = j->row_begin; r < j->row_end; ++r) {
        const int64_t mi = j->rows ? j->rows[r] : r;
        const uint16_t *arow = j->a + mi * j->k;
        for (int64_t ni = 0; ni < j->n; ++ni) {
            const uint16_t *brow = j->b + ni * j->k;
            double sum = 0.0;
            for (int64_t ki = 0; ki < j->k; ++ki) {
                sum += j->table[arow[ki]] * j->table[brow[ki]];
            }
            if (j->c) j->c[r * j->n + ni] = oracle_f64_to_f16(sum);
            if (j->c64) j->c64[r * j->n + ni] = sum;
        }
    }
    return NULL;
}

static int run(int64_t m, int64_t n, int64_t k, const uint16_t *a,
               const uint16_t *b, uint16_t *c, double *c64,
               const int64_t *rows, int64_t nrows, int nthreads)
{
    if (m < 0 || n < 0 || k < 0 || nrows < 0) return -1;
    if (nrows == 0 || n == 0) return 0;
    if ((k > 0 && (!a || !b)) || (!c && !c64)) return -2;
    if (rows) {
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= m) return -1;
    }
    double *table = (double *)malloc(sizeof(double) * 65536);
    if (!table) return -3;
    for (int h = 0; h < 65536; ++h) table[h] = oracle_f16_to_f64((uint16_t)h);

    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = (int)nrows;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    job_t *jobs = (job_t *)malloc(sizeof(job_t) * nthreads);
    if (!tid || !jobs) {
        free(table); free(tid); free(jobs);
        return -3;
    }
    /* Threads take disjoint row ranges; each output is still one sum in
     * increasing k, so the result does not depend on the thread count. */
    int started = 0, rc = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (job_t){m, n, k, a, b, c, c64, rows,
                          nrows * t / nthreads, nrows * (t + 1) / nthreads,
                          table};
        if (t == nthreads - 1) {
            run_rows(&jobs[t]);
        } else if (pthread_create(&tid[started], NULL, run_rows, &jobs[t]) == 0) {
            ++started;
        } else {
            run_rows(&jobs[t]);
        }
    }
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    free(table); free(tid); free(jobs);
    return rc;
}

/* Whole C.  Returns 0, -1 (bad size), -2 (null pointer), -3 (no memory). */
int oracle_gemm_f16_nt(int64_t m, int64_t n, int64_t k, const uint16_t *a,
                       const uint16_t *b, uint16_t *c, int nthreads)
{
    return run(m, n, k, a, b, c, NULL, NULL, m, nthreads);
}

/* Selected rows of C: c_rows is [nrows, n]; row r holds C[rows[r], :]. */
int oracle_gemm_f16_nt_rows(int64_t m, int64_t n, int64_t k, const uint16_t *a,
                            const uint16_t *b, const int64_t *rows,
                            int64_t nrows, uint16_t *c_rows, int nthreads)
{
    if (!rows && nrows > 0) return -2;
    return run(m, n, k, a, b, c_rows, NULL, rows, nrows, nthreads);
}

/* The unrounded fp64 sums, as the day-78 listing's reference keeps them. */
int oracle_gemm_f16_nt_f64(int64_t m, int64_t n, int64_t k, const uint16_t *a,
                           const uint16_t *b, double *c64, int nthreads)
{
    return run(m, n, k, a, b, NULL, c64, NULL, m, nthreads);
}

/* ---- the day-78 listing's own contract ---------------------------------
 * "wgmma_gemm.cu" computes D = A * B with A [M,K] row-major, B [K,N]
 * row-major (its producer reads b[(k)*N + n]) and keeps D in fp32; its CPU
 * reference (gemmCpu) is a triple loop over m, n, k in double that stores
 * the double sum unrounded.  This is that loop.  It also returns, per
 * output, the sum of |A[m][k] * B[k][n]| (in fp64), which bounds the error
 * of any fp32 summation order: |fl32(sum) - sum| <= gamma_K * sum|p|.     */

typedef struct {
    int64_t m, n, k;
    const uint16_t *a, *b;
    double *d64, *dabs;
    const int64_t *rows;
    int64_t row_begin, row_end;
    const double *table;
} job_nn_t;

static void *run_rows_nn(void *p)
{
    const job_nn_t *j = (const job_nn_t *)p;
    for (int64_t r = j->row_begin; r < j->row_end; ++r) {
        const int64_t mi = j->rows ? j->rows[r] : r;
        for (int64_t ni = 0; ni < j->n; ++ni) {
            double sum = 0.0, sabs = 0.0;
            for (int64_t ki = 0; ki < j->k; ++ki) {
                const double prod = j->table[j->a[mi * j->k + ki]] * j->table[j->b[ki * j->n + ni]];
                sum += prod;
                sabs += fabs(prod);
            }
            j->d64[r * j->n + ni] = sum;
            if (j->dabs) j->dabs[r * j->n + ni] = sabs;
        }
    }
    return NULL;
}

/* Rows `rows` (or all rows when rows == NULL, nrows == m) of D = A * B:
 * d64 and dabs are [nrows, n].  Returns 0, -1, -2 or -3 as above. */
int oracle_gemm_f16_nn_f64(int64_t m, int64_t n, int64_t k, const uint16_t *a,
                           const uint16_t *b, const int64_t *rows, int64_t nrows,
                           double *d64, double *dabs, int nthreads)
{
    if (m < 0 || n < 0 || k < 0 || nrows < 0) return -1;
    if (!rows && nrows != m) return -1;
    if (nrows == 0 || n == 0) return 0;
    if ((k > 0 && (!a || !b)) || !d64) return -2;
    if (rows) {
        for (int64_t r = 0; r < nrows; ++r)
            if (rows[r] < 0 || rows[r] >= m) return -1;
    }
    double *table = (double *)malloc(sizeof(double) * 65536);
    if (!table) return -3;
    for (int h = 0; h < 65536; ++h) table[h] = oracle_f16_to_f64((uint16_t)h);
    if (nthreads < 1) nthreads = 1;
    if (nthreads > nrows) nthreads = (int)nrows;
    pthread_t *tid = (pthread_t *)malloc(sizeof(pthread_t) * nthreads);
    job_nn_t *jobs = (job_nn_t *)malloc(sizeof(job_nn_t) * nthreads);
    if (!tid || !jobs) {
        free(table); free(tid); free(jobs);
        return -3;
    }
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        jobs[t] = (job_nn_t){m, n, k, a, b, d64, dabs, rows,
                             nrows * t / nthreads, nrows * (t + 1) / nthreads, table};
        if (t == nthreads - 1) {
            run_rows_nn(&jobs[t]);
        } else if (pthread_create(&tid[started], NULL, run_rows_nn, &jobs[t]) == 0) {
            ++started;
        } else {
            run_rows_nn(&jobs[t]);
        }
    }
    for (int t = 0; t < started; ++t) pthread_join(tid[t], NULL);
    free(table); free(tid); free(jobs);
    return 0;
}
