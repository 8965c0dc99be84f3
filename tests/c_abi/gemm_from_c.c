/*
 * Both GEMM contracts called from a C program through the library's C ABI,
 * with no Python in the process: device buffers come from the HIP runtime's
 * C API, the calls run on a stream of their own, and every output is
 * compared bit for bit with the C oracle (oracle/gemm_ref.c).
 *
 * Operands are k/8 with k drawn from -8..8, so every product is a multiple
 * of 1/64 and every partial sum is a multiple of 1/64 of magnitude at most
 * K: exact in fp32, in any order, while 64 K < 2^24.  C = A B^T then has one
 * correct fp16 value, and D = A B one correct fp32 value.  C and D sit
 * inside guard bands that must come back untouched.
 *
 * Exit status: 0 all cases pass, 1 a mismatch or wrong status, 2 a HIP or
 * host allocation failure.  Each case is printed before it runs.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include "gemm_f16.h"

/* The oracle's entry points (exported by oracle/libgemm_ref.so). */
int oracle_gemm_f16_nt(int64_t m, int64_t n, int64_t k, const uint16_t *a, const uint16_t *b, uint16_t *c,
                       int nthreads);
int oracle_gemm_f16_nn_f64(int64_t m, int64_t n, int64_t k, const uint16_t *a, const uint16_t *b,
                           const int64_t *rows, int64_t nrows, double *d64, double *dabs, int nthreads);

enum { GUARD = 64 };
static const uint16_t kSentinel16 = 0x7E00; /* an fp16 NaN */

#define HIP_OK(call)                                                                  \
    do {                                                                              \
        hipError_t e_ = (call);                                                       \
        if (e_ != hipSuccess) {                                                       \
            fprintf(stderr, "%s:%d: %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
            exit(2);                                                                  \
        }                                                                             \
    } while (0)

static void *host_alloc(size_t bytes) {
    void *p = malloc(bytes ? bytes : 1);
    if (!p) {
        fprintf(stderr, "out of host memory (%zu bytes)\n", bytes);
        exit(2);
    }
    return p;
}

/* fp16 bit pattern of i/8 for -8 <= i <= 8 (exact). */
static uint16_t eighth(int i) {
    if (i == 0) return 0;
    const uint16_t sign = i < 0 ? 0x8000 : 0;
    int v = i < 0 ? -i : i;
    int e = 0;
    while ((v >> (e + 1)) != 0) ++e; /* 2^e <= v < 2^(e+1) */
    const int mant = ((v << 10) >> e) & 0x3FF;
    return (uint16_t)(sign | (uint16_t)((e - 3 + 15) << 10) | (uint16_t)mant);
}

/* 64-bit linear congruential generator (Knuth's MMIX constants); the top
 * bits pick k in -8..8. */
static uint64_t lcg_state;
static int next_eighth(void) {
    lcg_state = lcg_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (int)((lcg_state >> 33) % 17) - 8;
}

static void fill(uint16_t *x, int64_t count) {
    for (int64_t i = 0; i < count; ++i) x[i] = eighth(next_eighth());
}

static int oracle_threads(void) {
    long n = sysconf(_SC_NPROCESSORS_ONLN);
    if (n < 1) n = 1;
    if (n > 16) n = 16;
    return (int)n;
}

/* C = A B^T on the device through gemm_f16_nt, against the oracle. */
static int case_nt(hipStream_t s, int64_t m, int64_t n, int64_t k, uint64_t seed) {
    printf("case: gemm_f16_nt m=%lld n=%lld k=%lld seed=%llu\n", (long long)m, (long long)n, (long long)k,
           (unsigned long long)seed);
    fflush(stdout);
    lcg_state = seed;
    const int64_t na = m * k, nb = n * k, nc = m * n, nbuf = nc + 2 * GUARD;
    uint16_t *a = host_alloc((size_t)(na ? na : 1) * 2), *b = host_alloc((size_t)(nb ? nb : 1) * 2);
    uint16_t *ref = host_alloc((size_t)nc * 2), *got = host_alloc((size_t)nbuf * 2);
    fill(a, na);
    fill(b, nb);
    if (oracle_gemm_f16_nt(m, n, k, a, b, ref, oracle_threads()) != 0) {
        fprintf(stderr, "oracle failed\n");
        exit(2);
    }
    for (int64_t i = 0; i < nbuf; ++i) got[i] = kSentinel16;

    void *da = NULL, *db = NULL, *dc = NULL;
    HIP_OK(hipMalloc(&da, (size_t)(na ? na : 1) * 2));
    HIP_OK(hipMalloc(&db, (size_t)(nb ? nb : 1) * 2));
    HIP_OK(hipMalloc(&dc, (size_t)nbuf * 2));
    if (na) HIP_OK(hipMemcpy(da, a, (size_t)na * 2, hipMemcpyHostToDevice));
    if (nb) HIP_OK(hipMemcpy(db, b, (size_t)nb * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dc, got, (size_t)nbuf * 2, hipMemcpyHostToDevice));

    const int rc = gemm_f16_nt(m, n, k, da, db, (uint16_t *)dc + GUARD, s);
    if (rc != GEMM_F16_OK) {
        fprintf(stderr, "gemm_f16_nt returned %d (%s)\n", rc, gemm_f16_status_string(rc));
        exit(1);
    }
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(got, dc, (size_t)nbuf * 2, hipMemcpyDeviceToHost));

    int bad = 0;
    for (int64_t i = 0; i < GUARD; ++i)
        if (got[i] != kSentinel16 || got[GUARD + nc + i] != kSentinel16) bad = 1;
    if (bad) fprintf(stderr, "write outside C\n");
    int64_t mismatches = 0, first = -1;
    for (int64_t i = 0; i < nc; ++i)
        if (got[GUARD + i] != ref[i]) {
            if (first < 0) first = i;
            ++mismatches;
        }
    if (mismatches) {
        fprintf(stderr, "%lld of %lld elements differ, first at (%lld, %lld): 0x%04x vs 0x%04x\n",
                (long long)mismatches, (long long)nc, (long long)(first / n), (long long)(first % n),
                got[GUARD + first], ref[first]);
        bad = 1;
    }
    HIP_OK(hipFree(da));
    HIP_OK(hipFree(db));
    HIP_OK(hipFree(dc));
    free(a);
    free(b);
    free(ref);
    free(got);
    return bad;
}

/* D = A B (B [K,N]) on the device through gemm_f16_nn_f32, against the
 * oracle's exact fp64 sums. */
static int case_nn(hipStream_t s, int64_t m, int64_t n, int64_t k, uint64_t seed) {
    printf("case: gemm_f16_nn_f32 m=%lld n=%lld k=%lld seed=%llu\n", (long long)m, (long long)n, (long long)k,
           (unsigned long long)seed);
    fflush(stdout);
    lcg_state = seed;
    const int64_t na = m * k, nb = k * n, nd = m * n, nbuf = nd + 2 * GUARD;
    uint16_t *a = host_alloc((size_t)na * 2), *b = host_alloc((size_t)nb * 2);
    double *ref = host_alloc((size_t)nd * sizeof(double));
    float *got = host_alloc((size_t)nbuf * sizeof(float));
    fill(a, na);
    fill(b, nb);
    if (oracle_gemm_f16_nn_f64(m, n, k, a, b, NULL, m, ref, NULL, oracle_threads()) != 0) {
        fprintf(stderr, "oracle failed\n");
        exit(2);
    }
    for (int64_t i = 0; i < nbuf; ++i) got[i] = -7.0f;

    void *da = NULL, *db = NULL, *dd = NULL;
    HIP_OK(hipMalloc(&da, (size_t)na * 2));
    HIP_OK(hipMalloc(&db, (size_t)nb * 2));
    HIP_OK(hipMalloc(&dd, (size_t)nbuf * sizeof(float)));
    HIP_OK(hipMemcpy(da, a, (size_t)na * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(db, b, (size_t)nb * 2, hipMemcpyHostToDevice));
    HIP_OK(hipMemcpy(dd, got, (size_t)nbuf * sizeof(float), hipMemcpyHostToDevice));

    const int rc = gemm_f16_nn_f32(m, n, k, da, db, (float *)dd + GUARD, s);
    if (rc != GEMM_F16_OK) {
        fprintf(stderr, "gemm_f16_nn_f32 returned %d (%s)\n", rc, gemm_f16_status_string(rc));
        exit(1);
    }
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(got, dd, (size_t)nbuf * sizeof(float), hipMemcpyDeviceToHost));

    int bad = 0;
    for (int64_t i = 0; i < GUARD; ++i)
        if (got[i] != -7.0f || got[GUARD + nd + i] != -7.0f) bad = 1;
    if (bad) fprintf(stderr, "write outside D\n");
    int64_t mismatches = 0, first = -1;
    for (int64_t i = 0; i < nd; ++i)
        if ((double)got[GUARD + i] != ref[i]) {
            if (first < 0) first = i;
            ++mismatches;
        }
    if (mismatches) {
        fprintf(stderr, "%lld of %lld elements differ, first at (%lld, %lld): %.9g vs %.17g\n", (long long)mismatches,
                (long long)nd, (long long)(first / n), (long long)(first % n), got[GUARD + first], ref[first]);
        bad = 1;
    }
    HIP_OK(hipFree(da));
    HIP_OK(hipFree(db));
    HIP_OK(hipFree(dd));
    free(a);
    free(b);
    free(ref);
    free(got);
    return bad;
}

/* Refusals that need device pointers: C overlapping A, and K = 0 (C := 0). */
static int case_edges(hipStream_t s) {
    printf("case: overlap and k = 0\n");
    fflush(stdout);
    enum { M = 40, N = 24, K = 16 };
    void *buf = NULL;
    HIP_OK(hipMalloc(&buf, (size_t)(M * K + N * K + M * N) * 2));
    uint16_t *a = buf, *b = a + M * K, *c = b + N * K;
    int bad = 0;
    if (gemm_f16_nt(M, N, K, a, b, a + 8, s) != GEMM_F16_EOVERLAP) bad = 1;
    uint16_t *host = host_alloc((size_t)M * N * 2);
    for (int i = 0; i < M * N; ++i) host[i] = kSentinel16;
    HIP_OK(hipMemcpy(c, host, (size_t)M * N * 2, hipMemcpyHostToDevice));
    if (gemm_f16_nt(M, N, 0, NULL, NULL, c, s) != GEMM_F16_OK) bad = 1;
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(host, c, (size_t)M * N * 2, hipMemcpyDeviceToHost));
    for (int i = 0; i < M * N; ++i)
        if (host[i] != 0) bad = 1;
    if (bad) fprintf(stderr, "overlap or k = 0 case failed\n");
    free(host);
    HIP_OK(hipFree(buf));
    return bad;
}

int main(void) {
    int count = 0;
    HIP_OK(hipGetDeviceCount(&count));
    if (count < 1) {
        fprintf(stderr, "no HIP device\n");
        return 2;
    }
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    int bad = 0;
    bad |= case_nt(s, 300, 520, 1000, 1);   /* ragged M, N and a K tail */
    bad |= case_nt(s, 1024, 1024, 512, 2);  /* whole 256x256 tiles */
    bad |= case_nt(s, 2048, 1536, 640, 3);  /* more tiles than CUs */
    bad |= case_nt(s, 37, 19, 8, 4);        /* one partial tile */
    bad |= case_nn(s, 300, 520, 1000, 5);
    bad |= case_nn(s, 1024, 512, 768, 6);
    bad |= case_edges(s);
    HIP_OK(hipStreamDestroy(s));
    if (bad) return 1;
    puts("ok");
    return 0;
}
