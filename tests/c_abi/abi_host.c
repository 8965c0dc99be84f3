/*
 * The library's C ABI from a C program: the header compiles as C99 and the
 * host-side entry points link and behave as include/gemm_f16.h states.
 * Every call here returns before any device is touched (argument errors are
 * reported first), so it runs on a host without a GPU.  Prints "ok" and
 * exits 0, or names the failed check and exits 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "gemm_f16.h"

#define CHECK(cond)                                                        \
    do {                                                                   \
        if (!(cond)) {                                                     \
            fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            return 1;                                                      \
        }                                                                  \
    } while (0)

static int status_strings(void) {
    const int codes[] = {GEMM_F16_OK,      GEMM_F16_EINVAL, GEMM_F16_ENULL,   GEMM_F16_EALIGN,
                         GEMM_F16_EDEVICE, GEMM_F16_EHIP,   GEMM_F16_EOVERLAP};
    const int n = (int)(sizeof codes / sizeof codes[0]);
    for (int i = 0; i < n; ++i) {
        const char *s = gemm_f16_status_string(codes[i]);
        CHECK(s != NULL && s[0] != '\0');
        for (int j = 0; j < i; ++j) CHECK(strcmp(s, gemm_f16_status_string(codes[j])) != 0);
    }
    CHECK(gemm_f16_status_string(12345) != NULL);
    CHECK(gemm_f16_status_string(-12345) != NULL);
    return 0;
}

/* Argument errors come back as codes, before the device gate. */
static int argument_errors(void) {
    uint16_t buf[64] = {0};
    float dbuf[16] = {0};
    uint16_t *a = buf, *b = buf + 16, *c = buf + 32;
    CHECK(gemm_f16_nt(-1, 4, 4, a, b, c, NULL) == GEMM_F16_EINVAL);
    CHECK(gemm_f16_nt(4, (int64_t)1 << 30, 4, a, b, c, NULL) == GEMM_F16_EINVAL);
    CHECK(gemm_f16_nt(4, 4, (int64_t)1 << 22, a, b, c, NULL) == GEMM_F16_EINVAL);
    CHECK(gemm_f16_nt(4, 4, 4, a, b, NULL, NULL) == GEMM_F16_ENULL);
    CHECK(gemm_f16_nt(4, 4, 4, NULL, b, c, NULL) == GEMM_F16_ENULL);
    CHECK(gemm_f16_nt(4, 4, 4, (const char *)a + 1, b, c, NULL) == GEMM_F16_EALIGN);
    CHECK(gemm_f16_nt(4, 4, 4, a, b, (char *)c + 1, NULL) == GEMM_F16_EALIGN);
    CHECK(gemm_f16_nt(4, 4, 4, a, b, buf + 8, NULL) == GEMM_F16_EOVERLAP); /* C over A */
    CHECK(gemm_f16_nt(4, 4, 4, a, b, buf + 20, NULL) == GEMM_F16_EOVERLAP); /* C over B */
    /* an empty C is a no-op, whatever the pointers */
    CHECK(gemm_f16_nt(0, 4, 4, NULL, NULL, NULL, NULL) == GEMM_F16_OK);
    CHECK(gemm_f16_nt(4, 0, 4, NULL, NULL, NULL, NULL) == GEMM_F16_OK);

    /* the second contract: D is fp32, 4-byte aligned */
    CHECK(gemm_f16_nn_f32(-1, 4, 4, a, b, dbuf, NULL) == GEMM_F16_EINVAL);
    CHECK(gemm_f16_nn_f32(4, 4, 4, a, b, NULL, NULL) == GEMM_F16_ENULL);
    CHECK(gemm_f16_nn_f32(4, 4, 4, a, b, (char *)dbuf + 2, NULL) == GEMM_F16_EALIGN);
    CHECK(gemm_f16_nn_f32(0, 4, 4, NULL, NULL, NULL, NULL) == GEMM_F16_OK);

    /* options */
    gemm_f16_options o;
    memset(&o, 0, sizeof o);
    o.xcd = -1;
    o.tile = 99;
    CHECK(gemm_f16_nt_ex(4, 4, 4, a, b, c, NULL, &o) == GEMM_F16_EINVAL);
    o.tile = 0;
    o.swizzle = -1;
    CHECK(gemm_f16_nt_ex(4, 4, 4, a, b, c, NULL, &o) == GEMM_F16_EINVAL);
    o.swizzle = 0;
    o.xcd = 2;
    CHECK(gemm_f16_nt_ex(4, 4, 4, a, b, c, NULL, &o) == GEMM_F16_EINVAL);
    o.xcd = -1;
    o.variant = 1; /* a variant needs an explicit block tile */
    CHECK(gemm_f16_nt_ex(4, 4, 64, a, b, c, NULL, &o) == GEMM_F16_EINVAL);
    return 0;
}

/* The scheduler is a bijection of the grid, with either XCD setting. */
static int scheduler(void) {
    enum { NM = 7, NN = 5 };
    for (int32_t sw = 1; sw <= 6; ++sw) {
        for (int32_t xcd = 0; xcd <= 1; ++xcd) {
            int seen[NM][NN];
            memset(seen, 0, sizeof seen);
            for (int64_t pid = 0; pid < NM * NN; ++pid) {
                int64_t mb = -1, nb = -1;
                CHECK(gemm_f16_tile_coord(pid, NM, NN, sw, xcd, &mb, &nb) == GEMM_F16_OK);
                CHECK(mb >= 0 && mb < NM && nb >= 0 && nb < NN);
                seen[mb][nb] += 1;
            }
            for (int i = 0; i < NM; ++i)
                for (int j = 0; j < NN; ++j) CHECK(seen[i][j] == 1);
        }
    }
    int64_t mb, nb;
    CHECK(gemm_f16_tile_coord(NM * NN, NM, NN, 1, 0, &mb, &nb) == GEMM_F16_EINVAL);
    CHECK(gemm_f16_tile_coord(0, NM, NN, 1, 0, NULL, &nb) == GEMM_F16_ENULL);
    CHECK(gemm_f16_select_xcd(16, 16, 4, 256) == 0);
    CHECK(gemm_f16_select_xcd(32, 8, 4, 256) == 1);
    CHECK(gemm_f16_select_xcd(0, 8, 4, 256) == GEMM_F16_EINVAL);
    const int t = gemm_f16_select_tile(8192, 8192, 8192);
    CHECK(t >= 1 && t <= GEMM_F16_TILE_LAST);
    CHECK(gemm_f16_select_tile(-1, 4, 4) == GEMM_F16_EINVAL);
    return 0;
}

int main(void) {
    if (status_strings() || argument_errors() || scheduler()) return 1;
    puts("ok");
    return 0;
}
