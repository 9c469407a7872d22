/* oracle_check.c -- the oracle's functions over every small shape, built with gcc under
 * AddressSanitizer and UndefinedBehaviorSanitizer by tests/test_sanitizers_cpu.py (no GPU).
 *
 * Every buffer is allocated at exactly the size the call may touch ((rows - 1) * ld + cols
 * elements), so a read or write past it is reported by the sanitizer.  Along the way the tiled
 * walks are compared with the plain definitions (the same self-consistency the Python pins check),
 * so the run also fails on a wrong result.  Exit status 0 when everything passes. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/oracle.h"

static long checked = 0, failed = 0;

#define CHECK(cond, ...)                                 \
    do {                                                 \
        ++checked;                                       \
        if (!(cond) && failed++ < 20) {                  \
            fprintf(stderr, "FAIL %s: ", #cond);         \
            fprintf(stderr, __VA_ARGS__);                \
            fprintf(stderr, "\n");                       \
        }                                                \
    } while (0)

static uint64_t state = 0x9E3779B97F4A7C15ull;
static float frand(float lo, float hi) {
    state ^= state << 13;
    state ^= state >> 7;
    state ^= state << 17;
    return lo + (hi - lo) * (float)((state >> 40) * (1.0 / 16777216.0));
}

static size_t span(int64_t rows, int64_t cols, int64_t ld) {
    return rows > 0 && cols > 0 ? (size_t)((rows - 1) * ld + cols) : 1;
}

static float *fill(size_t n, float lo, float hi) {
    float *p = malloc(n * sizeof *p);
    for (size_t i = 0; i < n; ++i)
        p[i] = frand(lo, hi);
    return p;
}

static void check_maps_and_reductions(void) {
    for (int64_t M = 0; M <= 17; ++M)
        for (int64_t N = 0; N <= 17; ++N) {
            const int64_t lds[3] = {N, N + 3, (N + 3) / 4 * 4};
            for (int k = 0; k < 3; ++k) {
                const int64_t ld = lds[k];
                const size_t n = span(M, N, ld);
                float *x = fill(n, -8.f, 8.f);
                float *y0 = malloc(n * sizeof *y0), *y1 = malloc(n * sizeof *y1);
                memset(y0, 0x7F, n * sizeof *y0);
                memcpy(y1, y0, n * sizeof *y1);
                orc_map_affine(x, ld, y0, ld, M, N, 0.75f, -0.25f);
                double *r0 = malloc((M ? M : 1) * sizeof *r0), *r1 = malloc((M ? M : 1) * sizeof *r1);
                double *c0 = malloc((N ? N : 1) * sizeof *c0);
                float *mx0 = malloc((M ? M : 1) * sizeof *mx0), *mx1 = malloc((M ? M : 1) * sizeof *mx1);
                float *sm0 = malloc((M ? M : 1) * sizeof *sm0), *sm1 = malloc((M ? M : 1) * sizeof *sm1);
                double *sl0 = malloc((M ? M : 1) * sizeof *sl0), *sl1 = malloc((M ? M : 1) * sizeof *sl1);
                orc_rowsum_f64(x, ld, M, N, r0);
                orc_colsum_f64(x, ld, M, N, c0);
                orc_rowmax(x, ld, M, N, mx0);
                orc_softmax_stats(x, ld, M, N, sm0, sl0);
                float *z = malloc(n * sizeof *z);
                orc_scale2d(x, ld, z, ld, M, N, 1.5f);
                orc_copy2d(x, ld, z, ld, M, N);
                for (int64_t i = 0; i < M; ++i)
                    CHECK(N == 0 || memcmp(z + i * ld, x + i * ld, (size_t)N * sizeof(float)) == 0,
                          "copy M=%ld N=%ld row %ld", (long)M, (long)N, (long)i);
                for (int64_t TM = 1; TM <= 16; TM *= 2)
                    for (int64_t TN = 1; TN <= 16; TN *= 2) {
                        memset(y1, 0x7F, n * sizeof *y1);
                        orc_map_affine_tiled(x, ld, y1, ld, M, N, 0.75f, -0.25f, TM, TN);
                        CHECK(memcmp(y0, y1, n * sizeof *y0) == 0, "tiled map M=%ld N=%ld ld=%ld TM=%ld TN=%ld",
                              (long)M, (long)N, (long)ld, (long)TM, (long)TN);
                    }
                for (int64_t T = 1; T <= 16; T *= 2) {
                    orc_rowsum_tiled_f64(x, ld, M, N, T, r1);
                    orc_rowmax_tiled(x, ld, M, N, T, -1.0e30f, mx1);
                    orc_softmax_stats_tiled(x, ld, M, N, T, -1.0e30f, sm1, sl1);
                    for (int64_t i = 0; i < M; ++i) {
                        CHECK(r0[i] == r1[i], "tiled rowsum M=%ld N=%ld T=%ld", (long)M, (long)N, (long)T);
                        CHECK(mx0[i] == mx1[i] && sm0[i] == mx0[i], "tiled rowmax M=%ld N=%ld T=%ld", (long)M,
                              (long)N, (long)T);
                        CHECK(fabs(sl0[i] - sl1[i]) <= 1e-13 * (sl0[i] > 1e-300 ? sl0[i] : 1e-300),
                              "tiled softmax M=%ld N=%ld T=%ld", (long)M, (long)N, (long)T);
                    }
                }
                for (int64_t TM = 1; TM <= 16; TM *= 2)
                    for (int64_t TN = 1; TN <= 16; TN *= 2) {
                        int64_t live = 0;
                        for (int64_t pm = 0; pm * TM < M; ++pm)
                            for (int64_t pn = 0; pn * TN < N; ++pn)
                                live += orc_tile_live(M, N, TM, TN, pm, pn);
                        CHECK(live == M * N, "tile_live sum M=%ld N=%ld", (long)M, (long)N);
                    }
                free(x); free(y0); free(y1); free(z); free(r0); free(r1); free(c0);
                free(mx0); free(mx1); free(sm0); free(sm1); free(sl0); free(sl1);
            }
        }
}

static void check_layout(void) {
    for (int64_t B = 1; B <= 3; ++B)
        for (int64_t M = 1; M <= 13; M += 3)
            for (int64_t N = 1; N <= 13; N += 4) {
                const int64_t ldx = N + 1, ldy = M + 2;
                const int64_t bsx = M * ldx, bsy = N * ldy;
                const size_t nx = (size_t)((B - 1) * bsx) + span(M, N, ldx);
                const size_t ny = (size_t)((B - 1) * bsy) + span(N, M, ldy);
                float *x = fill(nx, -1.f, 1.f), *y = malloc(ny * sizeof *y), *back = malloc(nx * sizeof *back);
                memset(y, 0, ny * sizeof *y);
                memset(back, 0, nx * sizeof *back);
                orc_transpose(x, ldx, bsx, y, ldy, bsy, B, M, N);
                orc_transpose(y, ldy, bsy, back, ldx, bsx, B, N, M);
                for (int64_t b = 0; b < B; ++b)
                    for (int64_t i = 0; i < M; ++i)
                        for (int64_t j = 0; j < N; ++j) {
                            CHECK(y[b * bsy + j * ldy + i] == x[b * bsx + i * ldx + j], "transpose B=%ld M=%ld N=%ld",
                                  (long)B, (long)M, (long)N);
                            CHECK(back[b * bsx + i * ldx + j] == x[b * bsx + i * ldx + j], "involution");
                        }
                free(x); free(y); free(back);
            }
    for (int64_t M = 1; M <= 9; ++M)
        for (int64_t N = 1; N <= 9; ++N) {
            const int64_t ld = N + 2;
            const size_t n = span(M, N, ld);
            float *x = fill(n, -2.f, 2.f), *y = malloc(n * sizeof *y);
            float *bias = fill((size_t)N, -1.f, 1.f), *scale = fill((size_t)N, 0.5f, 1.5f);
            orc_channel_affine(x, ld, NULL, bias, y, ld, M, N);
            for (int64_t i = 0; i < M; ++i)
                for (int64_t j = 0; j < N; ++j)
                    CHECK(y[i * ld + j] == x[i * ld + j] + bias[j], "bias add M=%ld N=%ld", (long)M, (long)N);
            orc_channel_affine(x, ld, scale, bias, y, ld, M, N);
            for (int64_t i = 0; i < M; ++i)
                for (int64_t j = 0; j < N; ++j)
                    CHECK(y[i * ld + j] == fmaf(x[i * ld + j], scale[j], bias[j]), "affine M=%ld N=%ld", (long)M,
                          (long)N);
            free(x); free(y); free(bias); free(scale);
        }
}

static void check_host_helpers(void) {
    for (int64_t K = 0; K <= 300; ++K)
        for (int64_t T = 1; T <= 70; ++T) {
            int64_t nf = -1, rem = -1;
            orc_split(K, T, &nf, &rem);
            CHECK(nf * T + rem == K && rem >= 0 && rem < T, "split K=%ld T=%ld", (long)K, (long)T);
        }
    for (int64_t M = 0; M <= 9; ++M)
        for (int64_t N = 0; N <= 9; ++N)
            for (int64_t TM = 1; TM <= 8; TM *= 2)
                for (int64_t TN = 1; TN <= 8; TN *= 2)
                    for (uint64_t base = 0x1000; base <= 0x1010; base += 4)
                        (void)orc_promise_holds(M, N, N + 1, N, TM, TN, base, base + 0x100);
}

int main(void) {
    check_maps_and_reductions();
    check_layout();
    check_host_helpers();
    printf("oracle_check: %ld checks, %ld failures\n", checked, failed);
    return failed == 0 ? 0 : 1;
}
