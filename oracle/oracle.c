/*
 * oracle.c -- plain CPU oracle for tiled f32 maps, copies and row/column reductions.
 *
 * TEST INFRASTRUCTURE ONLY (see oracle.h): loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product library.
 *
 * Plain, single-threaded C99.  Built with -O2 -ffp-contract=off and without fast-math, so every
 * float operation below is exactly the IEEE operation written: fmaf is the C99 correctly rounded
 * fused multiply-add, `a * b` is one rounded multiply, and sums accumulate in double in the order
 * of the loops.
 */
#include "oracle.h"

#include <math.h>
#include <string.h>

/* The mask fill of a maximum: the f32 nearest to -1.0e30 ([SLICING] "Reductions over a ragged
 * tile"). */
#define ORC_MAX_FILL (-1.0e30f)

void orc_split(int64_t K, int64_t T, int64_t *nfull, int64_t *rem)
{
    /* [SLICING] "Loops over a dynamic extent": whole tiles first, then what is left over. */
    *nfull = K / T;
    *rem = K - (*nfull) * T;
}

int64_t orc_tile_live(int64_t M, int64_t N, int64_t TM, int64_t TN, int64_t pm, int64_t pn)
{
    /* [SLICING] "Masking": count the tile's elements that exist, one by one. */
    int64_t live = 0;
    for (int64_t r = 0; r < TM; ++r) {
        for (int64_t c = 0; c < TN; ++c) {
            int64_t i = pm * TM + r;
            int64_t j = pn * TN + c;
            if (i < M && j < N)
                ++live;
        }
    }
    return live;
}

int orc_promise_holds(int64_t M, int64_t N, int64_t ld_in, int64_t ld_out, int64_t TM, int64_t TN,
                      uint64_t in_addr, uint64_t out_addr)
{
    /* [ALIGNED] "What it changes": the dimension is a whole number of tiles ... */
    if (M % TM != 0)
        return 0;
    if (N % TN != 0)
        return 0;
    /* ... and its rows may be moved as 16-byte vectors, which needs every row to start on a
     * 16-byte boundary ([LAYOUT] "The alignment constraint": four f32 elements): a 16-byte base
     * and, when there is more than one row, a row stride that is a multiple of 4 elements. */
    if (TN % 4 != 0)
        return 0;
    if (in_addr % 16 != 0)
        return 0;
    if (M > 1 && ld_in % 4 != 0)
        return 0;
    if (out_addr != 0) {
        if (out_addr % 16 != 0)
            return 0;
        if (M > 1 && ld_out % 4 != 0)
            return 0;
    }
    return 1;
}

void orc_map_affine(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
                    float alpha, float beta)
{
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            y[i * ldy + j] = fmaf(x[i * ldx + j], alpha, beta);
}

void orc_scale2d(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
                 float alpha)
{
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j)
            y[i * ldy + j] = alpha * x[i * ldx + j];
}

void orc_copy2d(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N)
{
    /* A byte copy of each row, so NaN payloads and signed zeros travel unchanged. */
    for (int64_t i = 0; i < M; ++i)
        if (N > 0)
            memmove(&y[i * ldy], &x[i * ldx], (size_t)N * sizeof(float));
}

void orc_rowsum_f64(const float *x, int64_t ldx, int64_t M, int64_t N, double *out)
{
    for (int64_t i = 0; i < M; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < N; ++j)
            acc += (double)x[i * ldx + j];
        out[i] = acc;
    }
}

void orc_colsum_f64(const float *x, int64_t ldx, int64_t M, int64_t N, double *out)
{
    for (int64_t j = 0; j < N; ++j) {
        double acc = 0.0;
        for (int64_t i = 0; i < M; ++i)
            acc += (double)x[i * ldx + j];
        out[j] = acc;
    }
}

void orc_rowmax(const float *s, int64_t lds, int64_t M, int64_t N, float *out)
{
    for (int64_t i = 0; i < M; ++i) {
        float m = ORC_MAX_FILL;
        for (int64_t j = 0; j < N; ++j) {
            float v = s[i * lds + j];
            if (v > m)
                m = v;
        }
        out[i] = m;
    }
}

void orc_map_affine_tiled(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
                          float alpha, float beta, int64_t TM, int64_t TN)
{
    int64_t tiles_m = (M + TM - 1) / TM;
    int64_t tiles_n = (N + TN - 1) / TN;
    for (int64_t pm = 0; pm < tiles_m; ++pm) {
        for (int64_t pn = 0; pn < tiles_n; ++pn) {
            for (int64_t r = 0; r < TM; ++r) {
                for (int64_t c = 0; c < TN; ++c) {
                    int64_t i = pm * TM + r;
                    int64_t j = pn * TN + c;
                    int inside = (i < M) && (j < N);
                    float v = inside ? x[i * ldx + j] : 0.0f; /* masked read gives 0 */
                    float res = fmaf(v, alpha, beta);
                    if (inside) /* masked store is skipped */
                        y[i * ldy + j] = res;
                }
            }
        }
    }
}

void orc_rowsum_tiled_f64(const float *x, int64_t ldx, int64_t M, int64_t N, int64_t TN,
                          double *out)
{
    int64_t nfull, rem;
    orc_split(N, TN, &nfull, &rem);
    for (int64_t i = 0; i < M; ++i) {
        double acc = 0.0;
        int64_t kt = 0;
        for (int64_t t = 0; t < nfull; ++t, kt += TN) /* whole tiles: no mask */
            for (int64_t c = 0; c < TN; ++c)
                acc += (double)x[i * ldx + kt + c];
        if (rem > 0) { /* one masked remainder tile */
            for (int64_t c = 0; c < TN; ++c) {
                float v = (c < N - kt) ? x[i * ldx + kt + c] : 0.0f;
                acc += (double)v;
            }
        }
        out[i] = acc;
    }
}

void orc_rowmax_tiled(const float *s, int64_t lds, int64_t M, int64_t N, int64_t BC, float fill,
                      float *out)
{
    int64_t nfull, rem;
    orc_split(N, BC, &nfull, &rem);
    for (int64_t i = 0; i < M; ++i) {
        float m = fill;
        int64_t kt = 0;
        for (int64_t t = 0; t < nfull; ++t, kt += BC) {
            for (int64_t c = 0; c < BC; ++c) {
                float v = s[i * lds + kt + c];
                if (v > m)
                    m = v;
            }
        }
        if (rem > 0) {
            for (int64_t c = 0; c < BC; ++c) {
                /* where(iota(1) < N - kt, s, fill) */
                float v = (c < N - kt) ? s[i * lds + kt + c] : fill;
                if (v > m)
                    m = v;
            }
        }
        out[i] = m;
    }
}

void orc_softmax_stats(const float *s, int64_t lds, int64_t M, int64_t N, float *m, double *l)
{
    orc_rowmax(s, lds, M, N, m);
    for (int64_t i = 0; i < M; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < N; ++j)
            acc += exp((double)s[i * lds + j] - (double)m[i]);
        l[i] = acc;
    }
}

void orc_softmax_stats_tiled(const float *s, int64_t lds, int64_t M, int64_t N, int64_t BC,
                             float fill, float *m, double *l)
{
    int64_t nfull, rem;
    orc_split(N, BC, &nfull, &rem);
    const int64_t ntiles = nfull + (rem > 0 ? 1 : 0);
    for (int64_t i = 0; i < M; ++i) {
        double run_m = (double)fill;
        double run_l = 0.0;
        for (int64_t t = 0; t < ntiles; ++t) {
            const int64_t kt = t * BC;
            /* the tile, with where(iota(1) < N - kt, s, fill) applied (a no-op on whole tiles) */
            double tile_max = (double)fill;
            for (int64_t c = 0; c < BC; ++c) {
                double v = (c < N - kt) ? (double)s[i * lds + kt + c] : (double)fill;
                if (v > tile_max)
                    tile_max = v;
            }
            double new_m = run_m > tile_max ? run_m : tile_max;
            double tile_sum = 0.0;
            for (int64_t c = 0; c < BC; ++c) {
                double v = (c < N - kt) ? (double)s[i * lds + kt + c] : (double)fill;
                tile_sum += exp(v - new_m);
            }
            run_l = run_l * exp(run_m - new_m) + tile_sum;
            run_m = new_m;
        }
        m[i] = (float)run_m;
        l[i] = run_l;
    }
}

void orc_transpose(const float *x, int64_t ldx, int64_t bsx, float *y, int64_t ldy, int64_t bsy,
                   int64_t B, int64_t M, int64_t N)
{
    for (int64_t b = 0; b < B; ++b)
        for (int64_t i = 0; i < M; ++i)
            for (int64_t j = 0; j < N; ++j)
                memcpy(&y[b * bsy + j * ldy + i], &x[b * bsx + i * ldx + j], sizeof(float));
}

void orc_channel_affine(const float *x, int64_t ldx, const float *scale, const float *bias, float *y,
                        int64_t ldy, int64_t M, int64_t N)
{
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t j = 0; j < N; ++j) {
            if (scale != 0)
                y[i * ldy + j] = fmaf(x[i * ldx + j], scale[j], bias[j]);
            else
                y[i * ldy + j] = x[i * ldx + j] + bias[j];
        }
    }
}
