/*
 * oracle.h -- plain CPU oracle for tiled f32 maps, copies and row/column reductions.
 *
 * TEST INFRASTRUCTURE ONLY.  This library defines what the tiled GPU path must compute.  Only the
 * test suite, the package's smoke check and the benchmark's CPU-baseline leg may load it; the
 * product library never links, loads or calls it, and it shares no header, helper or constant
 * with the product sources.
 *
 * Sources (web pages; cited by title and section):
 *   [ALIGNED]  Phobos docs, "@aligned" -- sections "A minimal kernel", "What it changes",
 *              "When the promise is broken".
 *   [P35]      Mojo GPU puzzles, puzzle 35 "Aligned Load & Store" -- sections "The exercise",
 *              "Solution".
 *   [SLICING]  Phobos docs, "Slicing, bounds and masking" -- sections "Masking", "Loops over a
 *              dynamic extent", "Promising whole tiles with @aligned", "Reductions over a ragged
 *              tile".
 *   [LAYOUT]   teenygrad kernels book, "Memory Coalescing and Tensor Layout" -- sections
 *              "What it actually costs", "Strides, and reading an index expression",
 *              "The alignment constraint".
 *
 * Conventions: every 2-D tensor is a row-major view with an explicit row stride `ld` (in
 * elements), element (i, j) at p[i*ld + j] ([LAYOUT] "Strides, and reading an index expression";
 * the passed stride is used, never the row length, per "The alignment constraint").
 * The oracle writes only the elements { y[i*ldy + j] : 0 <= i < M, 0 <= j < N } of an output.
 *
 * Parity status: every function below is pinned by a CPU test against values the pages print,
 * closed forms, library routines or brute force (see tests/test_oracle_pins.py).
 */
#ifndef TILEMAP_ORACLE_H
#define TILEMAP_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- loop remainder split ([SLICING] "Loops over a dynamic extent") ---------------------------
 * A loop over a run-time extent K in steps of T is a number of whole tiles plus at most one
 * masked remainder tile.  Writes the whole-tile count to *nfull and the remainder width to *rem.
 * Requires K >= 0, T > 0. */
void orc_split(int64_t K, int64_t T, int64_t *nfull, int64_t *rem);

/* ---- edge tiles ([SLICING] "Masking") ----------------------------------------------------------
 * Number of elements of tile (pm, pn) -- rows [pm*TM, pm*TM+TM), columns [pn*TN, pn*TN+TN) --
 * that lie inside an M x N tensor.  The tile's other TM*TN - live elements read as 0 and their
 * stores are skipped. */
int64_t orc_tile_live(int64_t M, int64_t N, int64_t TM, int64_t TN, int64_t pm, int64_t pn);

/* ---- the alignment promise ([ALIGNED] "What it changes", "When the promise is broken";
 * [LAYOUT] "The alignment constraint") ------------------------------------------------------------
 * Returns 1 when an M x N tensor pair keeps the whole-tile promise for TM x TN tiles and its rows
 * may move as 16-byte vectors: M % TM == 0, N % TN == 0, TN % 4 == 0, and every row of both
 * tensors starts on a 16-byte boundary (base % 16 == 0 and, when M > 1, row stride % 4 == 0).
 * `out_addr == 0` means there is no 2-D output (reductions); ld_out is then ignored.  Returns 0
 * otherwise.  Requires TM, TN > 0. */
int orc_promise_holds(int64_t M, int64_t N, int64_t ld_in, int64_t ld_out, int64_t TM, int64_t TN,
                      uint64_t in_addr, uint64_t out_addr);

/* ---- plain definitions ----------------------------------------------------------------------- */

/* y[i,j] = fmaf(x[i,j], alpha, beta): one correctly rounded multiply-add ([P35] "The exercise":
 * out = a*2 + 1, generalised to alpha, beta). */
void orc_map_affine(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
                    float alpha, float beta);

/* y[i,j] = alpha * x[i,j]: one IEEE single multiply ([ALIGNED] "A minimal kernel"). */
void orc_scale2d(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
                 float alpha);

/* y[i,j] = x[i,j], bit for bit ([SLICING] "Promising whole tiles with @aligned", kernel copy2d). */
void orc_copy2d(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N);

/* out[i] = sum_j x[i,j], accumulated left to right in double ([LAYOUT] "What it actually costs":
 * the row walk over a row-major matrix). */
void orc_rowsum_f64(const float *x, int64_t ldx, int64_t M, int64_t N, double *out);

/* out[j] = sum_i x[i,j], accumulated top to bottom in double ([LAYOUT] "What it actually costs":
 * the column walk over the same matrix). */
void orc_colsum_f64(const float *x, int64_t ldx, int64_t M, int64_t N, double *out);

/* out[i] = max over 0 <= j < N of s[i,j], starting from the mask fill -1.0e30f, so an empty row
 * gives -1.0e30f ([SLICING] "Reductions over a ragged tile").  NaN entries never win. */
void orc_rowmax(const float *s, int64_t lds, int64_t M, int64_t N, float *out);

/* Softmax row statistics: m[i] = the row maximum exactly as orc_rowmax computes it, and
 * l[i] = sum over 0 <= j < N of exp(s[i,j] - m[i]) in double ([SLICING] "Reductions over a ragged
 * tile": the masked maximum is what a softmax needs; l is the normaliser that goes with it).  An
 * empty row gives m = -1.0e30f and l = 0. */
void orc_softmax_stats(const float *s, int64_t lds, int64_t M, int64_t N, float *m, double *l);

/* Per-channel affine on an NC view: y[i,j] = fmaf(x[i,j], scale[j], bias[j]), or x[i,j] + bias[j]
 * when scale is NULL (one IEEE add).  Columns are channels: a (B, C, H, W) tensor stored NHWC is
 * the M = B*H*W by N = C view ([LAYOUT] "NCHW versus NHWC": per-channel scale and bias want the
 * channel dimension contiguous; the tree's channel_bias_add reads the tensor as NC with
 * N = B*H*W). */
void orc_channel_affine(const float *x, int64_t ldx, const float *scale, const float *bias, float *y,
                        int64_t ldy, int64_t M, int64_t N);

/* Batched transpose: y[b][j][i] = x[b][i][j] for b < B, i < M, j < N, bit for bit.  Batch b of x
 * starts at x + b*bsx with row stride ldx (M x N); batch b of y starts at y + b*bsy with row stride
 * ldy (N x M).  With x = [B][C][H*W] (M = C, N = H*W) this is the NCHW -> NHWC layout conversion
 * ([LAYOUT] "NCHW versus NHWC"; the flat index of [LAYOUT] "Strides, and reading an index
 * expression"). */
void orc_transpose(const float *x, int64_t ldx, int64_t bsx, float *y, int64_t ldy, int64_t bsy,
                   int64_t B, int64_t M, int64_t N);

/* ---- tiled walks: the pages' masked-tile procedure, step by step -----------------------------
 * These follow the tile-by-tile procedure (masked loads read as 0, masked stores skipped, loops
 * split into whole tiles plus a masked remainder).  The tests check that each one reproduces the
 * plain definition above, which pins the masking rules themselves. */

/* Walk ceil(M/TM) x ceil(N/TN) tiles; an element outside the tensor reads as 0.0f and its store
 * is skipped ([SLICING] "Masking"). */
void orc_map_affine_tiled(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
                          float alpha, float beta, int64_t TM, int64_t TN);

/* Row sums walking TN-wide column tiles: whole tiles unmasked, then one remainder tile whose
 * missing columns read as 0 ([SLICING] "Loops over a dynamic extent", "Masking"). */
void orc_rowsum_tiled_f64(const float *x, int64_t ldx, int64_t M, int64_t N, int64_t TN,
                          double *out);

/* Row maxima walking BC-wide column tiles: whole tiles unmasked, then one remainder tile in which
 * column c (tile-local index) keeps its score iff c < N - kt, else takes `fill`; the running maximum
 * starts at `fill` ([SLICING] "Reductions over a ragged tile").  The method uses fill = -1.0e30f;
 * fill = 0 reproduces the pages' counter-example. */
void orc_rowmax_tiled(const float *s, int64_t lds, int64_t M, int64_t N, int64_t BC, float fill,
                      float *out);

/* Softmax row statistics walking BC-wide column tiles online: for each tile (whole tiles, then one
 * remainder tile whose missing columns take `fill`, as in orc_rowmax_tiled) the tile maximum
 * t = max(tile), the new running maximum m' = max(m, t), and l' = l * exp(m - m') +
 * sum over the tile of exp(s - m'), all in double; the running values start at m = fill, l = 0.
 * With fill = -1.0e30f every masked column adds exp(-1e30 - m') = 0. */
void orc_softmax_stats_tiled(const float *s, int64_t lds, int64_t M, int64_t N, int64_t BC,
                             float fill, float *m, double *l);

#ifdef __cplusplus
}
#endif
#endif
