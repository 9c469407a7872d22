/*
 * tilemap.h -- C ABI of libtilemap.so: tiled, memory-bound f32 maps, copies and row/column
 * reductions on AMD Instinct MI355X (gfx950).
 *
 * Sources the operations follow (web pages, cited by title and section):
 *   [ALIGNED]  Phobos docs, "@aligned": sections "A minimal kernel", "What it changes",
 *              "When the promise is broken".
 *   [P35]      Mojo GPU puzzles, puzzle 35 "Aligned Load & Store": sections "The exercise",
 *              "Key API", "Solution".
 *   [SLICING]  Phobos docs, "Slicing, bounds and masking": sections "Masking", "Loops over a
 *              dynamic extent", "Promising whole tiles with @aligned", "Reductions over a ragged
 *              tile".
 *   [LAYOUT]   teenygrad kernels book, "Memory Coalescing and Tensor Layout": sections
 *              "Coalescing", "What it actually costs", "Seeing it in a real kernel",
 *              "The alignment constraint".
 *
 * ---- Common conventions -------------------------------------------------------------------------
 * Layout.  Every 2-D tensor is an M x N row-major view of f32 with an explicit row stride `ld`
 *   (elements, ld >= N): element (i, j) lives at p[i*ld + j].  The passed stride is always used,
 *   never N ([LAYOUT] "The alignment constraint").  1-D data is the case M = 1.
 * Tiles.  A call cuts the tensor into TM x TN tiles; tile (pm, pn) covers rows [pm*TM, pm*TM+TM) and
 *   columns [pn*TN, pn*TN+TN) ([SLICING] subscript form `pm*TM :+ TM`).  Tile extents are powers of
 *   two: TM (and BR) in {1, 2, 4, ..., 256}, TN (and BC) in {1, 2, 4, ..., 1024}.  A non-positive
 *   extent is invalid (TM_E_INVAL); any other value outside these menus is TM_E_UNSUPPORTED (the
 *   pages' tile must be a known constant, [ALIGNED] "When the promise is broken").
 * Two paths ([ALIGNED] "What it changes"; [SLICING] "Masking"):
 *   aligned = 0  ragged-edge path.  Any M, N >= 0 and ld >= N.  Elements past the tensor's edge
 *                read as 0 and their stores are skipped: no byte outside { p[i*ld + j] : i < M,
 *                j < N } of an output is ever written.
 *   aligned = 1  the caller promises whole tiles and 16-byte rows: M % TM == 0, N % TN == 0,
 *                TN % 4 == 0, and every row of every 2-D tensor starts on a 16-byte boundary
 *                (base address % 16 == 0 and, when M > 1, row stride % 4 == 0).
 *                The kernels then carry no masks and move rows as 16-byte vectors.  The promise is
 *                checked once on the host before anything is enqueued; a broken promise returns
 *                TM_E_ALIGN and writes nothing ([ALIGNED] "When the promise is broken" traps on the
 *                device instead; here the check never lets a launch write past a tensor).
 * Memory and ownership.  Every pointer is caller-owned DEVICE memory (4-byte aligned f32) that
 *   stays valid until the enqueued work completes.  The library allocates nothing and keeps no
 *   state between calls.  Pointers may be NULL only when the call has no work (M == 0 or N == 0).
 * Streams.  `stream` is a hipStream_t passed as void* (NULL = the null stream).  Work is enqueued
 *   asynchronously; a call returns once it is enqueued.  Stream priorities are never changed.
 * Errors.  All argument checks run synchronously on the host, before any HIP call.  On any error
 *   nothing is enqueued and no output byte changes.  When several checks fail, the first of
 *   TM_E_INVAL, TM_E_UNSUPPORTED, TM_E_WORKSPACE, TM_E_ALIGN in that order is returned.  A failed
 *   launch returns TM_E_HIP.  Nothing aborts, prints or traps.  Calls are thread-safe (no shared
 *   mutable state).
 * Empty work.  M == 0 or N == 0 is a no-op returning TM_OK for the maps and the copy.  A reduction
 *   over an empty extent still writes its result: tm_rowsum with N == 0 writes 0 to each of the M
 *   rows, tm_colsum with M == 0 writes 0 to each of the N columns, and tm_rowmax_masked with N == 0
 *   writes the fill -1.0e30f to each row.  Only an empty output makes a reduction a no-op.
 * Aliasing.  y == x with ldy == ldx is allowed for the maps and the copy; any other overlap of an
 *   output with an input is undefined.
 */
#ifndef TILEMAP_H
#define TILEMAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TM_OK = 0,
    TM_E_INVAL = -1,       /* malformed argument: negative extent, ld < N, tile <= 0, NULL with work,
                              pointer not 4-byte aligned, unknown enum value */
    TM_E_ALIGN = -2,       /* aligned = 1 but the promise is broken, or a 16-byte vector variant was
                              asked for on data whose rows are not 16-byte aligned */
    TM_E_UNSUPPORTED = -3, /* positive tile extent outside the compiled menu */
    TM_E_WORKSPACE = -4,   /* workspace NULL or smaller than tm_colsum_workspace_bytes() /
                              tm_rows_workspace_bytes() */
    TM_E_HIP = -5          /* the HIP runtime refused the launch */
} tm_status;

/* Access width of the element-wise maps ([P35] "The exercise"). */
typedef enum {
    TM_VAR_AUTO = 0,             /* VEC4 when legal, else 4-byte loads and stores, four
                                    elements per thread at a stride of the workgroup */
    TM_VAR_SCALAR = 1,           /* one element per thread, one 4-byte load and store each
                                    ([P35] "Solution": the scalar kernel), in workgroups of
                                    256 threads */
    TM_VAR_VEC4_UNDERSTATED = 2, /* 4 elements per thread, moved as four 4-byte accesses
                                    (alignment under-stated: [P35] "Key API"); needs TN % 4 == 0,
                                    else TM_E_UNSUPPORTED */
    TM_VAR_VEC4 = 3              /* 4 elements per thread as one 16-byte load and store; needs
                                    TN % 4 == 0 and rows starting on 16-byte boundaries (else
                                    TM_E_ALIGN) */
} tm_variant;

/* How tm_colsum walks the matrix ([LAYOUT] "What it actually costs"). */
typedef enum {
    TM_COL_NAIVE = 0,    /* each workgroup reads TM rows of ONE column: lane-varying term has stride
                            ld; workgroups in column order, as the pages' strided walk */
    TM_COL_LDS = 1,      /* lanes read rows with 16-byte coalesced loads; per-column partials are
                            folded through LDS ([LAYOUT] "Seeing it in a real kernel": tile once
                            into fast memory, then read it in any order) */
    TM_COL_NAIVE_XCD = 2 /* the naive walk with its workgroups spread so that each of the GPU's
                            XCDs (each with its own L2) takes a contiguous range of columns: the
                            neighbouring columns that share a 128-byte line are then read through
                            one L2, the reuse [LAYOUT] "What it actually costs" credits for the
                            strided walk's modest cost.  Same results as TM_COL_NAIVE. */
} tm_colwalk;

/* How the element-wise maps cut a call into work (reported by tm_map_walk). */
typedef enum {
    TM_MAP_NONE = 0,  /* nothing to launch (M or N is 0) */
    TM_MAP_FLAT = 1,  /* the view's rows are contiguous in both tensors: one flat row of 1 KiB work
                         items, only its end ragged */
    TM_MAP_SPAN = 2,  /* padded rows as one span of 1 KiB items on y's 1 KiB grid, the columns past
                         N masked per 16-byte chunk ([SLICING] "Masking"); x's row stride may differ
                         from y's, and x may start at another 4-byte phase than y (also: one
                         contiguous row that the flat plan cannot take) */
    TM_MAP_TILES = 3  /* the 2-D tile schedule: whole tiles unmasked, edge tiles masked */
} tm_mapwalk;

/* How tm_colsum cuts a call into work (reported by tm_col_walk). */
typedef enum {
    TM_COLFORM_NONE = 0,      /* nothing to launch (N is 0) */
    TM_COLFORM_ONE_PASS = 1,  /* the LDS walk over few rows: each thread adds one chunk of columns
                                 down all M rows and writes the sums; no partials */
    TM_COLFORM_TILES = 2,     /* two passes: one workgroup per (row slab, column strip) writes a
                                 partial per column, then a fixed-order sum of each column's
                                 partials (the naive walks: strips of one column) */
    TM_COLFORM_STRIPS = 3     /* two passes, the LDS walk over wide matrices: one workgroup per
                                 (row slab, strip of 256 columns), one 16-byte column chunk per
                                 lane of each of its 8 waves, which add an eighth of the slab's
                                 rows each, then the same fixed-order sum */
} tm_colform;

/* ---- element-wise maps over tiles --------------------------------------------------------------
 * x: input, M x N, row stride ldx.  y: output, M x N, row stride ldy.  TM, TN: tile.  aligned: 0|1.
 * variant: tm_variant.  The tile is what the alignment promise is made for.  How the work is cut
 * into workgroups, and which chunks take the masked code on the ragged path (the view's own edges:
 * nothing outside the M x N view is stored, and padding between rows is never written), is the
 * library's choice and never changes a result. */

/* y[i,j] = fmaf(x[i,j], alpha, beta): one correctly rounded multiply-add per element
 * ([P35] "The exercise": out = a*2 + 1; generalised to alpha, beta). */
int tm_map_affine(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
                  float alpha, float beta, int TM, int TN, int aligned, int variant, void *stream);

/* y[i,j] = alpha * x[i,j]: one IEEE multiply, so signed zeros are kept
 * ([ALIGNED] "A minimal kernel", kernel scale). */
int tm_scale2d(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
               float alpha, int TM, int TN, int aligned, int variant, void *stream);

/* y[i,j] = x[i,j], bit for bit: NaN payloads and signed zeros travel unchanged
 * ([SLICING] "Promising whole tiles with @aligned", kernel copy2d). */
int tm_copy2d(const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
              int TM, int TN, int aligned, int variant, void *stream);

/* Per-channel affine on an NC view: y[i,j] = fmaf(x[i,j], scale[j], bias[j]), one rounding per
 * element; scale == NULL means 1, which gives exactly the rounded sum x[i,j] + bias[j] (the bias
 * add).  Columns are channels: a (B, C, H, W) tensor stored NHWC is the M = B*H*W by N = C view
 * ([LAYOUT] "NCHW versus NHWC": per-channel scale and bias want the channels contiguous, and
 * reading the tensor as NC moves no data).  scale, bias: N floats each, device memory, 4-byte
 * aligned (16-byte aligned lets them load as 16-byte vectors); bias may be NULL only when there is
 * no work.  Tiles, paths and variants as for tm_map_affine (the promise covers x and y). */
int tm_channel_affine(const float *x, int64_t ldx, const float *scale, const float *bias, float *y,
                      int64_t ldy, int64_t M, int64_t N, int TM, int TN, int aligned, int variant,
                      void *stream);

/* ---- row and column reductions --------------------------------------------------------------
 * As for the maps, the caller's tile (TM x TN, BR x BC) is what the alignment promise is made
 * for.  The row walk takes the caller's column tile as its own when it suits the lanes of a row
 * (tm_row_walk reports the walk for any arguments); the lanes per row, and the slabs and strips of
 * the column walk, are the library's choice, set from M, N and the row alignment.  These choices
 * decide the order of floating-point additions (within the stated bounds), never a maximum.  A row is
 * walked by one workgroup at most, so a handful of very long rows cannot use the whole GPU; the
 * *_ws variants below take a workspace and split such rows across workgroups. */

/* out[i] = sum over j < N of x[i,j] for i < M (out: M floats, contiguous).  Rows are walked with
 * coalesced loads (16-byte when the rows start on 16-byte boundaries) in column tiles: whole tiles
 * unmasked, then one remainder tile whose missing columns read as 0 ([SLICING] "Loops over a
 * dynamic extent", "Masking"; [LAYOUT] "What it actually costs", the row walk).  Accumulation is
 * f32 in a fixed order; the result is within 1e-5 * sum_j |x[i,j]| of the exact sum.  aligned = 1
 * promises M % TM == 0, N % TN == 0 and 16-byte rows of x (out is not checked). */
int tm_rowsum(const float *x, int64_t ldx, float *out, int64_t M, int64_t N,
              int TM, int TN, int aligned, void *stream);

/* Bytes of device workspace tm_colsum needs for these arguments (0 when M == 0 or N == 0, and
 * also 0 for invalid arguments, which tm_colsum then rejects): 4 * N * (number of row slabs), where
 * a slab is TM rows for the naive walks and 256 rows for the LDS walk (taller, doubling, while
 * there would be more than 4096 slabs; shorter, halving, while there would be fewer than 1024
 * slabs x column strips of up to 128 columns, down to 32 rows, or 4096 / strip width rows for
 * narrower strips).  Wide matrices (N >= 1024, N % 4 == 0) may take the LDS walk's strip form, with
 * slabs of 64 rows (doubling while there would be more than 256) by 256-column strips, when that
 * makes at least 256 workgroups; the size then covers the larger of the two slab counts, since the
 * workspace's alignment (16 bytes for the strip form) is not known here.  0 when the LDS walk takes
 * its one-pass form (at most 64 rows, or at most 256 rows of at least 262144 columns: each thread
 * adds one 16-byte column chunk down all M rows and writes the sums, so there are no partials). */
size_t tm_colsum_workspace_bytes(int64_t M, int64_t N, int TM, int TN, int walk);

/* out[j] = sum over i < M of x[i,j] for j < N (out: N floats, contiguous).  Two passes: pass 1 writes
 * one partial per (row slab, column) into `ws`; pass 2 adds each column's partials in a fixed
 * order, so the result is deterministic (no atomics).  (The LDS walk over few rows is one pass in
 * a fixed order down each column and needs no workspace; ws may then be NULL.)  walk: tm_colwalk.  ws: caller-owned
 * device workspace of ws_bytes >= tm_colsum_workspace_bytes(...) bytes (contents on entry are
 * ignored; on return they are unspecified).  Same accuracy bound as tm_rowsum, over the column.
 * aligned = 1 promises M % TM == 0, N % TN == 0 and 16-byte rows of x; the naive walk moves single
 * elements whatever `aligned` says ([LAYOUT] "What it actually costs", the column walk). */
int tm_colsum(const float *x, int64_t ldx, float *out, int64_t M, int64_t N,
              int TM, int TN, int aligned, int walk, void *ws, size_t ws_bytes, void *stream);

/* The most workspace tm_colsum_noalloc can stand in for: 16 MiB per device. */
#define TM_COLSUM_NOALLOC_MAX_BYTES ((size_t)16 << 20)

/* tm_colsum for callers that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments (no workspace), same kernels,
 * same results bit for bit as tm_colsum with a workspace.  The slab partials live in a static
 * device array of TM_COLSUM_NOALLOC_MAX_BYTES that the library holds on every device it runs on
 * until the process ends; the call allocates nothing (no hipMalloc, no hipFree).  A call whose
 * tm_colsum_workspace_bytes(...) exceeds the array returns TM_E_WORKSPACE and enqueues nothing
 * (argument errors as tm_colsum, checked first, before any HIP call).  The first call on a device
 * looks up the array's device address (HIP calls that enqueue nothing); TM_E_HIP if that fails.
 * The array is shared by every call on a device and keeps the last call's partials: calls that
 * overlap on one device race, so issue them on one stream (which orders them) or serialize them. */
int tm_colsum_noalloc(const float *x, int64_t ldx, float *out, int64_t M, int64_t N, int TM, int TN,
                      int aligned, int walk, void *stream);

/* out[i] = max over j < N of s[i,j] (out: M floats, contiguous), walking column tiles: whole
 * tiles unmasked, then one remainder tile in which tile-local column c keeps s iff c < N - kt and
 * is otherwise replaced by -1.0e30f (f32 bits 0xF149F2CA); the running maximum starts at that fill,
 * so N == 0 gives -1.0e30f ([SLICING] "Reductions over a ragged tile").  Scores are assumed to lie
 * in [-1e30, +inf); NaN entries never win.  Bit-exact (max is order-free).  BR: rows per tile.
 * aligned = 1 promises M % BR == 0, N % BC == 0 and 16-byte rows of s. */
int tm_rowmax_masked(const float *s, int64_t lds, float *out, int64_t M, int64_t N,
                     int BR, int BC, int aligned, void *stream);

/* Softmax row statistics over column tiles: m[i] = max over j < N of s[i,j], exactly as
 * tm_rowmax_masked computes it (bit-exact), and l[i] = sum over j < N of exp(s[i,j] - m[i]), the
 * normaliser that goes with it ([SLICING] "Reductions over a ragged tile": the masked maximum is
 * what a softmax needs, and a 0 fill would corrupt both).  Tiles are walked as in
 * tm_rowmax_masked; each lane keeps a running maximum and a running sum that it rescales by
 * exp(m_old - m_new) whenever its maximum grows, and the lanes of a row are combined the same way.
 * Masked columns contribute nothing.  l is within 1e-5 relative of the exact sum (f32 sums;
 * e^x evaluated as 2^(x log2 e) with the hardware base-2 exponential).  N == 0 gives
 * m = -1.0e30f and l = 0; a row of -inf gives the same; a +inf score gives m = +inf and l = NaN
 * (e^(inf - inf)), a NaN score leaves m alone and makes l NaN.  m, l: M floats each, contiguous.
 * BR, BC, aligned and the score contract are those of tm_rowmax_masked. */
int tm_softmax_stats(const float *s, int64_t lds, float *m, float *l, int64_t M, int64_t N,
                     int BR, int BC, int aligned, void *stream);

/* ---- row reductions over a few long rows ----------------------------------------------------
 * tm_rowsum_ws, tm_rowmax_masked_ws and tm_softmax_stats_ws compute exactly what tm_rowsum,
 * tm_rowmax_masked and tm_softmax_stats compute, under the same contracts and bounds (maxima bit
 * for bit), and take a device workspace.  With fewer than 128 rows of at least 98304 elements, each
 * row is cut into segments of 1024 * K elements (K = 1, 2, 4, 8 or 16, chosen for about 2048
 * segments in all) that separate workgroups walk, each writing its segment's partial (sum,
 * maximum, or the pair (m, l) of [SLICING] "Reductions over a ragged tile" over the segment's live
 * columns) into the workspace; a second launch combines each row's partials in segment order
 * (for the softmax pair: m = max m_s, l = sum l_s * exp(m_s - m)).  Both are fixed-order folds, so
 * results are deterministic.  For other shapes the call is the one-pass call and the workspace is
 * not touched.  One row of 2^23 floats takes about 11 us this way and 0.58 ms in one pass. */

/* Bytes of device workspace the *_ws row calls need for M rows of N elements: 8 * M * (segments
 * per row) when rows are split, else 0 (also 0 for invalid extents, which the calls reject). */
size_t tm_rows_workspace_bytes(int64_t M, int64_t N);

/* tm_rowsum with a workspace: ws is caller-owned device memory of ws_bytes >=
 * tm_rows_workspace_bytes(M, N) bytes, 4-byte aligned (may be NULL when that is 0); contents on
 * entry are ignored and on return unspecified.  A missing or short workspace returns
 * TM_E_WORKSPACE (checked after the tile, before the promise). */
int tm_rowsum_ws(const float *x, int64_t ldx, float *out, int64_t M, int64_t N,
                 int TM, int TN, int aligned, void *ws, size_t ws_bytes, void *stream);

/* tm_rowmax_masked with a workspace (ws as for tm_rowsum_ws). */
int tm_rowmax_masked_ws(const float *s, int64_t lds, float *out, int64_t M, int64_t N,
                        int BR, int BC, int aligned, void *ws, size_t ws_bytes, void *stream);

/* tm_softmax_stats with a workspace (ws as for tm_rowsum_ws). */
int tm_softmax_stats_ws(const float *s, int64_t lds, float *m, float *l, int64_t M, int64_t N,
                        int BR, int BC, int aligned, void *ws, size_t ws_bytes, void *stream);

/* ---- layout conversion ----------------------------------------------------------------------- */

/* Batched transpose: y[b][j][i] = x[b][i][j] for b < B, i < M, j < N, bit for bit.  Batch b of x
 * (M x N, row stride ldx) starts at x + b*bsx; batch b of y (N x M, row stride ldy) at y + b*bsy.
 * With x = [B][C][H*W], M = C, N = H*W, ldx = H*W, bsx = C*H*W, ldy = C, bsy = H*W*C this converts
 * NCHW to NHWC; the same call with M and N swapped converts back ([LAYOUT] "NCHW versus NHWC": a
 * conversion costs one full pass over memory; "Strides, and reading an index expression").
 * x is staged through LDS in sub-tiles of 32 x 32 (for fewer than 32 rows or columns, as the
 * channels of an RGB image, as narrow as the tensor and up to 1024 elements long; when the narrow
 * side's rows are packed, C floats each, a work item moves that side as one contiguous block) so
 * that both the reads of x and the writes of y are coalesced rows ([LAYOUT] "Seeing it in a real
 * kernel"), in 16-byte chunks whenever every row of x and y starts on a 16-byte boundary, whatever
 * the tile; TM x TN is the tile the alignment promise is made for (under the promise the sub-tiles
 * are whole).  Ragged edges: elements past the tensor read as 0 and are never stored.  aligned = 1
 * promises
 * M % TM == 0, N % TN == 0, TM % 4 == 0, TN % 4 == 0 and 16-byte rows of x and y in every batch
 * (16-byte bases, row strides % 4 == 0, batch strides % 4 == 0 when B > 1), else TM_E_ALIGN.
 * For B > 1, bsy must be at least (N - 1)*ldy + M (batches of y may not overlap), else TM_E_INVAL.
 * x and y must not overlap.  B, M or N == 0 is a no-op. */
int tm_transpose(const float *x, int64_t ldx, int64_t bsx, float *y, int64_t ldy, int64_t bsy,
                 int64_t B, int64_t M, int64_t N, int TM, int TN, int aligned, void *stream);

/* ---- host-only helpers (no GPU needed) ------------------------------------------------------ */

/* The checks `aligned = 1` performs, as a pure host function: TM_OK when the promise holds,
 * TM_E_ALIGN when it is broken, TM_E_INVAL / TM_E_UNSUPPORTED for malformed arguments (checked
 * first).  out == NULL means there is no 2-D output (reductions); ld_out is then ignored.  The
 * addresses are only inspected, never dereferenced. */
int tm_check_promise(int64_t M, int64_t N, int64_t ld_in, int64_t ld_out, int TM, int TN,
                     const void *in, const void *out);

/* Loop remainder split ([SLICING] "Loops over a dynamic extent"): *nfull = K / T whole tiles and
 * *rem = K % T columns in the one masked remainder tile.  TM_E_INVAL if K < 0, T <= 0 or an output
 * pointer is NULL. */
int tm_split(int64_t K, int64_t T, int64_t *nfull, int64_t *rem);

/* The column walk of the one-pass row reductions (tm_rowsum, tm_rowmax_masked, tm_softmax_stats,
 * and the *_ws calls when they do not split rows) for these arguments, as a pure host function:
 * the walk's column tile *bc, its *nfull whole tiles, the *rem live columns of its one masked
 * remainder tile (0: none; [SLICING] "Loops over a dynamic extent", "Reductions over a ragged
 * tile") and the *lanes that share each row.  The caller's column tile BC (TN for tm_rowsum) is
 * the walk's whenever it holds whole chunks (16-byte chunks when every row of x starts on a
 * 16-byte boundary, else single floats), keeps at least half the lanes the row length and count
 * call for, one chunk each, and needs at most 4 chunks per lane per tile; otherwise the walk takes
 * its own tile, and the split follows the same rule.  8192 x 1000 with BC = 64 on 16-byte rows:
 * bc = 64, nfull = 15, rem = 40.  x is only inspected, never dereferenced.  TM_E_INVAL /
 * TM_E_UNSUPPORTED / TM_E_ALIGN as the reductions return them (no output vector is checked), or
 * TM_E_INVAL if an output pointer is NULL. */
int tm_row_walk(int64_t M, int64_t N, int64_t ld, int BR, int BC, int aligned, const void *x,
                int64_t *bc, int64_t *nfull, int64_t *rem, int *lanes);

/* The plan an element-wise map would run ([SLICING] "Masking": which elements are masked follows
 * from it).  op: 0 = tm_map_affine, 1 = tm_scale2d, 2 = tm_copy2d, 3 = tm_channel_affine with the
 * channel vector `bias` and no scale (bias is ignored for ops 0-2); the other arguments as for
 * that call.  Writes *walk (tm_mapwalk) and *items, the work items of the launch (one per
 * workgroup, before the grid is capped; 0 with TM_MAP_NONE).  Pointers are only inspected, never
 * dereferenced.  Returns what the call would return before launching (TM_E_INVAL, TM_E_ALIGN,
 * TM_E_UNSUPPORTED, and TM_E_INVAL for an op out of range or a NULL output pointer); the outputs
 * are written only on TM_OK. */
int tm_map_walk(int op, const void *x, int64_t ldx, const void *y, int64_t ldy, int64_t M, int64_t N,
                int TM, int TN, int aligned, int variant, const void *bias, int *walk, int64_t *items);

/* The plan tm_colsum would run for these arguments, as a pure host function ([LAYOUT] "What it
 * actually costs": the column walk; "Seeing it in a real kernel": the staged walk): *form
 * (tm_colform), *slab_rows (rows each work item adds down its columns: M for the one-pass form),
 * *strip_cols (columns per work item: 1 for the naive walks, the chunk width of a thread for the
 * one-pass form), *slabs and *strips (work items down and across; *slabs is the number of
 * partials per column of the two-pass forms, 0 when M is 0).  x, out and ws are only inspected,
 * never dereferenced (the strip form needs a 16-byte aligned ws).  Returns what tm_colsum would
 * return before launching (TM_E_INVAL, TM_E_ALIGN, TM_E_UNSUPPORTED, TM_E_WORKSPACE), or
 * TM_E_INVAL if an output pointer is NULL; the outputs are written only on TM_OK.  4096 x 4096
 * with the LDS walk and a 16-byte aligned workspace: TM_COLFORM_STRIPS, 64-row slabs by
 * 256-column strips, 64 x 16. */
int tm_col_walk(const void *x, int64_t ldx, const void *out, int64_t M, int64_t N, int TM, int TN,
                int aligned, int walk, const void *ws, size_t ws_bytes, int *form, int64_t *slab_rows,
                int64_t *strip_cols, int64_t *slabs, int64_t *strips);

/* Tile scheduler counts ([SLICING] "Masking"): *tiles_m = ceil(M / TM), *tiles_n = ceil(N / TN) and
 * *whole = the number of tiles lying entirely inside the M x N tensor; the other tiles are edge
 * tiles, whose out-of-range elements read as 0 and whose stores are skipped.  TM_E_INVAL /
 * TM_E_UNSUPPORTED as for the tile checks of the other calls, or TM_E_INVAL if an output pointer
 * is NULL or the whole-tile count does not fit 64 bits. */
int tm_plan_tiles(int64_t M, int64_t N, int TM, int TN, int64_t *tiles_m, int64_t *tiles_n,
                  int64_t *whole);

/* Padding that keeps the alignment promise ([ALIGNED] "Interactions": when a tuner picks the tile,
 * the host must pad or pick shapes that keep the promise for every candidate).  Writes the
 * smallest *Mp >= M and *Np >= N that are multiples of TM and TN, and *ldp = *Np, a row stride of
 * whole 16-byte units.  An Mp x Np tensor with row stride ldp on a 16-byte aligned base (its
 * padding zero-filled by the caller) then keeps the promise for TM x TN tiles; to keep it for every
 * tile of a set of candidates, pass the largest TM and TN of the set (menu extents are powers of
 * two, so the largest is a multiple of the others).  TM_E_ALIGN if TN % 4 != 0 (no tile row can be
 * 16-byte vectors); TM_E_INVAL / TM_E_UNSUPPORTED for malformed arguments or NULL outputs. */
int tm_pad_extents(int64_t M, int64_t N, int TM, int TN, int64_t *Mp, int64_t *Np, int64_t *ldp);

/* Tile-size sweep for the element-wise maps ([ALIGNED] "Interactions", @autotune; [LAYOUT] "What it
 * actually costs": measure rather than predict).  Runs op (0 = tm_map_affine, 1 = tm_scale2d,
 * 2 = tm_copy2d) from x to y with every tile of the menu (TM = 1..256, TN = 1..1024, powers of
 * two) that the call accepts -- with aligned = 1, only tiles that keep the promise -- reps times
 * each on `stream` after one warm-up launch, timing each candidate between the caller's two HIP
 * events (hipEvent_t passed as void*).  Returns the fastest tile in *TM_best, *TN_best and its mean
 * time per launch in *us_best.  If table != NULL it receives 9 x 11 floats, row i for TM = 2^i and
 * column j for TN = 2^j: the candidate's mean microseconds per launch, or -1 where it was not run.
 * The caller's buffers are used as they are: buffers that fit in the 256 MiB Infinity Cache time
 * cache bandwidth, not HBM.  In this library the tile states the promise (and, on the ragged path,
 * which elements are masked) but does not shape the work: the scheduler cuts every call into the
 * same work items whatever tile keeps the promise, so the candidates' times differ by launch noise
 * and the "fastest" is the fastest of this run, not a better tile.  The sweep is kept as the check
 * that no tile is a trap (each candidate's time is in `table`).  Synchronizes `stream`; y holds the
 * op's result afterwards.  x and y
 * must not overlap.  Errors: those of the op's own call for the shared arguments; TM_E_INVAL for
 * an unknown op, reps < 1, a NULL event or result pointer, or x == y; TM_E_ALIGN when no tile keeps
 * the promise; TM_E_HIP if a launch or event call fails. */
int tm_autotune_map(int op, const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
                    float alpha, float beta, int aligned, int variant, int reps, void *ev_start,
                    void *ev_stop, int *TM_best, int *TN_best, float *us_best, float *table,
                    void *stream);

/* Static, human-readable name of a status code ("TM_OK", ...; "unknown status" otherwise). */
const char *tm_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* TILEMAP_H */
