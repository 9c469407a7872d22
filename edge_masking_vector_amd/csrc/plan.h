// plan.h -- host-side argument checks, the alignment-promise checker and the tile scheduler of
// libtilemap.  Pure C++17: no HIP header, so this logic builds and runs on any CPU.
//
// Every tm_* entry point calls one plan_* function before touching the GPU.  A plan either
// rejects the call (status != TM_OK, nothing launched) or describes the launches completely:
// which kernel variant, how tiles map to workgroups, and how many workgroups.
#pragma once

#include <cstddef>
#include <cstdint>

#include "../../include/tilemap.h"

namespace tmp {

constexpr int kMaxTM = 256;   // row tile (TM, BR) menu: 1, 2, 4, ..., 256
constexpr int kMaxTN = 1024;  // column tile (TN, BC) menu: 1, 2, 4, ..., 1024
constexpr int kBlock = 256;   // threads per workgroup of the reductions (4 wave64s)
constexpr int kMapMinBlock = 64;    // map workgroups: at least one wave ...
constexpr int kMapMaxBlock = 1024;  // ... and at most 1024 threads
constexpr int kMapNarrowThreads = 256;  // ragged rows narrower than a segment: threads per work item
constexpr int kScalarChunksPerThread = 4;  // 4-byte chunks per thread (16-byte chunks: one)
constexpr int kLineBytes = 128;     // cache line
constexpr int kRowSegmentBytes = 512;  // map work items: bytes of each row they move, at least ...
constexpr int kStreamSegmentBytes = 1024;  // ... or one row segment of this many bytes, moved
                                           // with device-scope streaming buffer accesses
constexpr int64_t kChanFlatMax = 65535;  // channel op: flat views up to this many channels
constexpr int64_t kRowsSpanMinN = 64;      // padded rows in one span: rows of at least this many
                                           // floats and less than a line of padding between them
constexpr int64_t kRowsDiffMinN = 1024;    // ... and of at least this many when x's and y's row
                                           // strides differ
constexpr int64_t kRowsWideMinN = 2048;    // ... and padding past an eighth of the row off the line
                                           // grid: a quarter from this many floats on (16-byte
                                           // rows), half (rows off the 16-byte grid)
                                         // (C * C < 2^32 for the device's 32-bit modulo)
constexpr int kTrSub = 32;          // transpose: staged sub-tile edge (one 128-byte line of f32) ...
constexpr int64_t kTrWindowMinN = 12;  // transpose: line windows of y rows off the line grid need
                                       // x rows of at least this many floats (fewer: each window
                                       // item writes too short a stretch of y rows to pay)
constexpr int kTrPackBigC = 128;        // transpose: packed side of up to this many channels ...
constexpr int kTrPackBigElems = 4096;  // ... in work items of up to this many elements
constexpr int kTrSubElems = kTrSub * kTrSub;  // ... and elements; a narrow tensor's sub-tile is
                                              // narrower and longer (up to kTrSubElems long)
// Row reductions: rows of at most kTinyRowChunks 16-byte chunks are walked as one tile with
// about 4 chunks per lane, longer ones with about 8 per lane per pass; rows of more than
// kShortRowChunks* chunks are long: one wave each ...
constexpr int kTinyRowChunks = 64;
constexpr int kShortRowChunksVec = 256;
constexpr int kShortRowChunksScalar = 512;
// ... and below this many rows (one wave each), a longer row gets a workgroup of up to
// kRowMaxLanes threads, so that about this many waves run.
constexpr int kRowWideWaves = 2048;
constexpr int kRowMaxLanes = 1024;
// Rows of at least kRowLongChunks 16-byte chunks get kRowLongLanes lanes (a workgroup per row), so
// that each lane's chunks are in flight in one or two batches rather than many.
constexpr int64_t kRowLongChunks = 1024;
constexpr int kRowLongLanes = 256;
// The caller's column tile becomes the row walk's when it keeps at least half the lanes the
// row's length and count call for and needs at most this many chunks per lane per tile.
constexpr int64_t kRowTileMaxChunks = 4;
// Rows of more than kTinyRowChunks and at most kRowOnceK * 64 chunks (16-byte chunks; 4-byte
// chunks: kRowOnceKScalar * 64) are read in one batch: at least kRowOnceMinLanes lanes per row,
// every chunk in flight at once.
constexpr int kRowOnceK = 8;
constexpr int kRowOnceKScalar = 16;
constexpr int kRowOnceMinLanes = 16;
// 16-byte rows take up to this many lanes per row in one batch (past 64: one row per workgroup of
// that many threads, its waves combined through LDS); 4-byte rows at most one wave.
constexpr int kRowOnceMaxLanes = 256;
// Rows off the 16-byte grid of more than this many elements are read as 16-byte chunks from the
// 16-byte boundary at or before each row's start.
constexpr int64_t kRowShiftMinN = 2048;
// Rows of one lane each run on at most this many workgroups, each looping over several row groups.
constexpr int64_t kRowTinyGrid = 4096;
// Split rows (the row calls that take a workspace): fewer than kRowSplitRows rows of at least
// kRowSplitMinN elements are cut into segments of kRowSegUnit * K elements (K = 1, 2, 4, 8 or 16,
// chosen for about kRowSplitTarget segments in all), one workgroup each; a second kernel combines
// each row's partials in segment order.
constexpr int64_t kRowSplitRows = 128;
constexpr int64_t kRowSplitMinN = 98304;
constexpr int64_t kRowSplitTarget = 2048;
constexpr int kRowSegUnit = 1024;
constexpr int kRowSegMaxLogK = 4;
constexpr int kRowPartialBytes = 8;  // workspace per segment: one float, or the pair (m, l)
// LDS column walk: slabs of kColSlab rows (taller when there would be more than kColMaxSlabs of
// them) by strips of at most kColStrip columns.
constexpr int kColSlab = 256;
constexpr int64_t kColMaxSlabs = 4096;
constexpr int kColStrip = 128;
constexpr int64_t kColTargetWork = 1024;  // LDS walk: fewer (slab, strip) workgroups shorten the slabs
// LDS walk over wide matrices: strips of kColRowStrip columns (one 16-byte chunk per thread of a
// kBlock workgroup) by slabs of kColRowSlab rows (doubled while there would be more than
// kColRowMaxSlabs), when that makes at least kColRowMinWork workgroups.
constexpr int kColRowStrip = 1024;
constexpr int kColRowSlab = 64;
// The strip kernel itself: a workgroup of kColStripGroups x 64 threads takes a strip of
// kColStripCols columns (one 16-byte chunk per lane of a wave) of one slab, its row groups each
// adding an eighth of the slab's rows, folded through LDS.
constexpr int kColStripCols = 256;
constexpr int kColStripGroups = 8;
constexpr int64_t kColRowMaxSlabs = 256;
constexpr int64_t kColRowMinWork = 256;
// Column-sum pass 2: lanes per column chosen so that about this many threads run (one wave per
// column at most), or up to kFinishMaxLanes lanes (whole waves) while each lane would add more
// than kFinishBatchSlabs partials, the partials one lane loads at once.
constexpr int kFinishThreads = 16384;
constexpr int kFinishMaxLanes = 256;
constexpr int kFinishBatchSlabs = 16;
// The LDS walk goes direct (one thread per 16-byte column chunk down all rows, one pass) for at
// most kColDirectRows rows, or at most kColDirectRowsWide rows of at least kColDirectMinN columns.
constexpr int64_t kColDirectRows = 64;
constexpr int64_t kColDirectRowsWide = 256;
constexpr int64_t kColDirectMinN = int64_t{1} << 18;

enum MapOp { kAffine = 0, kScale = 1, kCopy = 2, kChannel = 3 };
// kScalar: 4-byte accesses, four elements per thread at a stride of the workgroup (what AUTO
// takes when rows are off the 16-byte grid); kScalar1: one element per thread, the scalar
// kernel of Mojo puzzle 35 "Solution" (TM_VAR_SCALAR), in workgroups of kScalar1Block threads.
enum Access { kScalar = 1, kVec4Understated = 2, kVec4 = 3, kScalar1 = 4 };
constexpr int kScalar1Block = 256;

int ilog2(int64_t v);  // v a power of two

// Division by a fixed divisor d >= 1 through a precomputed multiplier (Lemire, Kaser and Kurz,
// "Faster remainder by direct computation", 2019): with c = ceil(2^64 / d), every 32-bit a has
// a / d = the high 64 bits of c * a and a % d = the high 64 bits of (c * a mod 2^64) * d.  For
// d = 1 the multiplier (2^64) does not fit; c is then 0 and the device takes the identity.
struct Div32 {
    uint64_t c = 0;
    uint32_t d = 1;
};
Div32 make_div32(uint32_t d);

// ---- element-wise maps ---------------------------------------------------------------------
struct MapPlan {
    bool launch = false;          // false: valid call with no work
    int op = kAffine;
    int access = kScalar;         // resolved variant
    int aligned = 0;              // whole tiles promised and checked: kernels carry no masks
    int log_tm = 0, log_tn = 0;   // tile extents
    int log_vr = 0;               // log2(chunks per tile row), VR = TN / W
    // Work item = R rows x G tiles of one tile row band (R*G*VR chunks), one per workgroup.
    int log_r = 0;                // log2(R)
    int log_gv = 0;               // log2(G * VR): chunks per work-item row
    int log_strips = 0;           // log2(TM / R)
    int log_bs = 6;               // log2(threads per workgroup)
    bool guard = false;           // threads x chunks per thread exceed the work item's chunks
    bool share = false;           // channel op: a thread's chunks share one column's vectors
    bool stream = false;          // work item = one row segment of kStreamSegmentBytes (one wave,
                                  // 16-byte chunks); whole items use buffer accesses sc1 nt
    bool flat = false;            // one contiguous row in 1 KiB stream items, no channel op: the
                                  // kernel of mapflat.hip (item w = elements [256 w, 256 w + 256))
    uint32_t flat_last = 0;       // flat: elements of the last item inside the row (1 .. 256)
    // Padded rows in one span (mapflat.hip, map_rows): the view's rows lie ld apart in both
    // tensors; the span y[0 .. (M - 1) ld + N) is cut into 1 KiB items on y's 1 KiB grid, item 0
    // starting `head` floats before y[0].  Element f of the span is (row f / ld, column f % ld),
    // live when the column is below N.
    bool rows = false;
    uint32_t head = 0;            // rows: floats from the first item's start to y[0] (0 .. 255)
    uint32_t span = 0;            // rows: (M - 1) * ld + N
    Div32 ld_div;                 // rows: divisor ld (y's row stride)
    int32_t x_last = 0;           // rows: x's index of the chunk that holds the span's last element
    bool shift = false;           // rows: x at another 4-byte phase than y (4-byte aligned 16-byte loads)
    uint32_t group = 1;           // G
    uint32_t groups_n = 0;        // ceil(tiles_n / G)
    uint32_t tiles_n = 0;         // tiles along N
    uint32_t nwork = 0;           // work items: ceil(M / R) row strips * groups_n
    uint32_t grid = 0;            // workgroups
    const float *x = nullptr;
    float *y = nullptr;
    int64_t ldx = 0, ldy = 0, M = 0, N = 0;
    float alpha = 0.f, beta = 0.f;
    const float *scale = nullptr;  // per-column vectors of the channel op (scale may be null)
    const float *bias = nullptr;
    bool cvec16 = false;           // both column vectors 16-byte aligned (flat view: and C % 4 == 0)
    // Channel op over a view with contiguous rows, planned as one flat row: element (i, j) is flat
    // column i*C + j, whose channel is (flat column) mod C.  0: the channel is the column.
    uint32_t chan_n = 0;          // C
    Div32 chan;                   // divisor C
    uint32_t chan_step = 0;       // (columns per work item) mod C
};

int plan_map(int op, const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
             float alpha, float beta, int TM, int TN, int aligned, int variant, MapPlan *plan,
             const float *scale = nullptr, const float *bias = nullptr);

// ---- row reductions (sum, masked max) ------------------------------------------------------
enum RowOp { kRowSum = 0, kRowMax = 1, kRowSoftmax = 2 };

struct RowPlan {
    bool launch = false;
    int op = kRowSum;
    bool vec = false;             // 16-byte loads
    int lpr = 1;                  // lanes per row (power of two <= kRowMaxLanes)
    int block = kBlock;           // threads per workgroup: kBlock, or lpr when lpr > 64 (one row each)
    int per_tile = 1;             // vectors per lane per column tile
    int64_t nfull = 0;            // whole column tiles (unmasked)
    int64_t rem = 0;              // live columns of the remainder tile (0: none)
    int bc = 1;                   // column tile width
    // Rows read in one batch (row_once): every chunk of a row is in flight at once, `once_k`
    // chunks per lane at a stride of lpr chunks; chunks below nfull * bc / W are whole tiles.
    bool once = false;
    int once_k = 0;
    // Long rows off the 16-byte grid: each row is read in 16-byte chunks from the 16-byte boundary
    // at or before its start, with the elements before the row masked; bc, per_tile and lpr are
    // those of 16-byte chunks, and each row's split is that of N + (its start's offset) elements.
    bool shift = false;
    uint32_t grid = 0;
    const float *x = nullptr;
    float *out = nullptr;         // sums / maxima (softmax statistics: m)
    float *out2 = nullptr;        // softmax statistics: l
    int64_t ld = 0, M = 0, N = 0;
    // Split walk (only when the call brings a workspace and the rows are few and long): pass 1
    // writes one partial per row segment to ws, pass 2 combines them.
    bool split = false;
    int log_k = 0;                // segment = kRowSegUnit << log_k elements
    int64_t seg = 0;              // elements per segment
    uint32_t segs = 0;            // segments per row
    uint32_t nwork = 0;           // M * segs pass-1 workgroups' worth of segments
    float *ws = nullptr;
};

// Segment geometry of the split walk for M rows of N elements: false when the rows are walked in
// one pass (then no workspace is needed).
bool row_split_geometry(int64_t M, int64_t N, int *log_k, int64_t *seg, int64_t *segs);
size_t rows_ws_bytes(int64_t M, int64_t N);

// with_ws: the call brings a workspace (ws, ws_bytes), which licenses the split walk.
int plan_rows(int op, const float *x, int64_t ld, float *out, int64_t M, int64_t N, int TR, int TC,
              int aligned, RowPlan *plan, float *out2 = nullptr, bool with_ws = false,
              void *ws = nullptr, size_t ws_bytes = 0);

// The one-pass row walk for these arguments (what tm_rowsum, tm_rowmax_masked and
// tm_softmax_stats run): column tile *bc, *nfull whole tiles, *rem live columns of the masked
// remainder tile (0: none) and *lanes per row.  Argument errors as plan_rows (no output vector).
int row_walk_query(int64_t M, int64_t N, int64_t ld, int TR, int TC, int aligned, const void *x,
                   int64_t *bc, int64_t *nfull, int64_t *rem, int *lanes);

// ---- column sums ---------------------------------------------------------------------------
struct ColPlan {
    bool launch = false;          // pass 1 needed (M > 0)
    bool finish = false;          // pass 2 needed (N > 0)
    int walk = TM_COL_NAIVE;
    bool vec = false;
    int log_tm = 0;               // rows per slab: the caller's TM (naive walks) or the LDS walk's own
    int tw = 1;                   // columns per workgroup (LDS walk)
    bool whole = false;           // LDS walk: whole slabs and strips with 16-byte rows (no masks)
    bool direct = false;          // LDS walk over few rows or many columns: one pass, no partials
    bool out16 = false;           // direct walk: out is 16-byte aligned
    // LDS walk over wide matrices (col_strip + colsum_fold16): a workgroup per (slab, strip of
    // kColStripCols columns), each lane one 16-byte column chunk, kColStripGroups row groups;
    // partials as 16-byte vectors.
    bool strip = false;
    int fl = 1;                   // pass 2: lanes per column (power of two <= kFinishMaxLanes)
    int naive_block = 64;         // threads per workgroup (naive walk)
    uint32_t slabs = 0;           // ceil(M / rows per slab): partials per column
    uint32_t strips = 0;          // column strips (LDS walk) or columns (naive walk)
    const float *x = nullptr;
    float *out = nullptr;
    float *ws = nullptr;
    int64_t ld = 0, M = 0, N = 0;
};

bool col_direct(int64_t M, int64_t N, int walk);
size_t colsum_ws_bytes(int64_t M, int64_t N, int TM, int TN, int walk);

int plan_cols(const float *x, int64_t ld, float *out, int64_t M, int64_t N, int TM, int TN,
              int aligned, int walk, void *ws, size_t ws_bytes, ColPlan *plan);

// ---- batched transpose -----------------------------------------------------------------------

struct TransposePlan {
    bool launch = false;
    bool vec = false;             // 16-byte chunks on both sides (vx && vy)
    bool vx = false, vy = false;  // 16-byte chunks on the read side (x rows) / the write side (y rows)
    int aligned = 0;
    int sm = 1, sn = 1;           // staged sub-tile extents (powers of two, sm * sn <= sub)
    int sub = kTrSubElems;        // the kernel instance's largest sub-tile: kTrSubElems or twice that
    bool skew = false;            // one matrix, y rows off the 128-byte line grid: line-aligned y
                                  // windows (transpose_skew); subs_m = ceil((M + 31) / 64) item rows
                                  // in groups of 2^log_grp on one XCD, per_b the divisor of the group rows
    int log_g = 0;                // batches per work item: 2^log_g (whole matrices in one sub-tile)
    int log_grp = 0;              // skew: 2^log_grp vertically adjacent items on one XCD
    // Few channels with a packed side (transpose_packed): 1 = y rows of exactly M < kTrSub floats
    // (NCHW -> NHWC), 2 = x rows of exactly N < kTrSub floats (NHWC -> NCHW); 0 = neither.
    int packed = 0;
    bool pvec = false;            // packed kernel: the strided side moves 16-byte chunks
    bool flat16 = false;          // packed kernel: the packed block starts on 16-byte boundaries
    bool pbig = false;            // packed kernel: 32 to kTrPackBigC channels, items of up to
                                  // kTrPackBigElems elements
    uint32_t subs_m = 0, subs_n = 0;
    uint64_t nwork = 0;
    bool wide = false;            // nwork >= 2^32: 64-bit work-item arithmetic
    Div32 per_b, by_m, by_n;      // divisors subs_m * subs_n, subs_m, subs_n (when !wide)
    uint32_t grid = 0;
    const float *x = nullptr;
    float *y = nullptr;
    int64_t ldx = 0, ldy = 0, bsx = 0, bsy = 0, B = 0, M = 0, N = 0;
};

int plan_transpose(const float *x, int64_t ldx, int64_t bsx, float *y, int64_t ldy, int64_t bsy,
                   int64_t B, int64_t M, int64_t N, int TM, int TN, int aligned,
                   TransposePlan *plan);

// ---- pieces shared by the planners (exported through the C ABI as host helpers) -------------
// Loop remainder split: K columns in steps of T = *nfull whole tiles + one tile of *rem columns.
int split(int64_t K, int64_t T, int64_t *nfull, int64_t *rem);
int check_tile(int TM, int TN);
int check_promise(int64_t M, int64_t N, int64_t ld_in, int64_t ld_out, int TM, int TN,
                  const void *in, const void *out);
int plan_tiles(int64_t M, int64_t N, int TM, int TN, int64_t *tiles_m, int64_t *tiles_n,
               int64_t *whole);
int pad_extents(int64_t M, int64_t N, int TM, int TN, int64_t *Mp, int64_t *Np, int64_t *ldp);

}  // namespace tmp
