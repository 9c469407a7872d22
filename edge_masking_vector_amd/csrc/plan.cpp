// plan.cpp -- argument checks, the alignment-promise checker, the loop remainder split and the
// tile scheduler of libtilemap.  Pure host C++17 (no HIP), run before anything is enqueued.
//
// Sources (web pages): Phobos docs "@aligned" ("What it changes", "When the promise is broken");
// Phobos docs "Slicing, bounds and masking" ("Masking", "Loops over a dynamic extent");
// teenygrad "Memory Coalescing and Tensor Layout" ("The alignment constraint").
#include "plan.h"

#include <algorithm>
#include <climits>

namespace tmp {

namespace {

// Workgroups launched at most per kernel; larger jobs loop over their work inside the grid.
// 2^20 workgroups of 256 threads stays far inside the 2^32 work-item limit of one dispatch.
constexpr uint32_t kGridCap = 1u << 20;

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

bool aligned_to(const void *p, uintptr_t a) {
    return (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// a >= 0, b > 0; no intermediate sum, so it holds up to INT64_MAX (the size queries take any
// extents).
int64_t ceil_div(int64_t a, int64_t b) { return a / b + (a % b != 0); }

// One M x N view with row stride ld.  `work`: the call will touch it (M > 0 and N > 0).
int check_view(const void *p, int64_t M, int64_t N, int64_t ld, bool work) {
    if (M < 0 || N < 0 || ld < 0 || ld < N)
        return TM_E_INVAL;
    if (!work)
        return TM_OK;
    if (p == nullptr || !aligned_to(p, 4))
        return TM_E_INVAL;
    // (M - 1) * ld + N elements must be addressable with int64 byte offsets.
    const int64_t lim = (INT64_MAX / 4) - N;
    if (ld > 0 && (M - 1) > lim / ld)
        return TM_E_INVAL;
    return TM_OK;
}

// A contiguous vector of n floats (reduction outputs, workspaces).
int check_vector(const void *p, int64_t n) {
    if (n == 0)
        return TM_OK;
    if (p == nullptr || !aligned_to(p, 4))
        return TM_E_INVAL;
    return TM_OK;
}

// Every row of an M-row view with stride ld starts on a 16-byte boundary: a 16-byte base and,
// when there is more than one row, a stride of whole 16-byte units.
bool rows16(const void *p, int64_t M, int64_t ld) {
    return aligned_to(p, 16) && (M <= 1 || ld % 4 == 0);
}

// Whole tiles and 16-byte rows ([ALIGNED] "What it changes"; [LAYOUT] "The alignment constraint").
bool promise_holds(int64_t M, int64_t N, int64_t ld_in, int64_t ld_out, int TM, int TN,
                   const void *in, const void *out) {
    if (M % TM != 0 || N % TN != 0)
        return false;
    if (TN % 4 != 0 || !rows16(in, M, ld_in))
        return false;
    if (out != nullptr && !rows16(out, M, ld_out))
        return false;
    return true;
}

uint32_t cap_grid(int64_t work_items) {
    return static_cast<uint32_t>(std::min<int64_t>(work_items, kGridCap));
}

}  // namespace

Div32 make_div32(uint32_t d) {
    Div32 r;
    r.d = d;
    r.c = d > 1 ? ~uint64_t{0} / d + 1 : 0;  // ceil(2^64 / d) for d > 1
    return r;
}

int ilog2(int64_t v) {
    int l = 0;
    while (l < 62 && (int64_t{1} << l) < v)  // saturates at 2^62 (no shift past the sign bit)
        ++l;
    return l;
}

int split(int64_t K, int64_t T, int64_t *nfull, int64_t *rem) {
    // [SLICING] "Loops over a dynamic extent": whole tiles need no mask; what is left over (if
    // anything) is one masked tile.
    if (K < 0 || T <= 0 || nfull == nullptr || rem == nullptr)
        return TM_E_INVAL;
    *nfull = K / T;
    *rem = K - *nfull * T;
    return TM_OK;
}

int check_tile(int TM, int TN) {
    if (TM <= 0 || TN <= 0)
        return TM_E_INVAL;  // a divisor must be positive ([ALIGNED] "When the promise is broken")
    if (!is_pow2(TM) || TM > kMaxTM || !is_pow2(TN) || TN > kMaxTN)
        return TM_E_UNSUPPORTED;  // not a tile the kernels were built for
    return TM_OK;
}

int check_promise(int64_t M, int64_t N, int64_t ld_in, int64_t ld_out, int TM, int TN,
                  const void *in, const void *out) {
    if (M < 0 || N < 0 || ld_in < N || (out != nullptr && ld_out < N) || TM <= 0 || TN <= 0)
        return TM_E_INVAL;
    int st = check_tile(TM, TN);
    if (st != TM_OK)
        return st;
    return promise_holds(M, N, ld_in, ld_out, TM, TN, in, out) ? TM_OK : TM_E_ALIGN;
}

int plan_tiles(int64_t M, int64_t N, int TM, int TN, int64_t *tiles_m, int64_t *tiles_n,
               int64_t *whole) {
    if (tiles_m == nullptr || tiles_n == nullptr || whole == nullptr || M < 0 || N < 0)
        return TM_E_INVAL;
    int st = check_tile(TM, TN);
    if (st != TM_OK)
        return st;
    const int64_t wm = M / TM, wn = N / TN;  // whole tiles along each extent
    if (wn > 0 && wm > INT64_MAX / wn)
        return TM_E_INVAL;  // the whole-tile count does not fit 64 bits
    *tiles_m = ceil_div(M, TM);
    *tiles_n = ceil_div(N, TN);
    *whole = wm * wn;  // tiles with (pm+1)*TM <= M and (pn+1)*TN <= N
    return TM_OK;
}

int pad_extents(int64_t M, int64_t N, int TM, int TN, int64_t *Mp, int64_t *Np, int64_t *ldp) {
    if (Mp == nullptr || Np == nullptr || ldp == nullptr || M < 0 || N < 0 || TM <= 0 || TN <= 0)
        return TM_E_INVAL;
    int st = check_tile(TM, TN);
    if (st != TM_OK)
        return st;
    if (TN % 4 != 0)
        return TM_E_ALIGN;  // tile rows shorter than a 16-byte vector cannot keep the promise
    if (M > INT64_MAX / 4 - TM || N > INT64_MAX / 4 - TN)
        return TM_E_INVAL;
    *Mp = ceil_div(M, TM) * TM;
    *Np = ceil_div(N, TN) * TN;
    *ldp = *Np;  // a multiple of TN, hence of 4
    return TM_OK;
}

// ---- element-wise maps ------------------------------------------------------------------------

int plan_map(int op, const float *x, int64_t ldx, float *y, int64_t ldy, int64_t M, int64_t N,
             float alpha, float beta, int TM, int TN, int aligned, int variant, MapPlan *plan,
             const float *scale, const float *bias) {
    *plan = MapPlan{};
    if (op < kAffine || op > kChannel)
        return TM_E_INVAL;
    if (aligned != 0 && aligned != 1)
        return TM_E_INVAL;
    if (variant < TM_VAR_AUTO || variant > TM_VAR_VEC4)
        return TM_E_INVAL;
    if (M < 0 || N < 0 || TM <= 0 || TN <= 0)
        return TM_E_INVAL;
    const bool work = M > 0 && N > 0;
    int st;
    if ((st = check_view(x, M, N, ldx, work)) != TM_OK)
        return st;
    if ((st = check_view(y, M, N, ldy, work)) != TM_OK)
        return st;
    if (op == kChannel && work) {
        // per-column vectors: bias required, scale optional (1 when absent)
        if ((st = check_vector(bias, N)) != TM_OK)
            return st;
        if (scale != nullptr && (st = check_vector(scale, N)) != TM_OK)
            return st;
    }
    if ((st = check_tile(TM, TN)) != TM_OK)
        return st;
    if (aligned && !promise_holds(M, N, ldx, ldy, TM, TN, x, y))
        return TM_E_ALIGN;  // checked once, before any launch ([ALIGNED] "When the promise is broken")

    // 16-byte vectors are legal when every vector a thread moves starts on a 16-byte boundary.
    const bool vec16 = TN % 4 == 0 && rows16(x, M, ldx) && rows16(y, M, ldy);
    int access;
    switch (variant) {
    case TM_VAR_AUTO: access = vec16 ? kVec4 : kScalar; break;
    case TM_VAR_SCALAR: access = kScalar1; break;
    case TM_VAR_VEC4_UNDERSTATED:
        if (TN % 4 != 0)
            return TM_E_UNSUPPORTED;
        access = kVec4Understated;
        break;
    default:
        if (!vec16)
            return TM_E_ALIGN;
        access = kVec4;
        break;
    }
    if (!work)
        return TM_OK;

    // An element-wise map over views whose rows are contiguous in both tensors (row stride N) is
    // one flat row of M*N elements: the same elements at the same addresses, so the same results,
    // with the only ragged edge at the flat row's end.  Every work item inside is whole: the
    // 4100 x 1000 ragged map went from 7.7 to 6.9 us (its scalar variant from 10.2 to 7.0 us),
    // as fast as the aligned 4096 x 1024.  The per-channel op too, with the channel of a flat
    // column found as its remainder by C: a bias add of 2^24 elements over 3 channels (ragged,
    // TN = 1) went from 36 to 22 us, 16 channels from 31 to 22 us.  (Rows of a multiple of 32
    // channels, on the 128-byte line grid, keep the 2-D schedule when the tile allows 16-byte
    // chunks: whole rows already store as contiguous 1 KiB, and the flat view's channel lookup
    // cost the 64-channel bias add 1-3%.)  The promise was checked on the caller's view above and
    // carries over:
    // N % TN == 0 makes M*N a multiple of every scheduling tile.
    int64_t chan_n = 0;
    const bool chan_flat = N <= kChanFlatMax && (N % 32 != 0 || TN % 4 != 0);
    if (M > 1 && ldx == N && ldy == N && (op != kChannel || chan_flat)) {
        if (op == kChannel)
            chan_n = N;
        N *= M;  // fits: check_view bounded (M - 1) * ld + N
        ldx = ldy = N;
        M = 1;
        TM = 1;
        if (!aligned) {
            // On the ragged path the caller's tile no longer shapes anything (the only ragged edge
            // is the flat row's end): schedule row segments, and let AUTO move 16-byte chunks
            // whenever both bases allow them, whatever TN.  (Under the promise the tile must still
            // divide the flat row: every scheduling tile is taken whole.)
            TN = kRowSegmentBytes / 4;
            if (variant == TM_VAR_AUTO)
                access = aligned_to(x, 16) && aligned_to(y, 16) ? kVec4 : kScalar;
        }
    }

    // Padded rows (row stride ld > N, the same in both tensors, both bases the same distance past a
    // 16-byte boundary, padding under one 128-byte line or at most an eighth of the row, or wider
    // as below): on the ragged path the span from y[0] to the last element is cut into 1 KiB items
    // on y's 1 KiB grid, and each item moves 16-byte chunks with the columns past N masked
    // (mapflat.hip, map_rows);
    // the channel op takes each element's column as its channel.  Work items then never share a
    // line, where 2-D tiles over rows off the line grid shared the lines at both ends of every row
    // piece with the neighbouring items: a line written in parts by two XCDs reaches HBM3E as
    // partial writes, which the controller turns into read-modify-writes.  Only the lines that
    // hold padding are written in part here.  4100 x 4100 at row stride 4104: the map 33.6 ->
    // 21.6 us; at stride 4140 (40 floats of padding) the map 33.4 us and the bias add 54.3 us
    // under 2-D tiles.
    // Different row strides take the same span over y (DIFF in mapflat.hip) when they differ by a
    // multiple of 4 floats: the chunk of span element q, row r, then sits r (ldx - ldy) floats
    // further on in x, still 16-byte aligned; a chunk that crosses a row's end takes the next
    // row's elements from a second load.  y may then also be contiguous (x padded).
    // (Rows of both tensors on the 128-byte line grid keep the 2-D plan, whose work items are then
    // whole lines already, when the strides differ.)  x's rows drift against y's 1 KiB grid, so
    // an item's 1 KiB of x mostly spans nine lines, one of them fetched by two XCDs (11% more
    // reads); under 1024 floats a row the span then measured slower than the 2-D plan on 16-byte
    // rows: 4100 x 1000 at strides 1004 / 1008 8.1 us as a span, 7.8 under 2-D tiles, 16400 x
    // 1000 24.8 against 23.6; 4100 x 4100 at 4104 / 4108 23.5 against 33.5, 2733 x 1500 at 1504 /
    // 1508 8.1 against 8.4.  Rows off the 16-byte grid (where the 2-D plan moves 4-byte chunks)
    // take the span at any width: 62137 x 135 at 138 / 135 18.1 against 24.3 us, 7781 x 539 at
    // 539 / 607 10.5 against 12.9, 4100 x 1000 at 1001 / 1004 8.7 against 9.5, 16400 x 250 at
    // 251 / 256 9.0 against 9.5; it lost on 32768 x 100 at 101 / 103 (9.8 against 9.1) and
    // 8192 x 500 at 503 / 500 (9.7 against 9.1).
    const int64_t pad = ldy - N;
    const bool y_lines = aligned_to(y, kLineBytes) && ldy % (kLineBytes / 4) == 0;
    const bool both_lines = y_lines && aligned_to(x, kLineBytes) && ldx % (kLineBytes / 4) == 0;
    // Padding: under a line, or at most an eighth of the row; wider padding when y's rows miss the
    // line grid, where the 2-D plan's row pieces share lines between items (a wave wholly inside
    // the padding exits at once, so what wider padding costs is those waves' dispatch): a quarter
    // of the row for 16-byte rows of 2048 floats or more, and for rows off the 16-byte grid (which
    // the 2-D plan moves in 4-byte chunks) a quarter, or half from 2048 floats on.  Span against
    // 2-D tiles, HIP events over 1 GiB of rotating buffers: 4100 x 4100 at stride 4700 24.6 against
    // 33.8 us, 2048 x 4100 at 6150 14.2 against 24.5, 4096 x 2500 at 3750 16.8 against 23.4,
    // 8192 x 1000 at 1201 13.8 against 15.8; past those limits the span lost or tied: 8192 x 2048
    // at 3000 26.2 against 24.0, 4096 x 2048 at 2900 14.4 against 13.6, 32768 x 250 at 375 18.4
    // against 16.5, 8192 x 1000 at 1501 16.4 against 16.2.
    const bool y16 = aligned_to(y, 16) && ldy % 4 == 0;
    const bool pad_ok = pad < kLineBytes / 4 || pad * 8 <= N ||
                        (!y_lines && (pad * 4 <= N ? N >= kRowsWideMinN || !y16 : !y16 && N >= kRowsWideMinN && pad * 2 <= N));
    // x at another 4-byte phase than y's grid (bases not a multiple of 16 bytes apart, or strides
    // not a multiple of 4 floats apart): the same span over y, x's chunks moved as 4-byte aligned
    // 16-byte loads (SHIFT in mapflat.hip).  One flat row (contiguous rows, folded into one above)
    // takes the span too when the flat kernel cannot: x at another phase, or a base off the
    // 128-byte line grid (not the channel op, whose flat view finds channels by remainder).
    const bool shift = (reinterpret_cast<uintptr_t>(x) - reinterpret_cast<uintptr_t>(y)) % 16 != 0 ||
                       (M > 1 && (ldx - ldy) % 4 != 0);
    const bool padded = M > 1 && pad >= 0 && (ldx != ldy ? !both_lines && (N >= kRowsDiffMinN || access != kVec4) : pad > 0) && pad_ok;
    const bool flat_row = M == 1 && op != kChannel && (shift || !aligned_to(x, kLineBytes) || !aligned_to(y, kLineBytes));
    if (!aligned && (padded || flat_row) && N >= kRowsSpanMinN && (access == kVec4 || access == kScalar)) {
        if (M == 1)
            ldx = ldy = N;  // one row: the strides play no part
        const int64_t head = static_cast<int64_t>((reinterpret_cast<uintptr_t>(y) / 4) % 256);
        const int64_t span = (M - 1) * ldy + N;
        const int64_t xspan = (M - 1) * ldx + N;
        if (head + span + 256 <= INT32_MAX && xspan + 256 <= INT32_MAX && ldy <= UINT32_MAX) {  // 32-bit indexes
            const int64_t nwork = ceil_div(head + span, 256);
            const int64_t q_last = (span - 1) - ((span - 1 + head) & 3);
            plan->launch = true;
            plan->op = op;
            plan->access = access;
            plan->rows = true;
            plan->head = static_cast<uint32_t>(head);
            plan->span = static_cast<uint32_t>(span);
            plan->ld_div = make_div32(static_cast<uint32_t>(ldy));
            plan->x_last = static_cast<int32_t>(q_last + (M - 1) * (ldx - ldy));
            plan->shift = shift;
            plan->nwork = static_cast<uint32_t>(nwork);
            plan->grid = cap_grid(nwork);
            plan->x = x;
            plan->y = y;
            plan->ldx = ldx;
            plan->ldy = ldy;
            plan->M = M;
            plan->N = N;
            plan->alpha = alpha;
            plan->beta = beta;
            plan->scale = scale;
            plan->bias = bias;
            // a whole chunk's channels start on a column divisible by 4 when every chunk of the
            // span does (16-byte rows of y); then both vectors load as 16-byte chunks if aligned
            plan->cvec16 = op == kChannel && aligned_to(bias, 16) && aligned_to(scale, 16) && aligned_to(y, 16) &&
                           ldy % 4 == 0;
            return TM_OK;
        }
    }

    // Columns are scheduled in tiles at most one row segment wide: a wider tile (TN = 512, 1024)
    // is cut into row-segment columns.  The caller's tile only states the promise (already
    // checked) and, on the ragged path, which chunks take the masked body; neither changes a
    // result, and TN = 512 / 1024 tiles otherwise made work items of whole 2-4 KiB tile rows,
    // 6% slower on 8192 x 8192.
    //
    //
    // On the ragged path a row narrower than a row segment is scheduled as one tile exactly as
    // wide as the row's next power of two (at least one chunk), whatever the caller's tile: with
    // a 64-column tile, rows of 3 floats ran 3 live lanes of 64 (8.7M x 3 with row stride 7: 653
    // against 142 us).
    const int W = access == kScalar || access == kScalar1 ? 1 : 4;
    int TNs = static_cast<int>(std::min<int64_t>(TN, kRowSegmentBytes / 4));
    if (!aligned && N < kRowSegmentBytes / 4) {
        TNs = W;
        while (TNs < N)
            TNs *= 2;
    }
    int64_t tiles_m, tiles_n, whole;
    plan_tiles(M, N, TM, TNs, &tiles_m, &tiles_n, &whole);

    const int log_u = ilog2(access == kScalar ? kScalarChunksPerThread : 1);
    // Threads of a one-item workgroup on the line grid: one wave, or kScalar1Block threads for the
    // one-element-per-thread variant (a wave of single floats is only 256 bytes).
    const int log_item_threads = ilog2(access == kScalar1 ? kScalar1Block : kMapMinBlock);
    const int log_vr = ilog2(TNs / W);
    int log_tm = ilog2(TM);
    // A row that fits one scheduling tile cannot widen a work item, so on the ragged path (where
    // the tile's height shapes no result either) it is scheduled in tile rows tall enough for
    // 256 threads' chunks: a 1 x 64 tile over rows of 3 floats made work items of 3 elements.
    // (2M x 16 with row stride 17, 4-byte chunks: items of 16 / 64 / 256 rows took 68 / 61 /
    // 63 us; rows of 3, 5 or 8 floats within 3% of each other from 16 to 256 rows.)
    if (!aligned && tiles_n == 1)
        log_tm = std::max(log_tm, ilog2(kMapNarrowThreads) + log_u - log_vr);
    // Widest tile group: in the aligned path it must divide the tile count (no tile checks on the
    // device); in the ragged path it may run past the last tile (those lanes stay idle).
    int log_gcap = 0;
    if (aligned) {
        while (tiles_n % (int64_t{2} << log_gcap) == 0)
            ++log_gcap;
    } else {
        log_gcap = ilog2(tiles_n);
    }
    // Rows that start on cache lines: a work item is one wave's worth of chunks (64 x U, 1 KiB):
    // a strip of rows of a group of adjacent tiles, the group as wide as a 512-byte row segment
    // (whole lines, so no two work items share a line) and the strip as tall as the rest of the
    // 1 KiB allows.  On 8192 x 8192, 64-chunk work items with 128-, 256-, 512- and 1024-byte row
    // segments streamed 5.3, 5.85, 6.76 and 6.63 TB/s.  One-wave workgroups fill whatever wave
    // slots a CU has free; 1024-thread ones need 16 free slots on one CU at once.  Otherwise (rows
    // off the line grid) a work item spans as many tiles across the row band as fit in 1024 x U
    // chunks, so that workgroups share few lines.
    //
    // When the tile group can be a whole 1 KiB row segment, the work item is that one segment
    // instead, and whole items store it through a buffer resource with device scope and the
    // streaming hint (sc1 nt): on 4096 x 4096 21.1-21.2 us against 21.6-22.0 us for global nt
    // stores, with 16-byte chunks and with 4-byte ones alike (8192 x 8192: 79.6 against 79.7;
    // 4096 x 1024: 6.9 against 7.0).  The gain is the stores': the same policy on the loads
    // changed nothing, and on 2 x 512-byte items (21.9 us either way) or a transpose's 128-byte
    // row pieces it was no better or slower.
    const int64_t line = kLineBytes / 4;
    const bool line_rows = aligned_to(x, kLineBytes) && aligned_to(y, kLineBytes) &&
                           (M <= 1 || (ldx % line == 0 && ldy % line == 0));
    int log_r, log_g;
    bool stream = false;
    const int log_wave_chunks = log_item_threads + log_u;  // chunks of one (wave-sized) work item
    // (Not for the under-stated variant: each of its store instructions writes every fourth word.)
    const bool contiguous_stores = access != kVec4Understated;
    if (line_rows && contiguous_stores) {
        const int lg = ilog2(kStreamSegmentBytes / 4) - ilog2(TNs);  // tiles in one segment
        if (lg >= 0 && lg <= log_gcap && lg + log_vr == log_wave_chunks) {
            stream = true;
            log_g = lg;
            log_r = 0;
        }
    }
    if (stream) {
        // set above
    } else if (line_rows) {
        const int log_target = log_wave_chunks;
        log_g = std::min(log_gcap, std::max(0, ilog2(kRowSegmentBytes / 4) - ilog2(TNs)));
        log_r = std::min(log_tm, std::max(0, log_target - log_vr - log_g));
        log_g = std::min(log_gcap, std::max(log_g, log_target - log_vr - log_r));
    } else {
        const int log_target = ilog2(kMapMaxBlock) + log_u;
        // The channel op's U chunks per thread (4-byte chunks) share one read of the channel
        // vectors when the item spans at least U rows, so it keeps room for them (a bias add over
        // 4270 x 3017 with row stride 3049: 1024-column items of 4 rows instead of 4096-column
        // items of one row, of which 3017 columns live).
        const int log_rows_min = op == kChannel ? std::min(log_tm, log_u) : 0;
        log_g = std::min(log_gcap, std::max(0, log_target - log_vr - log_rows_min));
        log_r = std::min(log_tm, std::max(0, log_target - log_vr - log_g));
    }
    // A strip of whole rows of an output whose rows are contiguous (ldy == N) is one contiguous
    // 1 KiB block too: stored like a segment (100352 x 64 bias add: 9.35 against 9.44 us).
    if (!stream && line_rows && contiguous_stores && ldy == N && (int64_t{TNs} << log_g) == N &&
        log_r + log_g + log_vr == log_wave_chunks)
        stream = true;
    const int log_chunks = log_r + log_g + log_vr;
    const int64_t groups_n = ceil_div(tiles_n, int64_t{1} << log_g);
    // Row strips are numbered across the whole view (strip s = rows s*R .. s*R + R - 1; the kernel
    // splits s into tile row and strip within it), and only strips that hold a row are scheduled:
    // with 4 rows under a 64-row tile, 60 of every 64 strips used to launch, find no row and exit
    // (4 x 534137 with padded rows: 27 us for 17 MB).
    const int64_t nwork = ceil_div(M, int64_t{1} << log_r) * groups_n;
    if (nwork > INT32_MAX || tiles_n > INT32_MAX)
        return TM_E_UNSUPPORTED;  // work-item and tile ids are 32-bit on the device

    plan->launch = true;
    plan->op = op;
    plan->access = access;
    plan->aligned = aligned;
    plan->log_tm = log_tm;
    plan->log_tn = ilog2(TNs);
    plan->log_vr = log_vr;
    plan->log_r = log_r;
    plan->log_gv = log_g + log_vr;
    plan->log_strips = log_tm - log_r;
    plan->log_bs = std::max(ilog2(kMapMinBlock), log_chunks - log_u);
    plan->guard = plan->log_bs + log_u > log_chunks;
    // A thread's chunks t + u * threads share one column when the item is no wider than that.
    plan->share = op == kChannel && log_u > 0 && plan->log_gv <= plan->log_bs;
    plan->stream = stream;
    // One contiguous row cut into 1 KiB stream items (the scale, affine map and copy of any view
    // with contiguous rows on 128-byte lines): item w is elements [256 w, 256 w + 256) of the row,
    // and only the last can be ragged.  Such items go to a kernel that does nothing but that
    // (mapflat.hip).
    if (stream && M == 1 && op != kChannel && access != kVec4Understated) {
        plan->flat = true;
        plan->flat_last = static_cast<uint32_t>(N - (nwork - 1) * (kStreamSegmentBytes / 4));
    }
    plan->group = 1u << log_g;
    plan->groups_n = static_cast<uint32_t>(groups_n);
    plan->tiles_n = static_cast<uint32_t>(tiles_n);
    plan->nwork = static_cast<uint32_t>(nwork);
    plan->grid = cap_grid(nwork);
    plan->x = x;
    plan->y = y;
    plan->ldx = ldx;
    plan->ldy = ldy;
    plan->M = M;
    plan->N = N;
    plan->alpha = alpha;
    plan->beta = beta;
    plan->scale = scale;
    plan->bias = bias;
    // A flat channel chunk of 4 starts on a channel divisible by 4 and stays in one channel
    // vector chunk only when C % 4 == 0; otherwise its channels are gathered (and may wrap).
    plan->cvec16 = aligned_to(bias, 16) && aligned_to(scale, 16) && chan_n % 4 == 0;
    if (chan_n > 0) {
        plan->chan_n = static_cast<uint32_t>(chan_n);
        plan->chan = make_div32(static_cast<uint32_t>(chan_n));
        plan->chan_step = static_cast<uint32_t>((int64_t{TNs} << log_g) % chan_n);
    }
    return TM_OK;
}

// ---- row reductions ---------------------------------------------------------------------------

bool row_split_geometry(int64_t M, int64_t N, int *log_k, int64_t *seg, int64_t *segs) {
    if (M <= 0 || M >= kRowSplitRows || N < kRowSplitMinN)
        return false;
    // K: about kRowSplitTarget segments over all rows, at least one unit per segment.
    const int64_t units = ceil_div(N, kRowSegUnit) * M;
    int lk = 0;
    while (lk < kRowSegMaxLogK && (kRowSplitTarget << (lk + 1)) <= units)
        ++lk;
    *log_k = lk;
    *seg = int64_t{kRowSegUnit} << lk;
    *segs = ceil_div(N, *seg);
    return true;
}

size_t rows_ws_bytes(int64_t M, int64_t N) {
    int lk;
    int64_t seg, segs;
    if (!row_split_geometry(M, N, &lk, &seg, &segs))
        return 0;
    return static_cast<size_t>(M) * static_cast<size_t>(segs) * kRowPartialBytes;
}

// The one-pass row walk over M rows of N elements (16-byte chunks when vec) under the caller's
// column tile TC.
struct RowWalk {
    int lpr = 1;        // lanes per row (a power of two)
    int per_tile = 1;   // chunks per lane per column tile (the batched walk)
    int64_t bc = 1;     // column tile
    bool once = false;  // every chunk of a row in flight at once (row_once)
    int once_k = 0;     // chunks per lane of a one-batch row
};

static RowWalk row_walk(int64_t M, int64_t N, bool vec, int TC, bool once_ok = true) {
    const int W = vec ? 4 : 1;
    const int64_t chunks = ceil_div(N, W);  // chunks per row
    RowWalk rw;
    // Rows longer than a tiny row and short enough for one batch: lpr lanes (at least
    // kRowOnceMinLanes) with K chunks each cover the row, all issued before any arithmetic, and
    // the caller's tile decides which chunks are whole tiles (read without a mask) and which
    // belong to the one masked remainder tile; it cannot starve the row of lanes, so it is always
    // the walk's tile (a tile narrower than a chunk counts as one chunk).  Against the batched
    // walk below, on 8192 x 1000 masked maxima (1 GiB of rotating inputs, one process): 6.6-6.8 us
    // with 16, 32 or 64 lanes per row against 7.3-7.4 us.  Rows of more than half the batch's
    // lanes' reach with too few rows to fill the GPU keep the multi-wave walk.
    // 16-byte rows of up to kRowOnceMaxLanes * K chunks take 128 or 256 lanes per row, one row
    // per workgroup (4096 x 4096 sums, probe kernels of this shape, 1 GiB of rotating inputs: 128
    // or 256 lanes with 8 or 4 chunks each 11.2-11.3 us, where the batched walk below took 11.9;
    // one wave per row with 16 chunks per lane 12.5).
    const int K = vec ? kRowOnceK : kRowOnceKScalar;
    const bool few_long = chunks > int64_t{K} * 32 && M < kRowWideWaves;
    const int max_lanes = vec ? kRowOnceMaxLanes : 64;
    if (once_ok && chunks > int64_t{K} * kRowOnceMinLanes / 2 && chunks <= int64_t{K} * max_lanes && !few_long) {
        rw.once = true;
        rw.once_k = K;
        rw.lpr = std::max(kRowOnceMinLanes, 1 << ilog2(ceil_div(chunks, K)));
        rw.bc = std::max(TC, W);
        return rw;
    }
    // Lanes per row, fitted to HBM-streamed sweeps of forced lane counts (N = 4 to 2000 at 32 MB,
    // 1 GiB of rotating inputs, both chunk widths) and an interleaved comparison at 8192 x 1000
    // (16 / 32 / 64 lanes: 7.31 / 7.24 / 7.97 us): rows of up to 64 16-byte chunks are one tile
    // with about 4 chunks per lane; longer rows get about 8 chunks per lane per pass, up to a wave.
    int lpr, per_tile;
    if (vec && chunks <= kTinyRowChunks) {
        lpr = 1 << ilog2(ceil_div(chunks, 4));
        per_tile = 1 << ilog2(ceil_div(chunks, lpr));
    } else {
        lpr = 1 << std::min(6, ilog2(ceil_div(chunks, 8)));
        per_tile = 1;
    }
    if (chunks > (vec ? kShortRowChunksVec : kShortRowChunksScalar)) {
        // Long rows: one wave per row, walking tiles of 64 chunks (4-byte chunks: two per lane);
        // from 1024 16-byte chunks on, a 256-lane workgroup per row, whose lanes then have their
        // chunks in flight in one or two batches of 8 rather than two to eight one after another
        // (1 GiB of rotating inputs: 4096 x 4096 sums 12.1 -> 11.8 us, softmax statistics 13.0 ->
        // 12.4; 2048 x 8192 13.0 -> 11.9; 4096 x 16384 46.5 -> 41.0; at 2048 columns 128 or 256
        // lanes were 2-4% slower than 64).
        per_tile = vec ? 1 : 2;
        if (vec && chunks >= kRowLongChunks)
            lpr = kRowLongLanes;
        if (M < kRowWideWaves) {
            // Too few rows to fill the GPU with one wave each: a workgroup of several waves per
            // row, keeping at least 4 chunks per lane.
            int64_t l = int64_t{64} << ilog2(ceil_div(kRowWideWaves, M));
            l = std::min<int64_t>(std::max<int64_t>(l, lpr), kRowMaxLanes);
            while (l > 64 && l * 4 > chunks)
                l >>= 1;
            lpr = static_cast<int>(l);
            per_tile = 1;
        }
    }
    // The caller's column tile is the walk's whenever it holds whole chunks, keeps at least half
    // the lanes chosen above (one chunk each) and needs at most kRowTileMaxChunks chunks per lane
    // ([SLICING] "Reductions over a ragged tile": the 8192 x 1000 masked maximum in BC = 64
    // columns runs 15 whole tiles and one of 40 columns, 16 lanes per row where 32 were chosen;
    // 7.31 against 7.24 us).  Narrower tiles would starve the rows of lanes -- when the lanes per
    // row followed every tile, tiles 1 to 16 columns wide made a 4096 x 4096 row sum 4 to 58 times
    // slower -- and wider ones would put many chunks of the masked tile on each lane; both walk
    // the library's own tile of lpr * W * per_tile columns, split by the same rule into whole
    // tiles plus one masked remainder.
    if (TC % W == 0) {
        const int64_t tc = TC / W;  // chunks per caller tile (a power of two)
        const int64_t l = std::min<int64_t>(lpr, tc);
        if (2 * l >= lpr && tc / l <= kRowTileMaxChunks) {
            lpr = static_cast<int>(l);
            per_tile = static_cast<int>(tc / l);
        }
    }
    rw.lpr = lpr;
    rw.per_tile = per_tile;
    rw.bc = int64_t{lpr} * W * per_tile;
    return rw;
}

int plan_rows(int op, const float *x, int64_t ld, float *out, int64_t M, int64_t N, int TR, int TC,
              int aligned, RowPlan *plan, float *out2, bool with_ws, void *ws, size_t ws_bytes) {
    *plan = RowPlan{};
    if (op != kRowSum && op != kRowMax && op != kRowSoftmax)
        return TM_E_INVAL;
    if (aligned != 0 && aligned != 1)
        return TM_E_INVAL;
    if (M < 0 || N < 0 || TR <= 0 || TC <= 0)
        return TM_E_INVAL;
    int st;
    if ((st = check_view(x, M, N, ld, M > 0 && N > 0)) != TM_OK)
        return st;
    if ((st = check_vector(out, M)) != TM_OK)
        return st;
    if (op == kRowSoftmax && (st = check_vector(out2, M)) != TM_OK)
        return st;
    if ((st = check_tile(TR, TC)) != TM_OK)
        return st;
    int log_k = 0;
    int64_t seg = 0, segs = 0;
    const bool split_rows = with_ws && row_split_geometry(M, N, &log_k, &seg, &segs);
    if (split_rows && (ws == nullptr || ws_bytes < rows_ws_bytes(M, N) || !aligned_to(ws, 4)))
        return TM_E_WORKSPACE;
    if (aligned && !promise_holds(M, N, ld, 0, TR, TC, x, nullptr))
        return TM_E_ALIGN;
    if (M == 0)
        return TM_OK;
    if (split_rows) {
        // A few long rows: one workgroup per row would leave most of the GPU idle, so each row
        // segment gets a workgroup of its own.  Measured against the one-pass walk (1 GiB of
        // rotating inputs): 1 x 2^23 578 -> 11.1 us, 1 x 2^20 74.7 -> 7.3, 8 x 2^18 21.2 -> 7.5,
        // 64 x 2^18 23.1 -> 13.5, 96 x 2^17 13.8 -> 11.4; even at 65536 columns and from 128 rows
        // on (128 x 2^17 15.0 -> 13.5, 192 x 2^18 32.5 -> 34.9), slower at 32768 columns.
        if (M * segs > INT32_MAX)
            return TM_E_UNSUPPORTED;  // segment ids are 32-bit on the device
        plan->launch = true;
        plan->split = true;
        plan->op = op;
        plan->vec = rows16(x, M, ld);
        plan->log_k = log_k;
        plan->seg = seg;
        plan->segs = static_cast<uint32_t>(segs);
        plan->nwork = static_cast<uint32_t>(M * segs);
        plan->grid = cap_grid(M * segs);
        plan->block = kBlock;
        plan->x = x;
        plan->out = out;
        plan->out2 = out2;
        plan->ws = static_cast<float *>(ws);
        plan->ld = ld;
        plan->M = M;
        plan->N = N;
        return TM_OK;
    }

    // Lanes per row come from the row length and count; the column tile is the caller's BC
    // (TC here) whenever it suits the lanes (row_walk below).  Rows with 16-byte starts take
    // 16-byte chunks whatever N is: whole tiles hold whole chunks, and the remainder tile masks
    // the chunk that straddles N element by element.
    const bool vec = rows16(x, M, ld);
    // Long rows off the 16-byte grid are read in 16-byte chunks all the same: each from the 16-byte
    // boundary at or before its start (within the same aligned 16 bytes, so never past a page the
    // row does not touch), its first one to three elements masked, the walk laid out for N + 3
    // elements.  133 x 64954 at row stride 64986 read as 4-byte chunks streamed 2.8 TB/s.
    const bool shift = !vec && N > kRowShiftMinN;
    // (The one-batch kernel has no shifted form: such rows keep the batched walk.)
    const RowWalk rw = shift ? row_walk(M, N + 3, true, TC, false) : row_walk(M, N, vec, TC);
    const int lpr = rw.lpr;
    plan->launch = true;
    plan->op = op;
    plan->vec = vec;
    plan->shift = shift;
    plan->lpr = lpr;
    plan->block = lpr > 64 ? lpr : kBlock;
    plan->per_tile = rw.per_tile;
    plan->bc = static_cast<int>(rw.bc);
    plan->once = rw.once;
    plan->once_k = rw.once_k;
    split(N, plan->bc, &plan->nfull, &plan->rem);  // whole column tiles + one masked remainder tile
    const int64_t groups = ceil_div(M, plan->block / lpr);
    if (groups > INT32_MAX)
        return TM_E_UNSUPPORTED;  // row-group ids are 32-bit on the device
    // One lane per row (rows of a few elements): a wave's work is a few hundred bytes, so its fixed
    // cost dominates; workgroups that loop over several row groups spread it (1 GiB of rotating
    // inputs: 2^24 one-element rows 52.4 -> 38.8 us, 2^23 x 2 33.5 -> 27.2, 2^22 x 4 22.2 -> 17.5;
    // results unchanged, since each row is walked the same way).
    plan->grid = cap_grid(lpr == 1 ? std::min(groups, kRowTinyGrid) : groups);
    plan->x = x;
    plan->out = out;
    plan->out2 = out2;
    plan->ld = ld;
    plan->M = M;
    plan->N = N;
    return TM_OK;
}

int row_walk_query(int64_t M, int64_t N, int64_t ld, int TR, int TC, int aligned, const void *x,
                   int64_t *bc, int64_t *nfull, int64_t *rem, int *lanes) {
    if (bc == nullptr || nfull == nullptr || rem == nullptr || lanes == nullptr)
        return TM_E_INVAL;
    if (aligned != 0 && aligned != 1)
        return TM_E_INVAL;
    if (M < 0 || N < 0 || ld < N || TR <= 0 || TC <= 0)
        return TM_E_INVAL;
    if (M > 0 && N > 0 && (x == nullptr || !aligned_to(x, 4)))
        return TM_E_INVAL;
    const int st = check_tile(TR, TC);
    if (st != TM_OK)
        return st;
    if (aligned && !promise_holds(M, N, ld, 0, TR, TC, x, nullptr))
        return TM_E_ALIGN;
    const bool vec = rows16(x, M, ld);
    const RowWalk rw = !vec && N > kRowShiftMinN ? row_walk(M, N + 3, true, TC, false) : row_walk(M, N, vec, TC);
    *lanes = rw.lpr;
    *bc = rw.bc;
    return split(N, *bc, nfull, rem);
}

// ---- column sums ------------------------------------------------------------------------------

namespace {

// Rows per slab, as a power of two: the naive walks keep the caller's TM (one workgroup per TM
// rows of a column, the pages' geometry); the LDS walk uses kColSlab-row slabs, taller when more
// than kColMaxSlabs of them would leave pass 2 too many partials per column.  On 4096 x 4096 the
// LDS walk took 14.6-15.6 us with 64- to 256-row slabs and 64- or 128-column strips against
// 22-44 us with tiles 16-32 rows tall or 256-1024 columns wide.
int slab_log(int64_t M, int64_t N, int TM, int walk) {
    if (walk != TM_COL_LDS)
        return ilog2(TM);
    int l = ilog2(kColSlab);
    while (ceil_div(M, int64_t{1} << l) > kColMaxSlabs)
        ++l;
    // Few strips (narrow matrices): shorter slabs, halved while there would be fewer than
    // kColTargetWork workgroups, keeping at least 4 row steps per thread (a step is 1024 / TW rows
    // at 16-byte chunks).  1 GiB of rotating inputs: 1280 x 1338 14.7 -> 7.8 us (32-row slabs),
    // 2476 x 3397 15.8 -> 11.9, 21963 x 286 15.6 -> 11.4, 8192 x 1000 12.4 -> 11.9, 4096 x 1024
    // 10.6 -> 9.2; 4096 x 4096 within 1%; slabs below 4 row steps were slower (59048 x 59, 32
    // rows: 12.0 against 10.0 us).
    const int64_t tw = N >= kColStrip ? kColStrip : std::max<int64_t>(1, int64_t{1} << ilog2(N));
    const int64_t strips = ceil_div(N, tw);
    const int lmin = std::max(5, ilog2(std::max<int64_t>(1, 4096 / tw)));
    if (strips == 0)
        return l;  // N == 0: no columns, nothing to balance
    // slabs * strips < kColTargetWork, without the product: slabs < ceil(kColTargetWork / strips)
    const int64_t few = ceil_div(kColTargetWork, strips);
    while (l > lmin && ceil_div(M, int64_t{1} << l) < few)
        --l;
    return l;
}

}  // namespace

// The LDS walk over wide matrices (N >= kColRowStrip, whole 16-byte chunks): rows per slab for
// the strip kernel, or 0 when the shape takes the LDS-staged kernel instead.
int strip_slab_log(int64_t M, int64_t N, int walk) {
    if (walk != TM_COL_LDS || N < kColRowStrip || N % 4 != 0 || M <= 0)
        return 0;
    int l = ilog2(kColRowSlab);
    while (ceil_div(M, int64_t{1} << l) > kColRowMaxSlabs)
        ++l;
    const int64_t work = ceil_div(M, int64_t{1} << l) * ceil_div(N, kColRowStrip);
    return work >= kColRowMinWork ? l : 0;
}

// Measured against the two-pass walk (1 GiB of rotating inputs): 1 x 2^20 21.8 -> 6.5 us,
// 4 x 2^22 75.3 -> 18.2, 16 x 2^20 25.9 -> 15.0, 64 x 2^18 16.9 -> 13.1, 16 x 65536 7.3 -> 5.8,
// 256 x 2^18 45.2 -> 43.1; slower from 128 rows of fewer columns (256 x 65536: 14.5 against 28.1
// us; a thread walks its rows 16 loads at a time) and for tall inputs (4096 x 4096: 15 against
// 403 us: 1024 threads).
bool col_direct(int64_t M, int64_t N, int walk) {
    return walk == TM_COL_LDS && M > 0 &&
           (M <= kColDirectRows || (M <= kColDirectRowsWide && N >= kColDirectMinN));
}

size_t colsum_ws_bytes(int64_t M, int64_t N, int TM, int TN, int walk) {
    if (M <= 0 || N <= 0 || check_tile(TM, TN) != TM_OK)
        return 0;
    if (walk != TM_COL_NAIVE && walk != TM_COL_LDS && walk != TM_COL_NAIVE_XCD)
        return 0;
    if (col_direct(M, N, walk))
        return 0;  // one pass, no partials
    int64_t slabs = ceil_div(M, int64_t{1} << slab_log(M, N, TM, walk));
    // A wide matrix takes the strip kernel when the workspace is 16-byte aligned (and the rows
    // allow it), and the LDS-staged kernel otherwise: room for the larger of the two.
    if (const int ls = strip_slab_log(M, N, walk))
        slabs = std::max(slabs, ceil_div(M, int64_t{1} << ls));
    if (slabs > INT64_MAX / 4 / N)
        return 0;
    return static_cast<size_t>(slabs * N * 4);
}

int plan_cols(const float *x, int64_t ld, float *out, int64_t M, int64_t N, int TM, int TN,
              int aligned, int walk, void *ws, size_t ws_bytes, ColPlan *plan) {
    *plan = ColPlan{};
    if (walk != TM_COL_NAIVE && walk != TM_COL_LDS && walk != TM_COL_NAIVE_XCD)
        return TM_E_INVAL;
    if (aligned != 0 && aligned != 1)
        return TM_E_INVAL;
    if (M < 0 || N < 0 || TM <= 0 || TN <= 0)
        return TM_E_INVAL;
    int st;
    if ((st = check_view(x, M, N, ld, M > 0 && N > 0)) != TM_OK)
        return st;
    if ((st = check_vector(out, N)) != TM_OK)
        return st;
    if ((st = check_tile(TM, TN)) != TM_OK)
        return st;
    const int log_ts = M > 0 ? slab_log(M, N, TM, walk) : 0;
    const int64_t slabs = ceil_div(M, int64_t{1} << log_ts);
    const size_t need = colsum_ws_bytes(M, N, TM, TN, walk);
    const bool direct = col_direct(M, N, walk);
    if (slabs > INT32_MAX || (M > 0 && N > 0 && need == 0 && !direct))
        return TM_E_UNSUPPORTED;  // partial count or workspace size out of range
    if (need > 0 && (ws == nullptr || ws_bytes < need || !aligned_to(ws, 4)))
        return TM_E_WORKSPACE;
    if (aligned && !promise_holds(M, N, ld, 0, TM, TN, x, nullptr))
        return TM_E_ALIGN;
    if (N == 0)
        return TM_OK;
    if (direct) {
        // A column walk without partials: each thread adds one chunk of columns down all M rows.
        plan->direct = true;
        plan->finish = true;  // a call with work (callers launch when finish is set)
        plan->walk = walk;
        // 16-byte chunks, from 4-byte aligned addresses when the rows are off the 16-byte grid:
        // 16 x 2^20 at row stride 2^20 + 1 14.6 against 17.7 us with 4-byte chunks
        plan->vec = true;
        plan->out16 = aligned_to(out, 16);
        plan->x = x;
        plan->out = out;
        plan->ld = ld;
        plan->M = M;
        plan->N = N;
        return TM_OK;
    }

    plan->finish = true;
    plan->launch = M > 0;
    plan->walk = walk;
    plan->log_tm = log_ts;
    plan->slabs = static_cast<uint32_t>(slabs);
    // Wide matrices (at least kColRowStrip columns) with 16-byte rows and a 16-byte aligned
    // workspace: the strip kernel.  A workgroup takes one slab of a kColStripCols-column strip:
    // lane t of each of its kColStripGroups waves owns 16-byte column chunk t of the strip (each
    // row of the strip one 1 KiB run of memory), wave q adds its eighth of the slab's rows, 8
    // loads in flight, and the waves' sums meet in LDS in order.  On 4096 x 4096 (1 GiB of
    // rotating inputs) both passes took 14.3 us against 16.1 us when each thread of 256 walked
    // all 64 rows of a 1024-column strip 16 loads at a time (pass 1 alone 11.8 against 12.3 us;
    // the second launch then also started sooner), and 13.8 us was the LDS-staged kernel's
    // 128 x 128 tiles' pass 1 alone.
    // Rows off the 16-byte grid take the same walk with 4-byte aligned 16-byte loads (vec =
    // false: col_strip<..., U>) when N is a whole number of strips: 4096 x 4096 at row stride 4097
    // 17.9 -> 15.6 us against the LDS-staged kernel's 4-byte loads, with the base one float off
    // 19.2 -> 15.7, 8192 x 2048 at 2049 17.9 -> 16.3.  With a part-filled last strip the LDS-staged
    // kernel was faster (4096 x 3100 at 3101 15.0 against 16.7 us, 4096 x 4352 at 4353 19.0
    // against 20.1, 4096 x 4100 at 4103 19.0 against 20.3).
    const int lstrip = strip_slab_log(M, N, walk);
    const bool x16 = rows16(x, M, ld);
    const int64_t sslabs = lstrip > 0 ? ceil_div(M, int64_t{1} << lstrip) : 0;
    // (the grid's thread count, slabs x strips x workgroup threads, must fit 32 bits)
    const bool strip_grid = uint64_t(sslabs) * uint64_t(ceil_div(N, kColStripCols)) * (64u * kColStripGroups) <
                            (uint64_t{1} << 32);
    if (lstrip > 0 && strip_grid && aligned_to(ws, 16) && (x16 || N % kColRowStrip == 0)) {
        plan->strip = true;
        plan->vec = x16;
        plan->log_tm = lstrip;
        plan->slabs = static_cast<uint32_t>(sslabs);
        plan->tw = kColStripCols;
        plan->strips = static_cast<uint32_t>(ceil_div(N, kColStripCols));
        plan->whole = M % (int64_t{1} << lstrip) == 0 && N % kColStripCols == 0;
        plan->x = x;
        plan->out = out;
        plan->ws = static_cast<float *>(ws);
        plan->ld = ld;
        plan->M = M;
        plan->N = N;
        return TM_OK;
    }
    if (walk == TM_COL_LDS) {
        // Like the slabs, the strips are the walk's own: the caller's tile states the promise.
        // (16-byte chunks from 4-byte aligned addresses for rows off the 16-byte grid measured
        // slower here over narrow rows -- fewer lanes per row: 43690 x 96 at row stride 128 with
        // the base 3 floats off 13.0 against 11.7 us, 1677721 x 10 at 13 24.6 against 20.9 -- so
        // such rows keep 4-byte chunks.)
        plan->vec = rows16(x, M, ld);
        const int W = plan->vec ? 4 : 1;
        plan->tw = std::max(W, N >= kColStrip ? kColStrip : 1 << ilog2(N));
        const int64_t strips = ceil_div(N, plan->tw);
        if (strips > INT32_MAX)
            return TM_E_UNSUPPORTED;
        plan->strips = static_cast<uint32_t>(strips);
        // No masks when the shape is whole slabs by whole strips of 16-byte rows, promised or not.
        plan->whole = plan->vec && M % (int64_t{1} << log_ts) == 0 && N % plan->tw == 0;
    } else {
        plan->vec = TN % 4 == 0 && rows16(x, M, ld);
        plan->naive_block = std::max(64, TM);
        if (N > INT32_MAX)
            return TM_E_UNSUPPORTED;
        plan->strips = static_cast<uint32_t>(N);
    }
    // Pass 2: a group of fl lanes per column (each adding every fl-th slab in order, then a fixed
    // lane tree), so that tall, narrow inputs do not leave a few threads adding thousands of
    // partials one after another: up to 64 lanes (one wave), about kFinishThreads threads in
    // all, and up to kFinishMaxLanes while a lane would otherwise take more than one batch of
    // kFinishBatchSlabs partials (the waves of a column then meet in LDS): 2^20 x 64 (4096 slabs)
    // 50.9 -> 49.2 us, 1677721 x 10 at row stride 13 20.1 -> 18.6 (1 GiB of rotating inputs).
    {
        const int64_t fl = kFinishThreads / N;
        int l = 0;
        while (l < 6 && (int64_t{2} << l) <= fl)
            ++l;
        while ((int64_t{1} << l) < kFinishMaxLanes && (int64_t{kFinishBatchSlabs} << l) < slabs)
            ++l;
        plan->fl = std::min(1 << l, 1 << ilog2(std::max<int64_t>(slabs, 1)));
    }
    plan->x = x;
    plan->out = out;
    plan->ws = static_cast<float *>(ws);
    plan->ld = ld;
    plan->M = M;
    plan->N = N;
    return TM_OK;
}

// ---- batched transpose -------------------------------------------------------------------------

int plan_transpose(const float *x, int64_t ldx, int64_t bsx, float *y, int64_t ldy, int64_t bsy,
                   int64_t B, int64_t M, int64_t N, int TM, int TN, int aligned,
                   TransposePlan *plan) {
    *plan = TransposePlan{};
    if (aligned != 0 && aligned != 1)
        return TM_E_INVAL;
    if (B < 0 || M < 0 || N < 0 || bsx < 0 || bsy < 0 || TM <= 0 || TN <= 0)
        return TM_E_INVAL;
    const bool work = B > 0 && M > 0 && N > 0;
    int st;
    if ((st = check_view(x, M, N, ldx, work)) != TM_OK)   // x: M x N
        return st;
    if ((st = check_view(y, N, M, ldy, work)) != TM_OK)   // y: N x M
        return st;
    if (work && B > 1) {
        // batches of y must not overlap (their writes would race); x batches may be read twice
        if (bsy < (N - 1) * ldy + M || (bsx > 0 && (B - 1) > (INT64_MAX / 4) / bsx) ||
            (B - 1) > (INT64_MAX / 4) / std::max<int64_t>(bsy, 1))
            return TM_E_INVAL;
    }
    if ((st = check_tile(TM, TN)) != TM_OK)
        return st;
    // 16-byte chunks: x rows read along N, y rows written along M, every row on a 16-byte boundary
    // in every batch.  Whether they are used depends on the data only (a chunk that straddles the
    // edge of a ragged view moves element by element); the promise also covers the tile.
    const bool vx16 = rows16(x, M, ldx) && (B <= 1 || bsx % 4 == 0);
    const bool vy = rows16(y, N, ldy) && (B <= 1 || bsy % 4 == 0);
    const bool vec = vx16 && vy;
    if (aligned && !(M % TM == 0 && N % TN == 0 && TM % 4 == 0 && TN % 4 == 0 && vec))
        return TM_E_ALIGN;
    if (!work)
        return TM_OK;
    const bool y_lines = aligned_to(y, kLineBytes) && (N <= 1 || ldy % (kLineBytes / 4) == 0) &&
                         (B <= 1 || bsy % (kLineBytes / 4) == 0);
    const bool large = !aligned && M >= 2 * kTrSub && N >= kTrSub && M * N >= (int64_t{1} << 22);
    // (batches: the line windows of every batch, numbered as one matrix of B x subs_n strips)
    const bool skew = !aligned && M >= 2 * kTrSub && N >= kTrWindowMinN &&
                      M * N >= ceil_div(int64_t{1} << 22, std::max<int64_t>(B, 1)) && !y_lines;
    // x's reads move in 16-byte chunks also off the 16-byte grid, as 4-byte aligned 16-byte loads,
    // when its rows hold a whole sub-tile row.
    const bool vx = vx16 || N >= kTrSub;
    plan->launch = true;
    plan->vec = vec;
    plan->aligned = aligned;
    // Staged sub-tiles: kTrSub x kTrSub.  A narrow extent (fewer than kTrSub rows or columns, as
    // the 3 channels of an RGB image) gets a sub-tile just as narrow and as much longer, up to
    // kTrSubElems elements, so that no lanes are spent on rows or columns that do not exist.
    // Under the promise a sub-tile must divide the extents (whole sub-tiles, no masks): the
    // largest power of two up to the cap that divides the extent, which the promised tile
    // divides.  16-byte chunks need both sub-tile extents to be at least 4.
    // x rows (read along N) need sub-tiles at least a chunk wide (sn >= 4 for 16-byte reads), y
    // rows (written along M) likewise (sm >= 4 for 16-byte writes).
    auto fit = [&](int64_t extent, int64_t cap, int64_t lo) {
        int64_t e = aligned ? cap : std::min<int64_t>(cap, int64_t{1} << ilog2(extent));
        if (aligned)
            while (extent % e != 0)
                e /= 2;
        return static_cast<int>(std::max(e, lo));
    };
    const int64_t lo_n = vx ? 4 : 1, lo_m = vy ? 4 : 1;
    if (N < kTrSub && M >= kTrSub) {  // narrow rows of x: long along M
        plan->sn = fit(N, kTrSub, lo_n);
        plan->sm = fit(M, kTrSubElems / plan->sn, lo_m);
    } else {
        plan->sm = fit(M, kTrSub, lo_m);
        plan->sn = fit(N, kTrSubElems / plan->sm, lo_n);
    }
    // Rows on no 16-byte boundary on either side (odd strides): every 128-byte row piece straddles
    // two lines, and taller sub-tiles with longer y-row pieces did better.  64 x 16 against 32 x 32
    // (1 GiB of rotating buffers, outputs compared bit for bit): 4099 x 4099 66.5 -> 56.0 us,
    // 9163 x 1051 43.5 -> 31.8, 2951 x 2697 36.8 -> 32.2, 17827 x 767 64.0 -> 59.3; small
    // matrices (1001 x 1001: 5.0 against 5.4 us) keep 32 x 32.
    //
    // Rows of y off the 16-byte grid (4-byte stores; every y-row piece shares its end lines with
    // the neighbouring sub-tiles') do better still with 64 x 32 sub-tiles, staged in a 2048-element
    // instance: y-row pieces of 256 bytes, x-row pieces of 128.  Against 32 x 32 / 64 x 16, in the
    // kernel itself over 1 GiB of rotating buffers: 5450 x 2568 (y stride 5450) 63.2 / 51.8 ->
    // 47.9 us, 57348 x 252 (y stride 57349) 58.6 / 47.8 -> 45.3 us, 1707 x 7425 (strides 7428,
    // 1707) 48.7 / 43.7 -> 38.5 us, 4099 x 4099 with both sides off 65.4 / 55.2 -> 51.2 us;
    // 128 x 16, 128 x 32, 64 x 64 and 256 x 16 were slower than 64 x 32 on at least three of the
    // four.
    //
    // When y's rows are off the 128-byte line grid (16-byte rows or not), the lines at the ends of
    // each y-row piece are shared with the sub-tiles above and below, and a line written in parts
    // by two XCDs reaches HBM as partial writes (read-modify-write in the controller: 4096 x 4096
    // with y stride 4100 took 55.7 against 24.4 us with stride 4096).  One matrix then writes
    // line-aligned windows of its y rows instead of sub-tiles (transpose.hip, transpose_skew):
    // 64 elements of 32 y rows per work item, each window starting on a line, from a staged band
    // of 96 x rows.  Against 64 x 32 sub-tiles in vertical groups on one XCD (one process, 1 GiB of
    // rotating buffers): 4096 x 4096 at y stride 4100 30.3 -> 26.9 us, 4098 35.2 -> 27.3, 4097
    // 35.2 -> 27.6, both strides 4097 43.4 -> 32.5 (4-byte x reads), 5450 x 2568 36.9 -> 25.8,
    // 57348 x 252 39.4 -> 26.8, 1707 x 7425 37.9 -> 26.2, 4099 x 4099 48.2 -> 32.3.
    if ((large && !vy) || skew) {
        plan->sm = 2 * kTrSub;
        plan->sn = kTrSub;
        plan->sub = 2 * kTrSubElems;
        plan->skew = skew;
    }
    plan->vx = vx;
    plan->vy = vy;
    // skew: item rows of 64 windows each, one more when the windows' shift (up to 31 floats) can
    // leave the last rows of y uncovered
    const int64_t subs_m = skew ? ceil_div(M + kTrSub - 1, plan->sm) : ceil_div(M, plan->sm);
    const int64_t subs_n = ceil_div(N, plan->sn);
    if (subs_m > INT32_MAX || subs_n > INT32_MAX)
        return TM_E_UNSUPPORTED;
    plan->subs_m = static_cast<uint32_t>(subs_m);
    plan->subs_n = static_cast<uint32_t>(subs_n);
    if (subs_m * subs_n > INT64_MAX / B)
        return TM_E_UNSUPPORTED;
    // Small matrices (each in one sub-tile) are packed: a work item takes 2^log_g consecutive
    // batches, up to kTrSubElems elements in all, each staged in its own part of the LDS.  With one
    // matrix per 256-thread workgroup, 2^20 batches of 4 x 4 took 546 us.
    if (subs_m == 1 && subs_n == 1 && B > 1) {
        const int64_t room = kTrSubElems / (int64_t{plan->sm} * plan->sn);
        while ((int64_t{2} << plan->log_g) <= room && (int64_t{1} << plan->log_g) < B)
            ++plan->log_g;
    }
    plan->nwork = static_cast<uint64_t>(plan->log_g > 0 ? ceil_div(B, int64_t{1} << plan->log_g)
                                                        : B * subs_m * subs_n);
    // Few channels whose packed side is not 16-byte rows (3 channels: rows of 12 bytes): the packed
    // side of a work item is one contiguous block, moved in 16-byte chunks by transpose_packed.
    // (32, 3, 224, 224) NCHW -> NHWC and back: 13.9 -> 8.9 us; 1 to 31 channels gain 1.25-1.7x
    // (in one process, over 1 GiB of rotating buffers, outputs compared bit for bit).
    if (!vec && !plan->skew && plan->log_g == 0 && !(M < kTrSub && N < kTrSub)) {
        const bool bs16y = B <= 1 || bsy % 4 == 0, bs16x = B <= 1 || bsx % 4 == 0;
        if (M < kTrSub && ldy == M && subs_m == 1) {
            plan->packed = 1;
            plan->pvec = rows16(x, M, ldx) && bs16x;
            plan->flat16 = aligned_to(y, 16) && bs16y;
        } else if (N < kTrSub && ldx == N && subs_n == 1) {
            plan->packed = 2;
            plan->pvec = rows16(y, N, ldy) && bs16y;
            plan->flat16 = aligned_to(x, 16) && bs16x;
        }
        if (plan->packed != 0 && ((!plan->pvec && !plan->flat16) || plan->nwork > UINT32_MAX))
            plan->packed = 0;  // nothing to gain, or work ids beyond 32 bits
    }
    // 32 to kTrPackBigC channels whose packed rows (C floats) miss the 128-byte line grid: the
    // sub-tiles would write those rows in pieces that share lines with their neighbours (read-
    // modify-writes in HBM3E).  The packed kernel with larger items instead writes each item's
    // S positions x C channels as one block whose ends lie on lines (S a multiple of 32), S the
    // largest power of two with S C <= kTrPackBigElems; both sides in 16-byte chunks.  Against the
    // sub-tiles, NCHW -> NHWC / NHWC -> NCHW (one process, 1 GiB of rotating buffers): (32, 65,
    // 56, 56) 19.0 -> 12.6 / 16.2 -> 12.6 us, (64, 33, 56, 56) 21.0 -> 12.5 / 17.6 -> 12.8,
    // (16, 100, 56, 56) 13.6 -> 10.4 / 12.2 -> 9.8, (8, 127, 64, 64) 12.0 -> 8.8, one 100 x 262144
    // matrix 72.7 -> 40.1.  Items of up to 8192 elements took (32, 65, 56, 56) to 15.4 us, of
    // 16384 (two workgroups' LDS per CU) to 23.0.
    if (plan->packed == 0 && plan->log_g == 0 && !aligned) {
        const bool bs16y = B <= 1 || bsy % 4 == 0, bs16x = B <= 1 || bsx % 4 == 0;
        const int64_t line = kLineBytes / 4;
        int mode = 0;
        int64_t C = 0, P = 0;
        if (M >= kTrSub && M <= kTrPackBigC && ldy == M && N >= 2 * kTrSub && rows16(x, M, ldx) && bs16x &&
            aligned_to(y, 16) && bs16y && !(M % line == 0 && aligned_to(y, kLineBytes) && (B <= 1 || bsy % line == 0))) {
            mode = 1;
            C = M;
            P = N;
        } else if (N >= kTrSub && N <= kTrPackBigC && ldx == N && M >= 2 * kTrSub && rows16(y, N, ldy) && bs16y &&
                   aligned_to(x, 16) && bs16x && !(N % line == 0 && aligned_to(x, kLineBytes) && (B <= 1 || bsx % line == 0))) {
            mode = 2;
            C = N;
            P = M;
        }
        if (mode != 0) {
            int64_t S = kTrPackBigElems;
            while (S * C > kTrPackBigElems)
                S /= 2;
            const int64_t subs = ceil_div(P, S);
            if (B * subs <= UINT32_MAX && subs <= UINT32_MAX) {
                plan->packed = mode;
                plan->pbig = true;
                plan->pvec = true;
                plan->flat16 = true;
                plan->skew = false;
                plan->sub = kTrSubElems;
                if (mode == 1) {
                    plan->sm = static_cast<int>(C);
                    plan->sn = static_cast<int>(S);
                    plan->subs_m = 1;
                    plan->subs_n = static_cast<uint32_t>(subs);
                } else {
                    plan->sn = static_cast<int>(C);
                    plan->sm = static_cast<int>(S);
                    plan->subs_n = 1;
                    plan->subs_m = static_cast<uint32_t>(subs);
                }
                plan->nwork = static_cast<uint64_t>(B * subs);
            }
        }
    }
    if (plan->skew) {
        // Groups of G vertically adjacent items on one XCD: the upper neighbour's band rows are
        // still in that L2.  G = 4, 8 and 16 measured within 2-4% of each other; 8 with 16-byte x
        // reads, 4 with 4-byte ones.  (With 16-byte reads off the 16-byte grid, G = 8 against 4:
        // 17827 x 767 26.3 against 27.9 us, 5450 x 2568 with x stride 2569 26.9 against 28.1,
        // 9163 x 1051 19.7 against 20.2, 4096 x 4096 with both strides 4097 31.2-32.3 either way.)
        // Work items: 8 G per 8 groups (group r -> items 8 G (r / 8) + r mod 8 + 8 k, member k < G).
        plan->log_grp = vx ? 3 : 2;
        // few item rows (short y rows, as in batches): smaller groups, so that at most a quarter of
        // the group slots lie past the last item row (9 item rows in groups of 8 left 7 of 16 idle)
        while (plan->log_grp > 0 &&
               4 * (ceil_div(subs_m, int64_t{1} << plan->log_grp) * (int64_t{1} << plan->log_grp) - subs_m) >
                   ceil_div(subs_m, int64_t{1} << plan->log_grp) * (int64_t{1} << plan->log_grp))
            --plan->log_grp;
        const int64_t G = int64_t{1} << plan->log_grp;
        const int64_t grp_rows = ceil_div(subs_m, G);
        if (B > INT32_MAX || grp_rows * subs_n > UINT32_MAX / B)
            return TM_E_UNSUPPORTED;  // group ids are 32-bit
        const int64_t items = ceil_div(grp_rows * subs_n * B, 8) * 8 * G;
        if (items > UINT32_MAX)
            return TM_E_UNSUPPORTED;  // work ids are 32-bit in this order
        plan->nwork = static_cast<uint64_t>(items);
        plan->per_b = make_div32(static_cast<uint32_t>(grp_rows));
    }
    plan->wide = plan->nwork > UINT32_MAX;
    if (!plan->wide && !plan->skew)
        plan->per_b = make_div32(static_cast<uint32_t>(subs_m * subs_n));
    if (!plan->wide) {
        plan->by_m = make_div32(plan->subs_m);
        plan->by_n = make_div32(plan->subs_n);
    }
    plan->grid = cap_grid(static_cast<int64_t>(std::min<uint64_t>(plan->nwork, INT64_MAX)));
    plan->x = x;
    plan->y = y;
    plan->ldx = ldx;
    plan->ldy = ldy;
    plan->bsx = bsx;
    plan->bsy = bsy;
    plan->B = B;
    plan->M = M;
    plan->N = N;
    return TM_OK;
}

}  // namespace tmp
