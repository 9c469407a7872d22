// plan_check.cpp -- host checks of libtilemap's planner (edge_masking_vector_amd/csrc/plan.cpp),
// built with g++ under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers_cpu.py.  No GPU is involved.
//
// For every accepted call over a grid of shapes, strides, base offsets, tiles and paths, the
// device-side index mapping that the kernels apply to a plan is replayed here, and the test
// requires that it covers the tensor exactly:
//  * maps: every element (i, j) of the M x N view is moved by exactly one (work item, thread,
//    chunk), and on the aligned path (no masks) every chunk lies wholly inside the view;
//  * transpose: every staged sub-tile of every batch is visited by exactly one work item, with the
//    work-item number split by the plan's multiply-high divisors (checked against plain division).
// Row and column reduction plans are checked for their documented invariants, and the split row
// walk's segments and chunks are replayed.
//
// The replay restates the mapping the kernels document (map.hip: work item -> tile row pm, row
// strip, tile group gi, tile groups fastest; chunk q -> row q >> log_gv, tile (q & gv_mask) >>
// log_vr, chunk q & vr_mask.  transpose.hip: work item -> batch, then diagonal order pm = rest %
// subs_m, pn = (rest / subs_m + pm) % subs_n).  Exit status 0 when every check passes.
#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../edge_masking_vector_amd/csrc/plan.h"

static long g_checked = 0, g_failed = 0, g_flat = 0, g_rows = 0, g_skew = 0, g_dead_items = 0, g_pbig = 0;

#define CHECK(cond, ...)                                   \
    do {                                                   \
        if (!(cond)) {                                     \
            if (g_failed++ < 20) {                         \
                std::fprintf(stderr, "FAIL %s: ", #cond);  \
                std::fprintf(stderr, __VA_ARGS__);         \
                std::fprintf(stderr, "\n");                \
            }                                              \
        }                                                  \
    } while (0)

static const float *fake(uintptr_t addr) { return reinterpret_cast<const float *>(addr); }

static uint32_t umulhi_div(uint32_t a, const tmp::Div32 &d) {
    if (d.d == 1)
        return a;
    return static_cast<uint32_t>((static_cast<unsigned __int128>(d.c) * a) >> 64);
}
static uint32_t umulhi_mod(uint32_t a, const tmp::Div32 &d) {
    if (d.d == 1)
        return 0;
    const uint64_t low = d.c * a;
    return static_cast<uint32_t>((static_cast<unsigned __int128>(low) * d.d) >> 64);
}

// ---- maps --------------------------------------------------------------------------------------
// The replay walks the plan's own view (a contiguous caller view may be planned as one flat row)
// and counts the stores per output address; every element of the caller's view must be stored
// exactly once and no other address (row padding) at all.
// A flat plan (mapflat.hip): item w < nwhole moves elements [256 w, 256 w + 256) of the one
// contiguous row; item nwhole (when the last item is ragged) moves its first `tail` elements.  The
// workgroup's threads cover an item exactly: 64 x one 16-byte chunk, 64 x four 4-byte elements at
// a stride of 64, or 256 x one element.
static void replay_flat(const tmp::MapPlan &p, int64_t M, int64_t N, int64_t ld, const char *tag) {
    CHECK(p.M == 1 && p.stream && p.op != tmp::kChannel && p.access != tmp::kVec4Understated,
          "%s flat plan outside its case", tag);
    CHECK(p.M * p.N == M * N && (M == 1 || ld == N), "%s flat plan over a view that is not one row", tag);
    CHECK(p.grid >= 1 && p.grid <= p.nwork, "%s grid %u nwork %u", tag, p.grid, p.nwork);
    CHECK(p.flat_last >= 1 && p.flat_last <= 256, "%s last item of %u elements", tag, p.flat_last);
    const uint32_t nwhole = p.flat_last == 256 ? p.nwork : p.nwork - 1;
    const uint32_t tail = p.flat_last == 256 ? 0 : p.flat_last;
    const int threads = p.access == tmp::kScalar1 ? 256 : 64;
    const int per = p.access == tmp::kVec4 ? 1 : p.access == tmp::kScalar ? 4 : 1;
    const int W = p.access == tmp::kVec4 ? 4 : 1;
    std::vector<uint8_t> hits(size_t(M * N), 0);
    for (uint32_t w = 0; w < p.nwork; ++w) {
        const int64_t base = int64_t(w) * 256;
        for (int t = 0; t < threads; ++t)
            for (int u = 0; u < per; ++u) {
                // element of the item this (thread, slot) moves first, then W consecutive ones
                const int64_t e0 = p.access == tmp::kVec4 ? 4 * t : t + 64 * u;
                for (int e = 0; e < W; ++e) {
                    const int64_t el = e0 + e;
                    CHECK(el < 256, "%s element %ld beyond the item", tag, long(el));
                    const bool live = w < nwhole || el < int64_t(tail);
                    if (live) {
                        CHECK(base + el < M * N, "%s element %ld past the row", tag, long(base + el));
                        if (base + el < M * N)
                            ++hits[size_t(base + el)];
                    }
                }
            }
    }
    for (int64_t a = 0; a < M * N; ++a)
        if (hits[size_t(a)] != 1) {
            CHECK(false, "%s flat element %ld stored %d times", tag, long(a), int(hits[size_t(a)]));
            break;
        }
    ++g_checked;
    ++g_flat;
}

// Padded rows in one span (mapflat.hip, map_rows): item w, lane t moves the 16-byte chunk of span
// elements q .. q + 3, q = 256 w + 4 t - head; element f is row f / ld, column f % ld, live when the
// column is below N.  With a line or more of padding a chunk wholly inside it loads the row's last
// live chunk; loads are clamped to the chunks holding the span's first and last elements.  Every
// load must be a 16-byte aligned block of x inside a 128-byte line that holds a live element (so
// no line of padding alone is fetched, and no load leaves the view's lines); every live
// element must be stored exactly once and nothing else at all; whole-chunk stores must be aligned
// blocks inside the item's 1 KiB block of y, and for the channel op a whole chunk's channels are
// its columns c .. c + 3 (16-byte vector loads only when c is divisible by 4).
static void replay_rows(const tmp::MapPlan &p, int64_t M, int64_t N, int64_t ldx_, int64_t ldy_, const char *tag) {
    const int64_t ldx = ldx_, ldy = ldy_, ld = ldy, pad = ldy - N, dld = ldx - ldy;
    const bool diff = dld != 0;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(p.x), ya = reinterpret_cast<uintptr_t>(p.y);
    // padding: under a line, an eighth of the row, or (y's rows off the line grid) a quarter of
    // rows of 2048 floats or more on the 16-byte grid, a quarter or (2048 floats or more) half off it
    const bool y_lines = ya % 128 == 0 && ldy % 32 == 0, y16 = ya % 16 == 0 && ldy % 4 == 0;
    const bool wide_ok = !y_lines && (y16 ? N >= tmp::kRowsWideMinN && pad * 4 <= N
                                          : pad * 4 <= N || (N >= tmp::kRowsWideMinN && pad * 2 <= N));
    // x at another 4-byte phase than y: bases not a multiple of 16 bytes apart, or strides not a
    // multiple of 4 floats apart (then x's chunks are 4-byte aligned 16-byte loads)
    const bool shift = (xa - ya) % 16 != 0 || dld % 4 != 0;
    const bool one_row = M == 1 && ldx == N && ldy == N && p.op != tmp::kChannel &&
                         (shift || xa % 128 != 0 || ya % 128 != 0);
    const bool padded = M > 1 && pad >= 0 && (diff || pad > 0) && (pad < 32 || pad * 8 <= N || wide_ok) &&
                        (!diff || N >= tmp::kRowsDiffMinN || p.access != tmp::kVec4);
    CHECK(!p.aligned && p.ldx == ldx && p.ldy == ldy && (padded || one_row) && N >= tmp::kRowsSpanMinN &&
              p.shift == shift && (p.access == tmp::kVec4 || p.access == tmp::kScalar),
          "%s span plan outside its case", tag);
    const int64_t span = (M - 1) * ld + N, xspan = (M - 1) * ldx + N;
    CHECK(p.span == uint64_t(span) && p.head == (ya / 4) % 256 && p.ld_div.d == ld, "%s span geometry", tag);
    CHECK(p.nwork == uint64_t((p.head + span + 255) / 256) && p.grid >= 1 && p.grid <= p.nwork, "%s span items", tag);
    CHECK(!p.cvec16 || (p.op == tmp::kChannel && ya % 16 == 0 && ld % 4 == 0), "%s span channel vectors", tag);
    const int32_t q_first = -int32_t(p.head & 3u);
    const int32_t q_last = int32_t(span - 1) - int32_t((span - 1 + p.head) & 3u);
    CHECK(p.x_last == int32_t(q_last + (M - 1) * dld), "%s span x_last", tag);
    const bool wide = pad >= 32 || diff || shift;  // the kernels that redirect chunks wholly inside the padding
    auto in_x = [&](int64_t xi) { return xi >= 0 && xi < xspan; };
    std::vector<uint8_t> hits(size_t(span), 0);
    bool bad_load = false, bad_store = false, bad_source = false;
    // a 16-byte block of x at float index xi: aligned, and inside a line that holds a live element
    auto live_line = [&](int64_t xi) {
        if ((xa + 4 * xi) % 16 != 0)
            return false;
        const int64_t line = int64_t((xa + 4 * xi) / 128 * 128);
        for (int e = 0; e < 32; ++e) {
            const int64_t g = (line - int64_t(xa)) / 4 + e;  // x float index
            if (g >= 0 && g < (M - 1) * ldx + N && g % ldx < N)
                return true;
        }
        return false;
    };
    for (uint32_t w = 0; w < p.nwork; ++w) {
        if (wide) {
            // the wave exits when none of its chunks holds an element of a row or the next
            bool some = false;
            for (int t = 0; t < 64; ++t) {
                const int32_t q = int32_t(w * 256u + 4u * t) - int32_t(p.head);
                const uint32_t c = q > 0 ? uint32_t(q % ld) : 0u;
                some = some || (q + 3 >= 0 && q < span && (q < 0 || c < N || c + 3 >= ld));
            }
            if (!some) {
                ++g_dead_items;
                continue;
            }
        }
        for (int t = 0; t < 64; ++t) {
            const int32_t q = int32_t(w * 256u + 4u * t) - int32_t(p.head);
            uint32_t r = 0, c = 0;
            if (q > 0) {
                r = uint32_t(q / ld);
                c = uint32_t(q % ld);
                if (!diff && !shift && umulhi_mod(uint32_t(q), p.ld_div) != c)
                    bad_load = true;
                if ((diff || shift) && umulhi_div(uint32_t(q), p.ld_div) != r)
                    bad_load = true;
            }
            int64_t xa0 = q < q_first ? q_first : (q > q_last ? q_last : q), xb0 = xa0;
            if (wide) {
                int32_t qa = q;
                if (q >= 0 && c >= N && c + 3 < ld) {
                    const int32_t last = q - int32_t(c) + int32_t(N) - 1;
                    qa = last - int32_t((uint32_t(last) + p.head) & 3u);
                }
                xa0 = diff ? int64_t(qa) + int64_t(r) * dld : qa;
                if (!shift)
                    xa0 = q < q_first ? q_first : (q > q_last ? (diff ? p.x_last : q_last) : xa0);
                xb0 = xa0;
                if (diff || shift) {
                    const bool cross = q >= 0 && c + 3 >= ld && int64_t(q) - c + ld < span;
                    xb0 = cross ? xa0 + dld : xa0;
                    if (cross && c >= N)
                        xa0 = xb0;  // no element of the chunk is live in its own row
                }
            }
            // the span's end chunks of a shifted plan load their live elements one by one
            const bool edge = shift && !(q >= 0 && int64_t(q) + 3 < span);
            if (shift) {
                // every float of every 16-byte load inside x's view
                if (!edge)
                    for (int k = 0; k < 4; ++k)
                        if (!in_x(xa0 + k) || !in_x(xb0 + k))
                            bad_load = true;
            } else if (!live_line(xa0) || (diff && !live_line(xb0))) {
                bad_load = true;
            }
            const bool whole = q >= 0 && int64_t(q) + 3 < span && c + 3 < N;
            if (whole) {
                const uintptr_t blk = ya + 4 * (int64_t(w) * 256 - p.head);
                if (blk % 1024 != 0 || (ya + 4 * int64_t(q)) != blk + 16 * uintptr_t(t))
                    bad_store = true;
                if (p.cvec16 && c % 4 != 0)
                    bad_store = true;  // a 16-byte channel-vector load off its grid
            }
            for (int i = 0; i < 4; ++i) {
                const int32_t f = q + i;
                const uint32_t ci = q >= 0 ? c + i : uint32_t(f);
                const bool next = q >= 0 && ci >= ld;
                const uint32_t col = next ? ci - uint32_t(ld) : ci;
                if (f >= 0 && f < span && col < N) {
                    if (col != uint32_t(f % ld))
                        bad_store = true;
                    // the x element this output takes: row f / ldy, same column
                    const int64_t row = q >= 0 ? int64_t(r) + (next ? 1 : 0) : 0;
                    const int64_t src = edge ? f + row * dld : (next && diff ? xb0 : xa0) + i;
                    if (src != int64_t(f / ld) * ldx + col || !in_x(src))
                        bad_source = true;
                    ++hits[size_t(f)];
                }
            }
        }
    }
    CHECK(!bad_load, "%s span: a load off x's live lines (or a wrong row or column)", tag);
    CHECK(!bad_store, "%s span: a misplaced store", tag);
    CHECK(!bad_source, "%s span: an output element taken from the wrong x element", tag);
    for (int64_t f = 0; f < span; ++f) {
        const bool live = f % ld < N;
        if (hits[size_t(f)] != (live ? 1 : 0)) {
            CHECK(false, "%s span element %ld (live %d) stored %d times", tag, long(f), int(live), int(hits[size_t(f)]));
            break;
        }
    }
    ++g_checked;
    ++g_rows;
}

static void replay_map(const tmp::MapPlan &p, int64_t M, int64_t N, int64_t ld, uintptr_t xbase,
                       const char *tag) {
    if (p.flat) {
        replay_flat(p, M, N, ld, tag);
        return;
    }
    if (p.rows) {
        replay_rows(p, p.M, p.N, p.ldx, p.ldy, tag);  // the plan's view (contiguous rows: one row)
        return;
    }
    const int W = p.access == tmp::kScalar || p.access == tmp::kScalar1 ? 1 : 4;
    const int U = p.access == tmp::kScalar ? tmp::kScalarChunksPerThread : 1;
    const uint32_t bs = 1u << p.log_bs;
    const uint32_t chunks = 1u << (p.log_r + p.log_gv);
    const uint32_t vr_mask = (1u << p.log_vr) - 1u, gv_mask = (1u << p.log_gv) - 1u;
    const uint32_t strip_mask = (1u << p.log_strips) - 1u;
    const int64_t tm = int64_t(1) << p.log_tm, tn = int64_t(1) << p.log_tn;
    const int64_t PM = p.M, PN = p.N, pld = p.ldy;
    CHECK(p.grid >= 1 && p.grid <= p.nwork, "%s grid %u nwork %u", tag, p.grid, p.nwork);
    CHECK(bs >= 64 && bs <= 1024, "%s block %u", tag, bs);
    CHECK(uint64_t(bs) * U >= chunks, "%s block %u x %d < chunks %u", tag, bs, U, chunks);
    CHECK(p.guard == (uint64_t(bs) * U > chunks), "%s guard flag", tag);
    CHECK(tn * p.group * p.groups_n >= PN, "%s tile groups do not reach column N", tag);
    CHECK(PM * PN == M * N && (PM == M || (PM == 1 && ld == N && p.ldx == PN && pld == PN)),
          "%s planned view %ldx%ld is not the caller's or its flat row", tag, long(PM), long(PN));
    if (p.aligned) {
        CHECK(xbase % 16 == 0 && (PM <= 1 || p.ldx % 4 == 0) || W == 1, "%s 16-byte chunks off", tag);
    }
    if (p.stream) {
        CHECK(p.access != tmp::kVec4Understated && !p.guard && (int64_t(W) * chunks * 4 == tmp::kStreamSegmentBytes),
              "%s stream item is not one wave over 1 KiB", tag);
        CHECK(p.log_r == 0 || pld == PN, "%s stream item over rows that are not contiguous", tag);
    }
    // Channel op: a flat view carries C (the caller's N) and the device finds each element's
    // channel as (chan_base + col - col0) mod C, then steps it with a wrap at C.
    CHECK(p.chan_n == ((p.op == tmp::kChannel && PM != M) ? uint32_t(N) : 0u), "%s channel count %u", tag,
          p.chan_n);
    long chan_bad = 0;
    auto check_chan = [&](uint32_t gi, int64_t col0, int64_t col) {
        if (p.chan_n == 0)
            return;
        const uint64_t prod = uint64_t(umulhi_mod(gi, p.chan)) * p.chan_step;
        const uint64_t arg = uint64_t(umulhi_mod(uint32_t(prod), p.chan)) + uint64_t(col - col0);
        uint32_t c = umulhi_mod(uint32_t(arg), p.chan);
        if (prod > 0xFFFFFFFFull || arg > 0xFFFFFFFFull)
            ++chan_bad;
        for (int e = 0; e < W && col + e < PN; ++e) {
            if (c != uint32_t((col + e) % int64_t(p.chan_n)))
                ++chan_bad;
            c = c + 1 == p.chan_n ? 0 : c + 1;
        }
    };
    const int64_t span = (M - 1) * ld + N;  // addresses of the caller's view, in elements
    std::vector<uint8_t> hits(size_t(span), 0);
    for (uint32_t w = 0; w < p.nwork; ++w) {
        const uint32_t gi = w % p.groups_n, ps = w / p.groups_n;
        const uint32_t strip = ps & strip_mask, pm = ps >> p.log_strips;
        const int64_t row0 = (int64_t(pm) << p.log_tm) + (int64_t(strip) << p.log_r);
        const int64_t col0 = int64_t(gi) * p.group * tn;
        const bool item_whole = p.aligned || ((int64_t(pm) + 1) * tm <= PM && col0 + int64_t(p.group) * tn <= PN);
        for (uint32_t t = 0; t < bs; ++t) {
            for (int u = 0; u < U; ++u) {
                const uint32_t q = t + (uint32_t(u) << p.log_bs);
                if (q >= chunks)
                    continue;  // guarded lanes (or beyond the item) do nothing
                const uint32_t pn = gi * p.group + ((q & gv_mask) >> p.log_vr);
                const int64_t tile_col = col0 + int64_t((q & gv_mask) >> p.log_vr) * tn;
                const int64_t col = tile_col + int64_t(q & vr_mask) * W;
                const int64_t row = row0 + int64_t(q >> p.log_gv);
                if (item_whole) {
                    // unmasked body: the whole chunk moves
                    CHECK(row < PM && col + W <= PN, "%s unmasked chunk outside (%ld, %ld)", tag,
                          (long)row, (long)col);
                    if (p.stream) {
                        // the buffer store lands at byte 4 W q of the item's block
                        const int64_t a0 = row0 * pld + col0;
                        CHECK(row * pld + col == a0 + int64_t(q) * W, "%s stream chunk %u off its block", tag, q);
                    }
                    for (int e = 0; e < W; ++e)
                        if (row < PM && col + e < PN && row * pld + col + e < span)
                            ++hits[size_t(row * pld + col + e)];
                    check_chan(gi, col0, col);
                } else {
                    if (!(pn < p.tiles_n && row < PM && PN - col > 0))
                        continue;  // masked: nothing read or stored
                    check_chan(gi, col0, col);
                    for (int e = 0; e < W && col + e < PN; ++e)
                        if (row * pld + col + e < span)
                            ++hits[size_t(row * pld + col + e)];
                }
            }
        }
    }
    CHECK(chan_bad == 0, "%s %ld channel indices wrong", tag, chan_bad);
    for (int64_t a = 0; a < span; ++a) {
        const bool inside = ld == 0 || a % ld < N;
        if (hits[size_t(a)] != (inside ? 1 : 0)) {
            CHECK(false, "%s address %ld (element %ld, %ld) stored %d times", tag, long(a),
                  long(ld ? a / ld : 0), long(ld ? a % ld : a), int(hits[size_t(a)]));
            break;
        }
    }
    ++g_checked;
}

// Different row strides in x and y (the span's DIFF form when they differ by a multiple of 4 and
// the bases sit the same distance past a 16-byte boundary; the 2-D plan otherwise).
static void check_maps_diff() {
    long spans = 0;
    for (int64_t M : {int64_t{2}, int64_t{3}, int64_t{17}, int64_t{100}})
        for (int64_t N : {int64_t{1000}, int64_t{1024}, int64_t{1029}, int64_t{2000}})
            for (int dx : {0, 1, 4, 8, 40, 200})
                for (int dy : {0, 3, 4, 8, 31, 40})
                    for (uintptr_t xoff : {uintptr_t{0}, uintptr_t{4}, uintptr_t{12}})
                        for (uintptr_t yoff : {uintptr_t{0}, uintptr_t{4}})
                            for (int op : {int(tmp::kAffine), int(tmp::kChannel)})
                                for (int variant : {TM_VAR_AUTO, TM_VAR_VEC4}) {
                                    const int64_t ldx = N + dx, ldy = N + dy;
                                    if (ldx == ldy)
                                        continue;
                                    tmp::MapPlan p;
                                    const uintptr_t xb = 0x100000 + xoff, yb = 0x40000000 + yoff;
                                    const int st = tmp::plan_map(op, fake(xb), ldx, const_cast<float *>(fake(yb)), ldy, M, N,
                                                                 1.5f, 0.f, 64, 64, 0, variant, &p, nullptr, fake(0x200000));
                                    if (st != TM_OK || !p.launch)
                                        continue;
                                    char tag[160];
                                    std::snprintf(tag, sizeof tag, "map diff M=%ld N=%ld ldx=%ld ldy=%ld offs=%lu,%lu op=%d var=%d",
                                                  long(M), long(N), long(ldx), long(ldy), (unsigned long)xoff,
                                                  (unsigned long)yoff, op, variant);
                                    CHECK(!p.rows || N >= tmp::kRowsDiffMinN || p.access != tmp::kVec4,
                                          "%s: a span of 16-byte rows under the width minimum", tag);
                                    spans += p.rows;
                                    replay_map(p, M, N, ldy, xb, tag);
                                }
    CHECK(spans >= 500, "only %ld different-stride span plans", spans);
}

// Wide padding off the line grid: spans whose items lie wholly inside the padding (the waves that
// exit at once), rows on and off the 16-byte grid, on both sides of each width and padding limit.
static void check_maps_wide() {
    long spans = 0, tiles = 0;
    for (int64_t M : {int64_t{2}, int64_t{3}, int64_t{9}})
        for (int64_t N : {int64_t{1000}, int64_t{2047}, int64_t{2048}, int64_t{2500}, int64_t{4100}})
            for (int64_t pad : {N / 8 + 4, N / 4, N / 4 + 1, N / 4 + 2, N / 2 - 1, N / 2, N / 2 + 1, N / 2 + 3})
                for (int dx : {0, 4, -4})
                    for (uintptr_t off : {uintptr_t{0}, uintptr_t{4}, uintptr_t{8}, uintptr_t{64}})
                        for (int op : {int(tmp::kAffine), int(tmp::kChannel)}) {
                            const int64_t ldy = N + pad, ldx = std::max(N, ldy + dx);
                            tmp::MapPlan p;
                            const uintptr_t xb = 0x100000 + off, yb = 0x40000000 + off;
                            const int st = tmp::plan_map(op, fake(xb), ldx, const_cast<float *>(fake(yb)), ldy, M, N, 1.5f,
                                                         0.f, 64, 64, 0, TM_VAR_AUTO, &p, nullptr, fake(0x200000));
                            if (st != TM_OK || !p.launch)
                                continue;
                            char tag[160];
                            std::snprintf(tag, sizeof tag, "map wide M=%ld N=%ld ldx=%ld ldy=%ld off=%lu op=%d", long(M),
                                          long(N), long(ldx), long(ldy), (unsigned long)off, op);
                            spans += p.rows;
                            tiles += !p.rows && !p.flat;
                            replay_map(p, M, N, ldy, xb, tag);
                        }
    CHECK(spans >= 200 && tiles >= 200, "wide padding: %ld span and %ld tile plans", spans, tiles);
    CHECK(g_dead_items > 0, "no span wave wholly inside the padding was replayed");
}

static void check_maps() {
    const int64_t Ms[] = {0, 1, 3, 17, 64, 100, 1000};
    const int64_t Ns[] = {0, 1, 4, 17, 64, 129, 1000};
    const int TMs[] = {1, 4, 32, 256};
    const int TNs[] = {1, 4, 16, 128, 1024};
    const uintptr_t bases[] = {0x100000, 0x100004, 0x100010};  // line-aligned, 4-byte, 16-byte
    for (int64_t M : Ms)
        for (int64_t N : Ns) {
            const int64_t lds[] = {N, N + 3, (N + 3) / 4 * 4, (N + 31) / 32 * 32, N + 40, N + N / 8, N + N / 8 + 1};
            for (int64_t ld : lds)
                for (int TM : TMs)
                    for (int TN : TNs)
                        for (int aligned = 0; aligned <= 1; ++aligned)
                            for (int variant = 0; variant <= 3; ++variant)
                                for (uintptr_t base : bases)
                                    for (int op : {int(tmp::kScale), int(tmp::kChannel)}) {
                                        tmp::MapPlan p;
                                        const uintptr_t ybase = base + 0x40000000;
                                        const int st = tmp::plan_map(
                                            op, fake(base), ld, const_cast<float *>(fake(ybase)), ld,
                                            M, N, 1.5f, 0.f, TM, TN, aligned, variant, &p, nullptr,
                                            fake(0x200000));
                                        if (st != TM_OK || !p.launch)
                                            continue;
                                        char tag[160];
                                        std::snprintf(tag, sizeof tag,
                                                      "map M=%ld N=%ld ld=%ld TM=%d TN=%d al=%d var=%d base=%#lx op=%d",
                                                      long(M), long(N), long(ld), TM, TN, aligned, variant,
                                                      (unsigned long)base, op);
                                        replay_map(p, M, N, ld, base, tag);
                                    }
        }
}

// ---- transpose --------------------------------------------------------------------------------
static void replay_transpose(const tmp::TransposePlan &p, int64_t B, int64_t M, int64_t N, const char *tag) {
    CHECK(!p.wide, "%s small job planned as wide", tag);
    CHECK(p.subs_m == uint32_t((M + (p.skew ? tmp::kTrSub - 1 : 0) + p.sm - 1) / p.sm) &&
              p.subs_n == uint32_t((N + p.sn - 1) / p.sn),
          "%s sub-tile counts", tag);
    CHECK((p.log_g > 0 || p.skew || p.nwork == uint64_t(B) * p.subs_m * p.subs_n) && p.grid >= 1 &&
              p.grid <= p.nwork,
          "%s work", tag);
    // the instance's capacity: kTrSubElems, or twice that for the 64 x 32 sub-tiles of views whose
    // y rows are off the 16-byte grid (and for the line-aligned windows of one matrix)
    CHECK(p.sub == tmp::kTrSubElems || (p.sub == 2 * tmp::kTrSubElems && (!p.vy || p.skew) && p.log_g == 0 &&
                                        p.packed == 0 && p.sm == 2 * tmp::kTrSub && p.sn == tmp::kTrSub),
          "%s instance of %d elements", tag, p.sub);
    if (p.skew) {
        // transpose_skew: group order (G = 2^log_grp vertically adjacent items): item w -> group
        // 8 (w / 8G) + w mod 8, member (w / 8) mod G; pm = G (group mod group_rows) + member, pn =
        // group / group_rows; items past subs_m x subs_n do nothing.  Item (pm, pn) writes, in y row
        // 32 pn + j (j < 32), the 64 elements from the line boundary at or before y column 64 pm,
        // those inside [0, M); it reads band rows 64 pm - 32 .. 64 pm + 63 of
        // x clamped into [0, M).  Every element of y must be written exactly once, by the item whose
        // band holds its x row, and 16-byte stores must be aligned.
        const uint32_t G = 1u << p.log_grp;
        CHECK(B >= 1 && !p.wide && p.log_g == 0 && p.packed == 0 && p.log_grp >= 0 && p.log_grp <= 4 &&
                  p.nwork % (8 * G) == 0 && p.grid % (8 * G) == 0 && p.sm == 64 && p.sn == 32,
              "%s skew plan", tag);
        const uint32_t grp_rows = (p.subs_m + G - 1) / G;
        CHECK(p.per_b.d == grp_rows, "%s group divisor", tag);
        {
            // 16-byte x reads: chunk c of a band row reads columns col0 + 4c .. + 3, and the chunks
            // at or past the one holding the last live column read the 16 bytes that end at it;
            // every read lies inside the row, and every live column is staged by its own chunk or
            // by the clamped one
            const uintptr_t xa = reinterpret_cast<uintptr_t>(p.x);
            const bool x16 = xa % 16 == 0 && (M <= 1 || p.ldx % 4 == 0) && (B <= 1 || p.bsx % 4 == 0);
            CHECK(p.vx == (x16 || N >= tmp::kTrSub) && N >= tmp::kTrWindowMinN, "%s skew: x chunk width", tag);
            bool bad_read = false;
            for (uint32_t pn = 0; pn < p.subs_n; ++pn) {
                const int64_t col0 = int64_t(pn) * 32;
                const int cols_live = int(std::min<int64_t>(N - col0, 32));
                const int clast = (cols_live - 1) / 4, cend = cols_live - 4;
                std::vector<int> staged(32, 0);
                for (int c = 0; c < 8 && p.vx; ++c) {
                    const int cs = c < clast ? 4 * c : cend;
                    if (col0 + cs < 0 || col0 + cs + 4 > N)
                        bad_read = true;
                    for (int i = 0; i < 4; ++i)
                        if (cs + i >= 0 && cs + i < 32)
                            ++staged[size_t(cs + i)];
                }
                for (int j = 0; j < cols_live && p.vx; ++j)
                    if (staged[size_t(j)] == 0)
                        bad_read = true;
            }
            CHECK(!bad_read, "%s skew: a 16-byte read outside its row, or a live column not staged", tag);
        }
        const uintptr_t ya = reinterpret_cast<uintptr_t>(p.y);
        std::vector<uint8_t> hits(size_t(B) * size_t(N) * M, 0);
        bool bad = false;
        CHECK(p.nwork >= uint64_t(grp_rows) * p.subs_n * uint64_t(B) * G, "%s skew: too few items", tag);
        for (uint64_t w = 0; w < p.nwork; ++w) {
            const uint32_t w32 = uint32_t(w);
            const uint32_t grp = (w32 >> (3 + p.log_grp)) * 8 + (w32 & 7u), member = (w32 >> 3) & (G - 1);
            const uint32_t q = umulhi_div(grp, p.per_b);
            // the group's column strip runs over all batches: batch q / subs_n, strip q mod subs_n
            const uint32_t b = umulhi_div(q, p.by_n);
            const uint64_t pm = uint64_t(grp - q * p.per_b.d) * G + member, pn = q - b * p.subs_n;
            CHECK(q == grp / grp_rows && b == q / p.subs_n, "%s group division", tag);
            if (pm >= p.subs_m || int64_t(b) >= B)
                continue;
            const int64_t row0 = int64_t(pm) * 64, col0 = int64_t(pn) * 32;
            const int cols_live = int(std::min<int64_t>(N - col0, 32));
            for (int j = 0; j < cols_live; ++j) {
                const uintptr_t yr = ya + 4 * uintptr_t(int64_t(b) * p.bsy + (col0 + j) * p.ldy);
                const int sft = int(((yr + 4 * uintptr_t(row0)) >> 2) & 31u);
                for (int c = 0; c < 16; ++c) {
                    const int64_t i0 = row0 - sft + 4 * c;
                    const int br = 32 - sft + 4 * c;
                    if (br < 0 || br + 3 >= 96)
                        bad = true;  // outside the staged band
                    if (i0 >= 0 && i0 + 4 <= M && (yr + 4 * uintptr_t(i0)) % 16 != 0)
                        bad = true;  // a misaligned 16-byte store
                    for (int e = 0; e < 4; ++e) {
                        const int64_t i = i0 + e;
                        if (i >= 0 && i < M) {
                            if (i - (row0 - 32) != br + e)
                                bad = true;  // the band row is not this x row
                            ++hits[(size_t(b) * size_t(N) + size_t(col0 + j)) * M + i];
                        }
                    }
                }
            }
        }
        CHECK(!bad, "%s skew: a window outside the band or a misaligned store", tag);
        ++g_skew;
        for (size_t k = 0; k < hits.size(); ++k)
            if (hits[k] != 1) {
                CHECK(false, "%s skew: y element %zu written %d times", tag, k, int(hits[k]));
                break;
            }
        ++g_checked;
        return;
    }
    if (p.pbig) {
        // packed side of 32 to kTrPackBigC channels: items of S positions x C channels, S the
        // largest power of two with S C <= kTrPackBigElems, at least 32 (so each item's packed
        // block ends on a 128-byte line); 16-byte chunks on both sides; the LDS holds C rows of S + 1
        const bool m0 = p.packed == 1;
        const int64_t C = m0 ? M : N, S = m0 ? p.sn : p.sm, P = m0 ? N : M;
        CHECK((p.packed == 1 || p.packed == 2) && !p.aligned && !p.skew && p.log_g == 0 && p.pvec && p.flat16,
              "%s large packed mode", tag);
        CHECK(C >= tmp::kTrSub && C <= tmp::kTrPackBigC && (m0 ? p.ldy == M : p.ldx == N) && P >= 2 * tmp::kTrSub,
              "%s large packed shape", tag);
        CHECK((S & (S - 1)) == 0 && S >= 32 && S * C <= tmp::kTrPackBigElems && 2 * S * C > tmp::kTrPackBigElems &&
                  C * (S + 1) <= tmp::kTrPackBigElems + 2 * tmp::kTrPackBigC && (S * C * 4) % 128 == 0,
              "%s large packed item of %ld x %ld", tag, long(S), long(C));
        const uint32_t subs = uint32_t((P + S - 1) / S);
        CHECK((m0 ? (p.subs_m == 1 && p.subs_n == subs) : (p.subs_n == 1 && p.subs_m == subs)) &&
                  p.nwork == uint64_t(B) * subs,
              "%s large packed work", tag);
        ++g_checked;
        ++g_pbig;
        return;
    }
    CHECK((p.sm & (p.sm - 1)) == 0 && (p.sn & (p.sn - 1)) == 0 && int64_t(p.sm) * p.sn <= p.sub,
          "%s sub-tile %dx%d above %d elements", tag, p.sm, p.sn, p.sub);
    // the staged sub-tile (rows of stride SN + 1 floats) fits the instance's LDS of 2 * sub floats
    CHECK(int64_t(p.sm) * (p.sn + 1) <= 2 * p.sub, "%s staged sub-tile exceeds LDS", tag);
    // a narrow extent gets a narrow sub-tile (no sub-tile row or column is wholly outside the view,
    // beyond the minimum of 4 that 16-byte chunks need)
    auto p2 = [](int64_t v) { int64_t e = 1; while (e < v) e <<= 1; return e; };
    if (!p.aligned) {
        CHECK(p.sm <= std::max<int64_t>(p.vy ? 4 : 1, p2(M)) && p.sn <= std::max<int64_t>(p.vx ? 4 : 1, p2(N)),
              "%s sub-tile %dx%d wider than the view", tag, p.sm, p.sn);
        if (M >= tmp::kTrSub && N >= tmp::kTrSub) {
            // 32 x 32, or 64 x 32 for large views whose y rows are off the 16-byte grid (or, one
            // matrix, off the line grid)
            const bool tall = (!p.vy || p.skew) && M >= 2 * tmp::kTrSub && M * N >= (int64_t{1} << 22);
            CHECK(tall ? (p.sm == 2 * tmp::kTrSub && p.sn == tmp::kTrSub && p.sub == 2 * tmp::kTrSubElems)
                       : (p.sm == tmp::kTrSub && p.sn == tmp::kTrSub),
                  "%s wide view on %dx%d sub-tiles", tag, p.sm, p.sn);
        }
    }
    if (p.aligned)
        CHECK(M % p.sm == 0 && N % p.sn == 0, "%s promised sub-tiles are not whole", tag);
    CHECK(!p.vec || (p.vx && p.vy), "%s vec flag", tag);
    {
        // x read in 16-byte chunks: rows on the 16-byte grid, or rows of a whole sub-tile row
        const uintptr_t xa = reinterpret_cast<uintptr_t>(p.x);
        const bool x16 = xa % 16 == 0 && (M <= 1 || p.ldx % 4 == 0) && (B <= 1 || p.bsx % 4 == 0);
        CHECK(p.vx == (x16 || N >= tmp::kTrSub), "%s x chunk width", tag);
    }
    if (p.vx)
        CHECK(p.sn >= 4, "%s 16-byte reads need sub-tile rows of 4+", tag);
    if (p.vy)
        CHECK(p.sm >= 4, "%s 16-byte writes need sub-tile columns of 4+", tag);
    if (p.packed != 0) {
        // few channels with a packed side: C = the narrow extent, S positions per work item
        const bool m0 = p.packed == 1;
        const int64_t C = m0 ? M : N, S = m0 ? p.sn : p.sm;
        int64_t c2 = 1;
        while (c2 < C)
            c2 <<= 1;
        CHECK(!p.vec && p.log_g == 0 && C < tmp::kTrSub && (m0 ? M : N) == C, "%s packed mode", tag);
        CHECK(m0 ? (p.ldy == M && p.subs_m == 1 && N >= tmp::kTrSub) : (p.ldx == N && p.subs_n == 1 && M >= tmp::kTrSub),
              "%s packed side is not one block per work item", tag);
        CHECK(S >= 32 && S * c2 <= tmp::kTrSubElems && C * (S + 1) + 2 <= 2 * tmp::kTrSubElems,
              "%s packed work item of %ld x %ld exceeds the kernel", tag, long(C), long(S));
        CHECK(p.pvec || p.flat16, "%s packed mode with nothing in 16-byte chunks", tag);
    }
    if (p.log_g > 0) {
        // packed: every matrix in one sub-tile, work item w takes batches w * G .. w * G + G - 1
        const int64_t G = int64_t{1} << p.log_g;
        CHECK(p.subs_m == 1 && p.subs_n == 1 && B > 1, "%s packed plan with several sub-tiles", tag);
        CHECK(G * p.sm * p.sn <= tmp::kTrSubElems && G * p.sm * (p.sn + 1) <= 2 * tmp::kTrSubElems,
              "%s %ld packed sub-tiles of %dx%d exceed the work item", tag, long(G), p.sm, p.sn);
        CHECK(G < 2 * B, "%s more packed batches than needed", tag);
        CHECK(p.nwork == uint64_t((B + G - 1) / G), "%s packed work count", tag);
        std::vector<uint8_t> hit(size_t(B), 0);
        for (uint64_t w = 0; w < p.nwork; ++w)
            for (int64_t g = 0; g < G; ++g)
                if (int64_t(w) * G + g < B)
                    ++hit[size_t(int64_t(w) * G + g)];
        bool once = true;
        for (uint8_t h : hit)
            once = once && h == 1;
        CHECK(once, "%s packed batches not covered once", tag);
        ++g_checked;
        return;
    }
    CHECK(!(p.subs_m == 1 && p.subs_n == 1 && B > 1 && int64_t(p.sm) * p.sn * 2 <= tmp::kTrSubElems),
          "%s small matrices not packed", tag);
    std::vector<uint8_t> seen(size_t(p.nwork), 0);
    for (uint64_t w = 0; w < p.nwork; ++w) {
        const uint32_t w32 = uint32_t(w);
        const uint32_t b = umulhi_div(w32, p.per_b);
        const uint32_t rest = w32 - b * p.per_b.d;
        const uint32_t q = umulhi_div(rest, p.by_m);
        const uint32_t pm = rest - q * p.by_m.d;
        const uint32_t pn = umulhi_mod(q + pm, p.by_n);
        // the same split with plain division
        const uint32_t per_b = p.subs_m * p.subs_n;
        CHECK(b == w32 / per_b && rest == w32 % per_b && pm == rest % p.subs_m &&
                  pn == (rest / p.subs_m + rest % p.subs_m) % p.subs_n,
              "%s multiply-high split of work item %u", tag, w32);
        CHECK(b < B && pm < p.subs_m && pn < p.subs_n, "%s work item %u out of range", tag, w32);
        const uint64_t slot = (uint64_t(b) * p.subs_m + pm) * p.subs_n + pn;
        if (slot < seen.size())
            ++seen[size_t(slot)];
    }
    for (size_t k = 0; k < seen.size(); ++k) {
        if (seen[k] != 1) {
            CHECK(seen[k] == 1, "%s sub-tile %zu visited %d times", tag, k, int(seen[k]));
            break;
        }
    }
    ++g_checked;
}

// Views whose y rows miss the line grid, with bases at several offsets: the line-aligned windows.
static void check_skew_transposes() {
    struct S { int64_t M, N, ldx, ldy; };
    const S cases[] = {{4096, 4096, 4096, 4100}, {4099, 4099, 4099, 4099}, {5450, 2568, 2568, 5450},
                       {2049, 2050, 2051, 2049}, {8191, 513, 515, 8191}, {4103, 2049, 2052, 4108}};
    for (const S &c : cases)
        for (uintptr_t xoff : {uintptr_t{0}, uintptr_t{4}})
            for (uintptr_t yoff : {uintptr_t{0}, uintptr_t{12}, uintptr_t{68}}) {
                tmp::TransposePlan p;
                const int st = tmp::plan_transpose(fake(0x1000000 + xoff), c.ldx, 0,
                                                   const_cast<float *>(fake(0x40000000 + yoff)), c.ldy, 0, 1, c.M,
                                                   c.N, 1, 1, 0, &p);
                char tag[128];
                std::snprintf(tag, sizeof tag, "skew transpose %ldx%ld ldx=%ld ldy=%ld xoff=%lu yoff=%lu", long(c.M),
                              long(c.N), long(c.ldx), long(c.ldy), (unsigned long)xoff, (unsigned long)yoff);
                CHECK(st == TM_OK && p.launch && p.skew, "%s not planned as line-aligned windows", tag);
                if (st == TM_OK && p.launch)
                    replay_transpose(p, 1, c.M, c.N, tag);
            }
    // batches: y rows off the line grid in some batch (the row stride, the batch stride or the base)
    struct SB { int64_t B, M, N, ldx, ldy, bsx, bsy; };
    const SB bcases[] = {{8, 200, 4096, 4096, 200, 200 * 4096, 4096 * 200},    // NCHW -> NHWC, 200 channels
                         {3, 300, 5000, 5001, 300, 300 * 5001, 5000 * 300 + 7},  // padded batch stride
                         {4, 4096, 256, 256, 4096, 4096 * 256, 256 * 4096 + 4},  // rows on lines, batches not
                         {2, 129, 20000, 20000, 129, 129 * 20000, 20000 * 129},
                         {1, 1198372, 28, 68, 1198373, 0, 0},          // few columns, long y rows off the grid
                         {1, 1398101, 24, 24, 1398102, 0, 0},
                         {1, 900000, 12, 13, 900001, 0, 0},
                         {1, 330000, 13, 13, 330004, 0, 0}};
    for (const SB &c : bcases)
        for (uintptr_t yoff : {uintptr_t{0}, uintptr_t{16}}) {
            tmp::TransposePlan p;
            const int st = tmp::plan_transpose(fake(0x1000000), c.ldx, c.bsx, const_cast<float *>(fake(0x40000000 + yoff)),
                                               c.ldy, c.bsy, c.B, c.M, c.N, 1, 1, 0, &p);
            char tag[160];
            std::snprintf(tag, sizeof tag, "batched skew transpose B=%ld %ldx%ld ldy=%ld bsy=%ld yoff=%lu", long(c.B),
                          long(c.M), long(c.N), long(c.ldy), long(c.bsy), (unsigned long)yoff);
            CHECK(st == TM_OK && p.launch && p.skew, "%s not planned as line-aligned windows", tag);
            if (st == TM_OK && p.launch)
                replay_transpose(p, c.B, c.M, c.N, tag);
        }
}

// NCHW <-> NHWC with 32 to 128 channels: the packed kernel's large items when the packed rows miss
// the line grid, the sub-tiles when they lie on it (64 channels on a line-aligned base).
static void check_packed_big() {
    struct S { int64_t B, C, P; };
    const S cases[] = {{32, 65, 3136}, {4, 33, 100}, {2, 128, 4100}, {1, 100, 5000}, {3, 127, 64}, {8, 64, 3136},
                       {2, 32, 1000}};
    for (const S &c : cases)
        for (int rev = 0; rev <= 1; ++rev)
            for (uintptr_t off : {uintptr_t{0}, uintptr_t{16}, uintptr_t{4}}) {
                const int64_t M = rev ? c.P : c.C, N = rev ? c.C : c.P;
                tmp::TransposePlan p;
                const int st = tmp::plan_transpose(fake(0x100000 + off), N, M * N, const_cast<float *>(fake(0x40000000 + off)),
                                                   M, M * N, c.B, M, N, 1, 1, 0, &p);
                if (st != TM_OK)
                    continue;
                char tag[160];
                std::snprintf(tag, sizeof tag, "packed B=%ld C=%ld P=%ld rev=%d off=%lu", long(c.B), long(c.C),
                              long(c.P), rev, (unsigned long)off);
                const bool lines = c.C % 32 == 0 && off == 0;   // packed rows on the line grid
                CHECK(p.pbig == (!lines && off % 16 == 0 && c.P >= 64), "%s: large packed items %d", tag, int(p.pbig));
                replay_transpose(p, c.B, M, N, tag);
            }
}

static void check_transposes() {
    const int64_t Bs[] = {1, 3, 32, 1000};
    const int64_t Ms[] = {1, 2, 3, 4, 24, 64, 100, 50176};
    const int64_t Ns[] = {1, 3, 5, 16, 32, 100, 3136};
    for (int64_t B : Bs)
        for (int64_t M : Ms)
            for (int64_t N : Ns)
                for (int T : {4, 32, 64})
                    for (int aligned = 0; aligned <= 1; ++aligned) {
                        if (B * M * N > 100000000)
                            continue;  // the replay visits every work item
                        tmp::TransposePlan p;
                        const int64_t ldx = (N + 3) / 4 * 4, ldy = (M + 3) / 4 * 4;
                        const int st = tmp::plan_transpose(fake(0x100000), ldx, M * ldx,
                                                           const_cast<float *>(fake(0x40000000)), ldy,
                                                           N * ldy, B, M, N, T, T, aligned, &p);
                        if (st != TM_OK || !p.launch)
                            continue;
                        char tag[128];
                        std::snprintf(tag, sizeof tag, "transpose B=%ld M=%ld N=%ld T=%d al=%d", long(B),
                                      long(M), long(N), T, aligned);
                        replay_transpose(p, B, M, N, tag);
                    }
    // packed strides (NCHW <-> NHWC with few channels: y rows of exactly M, or x rows of exactly N)
    long packed_plans = 0;
    for (int64_t B : {int64_t{1}, int64_t{3}, int64_t{32}})
        for (int64_t C : {int64_t{1}, int64_t{2}, int64_t{3}, int64_t{5}, int64_t{31}})
            for (int64_t P : {int64_t{32}, int64_t{100}, int64_t{50176}})
                for (int dir = 0; dir < 2; ++dir)
                    for (uintptr_t off : {uintptr_t{0}, uintptr_t{4}}) {
                        const int64_t M = dir == 0 ? C : P, N = dir == 0 ? P : C;
                        tmp::TransposePlan p;
                        const int st = tmp::plan_transpose(fake(0x100000 + off), N, M * N,
                                                           const_cast<float *>(fake(0x40000000)), M, M * N, B, M,
                                                           N, 1, 1, 0, &p);
                        if (st != TM_OK || !p.launch)
                            continue;
                        packed_plans += p.packed != 0;
                        char tag[128];
                        std::snprintf(tag, sizeof tag, "packed transpose B=%ld M=%ld N=%ld off=%lu", long(B), long(M),
                                      long(N), (unsigned long)off);
                        replay_transpose(p, B, M, N, tag);
                    }
    CHECK(packed_plans > 0, "no packed-side transpose planned");
    // odd strides on both sides (no 16-byte rows): large views take 64 x 32 sub-tiles
    for (int64_t M : {int64_t{64}, int64_t{4099}, int64_t{9163}})
        for (int64_t N : {int64_t{33}, int64_t{1051}, int64_t{4099}}) {
            tmp::TransposePlan p;
            const int st = tmp::plan_transpose(fake(0x100004), N, 0, const_cast<float *>(fake(0x40000004)), M, 0, 1, M,
                                               N, 1, 1, 0, &p);
            CHECK(st == TM_OK && p.launch, "odd-stride transpose %ldx%ld refused", long(M), long(N));
            char tag[96];
            std::snprintf(tag, sizeof tag, "odd-stride transpose M=%ld N=%ld", long(M), long(N));
            replay_transpose(p, 1, M, N, tag);
        }
    // divisors of every size up to 5000, against plain division
    for (uint32_t d = 1; d <= 5000; ++d) {
        const tmp::Div32 v = tmp::make_div32(d);
        for (uint32_t a : {0u, 1u, d - 1, d, 2 * d + 1, 65535u, 0x7fffffffu, 0xffffffffu}) {
            CHECK(umulhi_div(a, v) == a / d && umulhi_mod(a, v) == a % d, "div32 a=%u d=%u", a, d);
        }
    }
    ++g_checked;
}

// ---- row and column reductions ----------------------------------------------------------------
static void check_reductions() {
    const int64_t Ms[] = {0, 1, 7, 300, 2047, 4096, 1048583};
    const int64_t Ns[] = {0, 1, 5, 64, 100, 257, 513, 1000, 2048, 2051, 4096, 5000, 1048576};
    for (int64_t M : Ms)
        for (int64_t N : Ns)
            for (int TR : {1, 4, 16, 256})
                for (int TC : {1, 4, 64, 256, 1024})
                    for (int aligned = 0; aligned <= 1; ++aligned)
                      for (int64_t ld : {(N + 3) / 4 * 4, N % 4 == 0 ? N + 1 : N}) {  // rows on / off the 16-byte grid
                        for (int op : {int(tmp::kRowSum), int(tmp::kRowMax), int(tmp::kRowSoftmax)}) {
                            tmp::RowPlan p;
                            float *o = const_cast<float *>(fake(0x200000));
                            const int st = tmp::plan_rows(op, fake(0x100000), ld, o, M, N, TR, TC, aligned, &p,
                                                          op == tmp::kRowSoftmax ? o + 4096 : nullptr);
                            if (st != TM_OK || !p.launch)
                                continue;
                            CHECK(p.lpr >= 1 && p.lpr <= tmp::kRowMaxLanes && (p.lpr & (p.lpr - 1)) == 0,
                                  "rows lpr %d", p.lpr);
                            CHECK(p.block == (p.lpr > 64 ? p.lpr : tmp::kBlock), "rows block %d", p.block);
                            CHECK(!(p.once && p.shift), "rows: a shifted walk planned as one batch (N=%ld)", long(N));
                            if (p.once) {
                                // one batch (row_once): lane g of a row takes chunks g + k * lpr for
                                // k < once_k; chunks below whole = nfull * bc / W load unmasked and
                                // must lie inside the row; every chunk of the row is taken once
                                const int W = p.vec ? 4 : 1;
                                const int64_t chunks = (N + W - 1) / W;
                                CHECK(p.bc == std::max(TC, W) && p.lpr >= tmp::kRowOnceMinLanes &&
                                          p.lpr <= (p.vec ? tmp::kRowOnceMaxLanes : 64) &&
                                          int64_t(p.lpr) * p.once_k >= chunks,
                                      "rows once bc %d lpr %d k %d N %ld", p.bc, p.lpr, p.once_k, long(N));
                                const int64_t whole = p.nfull * (p.bc / W);
                                std::vector<uint8_t> seen(size_t(chunks), 0);
                                for (int g = 0; g < p.lpr; ++g)
                                    for (int k = 0; k < p.once_k; ++k) {
                                        const int64_t c = int64_t(k) * p.lpr + g;
                                        if (c < whole)
                                            CHECK((c + 1) * W <= N, "rows once unmasked chunk %ld past N=%ld", long(c),
                                                  long(N));
                                        if (c < chunks)
                                            ++seen[size_t(c)];
                                    }
                                for (int64_t c = 0; c < chunks; ++c)
                                    if (seen[size_t(c)] != 1) {
                                        CHECK(false, "rows once chunk %ld taken %d times", long(c), int(seen[size_t(c)]));
                                        break;
                                    }
                            } else {
                                CHECK(p.bc == p.lpr * (p.vec || p.shift ? 4 : 1) * p.per_tile, "rows bc %d", p.bc);
                                CHECK(!p.shift || (!p.vec && N > tmp::kRowShiftMinN), "rows shift N=%ld", long(N));
                                CHECK(p.per_tile >= 1 && p.per_tile <= 4, "rows per_tile %d", p.per_tile);
                            }
                            CHECK(p.nfull * p.bc + p.rem == N && p.rem >= 0 && p.rem < p.bc,
                                  "rows split N=%ld bc=%d nfull=%ld rem=%ld", long(N), p.bc, long(p.nfull),
                                  long(p.rem));
                            {
                                const int64_t groups = (M + p.block / p.lpr - 1) / (p.block / p.lpr);
                                const int64_t cap = p.lpr == 1 ? tmp::kRowTinyGrid : int64_t{1} << 20;
                                CHECK(p.grid >= 1 && p.grid == uint32_t(groups < cap ? groups : cap),
                                      "rows grid %u for %ld row groups", p.grid, long(groups));
                            }
                            ++g_checked;
                        }
                        for (int walk : {TM_COL_NAIVE, TM_COL_LDS, TM_COL_NAIVE_XCD}) {
                            tmp::ColPlan c;
                            const size_t wsb = tmp::colsum_ws_bytes(M, N, TR, TC, walk);
                            const int st = tmp::plan_cols(fake(0x100000), ld, const_cast<float *>(fake(0x200000)),
                                                          M, N, TR, TC, aligned, walk,
                                                          const_cast<float *>(fake(0x300000)), wsb, &c);
                            if (st != TM_OK)
                                continue;
                            CHECK(c.direct == (N > 0 && tmp::col_direct(M, N, walk)), "cols direct M=%ld N=%ld", long(M),
                                  long(N));
                            if (c.direct)
                                CHECK(!c.launch && wsb == 0 && c.vec && c.out16,
                                      "cols direct plan M=%ld N=%ld", long(M), long(N));
                            if (c.strip) {
                                // strip walk: workgroup (slab, strip), lane t of each wave owns column
                                // chunk strip * 64 + t; its partial lands at ws[slab * N + 4 * chunk]; every
                                // (slab, column) partial is written exactly once, rows read stay < M;
                                // rows off the 16-byte grid only with whole strips (no partial chunk)
                                const int64_t ts = int64_t{1} << c.log_tm, nch = N / 4;
                                const bool x16 = M <= 1 || ld % 4 == 0;  // the fake base is 16-byte aligned
                                CHECK(walk == TM_COL_LDS && c.vec == x16 && N % 4 == 0 &&
                                          (x16 || N % tmp::kColRowStrip == 0) && ts >= tmp::kColRowSlab &&
                                          c.slabs == uint32_t((M + ts - 1) / ts) &&
                                          uint64_t(c.strips) * tmp::kColStripCols >= uint64_t(N) &&
                                          uint64_t(c.slabs) * c.strips * 64 * tmp::kColStripGroups < (uint64_t{1} << 32) &&
                                          ts % (tmp::kColStripGroups * 8) == 0 &&
                                          uint64_t(c.slabs) * uint64_t(N) * 4 <= wsb,
                                      "cols strip plan M=%ld N=%ld", long(M), long(N));
                                CHECK(!c.whole || (M % ts == 0 && N % tmp::kColStripCols == 0), "cols strip whole");
                                std::vector<uint8_t> hit(size_t(c.slabs) * size_t(nch), 0);
                                for (uint32_t b = 0; b < c.slabs * c.strips; ++b) {
                                    const uint32_t strip = b % c.strips, slab = b / c.strips;
                                    for (int t = 0; t < 64; ++t) {
                                        const int64_t ch = int64_t(strip) * 64 + t;
                                        if (ch < nch)
                                            ++hit[size_t(slab) * size_t(nch) + size_t(ch)];
                                    }
                                }
                                for (size_t k = 0; k < hit.size(); ++k)
                                    if (hit[k] != 1) {
                                        CHECK(false, "cols strip partial %zu written %d times", k, int(hit[k]));
                                        break;
                                    }
                            }
                            if (c.launch && !c.strip) {
                                const int64_t ts = int64_t{1} << c.log_tm;
                                CHECK(c.slabs == uint32_t((M + ts - 1) / ts), "cols slabs");
                                if (walk == TM_COL_LDS) {
                                    // 256-row slabs (taller past 4096 slabs), halved while there
                                    // would be fewer than kColTargetWork workgroups, to 32 rows
                                    CHECK(ts >= 32 && (ts >= tmp::kColSlab ||
                                                       int64_t((M + 2 * ts - 1) / (2 * ts)) * c.strips <
                                                           tmp::kColTargetWork),
                                          "cols slab rows %ld", long(ts));
                                } else {
                                    CHECK(ts == TR, "cols slab rows");
                                }
                                CHECK(c.fl >= 1 && c.fl <= tmp::kFinishMaxLanes && (c.fl & (c.fl - 1)) == 0 &&
                                          (c.fl <= 64 || int64_t(c.fl / 2) * tmp::kFinishBatchSlabs < int64_t(c.slabs)),
                                      "cols fl %d", c.fl);
                                if (walk == TM_COL_LDS) {
                                    CHECK(c.tw >= 1 && c.tw <= tmp::kColStrip && uint64_t(c.strips) * c.tw >= uint64_t(N),
                                          "cols strips");
                                    CHECK(!c.whole || (c.vec && M % ts == 0 && N % c.tw == 0), "cols whole");
                                }
                                CHECK(uint64_t(c.slabs) * uint64_t(N) * 4 <= wsb, "cols workspace too small");
                            }
                            if (wsb >= 4) {  // one float less is refused
                                const int st2 = tmp::plan_cols(fake(0x100000), ld,
                                                               const_cast<float *>(fake(0x200000)), M, N, TR, TC,
                                                               aligned, walk, const_cast<float *>(fake(0x300000)),
                                                               wsb - 4, &c);
                                CHECK(st2 == TM_E_WORKSPACE, "cols short workspace accepted (st %d)", st2);
                            }
                            ++g_checked;
                        }
                    }
}

// Split row walks (the calls with a workspace): the segments of a row cover its N columns once,
// each segment's chunks (C per thread at a stride of the workgroup's width, as row_split_partial
// documents) cover the segment once, and the workspace holds M * segs partials.
static void check_split_rows() {
    const int64_t Ms[] = {1, 2, 7, 63, 127, 128, 300};
    const int64_t Ns[] = {1000, 65536, 98303, 98304, 98305, 262144, (int64_t{1} << 23) + 3, int64_t{1} << 30};
    for (int64_t M : Ms)
        for (int64_t N : Ns)
            for (uintptr_t base : {uintptr_t{0x100000}, uintptr_t{0x100004}})
                for (int op : {int(tmp::kRowSum), int(tmp::kRowMax), int(tmp::kRowSoftmax)}) {
                    tmp::RowPlan p;
                    float *o = const_cast<float *>(fake(0x200000));
                    float *ws = const_cast<float *>(fake(0x400000));
                    const size_t wsb = tmp::rows_ws_bytes(M, N);
                    const int64_t ld = N + (N & 1);
                    const int st = tmp::plan_rows(op, fake(base), ld, o, M, N, 1, 1, 0, &p,
                                                  op == tmp::kRowSoftmax ? o + 4096 : nullptr, true, ws, wsb);
                    CHECK(st == TM_OK, "split rows status %d M=%ld N=%ld", st, long(M), long(N));
                    const bool want_split = M < tmp::kRowSplitRows && N >= tmp::kRowSplitMinN;
                    CHECK(p.split == want_split, "split chosen %d for M=%ld N=%ld", int(p.split), long(M), long(N));
                    CHECK(want_split == (wsb > 0), "workspace %zu for M=%ld N=%ld", wsb, long(M), long(N));
                    ++g_checked;
                    if (!p.split)
                        continue;
                    CHECK(p.log_k >= 0 && p.log_k <= tmp::kRowSegMaxLogK, "log_k %d", p.log_k);
                    CHECK(p.seg == (int64_t{tmp::kRowSegUnit} << p.log_k), "seg %ld", long(p.seg));
                    CHECK(int64_t(p.segs) * p.seg >= N && (int64_t(p.segs) - 1) * p.seg < N, "segs %u", p.segs);
                    CHECK(p.nwork == uint64_t(M) * p.segs, "nwork %u", p.nwork);
                    CHECK(p.grid == (p.nwork < (1u << 20) ? p.nwork : (1u << 20)), "grid %u", p.grid);
                    CHECK(uint64_t(M) * p.segs * tmp::kRowPartialBytes <= wsb, "workspace too small");
                    CHECK(p.vec == (base % 16 == 0 && (M <= 1 || ld % 4 == 0)), "vec %d", int(p.vec));
                    CHECK(p.ws == ws && p.block == tmp::kBlock, "ws / block");
                    // Fewer segments would do only with K = 16 (the largest) or when the target is met.
                    CHECK(p.log_k == tmp::kRowSegMaxLogK || int64_t(p.segs) * M >= tmp::kRowSplitTarget / 2 ||
                              p.log_k == 0,
                          "K too small: log_k %d segs %u", p.log_k, p.segs);
                    // one segment's columns: thread t, chunk c -> t * W + c * kBlock * W, W wide
                    const int W = p.vec ? 4 : 1;
                    const int C = tmp::kRowSegUnit / tmp::kBlock * (1 << p.log_k) / W;
                    std::vector<uint8_t> hit(size_t(p.seg), 0);
                    for (int t = 0; t < tmp::kBlock; ++t)
                        for (int c = 0; c < C; ++c)
                            for (int i = 0; i < W; ++i)
                                ++hit[size_t(int64_t(t) * W + int64_t(c) * tmp::kBlock * W + i)];
                    bool once = true;
                    for (uint8_t h : hit)
                        once = once && h == 1;
                    CHECK(once, "segment chunks do not cover the segment once (seg %ld)", long(p.seg));
                    if (wsb >= 4) {
                        const int st2 = tmp::plan_rows(op, fake(base), ld, o, M, N, 1, 1, 0, &p,
                                                       op == tmp::kRowSoftmax ? o + 4096 : nullptr, true, ws,
                                                       wsb - 4);
                        CHECK(st2 == TM_E_WORKSPACE, "rows short workspace accepted (st %d)", st2);
                    }
                    tmp::RowPlan q;
                    tmp::plan_rows(op, fake(base), ld, o, M, N, 1, 1, 0, &q,
                                   op == tmp::kRowSoftmax ? o + 4096 : nullptr);
                    CHECK(!q.split, "a call without a workspace was split");
                }
}

// Extreme extents: every planner either refuses the call or returns a plan, with no signed
// overflow (the build runs under UndefinedBehaviorSanitizer) in the shape rules: flat views, split
// rows, column slabs, transposes.
static void check_extremes() {
    const int64_t big[] = {int64_t{1} << 31, (int64_t{1} << 31) + 3, int64_t{1} << 40, int64_t{1} << 52,
                           INT64_MAX / 8, INT64_MAX / 4, INT64_MAX};
    float *o = const_cast<float *>(fake(0x200000));
    for (int64_t a : big)
        for (int64_t b : {int64_t{1}, int64_t{3}, int64_t{64}, int64_t{4096}, a}) {
            for (int dir = 0; dir < 2; ++dir) {
                const int64_t M = dir ? a : b, N = dir ? b : a;
                tmp::MapPlan mp;
                tmp::plan_map(tmp::kScale, fake(0x100000), N, o, N, M, N, 1.f, 0.f, 1, 4, 0, 0, &mp);
                tmp::plan_map(tmp::kChannel, fake(0x100000), N, o, N, M, N, 0.f, 0.f, 1, 1, 0, 0, &mp, nullptr,
                              fake(0x300000));
                tmp::RowPlan rp;
                tmp::plan_rows(tmp::kRowSoftmax, fake(0x100000), N, o, M, N, 1, 1, 0, &rp, o, true, o,
                               tmp::rows_ws_bytes(M, N));
                tmp::plan_rows(tmp::kRowSum, fake(0x100000), N, o, M, N, 1, 1, 0, &rp);
                tmp::ColPlan cp;
                const size_t w = tmp::colsum_ws_bytes(M, N, 1, 1, TM_COL_LDS);
                tmp::plan_cols(fake(0x100000), N, o, M, N, 1, 1, 0, TM_COL_LDS, o, w, &cp);
                tmp::TransposePlan tp;
                tmp::plan_transpose(fake(0x100000), N, 0, o, M, 0, 1, M, N, 1, 1, 0, &tp);
                tmp::plan_transpose(fake(0x100000), N, M * 0 + N, o, M, N, 2, M, N, 1, 1, 0, &tp);
                // the host helpers exported through the C ABI
                int64_t p1, p2, p3;
                tmp::split(M, N, &p1, &p2);
                tmp::split(M, 1, &p1, &p2);
                tmp::plan_tiles(M, N, 256, 1024, &p1, &p2, &p3);
                tmp::plan_tiles(M, N, 1, 1, &p1, &p2, &p3);
                tmp::pad_extents(M, N, 256, 1024, &p1, &p2, &p3);
                tmp::check_promise(M, N, N, N, 256, 1024, fake(0x100000), o);
                tmp::rows_ws_bytes(M, N);
                tmp::colsum_ws_bytes(M, N, 256, 64, TM_COL_NAIVE);
                ++g_checked;
            }
        }
}

int main() {
    check_extremes();
    check_maps();
    check_maps_diff();
    check_maps_wide();
    check_transposes();
    check_reductions();
    check_split_rows();
    check_skew_transposes();
    check_packed_big();
    CHECK(g_pbig >= 20, "only %ld large packed plans replayed", g_pbig);
    CHECK(g_rows > 0, "no padded-row span plan was replayed");
    CHECK(g_skew >= 36, "only %ld line-aligned window plans replayed", g_skew);
    std::printf("plan_check: %ld plans checked (%ld flat, %ld span), %ld failures\n", g_checked, g_flat, g_rows,
                g_failed);
    return g_failed == 0 ? 0 : 1;
}
