"""CPU tests of the C-ABI boundary: the library loads, exports every call include/tilemap.h declares,
and its host logic -- the promise checker, the loop split, the tile scheduler counts and the whole
error surface -- behaves as documented.  No kernel is launched: every call here either is a
host-only helper or fails validation, which happens before any HIP call.
"""
import ctypes
import os
import re

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tilemap.h")

tm = pytest.importorskip("edge_masking_vector_amd.tilemap")
torch = pytest.importorskip("torch")

# The error-path tests below pass fake device addresses that are never dereferenced because every
# call fails validation before any HIP call.  Where a GPU is visible, a slip in such a test could
# reach a launch with a fake address, so those tests only run on GPU-less hosts.
# (device_count() does not initialise the GPU.)
no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="fake-address error-path tests run only where no GPU is visible")

A16 = 0x7F0000000000          # a 16-byte aligned fake device address (never dereferenced)
B16 = 0x7F0000100000


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tm_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 11
    lib = ctypes.CDLL(tm.library_path())
    for n in names:
        assert hasattr(lib, n), n


def test_exports_nothing_else():
    out = os.popen("nm -D --defined-only '%s'" % tm.library_path()).read()
    exported = sorted(l.split()[-1] for l in out.splitlines() if " T " in l)
    assert exported == _declared()


def test_extension_binds_every_declared_call():
    """The _tilemap extension has one function per C call, under the same name, and so does the
    Python binding."""
    for n in _declared():
        assert hasattr(tm._ext, n), n
        assert callable(getattr(tm, n)), n


def test_extension_rejects_bad_arguments_before_calling():
    f = tm._ext.tm_map_affine
    good = [0, 16, 0, 16, 0, 16, 2.0, 1.0, 1, 1024, 0, 3, 0]   # M = 0: a no-op call
    assert f(*good) == tm.TM_OK
    with pytest.raises(TypeError):
        f(*good[:-1])                          # argument count
    with pytest.raises(TypeError):
        f(*(good[:1] + ["16"] + good[2:]))     # a string where a size goes
    with pytest.raises(OverflowError):
        f(*([-1] + good[1:]))                  # a negative address
    with pytest.raises(OverflowError):
        f(*(good[:8] + [1 << 40] + good[9:]))  # an int argument past C int
    with pytest.raises(TypeError):
        f(*(good[:6] + [None] + good[7:]))     # alpha must be a number
    assert tm._ext.tm_split(1000, 16) == (tm.TM_OK, 62, 8)
    assert tm._ext.tm_status_string(-2) == "TM_E_ALIGN"


def test_status_strings():
    for code, name in [(0, "TM_OK"), (-1, "TM_E_INVAL"), (-2, "TM_E_ALIGN"),
                       (-3, "TM_E_UNSUPPORTED"), (-4, "TM_E_WORKSPACE"), (-5, "TM_E_HIP")]:
        assert tm.tm_status_string(code) == name
    assert tm.tm_status_string(42) == "unknown status"


# ---- loop remainder split: the product's splitter against the pages and the oracle --------------

def test_split_matches_pages_and_oracle():
    assert tm.tm_split(1000, 16) == (tm.TM_OK, 62, 8)
    assert tm.tm_split(1000, 64) == (tm.TM_OK, 15, 40)
    for K in range(0, 200):
        for T in range(1, 33):
            st, nf, rm = tm.tm_split(K, T)
            assert st == tm.TM_OK and (nf, rm) == oracle.split(K, T)
    assert tm.tm_split(-1, 4)[0] == tm.TM_E_INVAL
    assert tm.tm_split(10, 0)[0] == tm.TM_E_INVAL


# ---- the row walk's column tiles ----------------------------------------------------------------

LINE = 0x100000  # a 128-byte-aligned address: inspected by the query, never dereferenced


def test_row_walk_honours_the_pages_masked_max_tile():
    """'Reductions over a ragged tile' walks Nk = 1000 columns in BC = 64 tiles: 15 whole tiles and
    one of 40 columns.  That is the walk the row reductions run on 8192 x 1000, with 16-byte rows
    and with rows off the 16-byte grid (row stride 1001) alike."""
    # rows of 250 16-byte chunks are read in one batch, 32 lanes of 8 chunks each; the tile
    # decides which chunks are read unmasked
    assert tm.tm_row_walk(8192, 1000, 1000, 16, 64, 0, LINE) == (tm.TM_OK, 64, 15, 40, 32)
    st, bc, nf, rem, lanes = tm.tm_row_walk(8192, 1000, 1001, 16, 64, 0, LINE)
    assert (st, bc, nf, rem) == (tm.TM_OK, 64, 15, 40)
    assert (nf, rem) == oracle.split(1000, 64)
    # its aligned counterpart: 16 whole tiles, no remainder
    assert tm.tm_row_walk(8192, 1024, 1024, 16, 64, 1, LINE) == (tm.TM_OK, 64, 16, 0, 32)
    # the loop split example of 'Loops over a dynamic extent': K = 1000 in 16-column tiles
    assert tm.tm_row_walk(8192, 1000, 1000, 16, 16, 0, LINE)[1:4] == (16, 62, 8)
    # the promise is checked as the reductions check it
    assert tm.tm_row_walk(8192, 1000, 1000, 16, 64, 1, LINE)[0] == tm.TM_E_ALIGN


def test_row_walk_split_is_the_remainder_rule():
    """Whatever tile the walk takes, nfull and rem are the remainder split of N by it.  The
    caller's tile (at least one chunk wide) is the walk's for rows read in one batch (more than
    half of 16 lanes' and at most 64 lanes' batch of chunks) and, for other rows, whenever it
    keeps at least half the lanes and at most 4 chunks per lane; otherwise the walk's own tile is
    a whole number of chunks per lane."""
    for M in (1, 7, 300, 4096):
        for N in (1, 5, 16, 63, 64, 100, 1000, 4096, 70000):
            for ld in (N + (-N) % 4, N + 1 if N % 4 == 0 else N):
                W = 4 if M <= 1 or ld % 4 == 0 else 1  # 16-byte chunks when every row starts on 16 bytes
                shifted = W == 1 and N > 2048  # long rows off the grid: 16-byte chunks from the boundary
                for BC in (1, 4, 16, 64, 256, 1024):
                    st, bc, nf, rem, lanes = tm.tm_row_walk(M, N, ld, 1, BC, 0, LINE)
                    assert st == tm.TM_OK
                    assert (nf, rem) == oracle.split(N, bc), (M, N, ld, BC)
                    chunks = -(-N // W)
                    K = 8 if W == 4 else 16
                    if 8 * K < chunks <= (256 if W == 4 else 64) * K and not (chunks > 32 * K and M < 2048):
                        # one batch: at least 16 lanes cover the row (up to 256 lanes for 16-byte
                        # chunks, 64 for 4-byte ones), and the tile is the caller's
                        assert lanes >= 16 and lanes * K >= chunks and bc == max(BC, W), (M, N, ld, BC)
                        continue
                    Wt = 4 if shifted else W
                    assert bc % (lanes * Wt) == 0 and 1 <= bc // (lanes * Wt) <= 4, (M, N, ld, BC, bc, lanes)
                    if bc == BC:
                        continue
                    # the caller's tile was not taken: it was not whole chunks, would leave fewer
                    # than half the lanes, or would need more than 4 chunks per lane
                    assert BC % Wt or BC // Wt < lanes // 2 or BC // Wt > 4 * lanes, (M, N, ld, BC, bc, lanes)


def test_row_walk_errors():
    assert tm.tm_row_walk(-1, 10, 10, 1, 64, 0, LINE)[0] == tm.TM_E_INVAL
    assert tm.tm_row_walk(4, 10, 9, 1, 64, 0, LINE)[0] == tm.TM_E_INVAL     # ld < N
    assert tm.tm_row_walk(4, 10, 10, 1, 0, 0, LINE)[0] == tm.TM_E_INVAL     # tile <= 0
    assert tm.tm_row_walk(4, 10, 10, 1, 48, 0, LINE)[0] == tm.TM_E_UNSUPPORTED
    assert tm.tm_row_walk(4, 10, 10, 1, 64, 0, None)[0] == tm.TM_E_INVAL   # NULL with work
    assert tm.tm_row_walk(4, 10, 10, 1, 64, 0, LINE + 2)[0] == tm.TM_E_INVAL  # not 4-byte aligned
    assert tm.tm_row_walk(0, 10, 10, 1, 64, 0, None)[0] == tm.TM_OK


# ---- the column sums' plan (tm_col_walk) ---------------------------------------------------------
def test_col_walk_reports_the_walks_the_column_sums_run():
    """teenygrad 'What it actually costs' walks 4096 x 4096 column by column (the naive walk: one
    column per workgroup, slabs of the caller's TM rows) and 'Seeing it in a real kernel' stages the
    reads so that they stay coalesced (the LDS walk, whose slabs and strips are its own)."""
    M = N = 4096
    wsb = tm.tm_colsum_workspace_bytes(M, N, 256, 64, tm.TM_COL_LDS)
    # wide matrix, 16-byte aligned workspace: the strip form, 64-row slabs by 256-column strips
    assert tm.tm_col_walk(LINE, N, LINE, M, N, 256, 64, 1, tm.TM_COL_LDS, LINE, wsb) == \
        (tm.TM_OK, tm.TM_COLFORM_STRIPS, 64, 256, 64, 16)
    # a workspace off the 16-byte grid: the LDS-staged slabs by 128-column strips instead
    st, form, srows, scols, slabs, strips = tm.tm_col_walk(LINE, N, LINE, M, N, 256, 64, 1, tm.TM_COL_LDS,
                                                           LINE + 4, wsb)
    assert (st, form, scols, strips) == (tm.TM_OK, tm.TM_COLFORM_TILES, 128, 32)
    assert slabs * srows >= M > (slabs - 1) * srows and slabs * N * 4 <= wsb
    # the naive walks: the caller's TM rows per slab, one column per workgroup
    for walk in (tm.TM_COL_NAIVE, tm.TM_COL_NAIVE_XCD):
        wsn = tm.tm_colsum_workspace_bytes(M, N, 256, 1, walk)
        assert tm.tm_col_walk(LINE, N, LINE, M, N, 256, 1, 0, walk, LINE, wsn) == \
            (tm.TM_OK, tm.TM_COLFORM_TILES, 256, 1, 16, N)
        assert wsn == 16 * N * 4
    # few rows: one pass, 16-byte column chunks down all rows, no workspace
    assert tm.tm_colsum_workspace_bytes(16, 1 << 20, 16, 64, tm.TM_COL_LDS) == 0
    assert tm.tm_col_walk(LINE, 1 << 20, LINE, 16, 1 << 20, 16, 64, 1, tm.TM_COL_LDS, None, 0) == \
        (tm.TM_OK, tm.TM_COLFORM_ONE_PASS, 16, 4, 1, 1 << 18)
    # nothing to launch without columns; only the zero-writing pass without rows
    assert tm.tm_col_walk(LINE, 10, LINE, 10, 0, 1, 1, 0, tm.TM_COL_LDS, None, 0)[:2] == (tm.TM_OK, tm.TM_COLFORM_NONE)
    assert tm.tm_col_walk(None, 10, LINE, 0, 10, 1, 1, 0, tm.TM_COL_LDS, None, 0)[:2] == (tm.TM_OK, tm.TM_COLFORM_TILES)


def test_col_walk_partials_fit_the_workspace():
    """Every two-pass plan's partials (slabs per column x N floats) fit the size
    tm_colsum_workspace_bytes reports, for any workspace alignment."""
    for M in (1, 63, 64, 300, 4096, 70000):
        for N in (1, 5, 127, 1024, 3000, 4096):
            for walk, TM, TN in ((tm.TM_COL_LDS, 64, 64), (tm.TM_COL_NAIVE, 256, 1), (tm.TM_COL_NAIVE_XCD, 64, 1)):
                wsb = tm.tm_colsum_workspace_bytes(M, N, TM, TN, walk)
                for ws in (LINE, LINE + 4):
                    st, form, srows, scols, slabs, strips = tm.tm_col_walk(LINE, N, LINE, M, N, TM, TN, 0, walk,
                                                                           ws if wsb else None, wsb)
                    assert st == tm.TM_OK, (M, N, walk, ws)
                    if form == tm.TM_COLFORM_ONE_PASS:
                        assert wsb == 0 and srows == M
                        continue
                    assert form in (tm.TM_COLFORM_TILES, tm.TM_COLFORM_STRIPS)
                    assert slabs * N * 4 <= wsb, (M, N, walk, ws, slabs, wsb)
                    assert slabs * srows >= M > (slabs - 1) * srows and strips * scols >= N > (strips - 1) * scols
                    assert form != tm.TM_COLFORM_STRIPS or (ws % 16 == 0 and scols == 256 and N >= 1024)


@no_gpu
def test_col_walk_errors():
    wsb = tm.tm_colsum_workspace_bytes(100, 100, 64, 64, tm.TM_COL_LDS)
    assert tm.tm_col_walk(A16, 100, B16, 100, 100, 64, 64, 0, 7, A16, wsb)[0] == tm.TM_E_INVAL       # walk
    assert tm.tm_col_walk(A16, 100, B16, 100, 100, 64, 64, 1, tm.TM_COL_LDS, A16, wsb)[0] == tm.TM_E_ALIGN
    assert tm.tm_col_walk(A16, 100, B16, 100, 100, 64, 64, 0, tm.TM_COL_LDS, A16, wsb - 4)[0] == tm.TM_E_WORKSPACE
    assert tm.tm_col_walk(A16, 100, None, 100, 100, 64, 64, 0, tm.TM_COL_LDS, A16, wsb)[0] == tm.TM_E_INVAL
    assert tm.tm_col_walk(A16, 99, B16, 100, 100, 64, 64, 0, tm.TM_COL_LDS, A16, wsb)[0] == tm.TM_E_INVAL  # ld < N


# ---- the maps' plan (tm_map_walk) ----------------------------------------------------------------

X0, Y0 = LINE, LINE + (1 << 30)   # two line-aligned bases (inspected only)


def walk(M, N, ldx, ldy, xoff=0, yoff=0, var=None, op=0, bias=None, aligned=0, TM=64, TN=64):
    var = tm.TM_VAR_AUTO if var is None else var
    st, w, items = tm.tm_map_walk(op, X0 + 4 * xoff, ldx, Y0 + 4 * yoff, ldy, M, N, TM, TN, aligned, var, bias)
    assert st == tm.TM_OK, (M, N, ldx, ldy, xoff, yoff, st)
    return w, items


def test_map_walk_bench_views():
    """The plans the benchmark's map paths are labelled with."""
    SPAN, TILES, FLAT = tm.TM_MAP_SPAN, tm.TM_MAP_TILES, tm.TM_MAP_FLAT
    assert walk(4100, 1000, 1000, 1000) == (FLAT, -(-4100 * 1000 // 256))   # one flat row of 1 KiB items
    assert walk(4096, 4096, 4096, 4096, var=tm.TM_VAR_VEC4, aligned=1, TM=32, TN=128) == (FLAT, 65536)
    for (M, N, ldx, ldy) in ((4100, 1000, 1001, 1001), (4100, 1000, 1004, 1004), (4100, 4100, 4104, 4104),
                             (4100, 4100, 4104, 4108), (4100, 4100, 4700, 4700)):
        # one span of 1 KiB items on y's 1 KiB grid from y[0] (line-aligned: head 0)
        assert walk(M, N, ldx, ldy) == (SPAN, -(-((M - 1) * ldy + N) // 256)), (M, N, ldx, ldy)
    assert walk(4100, 1000, 1004, 1008)[0] == TILES   # different strides, rows under 1024 floats
    assert walk(4100, 4100, 5120, 5120)[0] == TILES   # wide padding, rows on the line grid
    # the span's first item starts on y's 1 KiB grid: y 100 floats past it adds 100 to the span
    assert walk(4100, 1000, 1001, 1001, 100, 100) == (SPAN, -(-(100 + 4099 * 1001 + 1000) // 256))


def test_map_walk_span_limits():
    """Where the span stops and the 2-D tiles take over: one stride (or different strides over
    rows of 1024 floats or more, or off the 16-byte grid, unless both tensors' rows lie on the
    line grid), rows of 64
    floats or more, and padding under a line, at most an eighth of the row, or -- y's rows off
    the line grid -- a quarter of 16-byte rows of 2048 floats or more, a quarter of rows off the
    16-byte grid, or half of them from 2048 floats on; x at any 4-byte phase.  Contiguous rows
    are one row: the flat kernel's when both bases lie on the line grid at one phase, else a span."""
    SPAN, TILES = tm.TM_MAP_SPAN, tm.TM_MAP_TILES
    assert walk(100, 1000, 1031, 1031)[0] == SPAN     # under a line
    assert walk(100, 1000, 1125, 1125)[0] == SPAN     # an eighth
    assert walk(100, 1000, 1128, 1128)[0] == TILES    # past it, 16-byte rows under 2048 floats
    assert walk(100, 2048, 2556, 2556)[0] == SPAN     # a quarter of 16-byte rows of 2048 floats
    assert walk(100, 2048, 2564, 2564)[0] == TILES    # past it
    assert walk(100, 2044, 2552, 2552)[0] == TILES    # a quarter, rows under 2048 floats
    assert walk(100, 2048, 2560, 2560)[0] == TILES    # rows on the line grid: an eighth at most
    assert walk(100, 2048, 2304, 2304, 32, 32)[0] == SPAN
    assert walk(100, 2048, 2560, 2560, 4, 4)[0] == SPAN   # the same stride, bases off the line grid
    assert walk(100, 1000, 1249, 1249)[0] == SPAN     # a quarter of rows off the 16-byte grid
    assert walk(100, 1000, 1251, 1251)[0] == TILES
    assert walk(100, 2048, 3071, 3071)[0] == SPAN     # half of them from 2048 floats on
    assert walk(100, 2048, 3073, 3073)[0] == TILES
    assert walk(100, 2048, 3072, 3072, 2, 2)[0] == SPAN    # 16-byte stride, base off the 16-byte grid
    assert walk(100, 2047, 3071, 3071)[0] == TILES    # half, rows under 2048 floats
    assert walk(100, 1100, 1104, 1108)[0] == SPAN     # different strides, 1024 floats or more
    assert walk(100, 1000, 1004, 1008)[0] == TILES    # ... on the 16-byte grid under 1024 floats
    assert walk(100, 1000, 1003, 1007)[0] == SPAN     # ... off it, at any width
    assert walk(100, 1100, 1101, 1104)[0] == SPAN     # strides 3 apart: x's chunks 4-byte aligned
    assert walk(100, 1024, 1024, 1024 + 128, 0, 0)[0] == TILES   # both on the line grid, strides differ
    assert walk(100, 1000, 1001, 1001, 1, 0)[0] == SPAN    # bases at different 16-byte phases
    assert walk(100, 1000, 1000, 1000, 1, 0) == (SPAN, -(-100000 // 256))   # contiguous: one row
    assert walk(100, 1000, 1000, 1000, 4, 4)[0] == SPAN    # one phase, bases off the line grid
    assert walk(100, 1000, 1000, 1000, 32, 32)[0] == tm.TM_MAP_FLAT   # ... on it: the flat kernel
    assert walk(1, 100, 100, 100, 1, 0)[0] == SPAN     # one row at another phase
    assert walk(1, 63, 63, 63, 1, 0)[0] == TILES       # ... under 64 floats
    assert walk(100, 63, 64, 64)[0] == TILES          # rows under 64 floats
    assert walk(100, 1000, 1004, 1004, var=tm.TM_VAR_VEC4_UNDERSTATED)[0] == TILES
    assert walk(1, 1000, 1004, 1004)[0] == tm.TM_MAP_FLAT   # one row on the line grid is a flat row
    assert walk(0, 1000, 1004, 1004) == (tm.TM_MAP_NONE, 0)


def test_map_walk_channel_and_errors():
    assert walk(300, 1000, 1004, 1004, op=3, bias=LINE + (2 << 30))[0] == tm.TM_MAP_SPAN
    assert walk(300, 1000, 1000, 1000, op=3, bias=LINE + (2 << 30))[0] == tm.TM_MAP_FLAT
    assert tm.tm_map_walk(3, X0, 1004, Y0, 1004, 300, 1000, 64, 64, 0, 0, None)[0] == tm.TM_E_INVAL  # no bias
    assert tm.tm_map_walk(4, X0, 1004, Y0, 1004, 300, 1000, 64, 64, 0, 0)[0] == tm.TM_E_INVAL
    assert tm.tm_map_walk(0, X0, 1004, Y0, 1004, 4100, 1000, 64, 64, 1, 0)[0] == tm.TM_E_ALIGN
    assert tm.tm_map_walk(0, X0, 999, Y0, 1004, 4, 1000, 64, 64, 0, 0)[0] == tm.TM_E_INVAL   # ldx < N


# ---- tile scheduler counts ---------------------------------------------------------------------

def test_plan_tiles_workload_shapes():
    # ragged 4100 x 1000 under 64 x 64: 65 x 16 tiles, 64 x 15 = 960 whole
    assert tm.tm_plan_tiles(4100, 1000, 64, 64) == (tm.TM_OK, 65, 16, 960)
    # a whole-tile count beyond 64 bits is refused, not wrapped
    assert tm.tm_plan_tiles(1 << 40, 1 << 40, 1, 1)[0] == tm.TM_E_INVAL
    assert tm.tm_plan_tiles(1 << 40, 1 << 22, 1, 1) == (tm.TM_OK, 1 << 40, 1 << 22, 1 << 62)
    # 4096 x 4096 under 32 x 128: all 128 x 32 = 4096 tiles whole
    assert tm.tm_plan_tiles(4096, 4096, 32, 128) == (tm.TM_OK, 128, 32, 4096)
    # the pages' edge-tile example: 20 x 28 under 8 x 8
    assert tm.tm_plan_tiles(20, 28, 8, 8) == (tm.TM_OK, 3, 4, 6)


def test_plan_tiles_against_oracle_brute_force():
    for M in range(0, 19):
        for N in range(0, 19):
            for TM in (1, 2, 4, 8, 16):
                for TN in (1, 4, 8, 16):
                    st, tmm, tnn, whole = tm.tm_plan_tiles(M, N, TM, TN)
                    assert st == tm.TM_OK
                    assert tmm == -(-M // TM) and tnn == -(-N // TN)
                    full = sum(1 for pm in range(tmm) for pn in range(tnn)
                               if oracle.tile_live(M, N, TM, TN, pm, pn) == TM * TN)
                    assert whole == full, (M, N, TM, TN)


def test_plan_tiles_errors():
    assert tm.tm_plan_tiles(-1, 4, 4, 4)[0] == tm.TM_E_INVAL
    assert tm.tm_plan_tiles(4, 4, 0, 4)[0] == tm.TM_E_INVAL
    assert tm.tm_plan_tiles(4, 4, 3, 4)[0] == tm.TM_E_UNSUPPORTED
    assert tm.tm_plan_tiles(4, 4, 512, 4)[0] == tm.TM_E_UNSUPPORTED
    assert tm.tm_plan_tiles(4, 4, 4, 2048)[0] == tm.TM_E_UNSUPPORTED


# ---- the promise checker -------------------------------------------------------------------------

def test_promise_checker_matches_oracle():
    """Exhaustive over small shapes, strides and base alignments: TM_OK exactly when the oracle's
    predicate holds, TM_E_ALIGN otherwise (all arguments well-formed)."""
    for M in (0, 1, 4, 8, 12, 16, 20):
        for N in (0, 4, 8, 12, 16, 28, 32):
            for TM in (1, 4, 8):
                for TN in (1, 2, 4, 8, 16):
                    for ldi in (N, N + 1, N + 4):
                        for ldo in (N, N + 2):
                            for ia, oa in ((A16, B16), (A16 + 4, B16), (A16, B16 + 8), (A16, 0)):
                                st = tm.tm_check_promise(M, N, ldi, ldo, TM, TN, ia, oa or None)
                                want = oracle.promise_holds(M, N, ldi, ldo, TM, TN, ia, oa)
                                assert st == (tm.TM_OK if want else tm.TM_E_ALIGN), \
                                    (M, N, TM, TN, ldi, ldo, hex(ia), hex(oa))


def test_promise_checker_workloads():
    assert tm.tm_check_promise(4096, 4096, 4096, 4096, 32, 128, A16, B16) == tm.TM_OK
    assert tm.tm_check_promise(4100, 1000, 1000, 1000, 64, 64, A16, B16) == tm.TM_E_ALIGN
    assert tm.tm_check_promise(8192, 1000, 1000, 0, 16, 64, A16, None) == tm.TM_E_ALIGN


def test_promise_checker_malformed():
    assert tm.tm_check_promise(-4, 4, 4, 4, 4, 4, A16, B16) == tm.TM_E_INVAL
    assert tm.tm_check_promise(4, 8, 4, 8, 4, 4, A16, B16) == tm.TM_E_INVAL     # ld_in < N
    assert tm.tm_check_promise(4, 4, 4, 4, 0, 4, A16, B16) == tm.TM_E_INVAL
    assert tm.tm_check_promise(4, 4, 4, 4, 4, -8, A16, B16) == tm.TM_E_INVAL
    assert tm.tm_check_promise(4, 4, 4, 4, 6, 4, A16, B16) == tm.TM_E_UNSUPPORTED
    # precedence: INVAL before UNSUPPORTED
    assert tm.tm_check_promise(-4, 4, 4, 4, 6, 4, A16, B16) == tm.TM_E_INVAL


# ---- the error surface of every compute call (returns before any HIP call) ----------------------

S = 0  # null stream; never used, the calls fail validation first


@no_gpu
def test_map_errors():
    f = tm.tm_map_affine
    ok = dict(x=A16, ldx=4096, y=B16, ldy=4096, M=4096, N=4096, alpha=2.0, beta=1.0, TM=32, TN=128,
              aligned=1, variant=tm.TM_VAR_VEC4, stream=S)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["ldx"], a["y"], a["ldy"], a["M"], a["N"], a["alpha"], a["beta"],
                 a["TM"], a["TN"], a["aligned"], a["variant"], a["stream"])

    assert call(M=-1) == tm.TM_E_INVAL
    assert call(N=-5) == tm.TM_E_INVAL
    assert call(ldx=4095) == tm.TM_E_INVAL
    assert call(ldy=100) == tm.TM_E_INVAL
    assert call(x=0) == tm.TM_E_INVAL
    assert call(y=0) == tm.TM_E_INVAL
    assert call(x=A16 + 2) == tm.TM_E_INVAL            # not 4-byte aligned
    assert call(TM=0) == tm.TM_E_INVAL
    assert call(TN=-128) == tm.TM_E_INVAL
    assert call(aligned=2) == tm.TM_E_INVAL
    assert call(variant=7) == tm.TM_E_INVAL
    assert call(TM=48) == tm.TM_E_UNSUPPORTED
    assert call(TN=2048) == tm.TM_E_UNSUPPORTED
    assert call(TM=512) == tm.TM_E_UNSUPPORTED
    # broken promises
    assert call(M=4100, N=1000, ldx=1000, ldy=1000, TM=64, TN=64) == tm.TM_E_ALIGN
    assert call(x=A16 + 4) == tm.TM_E_ALIGN
    assert call(ldy=4098) == tm.TM_E_ALIGN
    # 16-byte variant on a ragged path whose rows are not 16-byte aligned
    assert call(aligned=0, x=A16 + 4) == tm.TM_E_ALIGN
    assert call(aligned=0, ldx=4099) == tm.TM_E_ALIGN
    assert call(aligned=0, variant=tm.TM_VAR_VEC4_UNDERSTATED, TN=2) == tm.TM_E_UNSUPPORTED
    # precedence
    assert call(M=-1, TM=48) == tm.TM_E_INVAL
    assert call(TM=48, x=A16 + 4) == tm.TM_E_UNSUPPORTED
    # no work: valid no-ops, even with NULL pointers
    assert call(M=0, x=0, y=0) == tm.TM_OK
    assert call(N=0, x=0, y=0, aligned=0) == tm.TM_OK


@no_gpu
def test_scale_copy_errors():
    assert tm.tm_scale2d(A16, 64, B16, 64, 64, 64, 1.5, 32, 128, 1, 0, S) == tm.TM_E_ALIGN
    assert tm.tm_scale2d(A16, 64, B16, 64, 64, 64, 1.5, 32, 3, 0, 0, S) == tm.TM_E_UNSUPPORTED
    assert tm.tm_copy2d(A16, 8, B16, 8, 4, 9, 4, 4, 0, 0, S) == tm.TM_E_INVAL
    assert tm.tm_copy2d(0, 8, 0, 8, 0, 8, 4, 4, 1, 0, S) == tm.TM_OK


@no_gpu
def test_reduction_errors():
    assert tm.tm_rowsum(A16, 1000, B16, -1, 1000, 4, 256, 0, S) == tm.TM_E_INVAL
    assert tm.tm_rowsum(A16, 1000, 0, 10, 1000, 4, 256, 0, S) == tm.TM_E_INVAL     # NULL out
    assert tm.tm_rowsum(A16, 1000, B16 + 2, 10, 1000, 4, 256, 0, S) == tm.TM_E_INVAL
    assert tm.tm_rowsum(A16, 1000, B16, 10, 1000, 4, 250, 0, S) == tm.TM_E_UNSUPPORTED
    assert tm.tm_rowsum(A16, 1000, B16, 8, 1000, 4, 256, 1, S) == tm.TM_E_ALIGN
    assert tm.tm_rowsum(A16, 1000, B16, 0, 1000, 4, 256, 0, S) == tm.TM_OK           # empty output
    # masked rowmax on the score workload: aligned=1 must fail (1000 % 64 = 40)
    assert tm.tm_rowmax_masked(A16, 1000, B16, 8192, 1000, 16, 64, 1, S) == tm.TM_E_ALIGN
    assert tm.tm_rowmax_masked(A16, 1000, B16, 8192, 1000, 16, 0, 0, S) == tm.TM_E_INVAL
    assert tm.tm_rowmax_masked(A16, 1000, B16, 8192, 1000, 16, 96, 0, S) == tm.TM_E_UNSUPPORTED
    # softmax statistics: both outputs are checked
    f = tm.tm_softmax_stats
    assert f(A16, 1000, B16, 0, 8192, 1000, 16, 64, 0, S) == tm.TM_E_INVAL        # NULL l
    assert f(A16, 1000, 0, B16, 8192, 1000, 16, 64, 0, S) == tm.TM_E_INVAL        # NULL m
    assert f(A16, 1000, B16, B16 + 6, 8192, 1000, 16, 64, 0, S) == tm.TM_E_INVAL  # l not 4-aligned
    assert f(A16, 1000, B16, B16 + 64, 8192, 1000, 16, 64, 1, S) == tm.TM_E_ALIGN
    assert f(A16, 1000, B16, B16 + 64, 8192, 1000, 16, 48, 0, S) == tm.TM_E_UNSUPPORTED
    assert f(A16, 1000, 0, 0, 0, 1000, 16, 64, 0, S) == tm.TM_OK                  # empty output


@no_gpu
def test_colsum_workspace_and_errors():
    W = tm.tm_colsum_workspace_bytes
    # LDS walk over a wide matrix: room for the strip kernel's 64-row slabs (64 of them here) and
    # for the LDS-staged kernel's (256-row slabs, halved while there would be fewer than 1024
    # (slab, strip) workgroups: 32 slabs of 128 rows), whichever is more
    assert W(4096, 4096, 256, 64, tm.TM_COL_LDS) == 64 * 4096 * 4
    assert W(4096, 4096, 256, 1, tm.TM_COL_NAIVE) == 16 * 4096 * 4
    assert W(4096, 4096, 256, 1, tm.TM_COL_NAIVE_XCD) == 16 * 4096 * 4
    assert W(4096, 4096, 256, 1, 3) == 0
    # the LDS walk's slabs are its own (256 rows; taller past 4096 slabs), not the caller's TM
    assert W(4100, 1000, 64, 64, tm.TM_COL_LDS) == 129 * 1000 * 4   # 8 strips: 32-row slabs
    assert W(4100, 1000, 1, 1, tm.TM_COL_LDS) == 129 * 1000 * 4
    assert W(59048, 59, 1, 1, tm.TM_COL_LDS) == 923 * 59 * 4      # 64-column strips: 64 rows at least
    assert W(65536, 512, 1, 1, tm.TM_COL_LDS) == 256 * 512 * 4    # 256 x 4 workgroups: 256 rows
    assert W(4100, 1000, 64, 1, tm.TM_COL_NAIVE) == 65 * 1000 * 4
    assert W(1 << 21, 8, 256, 8, tm.TM_COL_LDS) == 4096 * 8 * 4
    assert W((1 << 21) + 1, 8, 256, 8, tm.TM_COL_LDS) == 2049 * 8 * 4
    # the LDS walk's one-pass form needs no partials: at most 64 rows, or 256 rows of 2^18 columns
    assert W(64, 1000, 64, 64, tm.TM_COL_LDS) == 0
    assert W(64, 1000, 64, 1, tm.TM_COL_NAIVE) == 1000 * 4
    assert W(65, 1000, 64, 64, tm.TM_COL_LDS) == 3 * 1000 * 4
    assert W(256, 1 << 18, 64, 64, tm.TM_COL_LDS) == 0
    assert W(256, (1 << 18) - 1, 64, 64, tm.TM_COL_LDS) == ((1 << 18) - 1) * 4
    assert W(257, 1 << 18, 64, 64, tm.TM_COL_LDS) == 5 * (1 << 18) * 4   # strip kernel: 64-row slabs
    assert W(0, 1000, 64, 64, tm.TM_COL_LDS) == 0
    assert W(100, 0, 64, 64, tm.TM_COL_LDS) == 0
    assert W(100, 100, 3, 64, tm.TM_COL_LDS) == 0
    assert W(100, 100, 64, 64, 5) == 0
    f = tm.tm_colsum
    need = W(4096, 4096, 256, 64, tm.TM_COL_LDS)
    assert f(A16, 4096, B16, 4096, 4096, 256, 64, 1, 9, A16, need, S) == tm.TM_E_INVAL
    assert f(A16, 4096, B16, 4096, 4096, 256, 64, 1, tm.TM_COL_LDS, 0, need, S) == tm.TM_E_WORKSPACE
    assert f(A16, 4096, B16, 4096, 4096, 256, 64, 1, tm.TM_COL_LDS, A16, need - 4, S) == tm.TM_E_WORKSPACE
    assert f(A16, 4098, B16, 4096, 4096, 256, 64, 1, tm.TM_COL_LDS, A16, need, S) == tm.TM_E_ALIGN
    assert f(A16 + 8, 4096, B16, 4096, 4096, 256, 64, 1, tm.TM_COL_LDS, A16, need, S) == tm.TM_E_ALIGN
    assert f(A16, 4096, B16, 4096, 4096, 200, 64, 1, tm.TM_COL_LDS, A16, need, S) == tm.TM_E_UNSUPPORTED
    # precedence: WORKSPACE before ALIGN (M = 4100 breaks the promise and needs partials)
    assert f(A16, 4096, B16, 4100, 4096, 256, 64, 1, tm.TM_COL_LDS, 0, 0, S) == tm.TM_E_WORKSPACE
    assert f(A16, 4096, B16, 4096, 0, 256, 64, 0, tm.TM_COL_LDS, 0, 0, S) == tm.TM_OK  # empty output
    # a one-pass shape takes no workspace, so a missing one is no error (the promise still is)
    assert f(A16, 4098, B16, 64, 4096, 64, 64, 1, tm.TM_COL_LDS, 0, 0, S) == tm.TM_E_ALIGN
    assert f(A16, 4096, B16, 64, 4096, 64, 64, 1, tm.TM_COL_NAIVE, 0, 0, S) == tm.TM_E_WORKSPACE


@no_gpu
def test_rows_workspace_and_errors():
    W = tm.tm_rows_workspace_bytes
    # fewer than 128 rows of at least 98304 elements are split; K sized for about 2048 segments
    assert W(1, 1 << 23) == 1 * 2048 * 8        # K = 4: segments of 4096
    assert W(8, 1 << 18) == 8 * 256 * 8         # K = 1: segments of 1024
    assert W(63, 98304) == 63 * 48 * 8          # K = 2
    assert W(127, 1 << 20) == 127 * 64 * 8      # K = 16
    assert W(1, 98305) == 97 * 8                # a ragged last segment
    assert W(2, 1 << 30) == 2 * 65536 * 8       # K = 16 at most
    assert W(128, 1 << 20) == 0                 # enough rows: one pass
    assert W(8, 98303) == 0
    assert W(0, 1 << 20) == 0
    assert W(-1, 1 << 20) == 0
    assert W(8, -5) == 0
    M, N = 8, 1 << 18
    need = W(M, N)
    for f in (tm.tm_rowsum_ws, tm.tm_rowmax_masked_ws):
        assert f(A16, N, B16, M, N, 4, 256, 1, 0, need, S) == tm.TM_E_WORKSPACE
        assert f(A16, N, B16, M, N, 4, 256, 1, A16, need - 1, S) == tm.TM_E_WORKSPACE
        assert f(A16, N, B16, M, N, 4, 256, 1, A16 + 2, need, S) == tm.TM_E_WORKSPACE
        assert f(A16, N, B16, M, N, 4, 48, 1, 0, 0, S) == tm.TM_E_UNSUPPORTED   # tile before workspace
        assert f(A16, N - 1, B16, M, N, 4, 256, 1, 0, 0, S) == tm.TM_E_INVAL    # ld < N first
        assert f(A16, N + 2, B16, M, N, 4, 256, 1, 0, 0, S) == tm.TM_E_WORKSPACE  # before ALIGN
        assert f(A16, N + 2, B16, M, N, 4, 256, 1, A16, need, S) == tm.TM_E_ALIGN
        assert f(A16, N, 0, 0, N, 4, 256, 0, 0, 0, S) == tm.TM_OK              # empty output
    f = tm.tm_softmax_stats_ws
    assert f(A16, N, B16, 0, M, N, 4, 256, 0, A16, need, S) == tm.TM_E_INVAL    # NULL l
    assert f(A16, N, B16, B16 + 64, M, N, 4, 256, 0, 0, need, S) == tm.TM_E_WORKSPACE
    assert f(A16, N, B16, B16 + 64, M, N, 4, 256, 1, A16, 16, S) == tm.TM_E_WORKSPACE


@no_gpu
def test_transpose_errors():
    f = tm.tm_transpose
    # x: 64 x 128 (ldx 128), y: 128 x 64 (ldy 64)
    ok = dict(x=A16, ldx=128, bsx=0, y=B16, ldy=64, bsy=0, B=1, M=64, N=128, TM=32, TN=64, aligned=1)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["ldx"], a["bsx"], a["y"], a["ldy"], a["bsy"], a["B"], a["M"], a["N"],
                 a["TM"], a["TN"], a["aligned"], S)

    assert call(M=-1) == tm.TM_E_INVAL
    assert call(B=-1) == tm.TM_E_INVAL
    assert call(ldx=100) == tm.TM_E_INVAL          # ldx < N
    assert call(ldy=60) == tm.TM_E_INVAL           # ldy < M
    assert call(y=0) == tm.TM_E_INVAL
    assert call(B=2, bsy=64 * 127) == tm.TM_E_INVAL   # y batches would overlap
    assert call(TM=24) == tm.TM_E_UNSUPPORTED
    assert call(M=60, ldy=64) == tm.TM_E_ALIGN     # 60 % 32
    assert call(TM=2) == tm.TM_E_ALIGN             # y rows not whole 16-byte chunks
    assert call(ldy=66) == tm.TM_E_ALIGN
    assert call(B=2, bsx=64 * 128 + 2, bsy=128 * 64) == tm.TM_E_ALIGN
    assert call(B=0, x=0, y=0) == tm.TM_OK


@no_gpu
def test_channel_affine_errors():
    f = tm.tm_channel_affine
    C16 = 0x7F0000200000
    assert f(A16, 64, C16, 0, B16, 64, 128, 64, 64, 64, 1, 0, S) == tm.TM_E_INVAL        # NULL bias
    assert f(A16, 64, C16 + 2, C16, B16, 64, 128, 64, 64, 64, 1, 0, S) == tm.TM_E_INVAL  # scale not 4-aligned
    assert f(A16, 64, 0, C16 + 1, B16, 64, 128, 64, 64, 64, 1, 0, S) == tm.TM_E_INVAL    # bias not 4-aligned
    assert f(A16, 64, 0, C16, B16, 64, 130, 64, 64, 64, 1, 0, S) == tm.TM_E_ALIGN        # 130 % 64
    assert f(A16, 64, 0, C16, B16, 64, 128, 64, 64, 48, 0, 0, S) == tm.TM_E_UNSUPPORTED
    assert f(0, 64, 0, 0, 0, 64, 0, 64, 64, 64, 1, 0, S) == tm.TM_OK                     # no work


def test_pad_extents_keep_the_promise():
    """The padded extents keep the oracle's promise predicate and are the smallest that do."""
    for M in range(0, 40):
        for N in range(0, 40):
            for TM in (1, 2, 4, 8, 16):
                for TN in (4, 8, 16, 32):
                    st, Mp, Np, ldp = tm.tm_pad_extents(M, N, TM, TN)
                    assert st == tm.TM_OK
                    assert Mp >= M and Np >= N and ldp >= Np
                    assert oracle.promise_holds(Mp, Np, ldp, ldp, TM, TN, 0x1000, 0x2000)
                    assert not any(oracle.promise_holds(m, Np, ldp, ldp, TM, TN, 0x1000, 0x2000)
                                   for m in range(M, Mp))
                    assert not any(oracle.promise_holds(Mp, n, ldp, ldp, TM, TN, 0x1000, 0x2000)
                                   for n in range(N, Np))
    # the ragged workloads: 4100 x 1000 under 64 x 64 pads to 4160 x 1024
    assert tm.tm_pad_extents(4100, 1000, 64, 64) == (tm.TM_OK, 4160, 1024, 1024)
    assert tm.tm_pad_extents(8192, 1000, 16, 64) == (tm.TM_OK, 8192, 1024, 1024)
    assert tm.tm_pad_extents(10, 10, 4, 2)[0] == tm.TM_E_ALIGN
    assert tm.tm_pad_extents(10, 10, 3, 4)[0] == tm.TM_E_UNSUPPORTED
    assert tm.tm_pad_extents(-1, 10, 4, 4)[0] == tm.TM_E_INVAL


@no_gpu
def test_autotune_errors():
    E = 0x7F0000300000
    args = lambda op=1, x=A16, y=B16, reps=3, e0=E, e1=E: (op, x, 64, y, 64, 64, 64, 1.5, 0.0, 1, 0, reps,
                                                             e0, e1, S)
    assert tm.tm_autotune_map(*args(op=7), table=False)[0] == tm.TM_E_INVAL
    assert tm.tm_autotune_map(*args(reps=0), table=False)[0] == tm.TM_E_INVAL
    assert tm.tm_autotune_map(*args(e0=0))[0] == tm.TM_E_INVAL
    assert tm.tm_autotune_map(*args(y=A16))[0] == tm.TM_E_INVAL          # in place
    assert tm.tm_autotune_map(*args(x=A16 + 2))[0] == tm.TM_E_INVAL      # malformed shared argument
    # NULL result pointers, through the C ABI itself
    lib = ctypes.CDLL(tm.library_path())
    f = lib.tm_autotune_map
    f.restype = ctypes.c_int
    f.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                  ctypes.c_int64, ctypes.c_int64, ctypes.c_float, ctypes.c_float, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    i1, i2, u = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_float(0)
    base = (1, A16, 64, B16, 64, 64, 64, 1.5, 0.0, 1, 0, 3, E, E)
    assert f(*base, None, ctypes.byref(i2), ctypes.byref(u), None, S) == tm.TM_E_INVAL
    assert f(*base, ctypes.byref(i1), None, ctypes.byref(u), None, S) == tm.TM_E_INVAL
    assert f(*base, ctypes.byref(i1), ctypes.byref(i2), None, None, S) == tm.TM_E_INVAL
