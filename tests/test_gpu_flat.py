"""GPU parity of the maps over one contiguous row in 1 KiB work items (mapflat.hip), the kernel that
every view with contiguous rows on 128-byte lines reaches: rows of every length around the 256-element
item boundaries (whole items only, a ragged last item of 1 .. 255 elements), in the three access
kinds (16-byte chunks, four 4-byte elements per lane, one element per thread), for the affine map,
the scale and the copy, on the ragged and the aligned path.  Bit for bit against the oracle, with
line-sized 0x7F guard bands before and after the output.  Also the row walk that honours the
caller's column tile: the walk tm_row_walk reports is the one whose results are checked.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from edge_masking_vector_amd import inputs
from gpu_helpers import LINE_GUARD_FLOATS, Guarded, bits, sentinel_host

pytestmark = pytest.mark.gpu

tm = pytest.importorskip("edge_masking_vector_amd.tilemap")


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


LENGTHS = [1, 3, 4, 5, 63, 64, 255, 256, 257, 511, 512, 513, 1023, 1025, 4096 * 3 + 7, 65536, 1000003]
VARIANTS = [tm.TM_VAR_AUTO, tm.TM_VAR_SCALAR, tm.TM_VAR_VEC4]


def _run(op, X, Y, M, N, TM, TN, aligned, variant, alpha, beta):
    s = torch.cuda.current_stream()
    if op == "affine":
        return tm.tm_map_affine(X.ptr, N, Y.ptr, N, M, N, alpha, beta, TM, TN, aligned, variant, s)
    if op == "scale":
        return tm.tm_scale2d(X.ptr, N, Y.ptr, N, M, N, alpha, TM, TN, aligned, variant, s)
    return tm.tm_copy2d(X.ptr, N, Y.ptr, N, M, N, TM, TN, aligned, variant, s)


def _ref(op, x, y, M, N, alpha, beta):
    if op == "affine":
        oracle.map_affine(x, N, y, N, M, N, alpha, beta)
    elif op == "scale":
        oracle.scale2d(x, N, y, N, M, N, alpha)
    else:
        oracle.copy2d(x, N, y, N, M, N)


def _check(dev, op, M, N, TM, TN, aligned, variant, seed, alpha=0.75, beta=-0.25, expect=tm.TM_OK):
    n = M * N
    xh = inputs.uniform(seed, n, -8.0, 8.0)
    if op == "copy" and n >= 4:
        xh[:4] = np.array([0x7FC0BEEF, 0x80000000, 0x00000001, 0xFF800000], np.uint32).view(np.float32)
    X = Guarded(n, dev, guard=LINE_GUARD_FLOATS)   # the row starts on a 128-byte line
    X.upload(xh)
    Y = Guarded(n, dev, guard=LINE_GUARD_FLOATS)
    st = _run(op, X, Y, M, N, TM, TN, aligned, variant, alpha, beta)
    assert st == expect, (op, M, N, TM, TN, aligned, variant, tm.tm_status_string(st))
    torch.cuda.synchronize()
    want = sentinel_host(Y.buf.numel())
    if st == tm.TM_OK:   # a refused call writes nothing
        region = want[Y.off:Y.off + n].copy()
        _ref(op, xh, region, M, N, alpha, beta)
        want[Y.off:Y.off + n] = region
    assert np.array_equal(bits(Y.host()), bits(want)), (op, M, N, TM, TN, aligned, variant)
    assert X.guards_intact()


@pytest.mark.parametrize("op", ["affine", "scale", "copy"])
@pytest.mark.parametrize("variant", VARIANTS)
def test_flat_row_every_tail(dev, op, variant):
    """One row (M = 1) on the ragged path: every length around the item boundaries."""
    for k, n in enumerate(LENGTHS):
        note("flat row %s variant %d n %d" % (op, variant, n))
        _check(dev, op, 1, n, 1, 64, 0, variant, seed=1000 + k)


@pytest.mark.parametrize("variant", VARIANTS)
def test_flat_contiguous_2d_views(dev, variant):
    """Views with contiguous rows are one flat row: the ragged 4100 x 1000 workload, a view whose
    flat length is not a multiple of 4 (the last chunk straddles the end), and aligned views."""
    cases = [(4100, 1000, 64, 64, 0), (333, 17, 4, 16, 0), (7, 3, 1, 1, 0),
             (4096, 1024, 64, 64, 1), (256, 512, 32, 128, 1), (64, 12, 4, 4, 1)]
    for k, (M, N, TM, TN, aligned) in enumerate(cases):
        note("flat view %dx%d tile %dx%d aligned %d variant %d" % (M, N, TM, TN, aligned, variant))
        # 16-byte vectors asked for on rows off the 16-byte grid (row stride N % 4 != 0) are refused
        expect = tm.TM_E_ALIGN if variant == tm.TM_VAR_VEC4 and N % 4 else tm.TM_OK
        _check(dev, "affine", M, N, TM, TN, aligned, variant, seed=2000 + k, expect=expect)


def test_flat_scale_4096_full_size(dev):
    """The scale workload itself (4096 x 4096, 32 x 128 tiles, aligned, 16-byte chunks): bit for
    bit equal to alpha * x computed exactly in double and rounded once (exact for alpha = 1.5)."""
    M = N = 4096
    xh = inputs.scale_input(M, N)
    x = torch.from_numpy(xh).to(dev)
    y = torch.full_like(x, float("nan"))
    tm.check(tm.tm_scale2d(x, N, y, N, M, N, 1.5, 32, 128, 1, tm.TM_VAR_VEC4))
    want = (xh.astype(np.float64) * 1.5).astype(np.float32)
    assert np.array_equal(bits(y), bits(want))


def test_flat_large_row_loops(dev):
    """A row of more than 2^20 work items (2^28 + 77 floats, 1 GiB): the grid is capped and each
    workgroup loops; every element and the ragged end are still moved exactly once.  Checked on
    samples (the oracle on a stride of elements) and on the ends."""
    n = (1 << 28) + 77
    free, total = torch.cuda.mem_get_info()
    if free < 3 * 4 * n:
        pytest.skip("needs 3 GiB of free device memory")
    note("flat row of %d floats" % n)
    x = torch.arange(n, dtype=torch.float32, device=dev) * 0.5
    y = torch.full((n,), -1.0, device=dev)
    tm.check(tm.tm_map_affine(x, n, y, n, 1, n, 2.0, 1.0, 1, 1024, 0, tm.TM_VAR_VEC4))
    idx = torch.cat([torch.arange(0, 300, device=dev), torch.arange(n - 300, n, device=dev),
                     torch.randint(0, n, (100000,), device=dev, generator=torch.Generator(dev).manual_seed(3))])
    got = y[idx].cpu().numpy()
    xs = x[idx].cpu().numpy()
    want = np.empty_like(xs)
    oracle.map_affine(xs, xs.size, want, xs.size, 1, xs.size, 2.0, 1.0)
    assert np.array_equal(bits(got), bits(want))
    del x, y


# ---- the row walk honours the caller's column tile -----------------------------------------------

@pytest.mark.parametrize("BC,ld", [(64, 1000), (128, 1000), (256, 1000), (1024, 1000), (64, 1001), (16, 1000)])
def test_rowmax_walk_reported_and_exact(dev, BC, ld):
    """8192 x 1000 scores, all negative, masked row maximum and softmax statistics under BR x BC
    tiles: the walk tm_row_walk reports splits N by its tile as the oracle's splitter does, and
    the maxima equal the oracle bit for bit whichever tile the walk takes (BC = 64: 15 whole tiles
    and one of 40 columns, as 'Reductions over a ragged tile' walks it)."""
    M, N = 8192, 1000
    sh = inputs.matrix(inputs.scores_input(M, N), M, N, ld)
    s = torch.from_numpy(sh).to(dev)
    st, bc, nfull, rem, lanes = tm.tm_row_walk(M, N, ld, 16, BC, 0, s)
    assert st == tm.TM_OK and (nfull, rem) == oracle.split(N, bc)
    if BC == 64:
        assert (bc, nfull, rem) == (64, 15, 40)
    note("rowmax walk BC=%d ld=%d: bc %d, %d + %d, %d lanes" % (BC, ld, bc, nfull, rem, lanes))
    out = torch.empty(M, device=dev)
    tm.check(tm.tm_rowmax_masked(s, ld, out, M, N, 16, BC, 0))
    want = oracle.rowmax(sh, ld, M, N)
    assert np.array_equal(bits(out), bits(want))
    assert (out.cpu().numpy() < -1.0).all()   # never the 0 a zero fill would give
    m = torch.empty(M, device=dev)
    l = torch.empty(M, device=dev)
    tm.check(tm.tm_softmax_stats(s, ld, m, l, M, N, 16, BC, 0))
    wm, wl = oracle.softmax_stats(sh, ld, M, N)
    assert np.array_equal(bits(m), bits(wm))
    assert np.allclose(l.cpu().numpy(), wl, rtol=1e-5, atol=0)


# ---- padded rows in one span (mapflat.hip, map_rows) -------------------------------------------
def _check_strided(dev, op, M, N, ldx, ldy, xoff, yoff, variant, seed, alpha=0.75, beta=-0.25, walk=None):
    nx, ny = (M - 1) * ldx + N, (M - 1) * ldy + N
    xh = inputs.uniform(seed, nx, -8.0, 8.0)
    X = Guarded(nx, dev, offset=xoff, guard=LINE_GUARD_FLOATS)
    X.upload(xh)
    Y = Guarded(ny, dev, offset=yoff, guard=LINE_GUARD_FLOATS)
    s = torch.cuda.current_stream()
    if walk is not None:
        assert tm.tm_map_walk(0, X.ptr, ldx, Y.ptr, ldy, M, N, 64, 64, 0, variant)[:2] == (tm.TM_OK, walk)
    if op == "affine":
        st = tm.tm_map_affine(X.ptr, ldx, Y.ptr, ldy, M, N, alpha, beta, 64, 64, 0, variant, s)
    elif op == "scale":
        st = tm.tm_scale2d(X.ptr, ldx, Y.ptr, ldy, M, N, alpha, 64, 64, 0, variant, s)
    else:
        st = tm.tm_copy2d(X.ptr, ldx, Y.ptr, ldy, M, N, 64, 64, 0, variant, s)
    assert st == tm.TM_OK, tm.tm_status_string(st)
    torch.cuda.synchronize()
    want = sentinel_host(Y.buf.numel())
    region = want[Y.off:Y.off + ny].copy()   # the padding between rows keeps its sentinels
    if op == "affine":
        oracle.map_affine(xh, ldx, region, ldy, M, N, alpha, beta)
    elif op == "scale":
        oracle.scale2d(xh, ldx, region, ldy, M, N, alpha)
    else:
        oracle.copy2d(xh, ldx, region, ldy, M, N)
    want[Y.off:Y.off + ny] = region
    assert np.array_equal(bits(Y.host()), bits(want)), (op, M, N, ldx, ldy, xoff, yoff, variant)
    assert X.guards_intact()


@pytest.mark.parametrize("op,M,N,ld,off,variant", [
    ("affine", 3, 64, 65, 0, tm.TM_VAR_AUTO),         # the smallest rows taken, one float of padding
    ("scale", 7, 299, 320, 1, tm.TM_VAR_AUTO),        # the span starts 1 float past a line
    ("copy", 100, 1000, 1001, 3, tm.TM_VAR_AUTO),     # rows off the 16-byte grid
    ("affine", 100, 1000, 1004, 0, tm.TM_VAR_VEC4),   # 16-byte rows, a chunk of padding per row
    ("affine", 50, 4100, 4104, 2, tm.TM_VAR_AUTO),    # bases 8 bytes off the 16-byte grid
    ("scale", 1000, 257, 288, 5, tm.TM_VAR_AUTO),     # 31 floats of padding, ragged row ends
    ("copy", 513, 777, 808, 64, tm.TM_VAR_AUTO),      # the span starts mid 1 KiB block
    ("affine", 4100, 1000, 1001, 0, tm.TM_VAR_AUTO),  # the padded 4100 x 1000 workload
])
def test_padded_rows_one_span(dev, op, M, N, ld, off, variant):
    """Rows with less than a line of padding and one stride in both tensors are moved as one span
    of 1 KiB items on y's 1 KiB grid, 16-byte chunks whose columns past N are masked ([SLICING]
    "Masking": nothing past the view's edge is stored): bit for bit, the padding between rows and
    the guard bands untouched."""
    note("span %s %dx%d ld %d off %d variant %d" % (op, M, N, ld, off, variant))
    _check_strided(dev, op, M, N, ld, ld, off, off, variant, seed=M + N + ld)


@pytest.mark.parametrize("M,N,ldx,ldy,xoff,yoff", [
    (100, 1000, 1004, 1008, 0, 0),    # different strides over 16-byte rows under 1024 floats
    (100, 60, 61, 61, 0, 0),          # rows narrower than the span's minimum
    (100, 1000, 1500, 1500, 0, 0),    # half a row of padding, 16-byte rows under 2048 floats
    (50, 2048, 3072, 3072, 0, 0),     # wide padding between rows on the line grid
])
def test_padded_rows_outside_the_span(dev, M, N, ldx, ldy, xoff, yoff):
    """Padded views the span does not take (different strides or base offsets, narrow rows, wide
    padding on the 16-byte grid or on the line grid) keep the 2-D tile plan: the same results bit
    for bit."""
    note("no span %dx%d ldx %d ldy %d" % (M, N, ldx, ldy))
    _check_strided(dev, "affine", M, N, ldx, ldy, xoff, yoff, tm.TM_VAR_AUTO, seed=7 * M + N)


@pytest.mark.parametrize("ld,off", [(1003, 0), (1001, 1)])
def test_padded_rows_in_place(dev, ld, off):
    """x == y over padded rows (the span plan): every live element mapped once, the padding between
    rows untouched, as the oracle's out-of-place result."""
    M, N = 777, 1000
    n = (M - 1) * ld + N
    xh = inputs.uniform(41 + ld, n, -8.0, 8.0)
    X = Guarded(n, dev, offset=off, guard=LINE_GUARD_FLOATS)
    X.upload(xh)
    note("span in place %dx%d ld %d off %d" % (M, N, ld, off))
    assert tm.tm_map_affine(X.ptr, ld, X.ptr, ld, M, N, 0.75, -0.25, 64, 64, 0, tm.TM_VAR_AUTO) == tm.TM_OK
    torch.cuda.synchronize()
    want = sentinel_host(X.buf.numel())
    region = xh.copy()   # the padding keeps the input's values
    oracle.map_affine(xh, ld, region, ld, M, N, 0.75, -0.25)
    want[X.off:X.off + n] = region
    assert np.array_equal(bits(X.host()), bits(want))


SPAN, TILES = tm.TM_MAP_SPAN, tm.TM_MAP_TILES


@pytest.mark.parametrize("M,N,ldx,ldy,TM,TN,variant,walk,xoff", [
    (4100, 1000, 1001, 1001, 64, 64, tm.TM_VAR_AUTO, SPAN, 0),     # the bench's padded maps
    (4100, 1000, 1004, 1004, 64, 64, tm.TM_VAR_VEC4, SPAN, 0),
    (4100, 4100, 4104, 4104, 32, 128, tm.TM_VAR_VEC4, SPAN, 0),
    (4100, 4100, 4104, 4108, 32, 128, tm.TM_VAR_VEC4, SPAN, 0),    # different strides
    (4100, 4100, 4700, 4700, 32, 128, tm.TM_VAR_VEC4, SPAN, 0),    # 600 floats of padding
    (4100, 4100, 4104, 4104, 32, 128, tm.TM_VAR_AUTO, SPAN, 1),    # x one float past y's 16-byte phase
    (4100, 1000, 1004, 1008, 64, 64, tm.TM_VAR_VEC4, TILES, 0),
    (4100, 4100, 5120, 5120, 32, 128, tm.TM_VAR_VEC4, TILES, 0),
])
def test_bench_padded_maps_full_size(dev, M, N, ldx, ldy, TM, TN, variant, walk, xoff):
    """The padded-row maps the benchmark times, at their full sizes and in the same calls (ragged
    path, the same tiles and variants), bit for bit against the oracle, padding untouched, and on
    the plan the benchmark labels them with (tm_map_walk)."""
    note("bench padded map %dx%d ld %d/%d x offset %d" % (M, N, ldx, ldy, xoff))
    nx, ny = (M - 1) * ldx + N, (M - 1) * ldy + N
    xh = inputs.matrix(inputs.ragged_input(M, N, seed=12), M, N, ldx)[:nx].copy()
    X = Guarded(nx, dev, offset=xoff, guard=LINE_GUARD_FLOATS)
    X.upload(xh)
    Y = Guarded(ny, dev, guard=LINE_GUARD_FLOATS)
    assert tm.tm_map_walk(0, X.ptr, ldx, Y.ptr, ldy, M, N, TM, TN, 0, variant)[:2] == (tm.TM_OK, walk)
    assert tm.tm_map_affine(X.ptr, ldx, Y.ptr, ldy, M, N, 0.75, -0.25, TM, TN, 0, variant) == tm.TM_OK
    torch.cuda.synchronize()
    want = sentinel_host(Y.buf.numel())
    region = want[Y.off:Y.off + ny].copy()
    oracle.map_affine(xh, ldx, region, ldy, M, N, 0.75, -0.25)
    want[Y.off:Y.off + ny] = region
    assert np.array_equal(bits(Y.host()), bits(want))


@pytest.mark.parametrize("M,N,ld,off,boff,with_scale", [
    (300, 1000, 1004, 0, 0, False),   # 16-byte rows, bias as 16-byte vectors
    (300, 1000, 1004, 0, 1, True),    # vectors off their 16-byte grid: gathered one by one
    (257, 777, 800, 3, 0, True),      # rows off the 16-byte grid
    (100, 4100, 4140, 0, 0, False),   # 40 floats of padding: chunks wholly inside it load live data
    (64, 2000, 2250, 1, 2, True),     # padding of an eighth of the row
])
def test_padded_rows_channel_span(dev, M, N, ld, off, boff, with_scale):
    """The per-channel op over padded rows in one span: element (i, j) takes channel j, bit for
    bit against the oracle (one fmaf, scale 1 when absent), the padding untouched."""
    note("span channel %dx%d ld %d off %d boff %d scale %d" % (M, N, ld, off, boff, with_scale))
    n = (M - 1) * ld + N
    xh = inputs.uniform(61 + ld, n, -8.0, 8.0)
    bh = inputs.uniform(62 + ld, N, -1.0, 1.0)
    sh = inputs.uniform(63 + ld, N, 0.5, 1.5) if with_scale else None
    X = Guarded(n, dev, offset=off, guard=LINE_GUARD_FLOATS)
    X.upload(xh)
    Y = Guarded(n, dev, offset=off, guard=LINE_GUARD_FLOATS)
    B = Guarded(N, dev, offset=boff)
    B.upload(bh)
    S = None
    if with_scale:
        S = Guarded(N, dev, offset=boff)
        S.upload(sh)
    st = tm.tm_channel_affine(X.ptr, ld, S.ptr if S is not None else None, B.ptr, Y.ptr, ld, M, N, 64, 64, 0,
                              tm.TM_VAR_AUTO)
    assert st == tm.TM_OK, tm.tm_status_string(st)
    torch.cuda.synchronize()
    want = sentinel_host(Y.buf.numel())
    region = want[Y.off:Y.off + n].copy()
    oracle.channel_affine(xh, ld, sh, bh, region, ld, M, N)
    want[Y.off:Y.off + n] = region
    assert np.array_equal(bits(Y.host()), bits(want))
    assert X.guards_intact() and B.guards_intact()


@pytest.mark.parametrize("M,N,ld,off", [
    (100, 4100, 4140, 0), (300, 1000, 1125, 2), (41, 561, 593, 1),   # up to an eighth of the row
    (64, 4100, 4700, 0),     # a quarter of 16-byte rows of 2048 floats or more
    (100, 1000, 1201, 0),    # a quarter of rows off the 16-byte grid
    (40, 2500, 3750, 1),     # half of rows off the 16-byte grid, 2048 floats or more
    (16, 2048, 3072, 2),     # ... rows on the 16-byte grid, base off it
])
def test_padded_rows_wide_padding(dev, M, N, ld, off):
    """Padding of a line or more is still one span (up to an eighth of the row, or wider off the
    line grid); chunks wholly inside it load the row's last live chunk and store nothing, and
    waves wholly inside it exit at once."""
    note("span wide padding %dx%d ld %d off %d" % (M, N, ld, off))
    _check_strided(dev, "affine", M, N, ld, ld, off, off, tm.TM_VAR_AUTO, seed=M * 7 + ld)


@pytest.mark.parametrize("op,M,N,ldx,ldy,off", [
    ("affine", 300, 1100, 1104, 1108, 0),   # x rows 4 floats shorter than y's
    ("affine", 300, 1100, 1108, 1104, 0),   # ... and longer
    ("copy", 300, 1024, 1024, 1028, 0),     # x contiguous, y padded
    ("scale", 300, 1100, 1140, 1100, 2),    # x padded by 40, y contiguous
    ("affine", 257, 1777, 2801, 1781, 3),   # x padding far wider than y's
    ("affine", 64, 4100, 4104, 4108, 0),
    ("scale", 64, 4100, 4104, 4700, 0),     # y padded by 600 floats
    ("affine", 300, 1100, 1101, 1104, 1),   # strides 3 apart: x's chunks 4-byte aligned
    ("affine", 300, 1000, 1004, 1008, 0),   # 16-byte rows under 1024 floats: the 2-D tile plan
    ("affine", 300, 1000, 1003, 1007, 0),   # ... rows off the 16-byte grid: the span at any width
    ("copy", 500, 135, 138, 135, 1),        # narrow rows, y contiguous
])
def test_padded_rows_different_strides(dev, op, M, N, ldx, ldy, off):
    """Rows of 1024 floats or more with different strides in x and y (a multiple of 4 floats
    apart) as one span over y: the chunk of a row sits (ldx - ldy) floats further on in x per row,
    and a chunk that crosses a row's end takes the next row's elements from a second load; bit for
    bit, the padding of y untouched."""
    note("span %s %dx%d ldx %d ldy %d off %d" % (op, M, N, ldx, ldy, off))
    _check_strided(dev, op, M, N, ldx, ldy, off, off, tm.TM_VAR_AUTO, seed=M + 3 * ldx + ldy)


@pytest.mark.parametrize("op,M,N,ldx,ldy,xoff,yoff", [
    ("affine", 300, 1000, 1004, 1004, 1, 0),    # one stride, x one float past y's 16-byte phase
    ("scale", 300, 1000, 1001, 1001, 2, 1),     # rows off the 16-byte grid too
    ("copy", 257, 777, 800, 800, 3, 0),
    ("affine", 100, 4100, 4104, 4104, 1, 0),
    ("affine", 64, 4100, 4700, 4700, 2, 0),     # wide padding
    ("affine", 50, 2048, 3071, 3071, 1, 3),     # half a row of padding off the 16-byte grid
    ("affine", 300, 1100, 1107, 1104, 1, 2),    # strides 3 apart and bases at other phases
    ("copy", 64, 2048, 2049, 2048, 0, 0),       # y contiguous, x rows one float longer
    ("scale", 64, 2048, 2049, 2053, 3, 0),      # x rows shorter than y's
    ("affine", 100, 1000, 1000, 1000, 1, 0),    # contiguous rows: one row, x at another phase
    ("scale", 4096, 64, 64, 64, 2, 0),
    ("copy", 1, 100003, 100003, 100003, 3, 1),
    ("affine", 100, 1000, 1000, 1000, 4, 4),    # one phase, bases off the 128-byte line grid
    ("scale", 1, 65536, 65536, 65536, 8, 8),
    ("affine", 3, 64, 64, 64, 1, 0),            # a row of 192 floats: every chunk at an end
])
def test_shifted_phase_spans(dev, op, M, N, ldx, ldy, xoff, yoff):
    """x at another 4-byte phase than y's 1 KiB grid (bases not a multiple of 16 bytes apart,
    strides not a multiple of 4 floats apart), and contiguous views whose bases miss the 128-byte
    line grid: one span over y, x's chunks loaded as 4-byte aligned 16-byte vectors and the
    span's end chunks element by element; bit for bit, padding and guards untouched."""
    note("shifted span %s %dx%d ldx %d ldy %d offs %d,%d" % (op, M, N, ldx, ldy, xoff, yoff))
    _check_strided(dev, op, M, N, ldx, ldy, xoff, yoff, tm.TM_VAR_AUTO, seed=M + 5 * N + ldx + xoff,
                   walk=tm.TM_MAP_SPAN)


def test_shifted_phase_channel(dev):
    """The per-channel op over padded rows with x one float past y's phase."""
    M, N, ld = 300, 1000, 1004
    n = (M - 1) * ld + N
    xh = inputs.uniform(81, n, -8.0, 8.0)
    bh = inputs.uniform(82, N, -1.0, 1.0)
    sh = inputs.uniform(83, N, 0.5, 1.5)
    X = Guarded(n, dev, offset=1, guard=LINE_GUARD_FLOATS)
    X.upload(xh)
    Y = Guarded(n, dev, guard=LINE_GUARD_FLOATS)
    B = Guarded(N, dev)
    B.upload(bh)
    S = Guarded(N, dev)
    S.upload(sh)
    assert tm.tm_map_walk(3, X.ptr, ld, Y.ptr, ld, M, N, 64, 64, 0, 0, B.ptr)[:2] == (tm.TM_OK, tm.TM_MAP_SPAN)
    st = tm.tm_channel_affine(X.ptr, ld, S.ptr, B.ptr, Y.ptr, ld, M, N, 64, 64, 0, tm.TM_VAR_AUTO)
    assert st == tm.TM_OK, tm.tm_status_string(st)
    torch.cuda.synchronize()
    want = sentinel_host(Y.buf.numel())
    region = want[Y.off:Y.off + n].copy()
    oracle.channel_affine(xh, ld, sh, bh, region, ld, M, N)
    want[Y.off:Y.off + n] = region
    assert np.array_equal(bits(Y.host()), bits(want))


def test_padded_rows_different_strides_channel(dev):
    """The per-channel op over different strides in one span."""
    M, N, ldx, ldy = 300, 1100, 1112, 1104
    n_x, n_y = (M - 1) * ldx + N, (M - 1) * ldy + N
    xh = inputs.uniform(71, n_x, -8.0, 8.0)
    bh = inputs.uniform(72, N, -1.0, 1.0)
    sh = inputs.uniform(73, N, 0.5, 1.5)
    X = Guarded(n_x, dev, guard=LINE_GUARD_FLOATS)
    X.upload(xh)
    Y = Guarded(n_y, dev, guard=LINE_GUARD_FLOATS)
    B = Guarded(N, dev)
    B.upload(bh)
    S = Guarded(N, dev)
    S.upload(sh)
    note("span channel %dx%d ldx %d ldy %d" % (M, N, ldx, ldy))
    assert tm.tm_channel_affine(X.ptr, ldx, S.ptr, B.ptr, Y.ptr, ldy, M, N, 64, 64, 0, tm.TM_VAR_AUTO) == tm.TM_OK
    torch.cuda.synchronize()
    want = sentinel_host(Y.buf.numel())
    region = want[Y.off:Y.off + n_y].copy()
    oracle.channel_affine(xh, ldx, sh, bh, region, ldy, M, N)
    want[Y.off:Y.off + n_y] = region
    assert np.array_equal(bits(Y.host()), bits(want))
