"""GPU parity of the tiled maps (tm_map_affine, tm_scale2d, tm_copy2d, tm_channel_affine) against
the CPU oracle, through the C ABI.  Maps are compared bit for bit; every output sits between 0x7F
guard bands (64 bytes, or one 128-byte line where the views must start on lines) and its padding
columns start as 0x7F, and all of those bytes must survive the call.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from edge_masking_vector_amd import inputs
from gpu_helpers import (GUARD_FLOATS, LINE_GUARD_FLOATS, SENTINEL, SENTINEL_BITS, Guarded, bits,
                         sentinel_buffer, sentinel_host)

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


def run_map(op, x, ldx, y, ldy, M, N, alpha, beta, TM, TN, aligned, variant):
    s = torch.cuda.current_stream()
    if op == "affine":
        return tm.tm_map_affine(x, ldx, y, ldy, M, N, alpha, beta, TM, TN, aligned, variant, s)
    if op == "scale":
        return tm.tm_scale2d(x, ldx, y, ldy, M, N, alpha, TM, TN, aligned, variant, s)
    return tm.tm_copy2d(x, ldx, y, ldy, M, N, TM, TN, aligned, variant, s)


def ref_map(op, x, ldx, y, ldy, M, N, alpha, beta):
    if op == "affine":
        oracle.map_affine(x, ldx, y, ldy, M, N, alpha, beta)
    elif op == "scale":
        oracle.scale2d(x, ldx, y, ldy, M, N, alpha)
    else:
        oracle.copy2d(x, ldx, y, ldy, M, N)


def check_case(dev, op, M, N, ldx, ldy, TM, TN, aligned, variant, xh, alpha=0.75, beta=-0.25,
               xoff=0, yoff=0, expect=tm.TM_OK, guard=GUARD_FLOATS):
    """Run one map with guarded input and output and compare with the oracle bit for bit."""
    nx = max((M - 1) * ldx + N if M > 0 and N > 0 else 0, 1)
    ny = M * ldy if M > 0 else 0
    X = Guarded(nx, dev, xoff, guard)
    X.upload(np.resize(xh, nx).astype(np.float32))
    Y = Guarded(ny, dev, yoff, guard)
    st = run_map(op, X.ptr, ldx, Y.ptr, ldy, M, N, alpha, beta, TM, TN, aligned, variant)
    assert st == expect, (op, M, N, ldx, ldy, TM, TN, aligned, variant, tm.tm_status_string(st))
    torch.cuda.synchronize()
    want = sentinel_host(Y.buf.numel())
    if st == tm.TM_OK and M > 0 and N > 0:
        xin = X.host()[X.off:X.off + X.n].copy()
        region = want[Y.off:Y.off + Y.n].copy()
        ref_map(op, xin, ldx, region, ldy, M, N, alpha, beta)
        want[Y.off:Y.off + Y.n] = region
    got = Y.host()
    assert np.array_equal(bits(got), bits(want)), (op, M, N, ldx, ldy, TM, TN, aligned, variant)
    assert X.guards_intact()


# ---- the workload shapes at full size -----------------------------------------------------------

@pytest.mark.parametrize("variant,TN,aligned", [(tm.TM_VAR_SCALAR, 256, 1), (tm.TM_VAR_VEC4_UNDERSTATED, 1024, 1),
                                                (tm.TM_VAR_VEC4, 1024, 1), (tm.TM_VAR_VEC4, 1024, 0)])
def test_map1d_three_variants_closed_form(dev, variant, TN, aligned):
    """The 1M-element a*2+1 map, in each of the three access variants and on the ragged path,
    equals the closed form (k - 2**22) * 2**-22 computed from the generator's integers -- and
    hence the oracle."""
    n = 1 << 20
    note("map1d variant=%d TN=%d aligned=%d" % (variant, TN, aligned))
    a = inputs.map1d_input(n)
    k = inputs.u24(1, n)
    want = ((k - 2 ** 22) * 2.0 ** -22).astype(np.float32)
    x = torch.from_numpy(a).to(dev)
    Y = Guarded(n, dev)
    assert tm.tm_map_affine(x, n, Y.ptr, n, 1, n, 2.0, 1.0, 1, TN, aligned, variant) == tm.TM_OK
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y.payload()), bits(want))
    assert Y.guards_intact()
    ref = np.empty(n, np.float32)
    oracle.map_affine(a, n, ref, n, 1, n, 2.0, 1.0)
    assert np.array_equal(bits(Y.payload()), bits(ref))


def test_map1d_ragged_path_matches(dev):
    """The same map through the ragged path (aligned=0) on a length that is not a multiple of
    the tile or of 4."""
    n = (1 << 20) - 3
    a = inputs.map1d_input(n)
    for variant in (tm.TM_VAR_AUTO, tm.TM_VAR_SCALAR, tm.TM_VAR_VEC4_UNDERSTATED, tm.TM_VAR_VEC4):
        note("map1d ragged variant=%d" % variant)
        check_case(dev, "affine", 1, n, n, n, 1, 1024, 0, variant, a, 2.0, 1.0)


@pytest.mark.parametrize("aligned,variant", [(1, tm.TM_VAR_VEC4), (1, tm.TM_VAR_AUTO),
                                             (0, tm.TM_VAR_VEC4), (1, tm.TM_VAR_SCALAR),
                                             (1, tm.TM_VAR_VEC4_UNDERSTATED)])
def test_scale_4096(dev, aligned, variant):
    """Y = 1.5 X on the 4096 x 4096 N(0,1) matrix with 32 x 128 tiles, aligned and ragged paths."""
    M = N = 4096
    note("scale4096 aligned=%d variant=%d" % (aligned, variant))
    xh = inputs.scale_input(M, N)
    x = torch.from_numpy(xh).to(dev)
    Y = Guarded(M * N, dev)
    assert tm.tm_scale2d(x, N, Y.ptr, N, M, N, 1.5, 32, 128, aligned, variant) == tm.TM_OK
    torch.cuda.synchronize()
    want = np.empty_like(xh)
    oracle.scale2d(xh, N, want, N, M, N, 1.5)
    assert np.array_equal(bits(Y.payload()), bits(want))
    assert Y.guards_intact()


def test_ragged_affine_4100x1000_guards(dev):
    """Y = fmaf(X, 0.75, -0.25) on 4100 x 1000 under 64 x 64 tiles (65 x 16 tiles, 80 of them at
    an edge): bit-exact, guard bands untouched.  Rows are contiguous here, so the library walks
    the view as one row of 4.1M elements."""
    M, N = 4100, 1000
    xh = inputs.ragged_input(M, N)
    for variant in (tm.TM_VAR_AUTO, tm.TM_VAR_VEC4, tm.TM_VAR_SCALAR, tm.TM_VAR_VEC4_UNDERSTATED):
        note("ragged4100 variant=%d" % variant)
        check_case(dev, "affine", M, N, N, N, 64, 64, 0, variant, xh)


@pytest.mark.parametrize("ldx,ldy", [(1001, 1001), (1000, 1004), (1004, 1000), (1004, 1004)])
def test_ragged_affine_4100x1000_padded_rows(dev, ldx, ldy):
    """The same map over views whose rows are not contiguous in at least one tensor: the 2-D
    schedule (work items spanning the row band, rows off the 128-byte line grid or with 16-byte
    rows but ragged tiles), every padding column left at its 0x7F pre-fill."""
    M, N = 4100, 1000
    xh = inputs.uniform(31 + ldx + ldy, (M - 1) * ldx + N, -8.0, 8.0)
    for variant in (tm.TM_VAR_AUTO, tm.TM_VAR_SCALAR, tm.TM_VAR_VEC4_UNDERSTATED, tm.TM_VAR_VEC4):
        vec_ok = ldx % 4 == 0 and ldy % 4 == 0
        expect = tm.TM_E_ALIGN if variant == tm.TM_VAR_VEC4 and not vec_ok else tm.TM_OK
        note("ragged4100 ld=%d/%d variant=%d" % (ldx, ldy, variant))
        check_case(dev, "affine", M, N, ldx, ldy, 64, 64, 0, variant, xh, expect=expect)


def test_ragged_shape_refuses_aligned_and_writes_nothing(dev):
    """The promise is broken on 4100 x 1000 with 64 x 64 tiles: TM_E_ALIGN, and the output buffer
    -- guards included -- is byte-identical to its pre-fill."""
    M, N = 4100, 1000
    xh = inputs.ragged_input(M, N)
    x = torch.from_numpy(xh).to(dev)
    Y = Guarded(M * N, dev)
    before = bits(Y.buf).copy()
    for variant in (tm.TM_VAR_AUTO, tm.TM_VAR_VEC4, tm.TM_VAR_SCALAR):
        assert tm.tm_map_affine(x, N, Y.ptr, N, M, N, 0.75, -0.25, 64, 64, 1, variant) == tm.TM_E_ALIGN
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y.buf), before)


def test_aligned_counterpart_4096x1024(dev):
    M, N = 4096, 1024
    xh = inputs.ragged_input(M, N)
    note("aligned 4096x1024")
    check_case(dev, "affine", M, N, N, N, 64, 64, 1, tm.TM_VAR_VEC4, xh)


# ---- ops, variants, strides and tiles ----------------------------------------------------------

SHAPES = [
    # M, N, ldx, ldy
    (37, 45, 48, 52),      # ragged both ways, padded strides (16-byte rows)
    (100, 1000, 1000, 1000),
    (65, 130, 131, 133),   # strides not multiples of 4: 16-byte path illegal
    (300, 1001, 1004, 1004),  # N % 4 != 0 with 16-byte rows: chunks straddle column N
    (1, 5000, 5000, 5000),
    (513, 7, 7, 9),
]
TILES = [(8, 8), (16, 64), (32, 128), (64, 64), (1, 1024), (256, 4), (256, 1024), (2, 2)]


@pytest.mark.parametrize("op", ["affine", "scale", "copy"])
def test_ops_variants_shapes(dev, op):
    for (M, N, ldx, ldy) in SHAPES:
        xh = inputs.uniform(M * 7 + N, (M - 1) * ldx + N, -8.0, 8.0)
        vec_ok = ldx % 4 == 0 and ldy % 4 == 0
        for TM, TN in TILES:
            for variant in (tm.TM_VAR_AUTO, tm.TM_VAR_SCALAR, tm.TM_VAR_VEC4_UNDERSTATED, tm.TM_VAR_VEC4):
                expect = tm.TM_OK
                if variant == tm.TM_VAR_VEC4 and not (vec_ok and TN % 4 == 0):
                    expect = tm.TM_E_ALIGN
                if variant == tm.TM_VAR_VEC4_UNDERSTATED and TN % 4 != 0:
                    expect = tm.TM_E_UNSUPPORTED
                note("%s M=%d N=%d ld=%d/%d tile=%dx%d var=%d" % (op, M, N, ldx, ldy, TM, TN, variant))
                check_case(dev, op, M, N, ldx, ldy, TM, TN, 0, variant, xh, 1.5 if op == "scale" else 0.75,
                           -0.25, expect=expect)


def test_misaligned_bases_take_scalar_path(dev):
    """Bases 4 bytes off a 16-byte boundary: AUTO falls back to 4-byte accesses, VEC4 is refused,
    results and guards stay exact."""
    M, N, ld = 70, 200, 200
    xh = inputs.uniform(5, (M - 1) * ld + N, -2.0, 2.0)
    for xoff, yoff in ((1, 0), (0, 1), (3, 2)):
        note("misaligned xoff=%d yoff=%d" % (xoff, yoff))
        check_case(dev, "affine", M, N, ld, ld, 16, 64, 0, tm.TM_VAR_AUTO, xh, xoff=xoff, yoff=yoff)
        check_case(dev, "affine", M, N, ld, ld, 16, 64, 0, tm.TM_VAR_VEC4_UNDERSTATED, xh, xoff=xoff, yoff=yoff)
        check_case(dev, "affine", M, N, ld, ld, 16, 64, 0, tm.TM_VAR_VEC4, xh, xoff=xoff, yoff=yoff,
                   expect=tm.TM_E_ALIGN)


def test_brute_force_tiny_shapes(dev):
    """Every M, N in [0, 17], strides {N, N+3, N rounded up to 4}, tiles {1,2,4,8,16}^2, ragged
    path: one big batch of launches, each into its own guarded region, then one comparison."""
    cases = []
    for M in range(0, 18):
        for N in range(0, 18):
            for ld in sorted({max(N, 1), N + 3, max(4 * ((N + 3) // 4), 1)}):
                for TM in (1, 2, 4, 8, 16):
                    for TN in (1, 2, 4, 8, 16):
                        cases.append((M, N, ld, TM, TN))
    note("brute force: %d cases" % len(cases))
    span = lambda M, ld: M * ld + 2 * GUARD_FLOATS
    rnd = lambda v: (v + 15) // 16 * 16     # keep every region 64-byte aligned
    x_off, y_off, tot_x, tot_y = [], [], 0, 0
    for (M, N, ld, TM, TN) in cases:
        x_off.append(tot_x + GUARD_FLOATS); tot_x += rnd(span(M, ld))
        y_off.append(tot_y + GUARD_FLOATS); tot_y += rnd(span(M, ld))
    xh = inputs.uniform(77, tot_x, -4.0, 4.0)
    X = torch.from_numpy(xh).to(dev)
    Y = sentinel_buffer(tot_y, dev)
    xb, yb = X.data_ptr(), Y.data_ptr()
    s = torch.cuda.current_stream()
    for i, (M, N, ld, TM, TN) in enumerate(cases):
        st = tm.tm_map_affine(xb + 4 * x_off[i], ld, yb + 4 * y_off[i], ld, M, N, 0.75, -0.25, TM, TN,
                              0, tm.TM_VAR_AUTO, s)
        assert st == tm.TM_OK, cases[i]
    torch.cuda.synchronize()
    got = bits(Y)
    want = sentinel_host(tot_y)
    for i, (M, N, ld, TM, TN) in enumerate(cases):
        if M > 0 and N > 0:
            region = want[y_off[i]:y_off[i] + M * ld].copy()
            oracle.map_affine(xh[x_off[i]:x_off[i] + M * ld].copy(), ld, region, ld, M, N, 0.75, -0.25)
            want[y_off[i]:y_off[i] + M * ld] = region
    bad = np.nonzero(got != bits(want))[0]
    if bad.size:
        j = np.searchsorted(np.array(y_off), bad[0], side="right") - 1
        pytest.fail("first mismatch at float %d, case %r" % (bad[0], cases[max(j, 0)]))


def test_brute_force_aligned_promise(dev):
    """Tiny shapes with aligned=1: where the promise holds the output equals the oracle; where it
    is broken the call returns TM_E_ALIGN and writes nothing."""
    for M in (0, 4, 8, 12, 16, 20):
        for N in (0, 4, 8, 16, 28, 32):
            xh = inputs.uniform(M * 40 + N, max(M * N, 1), -3.0, 3.0)
            for TM in (1, 4, 8):
                for TN in (1, 4, 8, 16):
                    holds = oracle.promise_holds(M, N, N, N, TM, TN, 0x1000, 0x2000)
                    check_case(dev, "affine", M, N, max(N, 0), max(N, 0), TM, TN, 1, tm.TM_VAR_AUTO,
                               xh, expect=tm.TM_OK if holds else tm.TM_E_ALIGN)


# ---- edge cases ----------------------------------------------------------------------------------

def test_empty_is_noop(dev):
    Y = Guarded(64, dev)
    before = bits(Y.buf).copy()
    for M, N in ((0, 8), (8, 0), (0, 0)):
        for aligned in (0, 1):
            assert tm.tm_map_affine(0, 8, Y.ptr, 8, M, N, 2.0, 1.0, 4, 4, aligned, 0) == tm.TM_OK
            assert tm.tm_copy2d(0, 8, 0, 8, M, N, 4, 4, aligned, 0) == tm.TM_OK
    torch.cuda.synchronize()
    assert np.array_equal(bits(Y.buf), before)


def test_in_place(dev):
    M, N = 333, 1000
    xh = inputs.ragged_input(M, N)
    for variant in (tm.TM_VAR_VEC4, tm.TM_VAR_SCALAR, tm.TM_VAR_VEC4_UNDERSTATED):
        x = torch.from_numpy(xh).to(dev)
        assert tm.tm_map_affine(x, N, x, N, M, N, 0.75, -0.25, 64, 64, 0, variant) == tm.TM_OK
        want = np.empty_like(xh)
        oracle.map_affine(xh, N, want, N, M, N, 0.75, -0.25)
        torch.cuda.synchronize()
        assert np.array_equal(bits(x), bits(want))


def test_special_values(dev):
    """Copy keeps NaN payloads, infinities, signed zeros and subnormals bit for bit; scale keeps
    -0 (one IEEE multiply) and subnormal products (no flush to zero); affine rounds once."""
    specials = np.array([0x7FC00001, 0xFFC12345, 0x80000000, 0x00000000, 0x00000001, 0x807FFFFF,
                         0x7F800000, 0xFF800000, 0x7F7FFFFF, 0x00800000, 0x3F800001, 0xBF7FFFFF],
                        np.uint32)
    body = np.concatenate([specials, inputs.u32(3, 4096 - specials.size)]).view(np.float32).copy()
    M, N = 16, 256
    for op, alpha, beta in (("copy", 0, 0), ("scale", 1.5, 0), ("scale", 0.5, 0), ("affine", 0.75, -0.25),
                            ("affine", 3.0, 1e-40)):
        for variant in (tm.TM_VAR_VEC4, tm.TM_VAR_SCALAR):
            note("specials %s %g %g var=%d" % (op, alpha, beta, variant))
            check_case(dev, op, M, N, N, N, 16, 256, 1, variant, body, alpha, beta)


def test_max_tiles_and_odd_grids(dev):
    """Largest tiles (256 x 1024: 64 chunk passes per workgroup) and a tile count far above the
    number of CUs, on a ragged shape."""
    M, N = 1000, 3000
    xh = inputs.uniform(8, M * N, -1.0, 1.0)
    check_case(dev, "affine", M, N, N, N, 256, 1024, 0, tm.TM_VAR_AUTO, xh)
    check_case(dev, "affine", M, N, N, N, 1, 4, 0, tm.TM_VAR_AUTO, xh)


def test_side_stream(dev):
    """Work goes on the stream it is given."""
    M = N = 1024
    xh = inputs.scale_input(M, N, seed=12)
    x = torch.from_numpy(xh).to(dev)
    y = torch.zeros_like(x)
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        assert tm.tm_scale2d(x, N, y, N, M, N, 1.5, 32, 128, 1, tm.TM_VAR_VEC4, side) == tm.TM_OK
    side.synchronize()
    want = np.empty_like(xh)
    oracle.scale2d(xh, N, want, N, M, N, 1.5)
    assert np.array_equal(bits(y), bits(want))


def test_beyond_2g_elements(dev):
    """A tensor of more than 2**31 elements (64-bit addressing): 65792 x 32768 scaled on the
    aligned path; sampled rows, including those on both sides of element 2**31 and the last ones,
    against the oracle."""
    M, N = 65792, 32768
    note("beyond 2^31 elements: %d x %d" % (M, N))
    x = torch.empty(M * N, dtype=torch.float32, device=dev)
    # rows are filled from one seeded block of 64 rows (tiled), so any row is known on the host
    blk = inputs.uniform(9, 64 * N, -2.0, 2.0)
    x.view(M, N).copy_(torch.from_numpy(blk).to(dev).view(64, N).repeat((M + 63) // 64, 1)[:M])
    y = torch.empty_like(x)
    assert tm.tm_scale2d(x, N, y, N, M, N, 1.5, 256, 1024, 1, tm.TM_VAR_VEC4) == tm.TM_OK
    torch.cuda.synchronize()
    for r in (0, 1, 65535, 65536, M - 2, M - 1):
        got = y[r * N:(r + 1) * N].cpu().numpy()
        src = blk[(r % 64) * N:(r % 64 + 1) * N].copy()
        want = np.empty_like(src)
        oracle.scale2d(src, N, want, N, 1, N, 1.5)
        assert np.array_equal(bits(got), bits(want)), r
    del x, y
    torch.cuda.empty_cache()


# ---- work items on the 128-byte line grid ---------------------------------------------------------
# Inputs and outputs whose bases and row strides sit on 128-byte lines get one-wave work items of
# whole lines: one 1 KiB row segment when the tile group can span it, else strips of 512-byte
# segments; a whole item whose output is one contiguous 1 KiB is stored through a buffer resource
# (every access variant).  The guard bands here are one line long so that the regions start on a
# line.

LINE_CASES = [  # (M, N, ldx, ldy, TM, TN, aligned)
    (4096, 4096, 4096, 4096, 32, 128, 1),      # the bench's step configuration
    (4096, 4096, 4096, 4096, 32, 128, 0),      # its ragged path: every item whole
    (1000, 1000, 1024, 1024, 8, 128, 0),       # last tile group past column N: edge items
    (513, 777, 800, 832, 16, 64, 0),           # ragged in both directions, different pitches
    (64, 256, 256, 256, 4, 4, 1),              # 4-column tiles: 64 tiles per segment
    (32, 128, 128, 128, 32, 128, 1),           # one tile per row: 512-byte strips instead
    (1, (1 << 20) + 5, (1 << 20) + 32, (1 << 20) + 32, 1, 1024, 0),   # one long ragged row
    (256, 2048, 2048, 2048, 256, 1024, 1),     # wide tiles cut into scheduling tiles
    (1001, 64, 96, 64, 16, 64, 0),             # whole rows of a contiguous output, x pitch 96
    (4097, 128, 128, 128, 32, 128, 0),         # two contiguous rows per item, ragged last band
    (4096, 32, 32, 32, 32, 32, 1),             # eight contiguous rows per item
    (1000, 64, 64, 96, 16, 64, 0),             # output rows not contiguous: global stores
]


@pytest.mark.parametrize("case", LINE_CASES)
def test_line_grid_items_parity(dev, case):
    M, N, ldx, ldy, TM, TN, aligned = case
    xh = inputs.uniform(M * 7 + N, max((M - 1) * ldx + N, 1), -8.0, 8.0)
    for op in ("affine", "scale", "copy"):
        for variant in (tm.TM_VAR_VEC4, tm.TM_VAR_SCALAR, tm.TM_VAR_VEC4_UNDERSTATED):
            if variant == tm.TM_VAR_VEC4_UNDERSTATED and TN % 4:
                continue
            note("line grid %s %dx%d ld=%d/%d tile=%dx%d aligned=%d variant=%d"
                 % (op, M, N, ldx, ldy, TM, TN, aligned, variant))
            check_case(dev, op, M, N, ldx, ldy, TM, TN, aligned, variant, xh,
                       guard=LINE_GUARD_FLOATS)


def test_line_grid_channel_affine(dev):
    """The per-channel op through work items whose output is one contiguous 1 KiB (a 256-channel
    segment, or four rows of a contiguous 64-channel NC view), with and without a scale vector,
    aligned and ragged."""
    for (M, N, ld, aligned) in ((3136, 256, 256, 1), (1000, 520, 544, 0), (64, 1024, 1024, 1),
                                (3001, 64, 64, 0), (6272, 64, 64, 1)):
        for with_scale in (False, True):
            note("line grid channel %dx%d ld=%d aligned=%d scale=%d" % (M, N, ld, aligned, with_scale))
            check_channel(dev, M, N, ld, ld, 64 if aligned else 16, 64, aligned, tm.TM_VAR_VEC4, with_scale,
                          guard=LINE_GUARD_FLOATS)


# ---- per-channel affine on an NC view ----------------------------------------------------------------

def check_channel(dev, M, N, ldx, ldy, TM, TN, aligned, variant, with_scale, coff=0, seed=5,
                  expect=tm.TM_OK, guard=GUARD_FLOATS):
    xh = inputs.uniform(seed, max((M - 1) * ldx + N, 1), -8.0, 8.0)
    sh = inputs.uniform(seed + 1, max(N, 1), -2.0, 2.0)
    bh = inputs.uniform(seed + 2, max(N, 1), -1.0, 1.0)
    X = Guarded(xh.size, dev, 0, guard)
    X.upload(xh)
    Sv = Guarded(sh.size, dev, coff)
    Sv.upload(sh)
    Bv = Guarded(bh.size, dev, coff)
    Bv.upload(bh)
    Y = Guarded(max(M * ldy, 1), dev, 0, guard)
    st = tm.tm_channel_affine(X.ptr, ldx, Sv.ptr if with_scale else 0, Bv.ptr, Y.ptr, ldy, M, N, TM,
                              TN, aligned, variant)
    assert st == expect, (M, N, ldx, ldy, TM, TN, aligned, variant, tm.tm_status_string(st))
    torch.cuda.synchronize()
    want = sentinel_host(Y.buf.numel())
    if st == tm.TM_OK and M and N:
        region = want[Y.off:Y.off + Y.n].copy()
        oracle.channel_affine(xh, ldx, sh if with_scale else None, bh, region, ldy, M, N)
        want[Y.off:Y.off + Y.n] = region
    assert np.array_equal(bits(Y.host()), bits(want)), (M, N, ldx, ldy, TM, TN, aligned, variant, with_scale)
    assert Sv.guards_intact() and Bv.guards_intact() and X.guards_intact()


def test_channel_affine_nhwc_batches(dev):
    """(B, C, H, W) = (32, 64, 56, 56) stored NHWC as a 100352 x 64 NC view, aligned; then channel
    counts that are not multiples of the tile or of 4 (3 = RGB, 130) on the ragged path."""
    for with_scale in (False, True):
        note("channel affine nhwc 32x56x56x64 scale=%d" % with_scale)
        check_channel(dev, 32 * 56 * 56, 64, 64, 64, 64, 64, 1, tm.TM_VAR_AUTO, with_scale)
        for C in (3, 130):
            check_channel(dev, 8 * 28 * 28, C, C, C, 64, 64, 0, tm.TM_VAR_AUTO, with_scale)
    check_channel(dev, 100, 64, 64, 64, 64, 64, 1, tm.TM_VAR_AUTO, True, expect=tm.TM_E_ALIGN)


def test_channel_affine_variants_and_unaligned_vectors(dev):
    for variant in (tm.TM_VAR_SCALAR, tm.TM_VAR_VEC4_UNDERSTATED, tm.TM_VAR_VEC4):
        for coff in (0, 1):
            check_channel(dev, 257, 1000, 1000, 1004, 16, 64, 0, variant, True, coff=coff)


@pytest.mark.parametrize("C", [1, 2, 3, 4, 5, 8, 17, 64, 100])
def test_channel_affine_flat_views(dev, C):
    """Views whose rows are contiguous (ld = C) are walked as one flat row and each element finds
    its channel as (flat column) mod C: few and many channels, every access variant, with and
    without a scale, channel vectors 16-byte aligned or not (gathered), a ragged flat end."""
    M = 300007 // C
    for variant in (tm.TM_VAR_AUTO, tm.TM_VAR_SCALAR, tm.TM_VAR_VEC4_UNDERSTATED, tm.TM_VAR_VEC4):
        TN = 4 if variant == tm.TM_VAR_VEC4_UNDERSTATED else 1
        expect = tm.TM_OK
        if variant == tm.TM_VAR_VEC4:
            TN = 4
            expect = tm.TM_OK if C % 4 == 0 else tm.TM_E_ALIGN
        for with_scale, coff in ((False, 0), (True, 0), (True, 1)):
            note("flat channel C=%d M=%d var=%d scale=%d coff=%d" % (C, M, variant, with_scale, coff))
            check_channel(dev, M, C, C, C, 1, TN, 0, variant, with_scale, coff=coff, seed=C,
                          expect=expect)
    if C % 4 == 0:
        Mp = M - M % 64
        note("flat channel C=%d aligned" % C)
        check_channel(dev, Mp, C, C, C, 64, 4, 1, tm.TM_VAR_VEC4, True, seed=C + 1)


def test_channel_affine_flat_brute_force_tiny(dev):
    for M in (2, 3, 5, 17, 64):
        for N in (1, 2, 3, 4, 7, 16, 17):
            for (TM, TN) in ((1, 1), (2, 4), (8, 8), (16, 1024)):
                check_channel(dev, M, N, N, N, TM, TN, 0, tm.TM_VAR_AUTO, True, seed=M * 100 + N)


def test_channel_affine_brute_force_tiny(dev):
    for M in (1, 2, 5, 17):
        for N in (1, 3, 4, 7, 16, 17):
            for (TM, TN) in ((1, 1), (2, 4), (8, 8), (16, 1024)):
                for with_scale in (False, True):
                    check_channel(dev, M, N, N + 1, N + 2, TM, TN, 0, tm.TM_VAR_AUTO, with_scale,
                                  seed=M * 100 + N)


@pytest.mark.parametrize("N,ld", [(1, 3), (3, 7), (5, 6), (8, 12), (3, 32)])
def test_narrow_padded_rows(dev, N, ld):
    """Rows narrower than the tile on the ragged path are scheduled in narrower, taller tiles:
    rows of 1-8 floats with padded strides (16-byte rows for ld 12 and 32), tiles from 1 x 64 to
    64 x 1024, a row count that ends inside a tile row, every op and the channel op, bit for
    bit with the oracle and guard bands intact."""
    M = 70001
    xh = inputs.uniform(N * 31 + ld, (M - 1) * ld + N, -8.0, 8.0)
    for (TM, TN) in ((1, 64), (64, 64), (64, 1024), (4, 4)):
        for variant in (tm.TM_VAR_AUTO, tm.TM_VAR_SCALAR):
            for op in ("affine", "copy"):
                note("narrow rows %s M=%d N=%d ld=%d tile %dx%d var=%d" % (op, M, N, ld, TM, TN, variant))
                check_case(dev, op, M, N, ld, ld, TM, TN, 0, variant, xh)
            note("narrow rows channel M=%d N=%d ld=%d tile %dx%d var=%d" % (M, N, ld, TM, TN, variant))
            check_channel(dev, M, N, ld, ld, TM, TN, 0, variant, True, seed=N + ld)


# ---- tile-size sweep / autotune ------------------------------------------------------------------

def test_every_sweep_tile_at_8192(dev):
    """The tile sweep's workload at full size: Y = 1.5 X on 8192 x 8192 (aligned) with every menu
    tile that keeps the promise, and the 8192 x 8192 copy of the ceiling probe -- each output equal
    bit for bit to the oracle's, compared on the device against the oracle's result uploaded once."""
    M = N = 8192
    xh = inputs.scale_input(M, N, seed=9)
    want = np.empty_like(xh)
    oracle.scale2d(xh, N, want, N, M, N, 1.5)
    x = torch.from_numpy(xh).to(dev)
    ref = torch.from_numpy(want).to(dev)
    y = torch.empty_like(x)
    ran = 0
    for i in range(9):
        for j in range(11):
            TM, TN = 1 << i, 1 << j
            if not oracle.promise_holds(M, N, N, N, TM, TN, x.data_ptr(), y.data_ptr()):
                continue
            note("sweep tile %dx%d" % (TM, TN))
            y.fill_(-7.0)
            assert tm.tm_scale2d(x, N, y, N, M, N, 1.5, TM, TN, 1, tm.TM_VAR_AUTO) == tm.TM_OK
            assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), (TM, TN)
            ran += 1
    assert ran == 81
    note("copy 8192x8192 32x128")
    y.fill_(-7.0)
    assert tm.tm_copy2d(x, N, y, N, M, N, 32, 128, 1, tm.TM_VAR_VEC4) == tm.TM_OK
    assert torch.equal(y.view(torch.int32), x.view(torch.int32))


def test_autotune_map(dev):
    """The sweep runs every tile that keeps the promise (and only those), returns the fastest, and
    leaves y holding the op's result."""
    M = N = 1024
    xh = inputs.scale_input(M, N, seed=21)
    x = torch.from_numpy(xh).to(dev)
    y = torch.zeros_like(x)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st, TMb, TNb, us, table = tm.tm_autotune_map(1, x, N, y, N, M, N, 1.5, 0.0, 1,
                                                 tm.TM_VAR_AUTO, 3, e0, e1)
    assert st == tm.TM_OK
    want = np.empty_like(xh)
    oracle.scale2d(xh, N, want, N, M, N, 1.5)
    assert np.array_equal(bits(y), bits(want))
    ran = [(1 << i, 1 << j, table[i][j]) for i in range(9) for j in range(11) if table[i][j] >= 0]
    assert ran and all(oracle.promise_holds(M, N, N, N, a, b, x.data_ptr(), y.data_ptr()) for a, b, _ in ran)
    assert len(ran) == sum(oracle.promise_holds(M, N, N, N, 1 << i, 1 << j, x.data_ptr(), y.data_ptr())
                           for i in range(9) for j in range(11))
    assert (TMb, TNb) in [(a, b) for a, b, _ in ran] and us == min(t for _, _, t in ran) and us > 0
    # ragged shapes: all tiles run; no tile keeps the promise on an odd column count
    x2 = torch.from_numpy(inputs.ragged_input(99, 1001)).to(dev)
    y2 = torch.zeros_like(x2)
    st, TMb, TNb, us, table = tm.tm_autotune_map(0, x2, 1001, y2, 1001, 99, 1001, 0.75, -0.25, 0,
                                                 tm.TM_VAR_SCALAR, 1, e0, e1)
    assert st == tm.TM_OK and all(v >= 0 for row in table for v in row)
    want = np.empty(99 * 1001, np.float32)
    oracle.map_affine(x2.cpu().numpy(), 1001, want, 1001, 99, 1001, 0.75, -0.25)
    assert np.array_equal(bits(y2), bits(want))
    st = tm.tm_autotune_map(0, x2, 1001, y2, 1001, 99, 1001, 0.75, -0.25, 1, tm.TM_VAR_AUTO, 1, e0, e1)[0]
    assert st == tm.TM_E_ALIGN
