"""Pins for the CPU oracle: each test ties an oracle function to something other than itself --
values the pages print (tests/golden/), closed forms, exact special cases, library routines or
brute force on tiny shapes.  A plausible slip in the oracle (dropped term, wrong fill, fused vs
unfused rounding, a transposed index, accumulating in f32) fails at least one of them.

Sources: Phobos docs "@aligned" and "Slicing, bounds and masking"; Mojo GPU puzzle 35 "Aligned Load
& Store"; teenygrad "Memory Coalescing and Tensor Layout".
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from edge_masking_vector_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _bits(a):
    return np.ascontiguousarray(a, np.float32).view(np.uint32)


# ---- loop remainder split ------------------------------------------------------------------------

def test_split_worked_example():
    """'Slicing, bounds and masking', 'Loops over a dynamic extent': K=1000, TILE_K=16 -> 62 + 8."""
    g = _golden("split_loop.json")
    assert oracle.split(g["K"], g["TILE_K"]) == (g["whole_tiles"], g["remainder_cols"])


def test_split_masked_rowmax_shape():
    """The same rule on the score walk: Nk=1000 in BC=64 tiles -> 15 whole tiles + 40 columns."""
    assert oracle.split(1000, 64) == (15, 40)


def test_split_closed_form_exhaustive():
    """nfull*T + rem == K with 0 <= rem < T, for every small K and T."""
    for K in range(0, 300):
        for T in range(1, 40):
            nf, rm = oracle.split(K, T)
            assert nf * T + rm == K and 0 <= rm < T, (K, T, nf, rm)


# ---- edge tiles ----------------------------------------------------------------------------------

def test_edge_tile_worked_example():
    g = _golden("edge_tile.json")
    M, N = g["derived_shape"]["M"], g["derived_shape"]["N"]
    pm, pn = g["block"]
    live = oracle.tile_live(M, N, g["TM"], g["TN"], pm, pn)
    assert live == g["live"]
    assert g["TM"] * g["TN"] - live == g["masked"]


def test_edge_tile_shape_is_unique():
    """Among extents that are multiples of 4 (the pages' assumption) and that leave tile (2, 3) of
    an 8 x 8 tiling partly inside the tensor, only M=20, N=28 gives 16 live elements."""
    hits = []
    for M in range(4, 33, 4):
        for N in range(4, 41, 4):
            live = oracle.tile_live(M, N, 8, 8, 2, 3)
            if live == 16:
                hits.append((M, N))
    assert hits == [(20, 28)]


def test_edge_tile_brute_force_counts():
    """Brute force over tiny shapes: live count equals the overlap of row and column ranges."""
    for M in range(0, 14):
        for N in range(0, 14):
            for TM in (1, 2, 3, 4, 8):
                for TN in (1, 2, 4, 5, 8):
                    for pm in range(0, 4):
                        for pn in range(0, 4):
                            rows = len([i for i in range(pm * TM, pm * TM + TM) if i < M])
                            cols = len([j for j in range(pn * TN, pn * TN + TN) if j < N])
                            assert oracle.tile_live(M, N, TM, TN, pm, pn) == rows * cols


def test_edge_tile_stores_land_only_inside():
    """The masked tiled map on the worked example writes exactly the 16 live elements of tile
    (2, 3) and nothing outside the 20 x 28 tensor (48 masked stores skipped)."""
    M, N, ld = 20, 28, 32
    rows_alloc = 24
    x = np.arange(rows_alloc * ld, dtype=np.float32)
    sentinel = np.float32(3.25e38)
    y = np.full(rows_alloc * ld, sentinel, np.float32)
    oracle.map_affine_tiled(x, ld, y, ld, M, N, 2.0, 1.0, 8, 8)
    y2 = y.reshape(rows_alloc, ld)
    written = y2 != sentinel
    assert written[:M, :N].all()
    assert not written[M:, :].any() and not written[:, N:].any()
    tile = written[16:24, 24:32]
    assert tile.sum() == 16 and (~tile).sum() == 48


# ---- the affine map ------------------------------------------------------------------------------

def test_map_1d_closed_form():
    """'Aligned Load & Store': out = a*2 + 1 over the 1M-element buffer.  With a = (k - 2**23) *
    2**-23 (k a 24-bit integer), out = (k - 2**22) * 2**-22 exactly -- computed from integers."""
    n = 1 << 20
    a = inputs.map1d_input(n)
    k = inputs.u24(1, n)
    assert np.array_equal(a.astype(np.float64), (k - 2 ** 23) * 2.0 ** -23)
    want = ((k - 2 ** 22) * 2.0 ** -22).astype(np.float32)
    y = np.empty(n, np.float32)
    oracle.map_affine(a, n, y, n, 1, n, 2.0, 1.0)
    assert np.array_equal(_bits(y), _bits(want))


@pytest.mark.parametrize("alpha,beta,gen", [
    (0.75, -0.25, lambda: inputs.ragged_input(64, 1000)),
    (2.0, 1.0, lambda: inputs.map1d_input(1 << 16)),
])
def test_map_single_rounding(alpha, beta, gen):
    """fmaf is one rounding of the exact a*x + b.  For these inputs the double expression is exact
    (under 53 significant bits), so rounding it once to f32 is the correctly rounded result."""
    x = gen()
    exact = x.astype(np.float64) * alpha + beta
    # exactness of the double expression, checked with rationals on a sample
    for v in x[:200]:
        assert Fraction(float(v)) * Fraction(alpha) + Fraction(beta) == Fraction(float(v) * alpha + beta)
    want = exact.astype(np.float32)
    y = np.empty_like(x)
    oracle.map_affine(x, x.size, y, x.size, 1, x.size, alpha, beta)
    assert np.array_equal(_bits(y), _bits(want))


def test_map_fused_differs_from_unfused():
    """Negative control for the pin above: on the ragged workload's data, multiply-then-add in f32
    (two roundings) differs from the fused result for some elements, so the pin tells them apart."""
    x = inputs.ragged_input(64, 1000)
    unfused = (x * np.float32(0.75)) + np.float32(-0.25)
    y = np.empty_like(x)
    oracle.map_affine(x, x.size, y, x.size, 1, x.size, 0.75, -0.25)
    assert (_bits(unfused) != _bits(y)).sum() > 0


def test_map_respects_strides():
    """Row strides are the passed ones ('The alignment constraint'): padding is never read or
    written, and swapping ldx/ldy misplaces data."""
    M, N, ldx, ldy = 5, 7, 9, 11
    x = np.arange(M * ldx, dtype=np.float32)
    y = np.full(M * ldy, -7.0, np.float32)
    oracle.map_affine(x, ldx, y, ldy, M, N, 2.0, 1.0)
    for i in range(M):
        for j in range(ldy):
            if j < N:
                assert y[i * ldy + j] == 2.0 * x[i * ldx + j] + 1.0
            else:
                assert y[i * ldy + j] == -7.0


# ---- scale and copy ------------------------------------------------------------------------------

def test_scale_is_ieee_multiply():
    """Y = alpha*X is one IEEE f32 multiply: numpy's f32 multiply is that operation.  Signed zeros
    survive (1.5 * -0 = -0), which a fused alpha*x + 0 would turn into +0."""
    x = inputs.scale_input(64, 512)
    x[:4] = [-0.0, 0.0, 1e-40, -1e-40]   # signed zeros and subnormals
    y = np.empty_like(x)
    oracle.scale2d(x, 512, y, 512, 64, 512, 1.5)
    want = np.float32(1.5) * x
    assert np.array_equal(_bits(y), _bits(want))
    assert _bits(y)[0] == 0x80000000


def test_scale_exact_in_double():
    """For alpha = 1.5 the product of an f32 with 1.5 is exact in double; rounding once to f32
    reproduces the f32 multiply."""
    x = inputs.scale_input(128, 1024)
    y = np.empty_like(x)
    oracle.scale2d(x, 1024, y, 1024, 128, 1024, 1.5)
    assert np.array_equal(_bits(y), _bits((x.astype(np.float64) * 1.5).astype(np.float32)))


def test_copy_is_bitwise():
    specials = np.array([0x7FC00001, 0xFFC12345, 0x80000000, 0x00000001, 0x7F800000,
                         0xFF800000, 0x7FA00000], np.uint32)
    x = np.concatenate([specials, inputs.u32(9, 57)]).view(np.float32).copy()
    y = np.zeros(64 * 2, np.float32)
    oracle.copy2d(x, 64, y, 128, 1, 64)
    assert np.array_equal(_bits(y[:64]), _bits(x))
    assert not _bits(y[64:]).any()


# ---- tiled walks vs plain definitions: brute force on tiny shapes --------------------------------

def _tiny_cases():
    for M in range(0, 18):
        for N in range(0, 18):
            for ld in sorted({max(N, 1), N + 3, max(4 * ((N + 3) // 4), 1)}):
                yield M, N, ld


def test_tiled_map_equals_plain_brute_force():
    """'Masking': masked reads give 0, masked stores are skipped.  For every tiny shape and tile
    the tiled walk writes exactly the plain map's values, and never touches padding or the
    rows past M (sentinels)."""
    sentinel = np.float32(3.0e38)
    for M, N, ld in _tiny_cases():
        x = inputs.uniform(M * 131 + N * 7 + ld, (M + 1) * ld + 1, -4.0, 4.0)
        ref = np.full(x.size, sentinel, np.float32)
        oracle.map_affine(x, ld, ref, ld, M, N, 0.75, -0.25)
        for TM in (1, 2, 4, 8, 16):
            for TN in (1, 2, 4, 8, 16):
                y = np.full(x.size, sentinel, np.float32)
                oracle.map_affine_tiled(x, ld, y, ld, M, N, 0.75, -0.25, TM, TN)
                assert np.array_equal(_bits(y), _bits(ref)), (M, N, ld, TM, TN)


def test_tiled_rowsum_equals_plain_brute_force():
    """Whole tiles + one zero-filled remainder give the plain fp64 row sum bit for bit."""
    for M, N, ld in _tiny_cases():
        if M == 0:
            continue
        x = inputs.uniform(M * 17 + N + 5 * ld, M * ld, -3.0, 3.0)
        ref = oracle.rowsum_f64(x, ld, M, N)
        for T in (1, 2, 4, 8, 16):
            got = oracle.rowsum_tiled_f64(x, ld, M, N, T)
            assert np.array_equal(got, ref), (M, N, ld, T)


def test_tiled_rowmax_equals_plain_brute_force():
    """With the -1e30 fill the masked remainder never wins, so the tiled walk equals the plain max."""
    for M, N, ld in _tiny_cases():
        if M == 0:
            continue
        s = inputs.uniform(M * 29 + N + 3 * ld, M * ld, -10.0, -1.0)
        ref = oracle.rowmax(s, ld, M, N)
        for BC in (1, 2, 4, 8, 16):
            got = oracle.rowmax_tiled(s, ld, M, N, BC)
            assert np.array_equal(_bits(got), _bits(ref)), (M, N, ld, BC)


# ---- reductions ----------------------------------------------------------------------------------

def test_rowmax_fill_value_bits():
    """-1.0e30 in f32 is the nearest float, 0xF149F2CA."""
    assert int(np.array([oracle.MAX_FILL], np.float32).view(np.uint32)[0]) == 0xF149F2CA
    s = np.zeros(4, np.float32)
    out = oracle.rowmax(s, 1, 3, 0)        # empty rows
    assert (_bits(out) == 0xF149F2CA).all()


def test_rowmax_all_negative_never_zero():
    """'Reductions over a ragged tile': a ragged row of negative scores keeps its true (negative)
    maximum under the -1e30 fill ..."""
    M, N, BC = 64, 1000, 64
    s = inputs.scores_input(M, N)
    got = oracle.rowmax_tiled(s, N, M, N, BC)
    assert (got < 0).all()
    assert np.array_equal(got, s.reshape(M, N).max(axis=1))


def test_rowmax_zero_fill_negative_control():
    """... and the same walk with a 0 fill reports 0, the wrong answer the pages warn about."""
    M, N, BC = 64, 1000, 64
    s = inputs.scores_input(M, N)
    got = oracle.rowmax_tiled(s, N, M, N, BC, fill=0.0)
    assert (got == 0).all()


def test_rowmax_matches_numpy_full_shape():
    """Max is exact and order-free: the masked-rowmax workload (8192 x 1000) against numpy's max."""
    M, N = 8192, 1000
    s = inputs.scores_input(M, N)
    got = oracle.rowmax(s, N, M, N)
    assert np.array_equal(_bits(got), _bits(s.reshape(M, N).max(axis=1)))


def test_rowmax_nan_never_wins():
    s = np.array([-3.0, np.nan, -2.0, -5.0], np.float32)
    assert oracle.rowmax(s, 4, 1, 4)[0] == np.float32(-2.0)


def test_sums_integer_inputs_exact():
    """Integer inputs in [0, 16): every sum is an exact integer; compare with Python integers."""
    M, N = 96, 200
    x = inputs.integers(11, M * N, 0, 16)
    xi = x.astype(np.int64).reshape(M, N)
    assert np.array_equal(oracle.rowsum_f64(x, N, M, N), xi.sum(axis=1).astype(np.float64))
    assert np.array_equal(oracle.colsum_f64(x, N, M, N), xi.sum(axis=0).astype(np.float64))


def test_sums_constant_closed_form():
    M, N, c = 300, 700, 0.125
    x = np.full(M * N, c, np.float32)
    assert (oracle.rowsum_f64(x, N, M, N) == N * c).all()
    assert (oracle.colsum_f64(x, N, M, N) == M * c).all()


def test_sums_accumulate_in_double():
    """A large term followed by many tiny ones: an f32 accumulator would drop the tiny terms, the
    fp64 one keeps them.  Compared with math.fsum (exactly rounded)."""
    N = 4096
    row = np.full(N, 2.0 ** -30, np.float32)
    row[0] = 1.0
    got = oracle.rowsum_f64(row, N, 1, N)[0]
    assert got == math.fsum(float(v) for v in row)
    assert got > 1.0 + 1e-6


def test_sums_against_fsum():
    """Row and column sums of the 4096 x 4096 U[0,1) workload against math.fsum on sampled lines
    (fp64 left-to-right accumulation of 4096 terms is within 4096 * 2**-53 relative)."""
    M = N = 4096
    x = inputs.colrow_input(M, N)
    rs = oracle.rowsum_f64(x, N, M, N)
    cs = oracle.colsum_f64(x, N, M, N)
    X = x.reshape(M, N)
    for i in (0, 1, 777, 2048, 4095):
        ref = math.fsum(X[i, :].astype(np.float64))
        assert abs(rs[i] - ref) <= 1e-12 * ref
        ref = math.fsum(X[:, i].astype(np.float64))
        assert abs(cs[i] - ref) <= 1e-12 * ref


def test_colsum_is_rowsum_of_transpose():
    """Column sums of X equal row sums of X^T, bit for bit (same terms, same order)."""
    M, N = 123, 77
    x = inputs.uniform(21, M * N, -1.0, 1.0)
    xt = np.ascontiguousarray(x.reshape(M, N).T).reshape(-1)
    assert np.array_equal(oracle.colsum_f64(x, N, M, N), oracle.rowsum_f64(xt, M, N, M))


def test_sums_respect_stride_padding():
    M, N, ld = 33, 10, 13
    x = np.full(M * ld, 1000.0, np.float32)
    x.reshape(M, ld)[:, :N] = 1.0
    assert (oracle.rowsum_f64(x, ld, M, N) == N).all()
    assert (oracle.colsum_f64(x, ld, M, N) == M).all()


# ---- the alignment promise -----------------------------------------------------------------------

def test_promise_worked_shapes():
    """The scale kernel's shape (4096 x 4096, 32 x 128 tiles) keeps the promise; the ragged shape
    (4100 x 1000 under 64 x 64 tiles: 4100 % 64 = 4, 1000 % 64 = 40) breaks it."""
    assert oracle.promise_holds(4096, 4096, 4096, 4096, 32, 128, 0x10000, 0x20000)
    assert not oracle.promise_holds(4100, 1000, 1000, 1000, 64, 64, 0x10000, 0x20000)
    assert not oracle.promise_holds(4096, 1000, 1000, 1000, 64, 64, 0x10000, 0x20000)
    assert not oracle.promise_holds(4100, 1024, 1024, 1024, 64, 64, 0x10000, 0x20000)
    assert oracle.promise_holds(4096, 1024, 1024, 1024, 64, 64, 0x10000, 0x20000)


def test_promise_needs_16_byte_rows():
    """Whole tiles are not enough: rows must start on 16-byte boundaries ('@aligned' licenses
    16-byte vectors; 'The alignment constraint' asks for 16-byte rows)."""
    ok = dict(M=64, N=64, ld_in=64, ld_out=64, TM=8, TN=8, in_addr=0x1000, out_addr=0x2000)
    assert oracle.promise_holds(**ok)
    for k, v in [("ld_in", 66), ("ld_out", 65), ("in_addr", 0x1004), ("out_addr", 0x2008)]:
        bad = dict(ok, **{k: v})
        assert not oracle.promise_holds(**bad), k
    assert not oracle.promise_holds(**dict(ok, N=2 * 2, TN=2))      # 8-byte tile rows
    # reductions have no 2-D output: only the input side counts
    assert oracle.promise_holds(**dict(ok, ld_out=3, out_addr=0))
    # a single row starts at the base: its stride plays no part
    one = dict(ok, M=1, TM=1)
    assert oracle.promise_holds(**dict(one, ld_in=65, ld_out=67))
    assert not oracle.promise_holds(**dict(one, in_addr=0x1004))


def test_coalescing_table_byte_accounting():
    """'What it actually costs': the printed bandwidths are the 64 MiB read over the printed
    times in decimal GB/s (to the printed rounding)."""
    g = _golden("coalescing_table.json")
    M, N = g["matrix"]
    assert M * N * 4 == g["bytes_read"]
    for walk in ("rows", "columns"):
        gbs = g["bytes_read"] / (g[walk]["time_us"] * 1e-6) / 1e9
        assert abs(gbs - g[walk]["gbs"]) < 0.3
    assert round(g["columns"]["time_us"] / g["rows"]["time_us"], 1) == g["slowdown"]


def test_promise_whole_tiles_brute_force():
    """'A dimension is a whole number of tiles' restated through the edge-tile count: with 16-byte
    rows and bases, the promise holds exactly when every tile of the ceil(M/TM) x ceil(N/TN) grid
    is full (no element of any tile masked)."""
    for M in range(1, 25):
        for N in range(4, 41, 4):
            for TM in (1, 2, 4, 8, 16):
                for TN in (4, 8, 16, 32):
                    tiles_m, tiles_n = -(-M // TM), -(-N // TN)
                    full = all(oracle.tile_live(M, N, TM, TN, pm, pn) == TM * TN
                               for pm in range(tiles_m) for pn in range(tiles_n))
                    got = oracle.promise_holds(M, N, N + (-N % 4), 4 * ((N + 7) // 4), TM, TN,
                                               0x4000, 0x8000)
                    assert got == full, (M, N, TM, TN)


# ---- softmax row statistics (the masked maximum's consumer) -------------------------------------

def test_softmax_stats_constant_row():
    """s == c: m = c and every exp(s - m) is exactly 1, so l = N."""
    M, N = 5, 777
    s = np.full(M * N, -3.25, np.float32)
    m, l = oracle.softmax_stats(s, N, M, N)
    assert (m == np.float32(-3.25)).all() and (l == N).all()


def test_softmax_stats_geometric_closed_form():
    """s_j = -j (exact in f32): m = 0 and l = sum_j e^-j = (1 - e^-N) / (1 - e^-1)."""
    N = 1000
    s = -np.arange(N, dtype=np.float32)
    m, l = oracle.softmax_stats(s, N, 1, N)
    want = (1.0 - math.exp(-N)) / (1.0 - math.exp(-1.0))
    assert m[0] == 0.0 and abs(l[0] - want) <= 1e-14 * want


def test_softmax_stats_against_logsumexp():
    """l = exp(logsumexp(s) - m), with scipy's logsumexp (a different algorithm) as the reference."""
    from scipy.special import logsumexp
    M, N = 64, 1000
    s = inputs.scores_input(M, N)
    m, l = oracle.softmax_stats(s, N, M, N)
    S = s.reshape(M, N).astype(np.float64)
    assert np.array_equal(m, s.reshape(M, N).max(axis=1))
    want = np.exp(logsumexp(S, axis=1) - m.astype(np.float64))
    assert np.all(np.abs(l - want) <= 1e-12 * want)


def test_softmax_stats_shift_invariance():
    """Adding 0.5 to every score (exact here) moves m by 0.5 and leaves l unchanged."""
    M, N = 16, 300
    s = inputs.scores_input(M, N)
    m0, l0 = oracle.softmax_stats(s, N, M, N)
    m1, l1 = oracle.softmax_stats((s + np.float32(0.5)).astype(np.float32), N, M, N)
    assert np.array_equal(m1, m0 + np.float32(0.5))
    assert np.all(np.abs(l1 - l0) <= 1e-13 * l0)


def test_softmax_stats_tiled_equals_plain():
    """The online tile-by-tile update with the -1e30 fill reproduces the plain statistics, for
    every small shape and tile width (m bit for bit, l to double rounding)."""
    for M, N, ld in _tiny_cases():
        if M == 0:
            continue
        s = inputs.uniform(M * 13 + N + ld, M * ld, -10.0, -1.0)
        m, l = oracle.softmax_stats(s, ld, M, N)
        for BC in (1, 2, 4, 8, 16):
            mt, lt = oracle.softmax_stats_tiled(s, ld, M, N, BC)
            assert np.array_equal(mt, m), (M, N, ld, BC)
            assert np.all(np.abs(lt - l) <= 1e-13 * np.maximum(l, 1e-300)), (M, N, ld, BC)


def test_softmax_stats_zero_fill_negative_control():
    """With a 0 fill the ragged tile's missing columns win the maximum and corrupt the normaliser
    (the pages' warning about softmax); the -1e30 fill does not."""
    M, N, BC = 8, 1000, 64
    s = inputs.scores_input(M, N)
    m, l = oracle.softmax_stats(s, N, M, N)
    mz, lz = oracle.softmax_stats_tiled(s, N, M, N, BC, fill=0.0)
    assert (mz == 0).all() and np.all(np.abs(lz - l) > 1.0)


def test_softmax_stats_empty_row():
    m, l = oracle.softmax_stats(np.zeros(1, np.float32), 1, 3, 0)
    assert (m.view(np.uint32) == 0xF149F2CA).all() and (l == 0).all()


# ---- transpose / layout conversion ------------------------------------------------------------------

def test_transpose_nchw_to_nhwc_index_formula():
    """'Strides, and reading an index expression': in NCHW the element (b, c, h, w) sits at
    b*(C*H*W) + c*(H*W) + h*W + w; in NHWC at b*(H*W*C) + (h*W + w)*C + c.  Fill x with its own
    NCHW flat index; after the conversion each y element must hold the NCHW index of the element
    that belongs at its NHWC position."""
    B, C, H, W = 3, 5, 4, 7
    HW = H * W
    x = np.arange(B * C * HW, dtype=np.float32)
    y = np.full(B * HW * C, -1.0, np.float32)
    oracle.transpose(x, HW, C * HW, y, C, HW * C, B, C, HW)
    for b in range(B):
        for c in range(C):
            for h in range(H):
                for w in range(W):
                    assert y[b * HW * C + (h * W + w) * C + c] == b * C * HW + c * HW + h * W + w


def test_transpose_matches_numpy_and_is_an_involution():
    M, N = 37, 53
    x = inputs.uniform(4, M * N, -1.0, 1.0)
    y = np.empty(N * M, np.float32)
    oracle.transpose(x, N, 0, y, M, 0, 1, M, N)
    assert np.array_equal(y.view(np.uint32), np.ascontiguousarray(x.reshape(M, N).T).reshape(-1).view(np.uint32))
    z = np.empty_like(x)
    oracle.transpose(y, M, 0, z, N, 0, 1, N, M)
    assert np.array_equal(z.view(np.uint32), x.view(np.uint32))


def test_transpose_strides_and_bits():
    """Padded strides are honoured (padding never written) and NaN payloads survive."""
    M, N, ldx, ldy = 4, 6, 9, 7
    x = np.arange(M * ldx, dtype=np.float32)
    x[0] = np.array([0x7FC01234], np.uint32).view(np.float32)[0]
    y = np.full(N * ldy, 5.0, np.float32)
    oracle.transpose(x, ldx, 0, y, ldy, 0, 1, M, N)
    Y = y.reshape(N, ldy)
    assert (Y[:, M:] == 5.0).all()
    assert Y[0, 0].view(np.uint32) == 0x7FC01234
    assert all(Y[j, i] == x[i * ldx + j] for i in range(1, M) for j in range(N))


# ---- per-channel affine on an NC view ----------------------------------------------------------------

def test_channel_bias_add_is_ieee_add():
    """Without a scale the op is one f32 add per element: numpy's f32 add is that operation."""
    M, N = 50, 70
    x = inputs.uniform(1, M * N, -4.0, 4.0)
    b = inputs.uniform(2, N, -1.0, 1.0)
    y = np.empty_like(x)
    oracle.channel_affine(x, N, None, b, y, N, M, N)
    assert np.array_equal(y.view(np.uint32), (x.reshape(M, N) + b[None, :]).reshape(-1).view(np.uint32))


def test_channel_affine_single_rounding():
    """With a scale it is one fused multiply-add: scale values 0.75 and 1.5 keep the double
    expression exact on these inputs, so rounding it once is the correctly rounded result."""
    M, N = 40, 64
    x = inputs.ragged_input(M, N)
    s = np.where(np.arange(N) % 2 == 0, 0.75, 1.5).astype(np.float32)
    b = (inputs.integers(3, N, -64, 64) * np.float32(0.25)).astype(np.float32)
    y = np.empty_like(x)
    oracle.channel_affine(x, N, s, b, y, N, M, N)
    want = (x.reshape(M, N).astype(np.float64) * s[None, :] + b[None, :]).astype(np.float32).reshape(-1)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32))


def test_channel_affine_broadcasts_along_columns():
    """Rows of constant x with a distinct bias per column: y[i, j] depends on j through the bias
    (a transposed broadcast would make it depend on i)."""
    M, N = 6, 9
    x = np.repeat(np.arange(M, dtype=np.float32), N)
    b = np.arange(N, dtype=np.float32) * 100
    y = np.empty_like(x)
    oracle.channel_affine(x, N, None, b, y, N, M, N)
    assert all(y[i * N + j] == i + 100 * j for i in range(M) for j in range(N))


def test_channel_affine_on_nhwc_view():
    """A (B, C, H, W) tensor stored NHWC is the (B*H*W) x C view: element (b, c, h, w) sits at
    ((b*H + h)*W + w)*C + c and receives bias[c]."""
    B, C, H, W = 2, 3, 4, 5
    x = np.zeros(B * H * W * C, np.float32)
    b = np.array([1.0, 20.0, 300.0], np.float32)
    y = np.empty_like(x)
    oracle.channel_affine(x, C, None, b, y, C, B * H * W, C)
    for bb in range(B):
        for c in range(C):
            for h in range(H):
                for w in range(W):
                    assert y[((bb * H + h) * W + w) * C + c] == b[c]


# ---- row strides of scale, copy and the per-channel op ------------------------------------------
# teenygrad "Memory Coalescing and Tensor Layout", "The alignment constraint" (and item 5 of "A
# checklist"): a kernel must use the row stride it is passed, never the row length, because rows
# may be padded.  Each function below gets M > 1 rows with ldx != ldy (both ways round), inputs
# whose padding columns hold sentinels, outputs pre-filled with another sentinel, and an
# expectation built index by index from the passed strides: element (i, j) of y at i*ldy + j
# comes from i*ldx + j of x, and nothing else in y changes.

_STRIDE_CASES = [(6, 5, 9, 7), (5, 7, 7, 12), (4, 3, 3, 8), (7, 4, 11, 4)]  # (M, N, ldx, ldy)
_X_PAD = np.float32(-9.5e37)   # never a legal output of the ops on these inputs
_Y_PAD = np.float32(7.25e37)


def _strided_input(M, N, ldx, ldy, seed):
    """x with distinct values in its M x N window, sentinels in its padding, and room for a reader
    that uses the wrong stride (M * max(ldx, ldy) elements) so that such a mistake reads
    sentinels instead of running off the buffer."""
    size = M * max(ldx, ldy) + 1
    x = np.full(size, _X_PAD, np.float32)
    vals = inputs.uniform(seed, M * N, 1.0, 2.0)
    for i in range(M):
        x[i * ldx:i * ldx + N] = vals[i * N:(i + 1) * N]
    return x


def _expect(x, ldx, ldy, M, N, size, f):
    """Expected y, built element by element from the passed strides."""
    want = np.full(size, _Y_PAD, np.float32)
    for i in range(M):
        for j in range(N):
            want[i * ldy + j] = f(x[i * ldx + j], j)
    return want


def test_scale_uses_passed_strides():
    for k, (M, N, ldx, ldy) in enumerate(_STRIDE_CASES):
        x = _strided_input(M, N, ldx, ldy, 40 + k)
        size = M * max(ldx, ldy) + 1
        y = np.full(size, _Y_PAD, np.float32)
        oracle.scale2d(x, ldx, y, ldy, M, N, 1.5)
        want = _expect(x, ldx, ldy, M, N, size, lambda v, j: np.float32(1.5) * v)
        assert np.array_equal(_bits(y), _bits(want)), (M, N, ldx, ldy)


def test_copy_uses_passed_strides():
    for k, (M, N, ldx, ldy) in enumerate(_STRIDE_CASES):
        x = _strided_input(M, N, ldx, ldy, 50 + k)
        x[0] = np.array([0x7FC0BEEF], np.uint32).view(np.float32)[0]  # a NaN payload travels too
        size = M * max(ldx, ldy) + 1
        y = np.full(size, _Y_PAD, np.float32)
        oracle.copy2d(x, ldx, y, ldy, M, N)
        want = _expect(x, ldx, ldy, M, N, size, lambda v, j: v)
        assert np.array_equal(_bits(y), _bits(want)), (M, N, ldx, ldy)


def test_channel_affine_uses_passed_strides():
    for k, (M, N, ldx, ldy) in enumerate(_STRIDE_CASES):
        x = _strided_input(M, N, ldx, ldy, 60 + k)
        size = M * max(ldx, ldy) + 1
        b = (np.arange(N, dtype=np.float32) + 1) * np.float32(0.5)
        s = np.where(np.arange(N) % 2 == 0, 0.75, 1.5).astype(np.float32)
        y = np.full(size, _Y_PAD, np.float32)
        oracle.channel_affine(x, ldx, None, b, y, ldy, M, N)
        want = _expect(x, ldx, ldy, M, N, size, lambda v, j: v + b[j])
        assert np.array_equal(_bits(y), _bits(want)), ("bias", M, N, ldx, ldy)
        y = np.full(size, _Y_PAD, np.float32)
        oracle.channel_affine(x, ldx, s, b, y, ldy, M, N)
        # fmaf(v, s, b) with s in {0.75, 1.5} and these inputs is exact in double: one rounding
        want = _expect(x, ldx, ldy, M, N, size,
                       lambda v, j: np.float32(np.float64(v) * np.float64(s[j]) + np.float64(b[j])))
        assert np.array_equal(_bits(y), _bits(want)), ("scale", M, N, ldx, ldy)
