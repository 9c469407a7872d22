"""Seeded random parity cases: medium shapes, strides, base offsets, tiles, variants and paths drawn
at random (fixed seeds), every call checked against the oracle -- bit for bit for maps, copies,
maxima and transposes, within the sum tolerance for sums and softmax normalisers -- with guard
bands around every output.  A call the library refuses must return the status the argument rules
give and leave its output untouched.
"""
import random
import sys

import numpy as np
import pytest
import torch

import oracle
from edge_masking_vector_amd import inputs
from gpu_helpers import LINE_GUARD_FLOATS, Guarded, bits, sentinel_host, sum_tol

pytestmark = pytest.mark.gpu
tm = pytest.importorskip("edge_masking_vector_amd.tilemap")

TMS = [1, 2, 4, 8, 16, 32, 64, 128, 256]
TNS = [1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024]


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")


def rows16(addr, M, ld):
    return addr % 16 == 0 and (M <= 1 or ld % 4 == 0)


def draw_view(rng, aligned_wanted, TM, TN):
    """(M, N, ld_x, ld_y, off_x, off_y), shaped to keep the promise when aligned_wanted."""
    if aligned_wanted:
        M = TM * rng.randint(1, max(1, 300 // TM))
        N = TN * rng.randint(1, max(1, 1100 // TN))
        ldx = N + 4 * rng.randint(0, 8)
        ldy = N + 4 * rng.randint(0, 8)
        offx, offy = 4 * rng.randint(0, 3), 4 * rng.randint(0, 3)
    else:
        M, N = rng.randint(1, 300), rng.randint(1, 1100)
        ldx, ldy = N + rng.randint(0, 40), N + rng.randint(0, 40)
        offx, offy = rng.choice([0, 1, 2, 3, 4, 8, 32]), rng.choice([0, 1, 2, 3, 4, 8, 32])
    return M, N, ldx, ldy, offx, offy


def expected_map_status(X, Y, M, N, ldx, ldy, TM, TN, aligned, variant):
    if aligned and not oracle.promise_holds(M, N, ldx, ldy, TM, TN, X.ptr, Y.ptr):
        return tm.TM_E_ALIGN
    if variant == tm.TM_VAR_VEC4_UNDERSTATED and TN % 4:
        return tm.TM_E_UNSUPPORTED
    if variant == tm.TM_VAR_VEC4 and not (TN % 4 == 0 and rows16(X.ptr, M, ldx) and rows16(Y.ptr, M, ldy)):
        return tm.TM_E_ALIGN
    return tm.TM_OK


def test_fuzz_maps(dev):
    rng = random.Random(2024)
    ran = {"ok": 0, "refused": 0}
    for case in range(400):
        op = rng.choice(["affine", "scale", "copy", "channel", "channel_scale"])
        TM, TN = rng.choice(TMS), rng.choice(TNS)
        aligned = rng.random() < 0.4 and TN % 4 == 0
        variant = rng.choice([tm.TM_VAR_AUTO, tm.TM_VAR_SCALAR, tm.TM_VAR_VEC4_UNDERSTATED, tm.TM_VAR_VEC4])
        M, N, ldx, ldy, offx, offy = draw_view(rng, aligned, TM, TN)
        note("fuzz map %d: %s M=%d N=%d ldx=%d ldy=%d offs=%d,%d tile=%dx%d aligned=%d variant=%d"
             % (case, op, M, N, ldx, ldy, offx, offy, TM, TN, aligned, variant))
        nx, ny = (M - 1) * ldx + N, M * ldy
        xh = inputs.uniform(case, nx, -8.0, 8.0)
        X = Guarded(nx, dev, offx)
        X.upload(xh)
        Y = Guarded(ny, dev, offy)
        alpha, beta = 0.75, -0.25
        if op.startswith("channel"):
            bh = inputs.uniform(1000 + case, N, -1.0, 1.0)
            B = Guarded(N, dev, rng.choice([0, 1, 4]))
            B.upload(bh)
            sh = None
            if op == "channel_scale":
                sh = inputs.uniform(2000 + case, N, 0.5, 1.5)
                S = Guarded(N, dev, rng.choice([0, 4]))
                S.upload(sh)
            st = tm.tm_channel_affine(X.ptr, ldx, S.ptr if sh is not None else None, B.ptr, Y.ptr, ldy, M, N,
                                      TM, TN, int(aligned), variant)
        elif op == "affine":
            st = tm.tm_map_affine(X.ptr, ldx, Y.ptr, ldy, M, N, alpha, beta, TM, TN, int(aligned), variant)
        elif op == "scale":
            st = tm.tm_scale2d(X.ptr, ldx, Y.ptr, ldy, M, N, 1.5, TM, TN, int(aligned), variant)
        else:
            st = tm.tm_copy2d(X.ptr, ldx, Y.ptr, ldy, M, N, TM, TN, int(aligned), variant)
        assert st == expected_map_status(X, Y, M, N, ldx, ldy, TM, TN, aligned, variant), tm.tm_status_string(st)
        torch.cuda.synchronize()
        want = sentinel_host(Y.buf.numel())
        if st == tm.TM_OK:
            region = want[Y.off:Y.off + Y.n].copy()
            if op == "affine":
                oracle.map_affine(xh, ldx, region, ldy, M, N, alpha, beta)
            elif op == "scale":
                oracle.scale2d(xh, ldx, region, ldy, M, N, 1.5)
            elif op == "copy":
                oracle.copy2d(xh, ldx, region, ldy, M, N)
            else:
                oracle.channel_affine(xh, ldx, sh, bh, region, ldy, M, N)
            want[Y.off:Y.off + Y.n] = region
            ran["ok"] += 1
        else:
            ran["refused"] += 1
        assert np.array_equal(bits(Y.host()), bits(want)), "case %d" % case
        assert X.guards_intact()
    note("fuzz maps: %s" % ran)
    assert ran["ok"] >= 200


def test_fuzz_maps_line_grid(dev):
    """Maps on views whose bases and row strides sit on 128-byte lines (one-wave work items of
    whole lines; with 16-byte chunks mostly one 1 KiB row segment moved with buffer accesses):
    random shapes, tiles, variants and paths, bit for bit against the oracle, one-line guards."""
    rng = random.Random(2025)
    ran = 0
    for case in range(200):
        op = rng.choice(["affine", "scale", "copy", "channel"])
        TM, TN = rng.choice(TMS), rng.choice(TNS)
        variant = rng.choice([tm.TM_VAR_AUTO, tm.TM_VAR_VEC4, tm.TM_VAR_VEC4, tm.TM_VAR_SCALAR])
        aligned = rng.random() < 0.4 and TN % 4 == 0
        if aligned:
            M = TM * rng.randint(1, max(1, 300 // TM))
            N = TN * rng.randint(1, max(1, 2100 // TN))
        else:
            M, N = rng.randint(1, 300), rng.randint(1, 2100)
        ldx = (N + 31) // 32 * 32 + 32 * rng.randint(0, 2)
        ldy = (N + 31) // 32 * 32 + 32 * rng.randint(0, 2)
        note("fuzz line-grid map %d: %s M=%d N=%d ldx=%d ldy=%d tile=%dx%d aligned=%d variant=%d"
             % (case, op, M, N, ldx, ldy, TM, TN, aligned, variant))
        nx, ny = (M - 1) * ldx + N, M * ldy
        xh = inputs.uniform(3000 + case, nx, -8.0, 8.0)
        X = Guarded(nx, dev, 0, LINE_GUARD_FLOATS)
        X.upload(xh)
        Y = Guarded(ny, dev, 0, LINE_GUARD_FLOATS)
        if op == "channel":
            bh = inputs.uniform(4000 + case, N, -1.0, 1.0)
            sh = inputs.uniform(5000 + case, N, 0.5, 1.5) if rng.random() < 0.5 else None
            B = Guarded(N, dev)
            B.upload(bh)
            S = Guarded(N, dev)
            if sh is not None:
                S.upload(sh)
            st = tm.tm_channel_affine(X.ptr, ldx, S.ptr if sh is not None else None, B.ptr, Y.ptr, ldy, M, N,
                                      TM, TN, int(aligned), variant)
        elif op == "affine":
            st = tm.tm_map_affine(X.ptr, ldx, Y.ptr, ldy, M, N, 0.75, -0.25, TM, TN, int(aligned), variant)
        elif op == "scale":
            st = tm.tm_scale2d(X.ptr, ldx, Y.ptr, ldy, M, N, 1.5, TM, TN, int(aligned), variant)
        else:
            st = tm.tm_copy2d(X.ptr, ldx, Y.ptr, ldy, M, N, TM, TN, int(aligned), variant)
        assert st == expected_map_status(X, Y, M, N, ldx, ldy, TM, TN, aligned, variant), tm.tm_status_string(st)
        torch.cuda.synchronize()
        want = sentinel_host(Y.buf.numel())
        if st == tm.TM_OK:
            region = want[Y.off:Y.off + Y.n].copy()
            if op == "affine":
                oracle.map_affine(xh, ldx, region, ldy, M, N, 0.75, -0.25)
            elif op == "scale":
                oracle.scale2d(xh, ldx, region, ldy, M, N, 1.5)
            elif op == "copy":
                oracle.copy2d(xh, ldx, region, ldy, M, N)
            else:
                oracle.channel_affine(xh, ldx, sh, bh, region, ldy, M, N)
            want[Y.off:Y.off + Y.n] = region
            ran += 1
        assert np.array_equal(bits(Y.host()), bits(want)), "case %d" % case
        assert X.guards_intact()
    note("fuzz line-grid maps: %d ran" % ran)
    assert ran >= 120


def test_fuzz_reductions(dev):
    rng = random.Random(77)
    for case in range(250):
        kind = rng.choice(["rowsum", "rowmax", "softmax", "colsum"])
        TM, TN = rng.choice(TMS), rng.choice(TNS)
        aligned = rng.random() < 0.3 and TN % 4 == 0
        M, N, ld, _, off, _ = draw_view(rng, aligned, TM, TN)
        walk = rng.choice([tm.TM_COL_NAIVE, tm.TM_COL_LDS, tm.TM_COL_NAIVE_XCD])
        note("fuzz reduction %d: %s M=%d N=%d ld=%d off=%d tile=%dx%d aligned=%d walk=%d"
             % (case, kind, M, N, ld, off, TM, TN, aligned, walk))
        n = (M - 1) * ld + N
        lo, hi = (0.0, 1.0) if kind in ("rowsum", "colsum") else (-10.0, -1.0)
        xh = inputs.uniform(500 + case, n, lo, hi)
        X = Guarded(n, dev, off)
        X.upload(xh)
        promise = oracle.promise_holds(M, N, ld, ld, TM, TN, X.ptr, 0)
        want_st = tm.TM_E_ALIGN if aligned and not promise else tm.TM_OK
        if kind == "colsum":
            O = Guarded(N, dev)
            wsb = tm.tm_colsum_workspace_bytes(M, N, TM, TN, walk)
            W = Guarded(max(wsb // 4, 1), dev)
            st = tm.tm_colsum(X.ptr, ld, O.ptr, M, N, TM, TN, int(aligned), walk, W.ptr, wsb)
            assert st == want_st, tm.tm_status_string(st)
            torch.cuda.synchronize()
            if st == tm.TM_OK:
                ref = oracle.colsum_f64(xh, ld, M, N)
                got = O.payload().cpu().numpy().astype(np.float64)
                assert (np.abs(got - ref) <= sum_tol(ref)).all(), "case %d" % case
            assert O.guards_intact()
            continue
        O = Guarded(M, dev)
        if kind == "rowsum":
            st = tm.tm_rowsum(X.ptr, ld, O.ptr, M, N, TM, TN, int(aligned))
        elif kind == "rowmax":
            st = tm.tm_rowmax_masked(X.ptr, ld, O.ptr, M, N, TM, TN, int(aligned))
        else:
            L = Guarded(M, dev)
            st = tm.tm_softmax_stats(X.ptr, ld, O.ptr, L.ptr, M, N, TM, TN, int(aligned))
        assert st == want_st, tm.tm_status_string(st)
        torch.cuda.synchronize()
        if st != tm.TM_OK:
            assert (bits(O.buf) == bits(sentinel_host(1))[0]).all()
            continue
        got = O.payload().cpu().numpy()
        if kind == "rowsum":
            ref = oracle.rowsum_f64(xh, ld, M, N)
            assert (np.abs(got.astype(np.float64) - ref) <= sum_tol(ref)).all(), "case %d" % case
        elif kind == "rowmax":
            assert np.array_equal(bits(got), bits(oracle.rowmax(xh, ld, M, N))), "case %d" % case
        else:
            m_ref, l_ref = oracle.softmax_stats(xh, ld, M, N)
            assert np.array_equal(bits(got), bits(m_ref)), "case %d" % case
            l = L.payload().cpu().numpy().astype(np.float64)
            assert (np.abs(l - l_ref) <= 1e-5 * l_ref).all(), "case %d" % case
            assert L.guards_intact()
        assert O.guards_intact()


def test_fuzz_long_rows(dev):
    """Row reductions on long rows (N from 1025 to 60000) with few to many rows (M from 1 to 4000,
    at most 6M elements): rows of one wave and rows of a 128- to 1024-lane workgroup whose waves
    combine through LDS, on 16-byte and 4-byte rows (random strides and base offsets)."""
    rng = random.Random(78)
    for case in range(40):
        kind = rng.choice(["rowsum", "rowmax", "softmax"])
        N = int(1025 * (60000 / 1025) ** rng.random())               # log-uniform
        M = max(1, int(min(4000, 6_000_000 // N) ** rng.random()))   # log-uniform from 1
        ld = N + rng.choice([0, 0, 0, 4, 1, 3])
        off = rng.choice([0, 0, 0, 1])
        TM, TN = rng.choice(TMS), rng.choice(TNS)
        note("fuzz long rows %d: %s M=%d N=%d ld=%d off=%d tile=%dx%d" % (case, kind, M, N, ld, off, TM, TN))
        n = (M - 1) * ld + N
        lo, hi = (0.0, 1.0) if kind == "rowsum" else (-10.0, -1.0)
        xh = inputs.uniform(900 + case, n, lo, hi)
        X = Guarded(n, dev, off)
        X.upload(xh)
        O = Guarded(M, dev)
        if kind == "rowsum":
            st = tm.tm_rowsum(X.ptr, ld, O.ptr, M, N, TM, TN, 0)
        elif kind == "rowmax":
            st = tm.tm_rowmax_masked(X.ptr, ld, O.ptr, M, N, TM, TN, 0)
        else:
            L = Guarded(M, dev)
            st = tm.tm_softmax_stats(X.ptr, ld, O.ptr, L.ptr, M, N, TM, TN, 0)
        assert st == tm.TM_OK, tm.tm_status_string(st)
        torch.cuda.synchronize()
        got = O.payload().cpu().numpy()
        if kind == "rowsum":
            ref = oracle.rowsum_f64(xh, ld, M, N)
            assert (np.abs(got.astype(np.float64) - ref) <= sum_tol(ref)).all(), "case %d" % case
        elif kind == "rowmax":
            assert np.array_equal(bits(got), bits(oracle.rowmax(xh, ld, M, N))), "case %d" % case
        else:
            m_ref, l_ref = oracle.softmax_stats(xh, ld, M, N)
            assert np.array_equal(bits(got), bits(m_ref)), "case %d" % case
            l = L.payload().cpu().numpy().astype(np.float64)
            assert (np.abs(l - l_ref) <= 1e-5 * l_ref).all(), "case %d" % case
            assert L.guards_intact()
        assert O.guards_intact()


def test_fuzz_split_rows(dev):
    """The row calls with a workspace on random shapes around the split rule (M from 1 to 200,
    N from 60000 to 600000, at most 12M elements): split and one-pass walks, 16-byte and 4-byte
    rows, random strides, base offsets and tiles; a workspace of exactly the reported size between
    guard bands."""
    rng = random.Random(79)
    for case in range(40):
        kind = rng.choice(["rowsum", "rowmax", "softmax"])
        N = int(60000 * 10 ** rng.random())                          # log-uniform
        M = max(1, int(min(200, 12_000_000 // N) ** rng.random()))   # log-uniform from 1
        ld = N + rng.choice([0, 0, 0, 4, 1, 3])
        off = rng.choice([0, 0, 0, 1])
        TM, TN = rng.choice(TMS), rng.choice(TNS)
        wsb = tm.tm_rows_workspace_bytes(M, N)
        note("fuzz split rows %d: %s M=%d N=%d ld=%d off=%d tile=%dx%d ws=%d" % (case, kind, M, N, ld, off,
                                                                                TM, TN, wsb))
        n = (M - 1) * ld + N
        lo, hi = (0.0, 1.0) if kind == "rowsum" else (-10.0, -1.0)
        xh = inputs.uniform(950 + case, n, lo, hi)
        X = Guarded(n, dev, off)
        X.upload(xh)
        O = Guarded(M, dev)
        W = Guarded(max(wsb // 4, 1), dev)
        if kind == "rowsum":
            st = tm.tm_rowsum_ws(X.ptr, ld, O.ptr, M, N, TM, TN, 0, W.ptr, wsb)
        elif kind == "rowmax":
            st = tm.tm_rowmax_masked_ws(X.ptr, ld, O.ptr, M, N, TM, TN, 0, W.ptr, wsb)
        else:
            L = Guarded(M, dev)
            st = tm.tm_softmax_stats_ws(X.ptr, ld, O.ptr, L.ptr, M, N, TM, TN, 0, W.ptr, wsb)
        assert st == tm.TM_OK, tm.tm_status_string(st)
        torch.cuda.synchronize()
        got = O.payload().cpu().numpy()
        if kind == "rowsum":
            ref = oracle.rowsum_f64(xh, ld, M, N)
            assert (np.abs(got.astype(np.float64) - ref) <= sum_tol(ref)).all(), "case %d" % case
        elif kind == "rowmax":
            assert np.array_equal(bits(got), bits(oracle.rowmax(xh, ld, M, N))), "case %d" % case
        else:
            m_ref, l_ref = oracle.softmax_stats(xh, ld, M, N)
            assert np.array_equal(bits(got), bits(m_ref)), "case %d" % case
            l = L.payload().cpu().numpy().astype(np.float64)
            assert (np.abs(l - l_ref) <= 1e-5 * l_ref).all(), "case %d" % case
            assert L.guards_intact()
        assert O.guards_intact() and W.guards_intact()


def test_fuzz_transposes(dev):
    rng = random.Random(5150)
    ok = 0
    for case in range(200):
        TM, TN = rng.choice(TMS), rng.choice(TNS)
        aligned = rng.random() < 0.35 and TM % 4 == 0 and TN % 4 == 0
        B = rng.randint(1, 4)
        if aligned:
            M = TM * rng.randint(1, max(1, 200 // TM))
            N = TN * rng.randint(1, max(1, 400 // TN))
            ldx, ldy = N + 4 * rng.randint(0, 4), M + 4 * rng.randint(0, 4)
            offx, offy = 4 * rng.randint(0, 2), 4 * rng.randint(0, 2)
        else:
            M, N = rng.randint(1, 200), rng.randint(1, 400)
            ldx, ldy = N + rng.randint(0, 9), M + rng.randint(0, 9)
            offx, offy = rng.choice([0, 1, 3, 4]), rng.choice([0, 2, 4])
        bsx = (M - 1) * ldx + N + (4 * rng.randint(0, 3) if aligned else rng.randint(0, 5))
        bsy = (N - 1) * ldy + M + (4 * rng.randint(0, 3) if aligned else rng.randint(0, 5))
        if aligned:
            bsx, bsy = -(-bsx // 4) * 4, -(-bsy // 4) * 4
        note("fuzz transpose %d: B=%d M=%d N=%d ld=%d,%d bs=%d,%d offs=%d,%d tile=%dx%d aligned=%d"
             % (case, B, M, N, ldx, ldy, bsx, bsy, offx, offy, TM, TN, aligned))
        nx, ny = (B - 1) * bsx + (M - 1) * ldx + N, (B - 1) * bsy + (N - 1) * ldy + M
        xh = inputs.uniform(900 + case, nx, -4.0, 4.0)
        X = Guarded(nx, dev, offx)
        X.upload(xh)
        Y = Guarded(ny, dev, offy)
        st = tm.tm_transpose(X.ptr, ldx, bsx, Y.ptr, ldy, bsy, B, M, N, TM, TN, int(aligned))
        vec = (TM % 4 == 0 and TN % 4 == 0 and rows16(X.ptr, M, ldx) and rows16(Y.ptr, N, ldy)
               and (B <= 1 or (bsx % 4 == 0 and bsy % 4 == 0)))
        want_st = tm.TM_E_ALIGN if aligned and not (M % TM == 0 and N % TN == 0 and vec) else tm.TM_OK
        assert st == want_st, tm.tm_status_string(st)
        torch.cuda.synchronize()
        want = sentinel_host(Y.buf.numel())
        if st == tm.TM_OK:
            region = want[Y.off:Y.off + Y.n].copy()
            oracle.transpose(xh, ldx, bsx, region, ldy, bsy, B, M, N)
            want[Y.off:Y.off + Y.n] = region
            ok += 1
        assert np.array_equal(bits(Y.host()), bits(want)), "case %d" % case
        assert X.guards_intact()
    assert ok >= 140


def test_fuzz_padded_spans(dev):
    """Padded rows (the span plan of 1 KiB items on y's 1 KiB grid when y's padding is under a
    line, at most an eighth of the row or (rows off the line grid) up to half of it, and x's
    stride is the same or, over rows of 1024 floats or more, another; x at any 4-byte phase;
    the 2-D tile plan otherwise): random shapes, paddings, strides, offsets, ops (the channel op
    too) and variants, bit for bit, the padding between rows untouched."""
    rng = random.Random(4242)
    for case in range(150):
        op = rng.choice(["affine", "scale", "copy", "channel", "channel_scale"])
        variant = rng.choice([tm.TM_VAR_AUTO, tm.TM_VAR_AUTO, tm.TM_VAR_VEC4, tm.TM_VAR_SCALAR])
        # x's stride: mostly the same, else a multiple of 4 floats away, or not (the span over
        # 16-byte rows from 1024 floats on, over rows off the 16-byte grid at any width)
        diff = rng.random() >= 0.6
        M = rng.randint(2, 300)
        N = rng.randint(64, 2600) if diff else (rng.randint(64, 1100) if rng.random() < 0.7 else rng.randint(1024, 4200))
        u = rng.random()   # y's padding: under a line, up to an eighth of the row, or wider
        ld = N + (rng.randint(1, 31) if u < 0.55 else rng.randint(32, max(32, N // 8 + 3)) if u < 0.8
                  else rng.randint(N // 8, N // 2 + 3))
        ldx = max(N, ld + rng.choice([-8, -4, 4, 8, 12, 40, 3, -1])) if diff else ld
        offx = rng.choice([0, 1, 2, 3, 5, 64, 100])
        offy = offx if rng.random() < 0.8 else rng.choice([0, 1, 2, 3])
        note("fuzz span %d: %s M=%d N=%d ldx=%d ld=%d offs=%d,%d variant=%d" % (case, op, M, N, ldx, ld, offx, offy, variant))
        n = (M - 1) * ld + N
        nx = (M - 1) * ldx + N
        xh = inputs.uniform(7000 + case, nx, -8.0, 8.0)
        X = Guarded(nx, dev, offx, LINE_GUARD_FLOATS)
        X.upload(xh)
        Y = Guarded(n, dev, offy, LINE_GUARD_FLOATS)
        sh = None
        if op.startswith("channel"):
            bh = inputs.uniform(7500 + case, N, -1.0, 1.0)
            Bv = Guarded(N, dev, rng.choice([0, 1, 4]))
            Bv.upload(bh)
            if op == "channel_scale":
                sh = inputs.uniform(7700 + case, N, 0.5, 1.5)
                Sv = Guarded(N, dev, rng.choice([0, 4]))
                Sv.upload(sh)
            st = tm.tm_channel_affine(X.ptr, ldx, Sv.ptr if sh is not None else None, Bv.ptr, Y.ptr, ld, M, N,
                                      64, 64, 0, variant)
        elif op == "affine":
            st = tm.tm_map_affine(X.ptr, ldx, Y.ptr, ld, M, N, 0.75, -0.25, 64, 64, 0, variant)
        elif op == "scale":
            st = tm.tm_scale2d(X.ptr, ldx, Y.ptr, ld, M, N, 1.5, 64, 64, 0, variant)
        else:
            st = tm.tm_copy2d(X.ptr, ldx, Y.ptr, ld, M, N, 64, 64, 0, variant)
        vec_ok = rows16(X.ptr, M, ldx) and rows16(Y.ptr, M, ld)
        assert st == (tm.TM_OK if variant != tm.TM_VAR_VEC4 or vec_ok else tm.TM_E_ALIGN), tm.tm_status_string(st)
        torch.cuda.synchronize()
        want = sentinel_host(Y.buf.numel())
        if st == tm.TM_OK:
            region = want[Y.off:Y.off + n].copy()
            if op == "affine":
                oracle.map_affine(xh, ldx, region, ld, M, N, 0.75, -0.25)
            elif op == "scale":
                oracle.scale2d(xh, ldx, region, ld, M, N, 1.5)
            elif op == "copy":
                oracle.copy2d(xh, ldx, region, ld, M, N)
            else:
                oracle.channel_affine(xh, ldx, sh, bh, region, ld, M, N)
            want[Y.off:Y.off + n] = region
        assert np.array_equal(bits(Y.host()), bits(want)), "case %d" % case
        assert X.guards_intact()


def test_fuzz_line_windows(dev):
    """One large matrix whose y rows miss the 128-byte line grid (line-aligned y windows from a band
    of x rows): random shapes of 4-7M elements, strides and base offsets, bit for bit."""
    rng = random.Random(777)
    for case in range(10):
        N = rng.randint(40, 3000)
        M = max(64, (rng.randint(4_200_000, 7_000_000) // N))
        ldx = N + rng.choice([0, 1, 3, 4, 7, 32])
        ldy = M + rng.choice([1, 2, 3, 4, 5, 17, 33])
        offx, offy = rng.choice([0, 1, 4]), rng.choice([0, 1, 2, 3, 9])
        note("fuzz line windows %d: M=%d N=%d ld=%d,%d offs=%d,%d" % (case, M, N, ldx, ldy, offx, offy))
        nx, ny = (M - 1) * ldx + N, (N - 1) * ldy + M
        xh = inputs.uniform(8000 + case, nx, -4.0, 4.0)
        X = Guarded(nx, dev, offx)
        X.upload(xh)
        Y = Guarded(ny, dev, offy)
        assert tm.tm_transpose(X.ptr, ldx, 0, Y.ptr, ldy, 0, 1, M, N, 1, 1, 0) == tm.TM_OK
        torch.cuda.synchronize()
        want = sentinel_host(Y.buf.numel())
        region = want[Y.off:Y.off + Y.n].copy()
        oracle.transpose(xh, ldx, 0, region, ldy, 0, 1, M, N)
        want[Y.off:Y.off + Y.n] = region
        assert np.array_equal(bits(Y.host()), bits(want)), "case %d" % case
        assert X.guards_intact()
