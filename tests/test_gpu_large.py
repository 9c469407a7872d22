"""Reductions, the transpose and a padded-row map on a tensor of more than 2**31 elements (64-bit addressing):
65792 x 32768 f32 (8.6 GB), built on the device by tiling one seeded block of 64 rows, so that
any row is known on the host.  Sampled rows (including those around element 2**31 and the last
ones) are checked against the oracle; column sums against the oracle's sums of the block times
the 1028 repetitions; the transpose on whole sampled output rows.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from edge_masking_vector_amd import inputs
from gpu_helpers import SENTINEL, bits, sum_tol

pytestmark = pytest.mark.gpu
tm = pytest.importorskip("edge_masking_vector_amd.tilemap")

M, N, BLK = 65792, 32768, 64          # M = 1028 * 64 = 257 * 256; M * N > 2**31
ROWS = (0, 1, 63, 64, 65535, 65536, 65537, M - 2, M - 1)   # row 65536 starts at element 2**31


def note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def big():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = torch.device("cuda:0")
    blk = inputs.uniform(19, BLK * N, -10.0, -1.0)
    x = torch.empty(M, N, dtype=torch.float32, device=dev)
    x.copy_(torch.from_numpy(blk).to(dev).view(BLK, N).repeat(M // BLK, 1))
    torch.cuda.synchronize()
    yield dev, x, blk
    del x
    torch.cuda.empty_cache()


def block_row(blk, r):
    return blk[(r % BLK) * N:(r % BLK + 1) * N].copy()


def test_row_reductions_beyond_2g(big):
    dev, x, blk = big
    out = torch.empty(M, device=dev)
    l = torch.empty(M, device=dev)
    note("rowsum %dx%d" % (M, N))
    assert tm.tm_rowsum(x, N, out, M, N, 4, 256, 1) == tm.TM_OK
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    for r in ROWS:
        ref = oracle.rowsum_f64(block_row(blk, r), N, 1, N)
        assert abs(got[r] - ref[0]) <= sum_tol(abs(ref[0])), r
    note("rowmax %dx%d" % (M, N))
    assert tm.tm_rowmax_masked(x, N, out, M, N, 16, 64, 1) == tm.TM_OK
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for r in ROWS:
        assert bits(got[r:r + 1])[0] == bits(oracle.rowmax(block_row(blk, r), N, 1, N))[0], r
    note("softmax statistics %dx%d" % (M, N))
    assert tm.tm_softmax_stats(x, N, out, l, M, N, 16, 64, 1) == tm.TM_OK
    torch.cuda.synchronize()
    m_got, l_got = out.cpu().numpy(), l.cpu().numpy().astype(np.float64)
    for r in ROWS:
        m_ref, l_ref = oracle.softmax_stats(block_row(blk, r), N, 1, N)
        assert bits(m_got[r:r + 1])[0] == bits(m_ref)[0], r
        assert abs(l_got[r] - l_ref[0]) <= 1e-5 * l_ref[0], r


def test_column_sums_beyond_2g(big):
    dev, x, blk = big
    ref = oracle.colsum_f64(blk, N, BLK, N) * (M // BLK)
    absref = oracle.colsum_f64(np.abs(blk), N, BLK, N) * (M // BLK)
    out = torch.empty(N, device=dev)
    for walk, TM, TN in ((tm.TM_COL_LDS, 256, 64), (tm.TM_COL_NAIVE_XCD, 256, 1)):
        note("colsum %dx%d walk=%d" % (M, N, walk))
        wsb = tm.tm_colsum_workspace_bytes(M, N, TM, TN, walk)
        ws = torch.empty(wsb // 4, device=dev)
        assert tm.tm_colsum(x, N, out, M, N, TM, TN, int(walk == tm.TM_COL_LDS), walk, ws, wsb) == tm.TM_OK
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        assert (np.abs(got - ref) <= sum_tol(absref)).all(), walk
        del ws


def test_direct_column_sums_across_2g(big):
    """The one-pass column walk (64 rows) over rows 65504 .. 65567, which straddle element 2^31:
    every column against the oracle's sum of the same block rows."""
    dev, x, blk = big
    r0, M = 65504, 64
    assert tm.tm_colsum_workspace_bytes(M, N, 64, 64, tm.TM_COL_LDS) == 0
    view = x.view(-1)[r0 * N:]
    rows = np.concatenate([block_row(blk, r) for r in range(r0, r0 + M)])
    ref = oracle.colsum_f64(rows, N, M, N)
    absref = oracle.colsum_f64(np.abs(rows), N, M, N)
    out = torch.empty(N, device=dev)
    note("direct colsum rows %d..%d" % (r0, r0 + M - 1))
    assert tm.tm_colsum(view, N, out, M, N, 64, 64, 1, tm.TM_COL_LDS, None, 0) == tm.TM_OK
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert (np.abs(got - ref) <= sum_tol(absref)).all()


def test_transpose_beyond_2g(big):
    dev, x, blk = big
    note("transpose %dx%d" % (M, N))
    y = torch.empty(N, M, dtype=torch.float32, device=dev)
    assert tm.tm_transpose(x, N, 0, y, M, 0, 1, M, N, 32, 32, 1) == tm.TM_OK
    torch.cuda.synchronize()
    B = blk.reshape(BLK, N)
    for j in (0, 1, 31, 32, 16383, 16384, N - 1):
        got = y[j].cpu().numpy()                 # y row j = x column j
        want = np.tile(B[:, j], M // BLK)
        assert np.array_equal(bits(got), bits(want)), j
    del y
    torch.cuda.empty_cache()


def test_padded_map_near_and_beyond_2g(big):
    """The affine map over the big tensor read as padded rows (N - 5 of every N floats): with
    64000 rows the view is one span of just under 2**31 floats (32-bit span indexes near their
    limit), with every row it is more, and the 2-D tile plan takes it.  Sampled rows bit for bit
    against the oracle, the 5 padding floats of each and the rows past the view untouched."""
    dev, x, blk = big
    Np = N - 5
    y = torch.empty(M, N, dtype=torch.float32, device=dev)
    for Mr in (64000, M):
        y.fill_(float(SENTINEL))
        note("padded map %dx%d at stride %d" % (Mr, Np, N))
        assert tm.tm_map_affine(x, N, y, N, Mr, Np, 0.75, -0.25, 64, 64, 0, tm.TM_VAR_AUTO) == tm.TM_OK
        torch.cuda.synchronize()
        for r in sorted(set(ROWS + (Mr - 1, min(Mr, M - 1)))):
            got = y[r].cpu().numpy()
            want = np.full(N, SENTINEL, np.float32)
            if r < Mr:
                row = block_row(blk, r)
                oracle.map_affine(row, N, want, N, 1, Np, 0.75, -0.25)
            assert np.array_equal(bits(got), bits(want)), (Mr, r)
    del y
    torch.cuda.empty_cache()


def test_transpose_off_the_line_grid_beyond_2g(big):
    """The transpose of the big tensor into y rows of stride M + 3 (off the 128-byte line grid):
    line-aligned y windows with 64-bit addresses; sampled y rows bit for bit, their 3 padding
    floats untouched."""
    dev, x, blk = big
    ldy = M + 3
    note("transpose %dx%d to y stride %d" % (M, N, ldy))
    y = torch.empty(N * ldy, dtype=torch.float32, device=dev)
    y.fill_(float(SENTINEL))
    assert tm.tm_transpose(x, N, 0, y, ldy, 0, 1, M, N, 1, 1, 0) == tm.TM_OK
    torch.cuda.synchronize()
    B = blk.reshape(BLK, N)
    for j in (0, 1, 31, 32, 16383, 16384, N - 1):
        got = y[j * ldy:(j + 1) * ldy].cpu().numpy() if j < N - 1 else y[j * ldy:].cpu().numpy()
        want = np.full(got.size, SENTINEL, np.float32)
        want[:M] = np.tile(B[:, j], M // BLK)
        assert np.array_equal(bits(got), bits(want)), j
    del y
    torch.cuda.empty_cache()
