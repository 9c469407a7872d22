"""GPU parity of the LDS walk's kernel for wide matrices (a workgroup per slab of rows and strip of
256 columns, each lane of its 8 waves one 16-byte column chunk over an eighth of the slab's rows;
then a fold of the slab partials), against the
fp64 oracle: the column-sum workload, matrices ragged in rows and columns, integer data (every
partial sum exact, so the result is exact too), and the same call with a workspace off the
16-byte grid, which takes the LDS-staged kernel instead and must agree within the bound.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from edge_masking_vector_amd import inputs
from gpu_helpers import Guarded, bits, sum_tol

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


def _colsum(dev, xh, M, N, ld, TM, TN, aligned, ws_offset=0):
    x = torch.from_numpy(xh).to(dev)
    wsb = tm.tm_colsum_workspace_bytes(M, N, TM, TN, tm.TM_COL_LDS)
    ws = torch.empty(wsb // 4 + 8, device=dev)
    out = Guarded(N, dev)
    st = tm.tm_colsum(x, ld, out.ptr, M, N, TM, TN, aligned, tm.TM_COL_LDS, ws.data_ptr() + 4 * ws_offset,
                      wsb, torch.cuda.current_stream())
    assert st == tm.TM_OK, tm.tm_status_string(st)
    torch.cuda.synchronize()
    assert out.guards_intact()
    return out.payload().cpu().numpy()


@pytest.mark.parametrize("M,N,ld,TM,TN,aligned", [
    (4096, 4096, 4096, 256, 64, 1),     # the column-sum workload
    (7000, 3000, 3000, 1, 4, 0),        # ragged rows (7000 = 109 slabs of 64 + 24) and strips (11 x 256 + 184)
    (16384, 1024, 1028, 64, 256, 0),    # padded rows, four strips
    (2048, 8192, 8192, 64, 1024, 1),    # short and wide
    (20000, 4096, 4096, 1, 4, 0),       # tall: 157 slabs of 128 rows (16 per wave, 2 batches), the last of 32
])
def test_strip_walk_against_oracle(dev, M, N, ld, TM, TN, aligned):
    note("strip colsum %dx%d ld %d" % (M, N, ld))
    xh = inputs.matrix(inputs.uniform(M + N, M * N, 0.0, 1.0), M, N, ld)
    got = _colsum(dev, xh, M, N, ld, TM, TN, aligned)
    want = oracle.colsum_f64(xh, ld, M, N)
    assert np.all(np.abs(got.astype(np.float64) - want) <= sum_tol(want))
    # the same call with the workspace 4 bytes off the 16-byte grid runs the LDS-staged kernel
    other = _colsum(dev, xh, M, N, ld, TM, TN, aligned, ws_offset=1)
    assert np.all(np.abs(other.astype(np.float64) - want) <= sum_tol(want))


def test_strip_walk_exact_on_integers(dev):
    """Integers 0..15: every partial sum is an exact f32 integer, so the sums are bit-exact."""
    M, N = 7000, 3000
    xh = inputs.integers(5, M * N, 0, 16).astype(np.float32)
    got = _colsum(dev, xh, M, N, N, 1, 4, 0)
    want = oracle.colsum_f64(xh, N, M, N)
    assert np.array_equal(got.astype(np.float64), want)


def test_strip_workspace_query_covers_both_kernels(dev):
    """The size query does not know the workspace's alignment: it covers the strip kernel's slabs
    and the LDS-staged kernel's, whichever is more."""
    for M, N in ((4096, 4096), (7000, 3000), (16384, 1024)):
        wsb = tm.tm_colsum_workspace_bytes(M, N, 1, 4, tm.TM_COL_LDS)
        assert wsb >= -(-M // 64) * N * 4 or wsb >= 256 * N * 4


@pytest.mark.parametrize("M,N,ld,xoff", [
    (4096, 4096, 4097, 0),    # rows off the 16-byte grid, whole strips: the strip walk
    (4096, 4096, 4096, 1),    # the base one float off it
    (1000, 3072, 3072, 3),    # ragged slabs
    (64, 1024, 1027, 0),      # one slab
    (2048, 2051, 2051, 0),    # a part-filled last strip: the LDS-staged walk
    (3000, 1025, 1030, 3),
    (700, 5002, 5002, 2),
])
def test_strip_walk_unaligned_rows(dev, M, N, ld, xoff):
    """Rows off the 16-byte grid: with whole strips, the strip walk with 4-byte aligned 16-byte
    loads; otherwise the LDS-staged walk.  The padding between rows and the floats past the view
    hold NaN, so a sum that took any of them would be NaN; within the bound on U[0,1) data and
    bit-exact on integers."""
    note("strip colsum unaligned %dx%d ld %d off %d" % (M, N, ld, xoff))
    n = (M - 1) * ld + N
    for data in ("uniform", "integers"):
        vals = (inputs.uniform(M + N + xoff, M * N, 0.0, 1.0) if data == "uniform"
                else inputs.integers(M + 3 * N, M * N, 0, 16).astype(np.float32))
        xh = inputs.matrix(vals, M, N, ld, pad=np.nan)[:n]
        buf = np.concatenate([np.zeros(xoff, np.float32), xh, np.full(64, np.nan, np.float32)])
        x = torch.from_numpy(buf).to(dev)
        wsb = tm.tm_colsum_workspace_bytes(M, N, 1, 4, tm.TM_COL_LDS)
        ws = torch.empty(wsb // 4 + 8, device=dev)
        out = Guarded(N, dev)
        st = tm.tm_colsum(x.data_ptr() + 4 * xoff, ld, out.ptr, M, N, 1, 4, 0, tm.TM_COL_LDS, ws, wsb,
                          torch.cuda.current_stream())
        assert st == tm.TM_OK, tm.tm_status_string(st)
        torch.cuda.synchronize()
        assert out.guards_intact()
        got = out.payload().cpu().numpy().astype(np.float64)
        want = oracle.colsum_f64(xh, ld, M, N)
        assert np.all(np.isfinite(got)), data
        if data == "integers":
            assert np.array_equal(got, want)
        else:
            assert np.all(np.abs(got - want) <= sum_tol(want))


@pytest.mark.parametrize("M,N,ld,xoff", [
    (16, 1 << 20, (1 << 20) + 1, 0),   # rows off the 16-byte grid
    (64, 262147, 262147, 1),           # N % 4 == 3, the base one float off
    (1, 1001, 1001, 3),                # one row
    (7, 5003, 5010, 2),
])
def test_direct_walk_unaligned_rows(dev, M, N, ld, xoff):
    """Few rows take the one-pass walk (no workspace), whose 16-byte column chunks are loads from
    4-byte aligned addresses when the rows are off the 16-byte grid and whose last chunk of a row
    moves element by element.  NaN in the padding and past the view must reach no sum; within the
    bound on U[0,1) data, bit-exact on integers."""
    note("direct colsum unaligned %dx%d ld %d off %d" % (M, N, ld, xoff))
    assert tm.tm_colsum_workspace_bytes(M, N, 1, 4, tm.TM_COL_LDS) == 0   # the one-pass walk
    n = (M - 1) * ld + N
    for data in ("uniform", "integers"):
        vals = (inputs.uniform(M + N + xoff, M * N, 0.0, 1.0) if data == "uniform"
                else inputs.integers(M + 3 * N, M * N, 0, 16).astype(np.float32))
        xh = inputs.matrix(vals, M, N, ld, pad=np.nan)[:n]
        buf = np.concatenate([np.zeros(xoff, np.float32), xh, np.full(64, np.nan, np.float32)])
        x = torch.from_numpy(buf).to(dev)
        out = Guarded(N, dev)
        st = tm.tm_colsum(x.data_ptr() + 4 * xoff, ld, out.ptr, M, N, 1, 4, 0, tm.TM_COL_LDS, None, 0,
                          torch.cuda.current_stream())
        assert st == tm.TM_OK, tm.tm_status_string(st)
        torch.cuda.synchronize()
        assert out.guards_intact()
        got = out.payload().cpu().numpy().astype(np.float64)
        want = oracle.colsum_f64(xh, ld, M, N)
        assert np.all(np.isfinite(got)), data
        if data == "integers":
            assert np.array_equal(got, want)
        else:
            assert np.all(np.abs(got - want) <= sum_tol(want))
