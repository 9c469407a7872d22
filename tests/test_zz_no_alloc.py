"""tm_colsum_noalloc (the column sum without a workspace, its partials in the library's static
device array) against tm_colsum with a caller workspace, through the C ABI: two calls in a row,
the second on a smaller input, so the second call reads the array after the first call's partials
were left in it.  Same kernels, same fold order: the sums must agree bit for bit (and with the
fp64 oracle within 1e-5 of sum |x|).  Output guard bands stay untouched; a call needing more
partials than the array holds is refused before anything is enqueued.
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


def _both(dev, M, N, TM, TN, aligned, walk, seed):
    note("noalloc colsum %dx%d tile %dx%d aligned %d walk %d" % (M, N, TM, TN, aligned, walk))
    xh = inputs.uniform(seed, M * N, 0.0, 1.0)
    x = torch.from_numpy(xh).to(dev)
    s = torch.cuda.current_stream()
    # reference: the workspace call
    wsb = tm.tm_colsum_workspace_bytes(M, N, TM, TN, walk)
    assert wsb <= tm.TM_COLSUM_NOALLOC_MAX_BYTES
    ws = torch.empty(max(wsb // 4, 1), device=dev)
    ref = Guarded(N, dev)
    assert tm.tm_colsum(x, N, ref.ptr, M, N, TM, TN, aligned, walk, ws, wsb, s) == tm.TM_OK
    got = Guarded(N, dev)
    assert tm.tm_colsum_noalloc(x, N, got.ptr, M, N, TM, TN, aligned, walk, s) == tm.TM_OK
    torch.cuda.synchronize()
    assert got.guards_intact() and ref.guards_intact()
    g, r = got.payload().cpu().numpy(), ref.payload().cpu().numpy()
    assert np.array_equal(bits(g), bits(r)), (M, N, walk)
    want = oracle.colsum_f64(xh, N, M, N)
    assert np.all(np.abs(g.astype(np.float64) - want) <= sum_tol(want))


@pytest.mark.parametrize("walk", [tm.TM_COL_LDS, tm.TM_COL_NAIVE])
def test_noalloc_matches_workspace_call_twice(dev, walk):
    """The column-sum workload (4096 x 4096, aligned), then a smaller ragged matrix (1000 x 777)."""
    if walk == tm.TM_COL_LDS:
        _both(dev, 4096, 4096, 256, 64, 1, walk, seed=81)
    else:
        _both(dev, 4096, 4096, 256, 1, 0, walk, seed=81)
    _both(dev, 1000, 777, 64, 64, 0, walk, seed=82)


def test_noalloc_refuses_more_than_the_array(dev):
    """4 * 2^20 partials do not fit 16 MiB: TM_E_WORKSPACE, nothing enqueued, out untouched."""
    M, N = 1 << 20, 4096
    need = tm.tm_colsum_workspace_bytes(M, N, 256, 64, tm.TM_COL_LDS)
    assert need > tm.TM_COLSUM_NOALLOC_MAX_BYTES
    x = torch.zeros(16, device=dev)       # never read: the call is refused on the host
    out = Guarded(16, dev)
    st = tm.tm_colsum_noalloc(x, N, out.ptr, M, N, 256, 64, 0, tm.TM_COL_LDS)
    assert st == tm.TM_E_WORKSPACE
    torch.cuda.synchronize()
    assert out.guards_intact()
    assert (bits(out.payload()) == 0x7F7F7F7F).all()
    # argument errors come first, as for tm_colsum
    assert tm.tm_colsum_noalloc(x, N, out.ptr, M, N, 256, 63, 0, tm.TM_COL_LDS) == tm.TM_E_UNSUPPORTED
