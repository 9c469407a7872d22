"""The library's calls captured into a HIP graph: they only enqueue kernels on the caller's stream,
so a captured sequence replays the same work.  The sequence -- scale, row sum, LDS column sum,
softmax statistics, transpose -- is replayed several times with eager work and synchronisations
between the replays, and every replay must reproduce the eager results bit for bit.
"""
import sys

import numpy as np
import pytest
import torch

from edge_masking_vector_amd import inputs

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


def run_sequence(bufs):
    x, y, rs, cs, ws, m, l, t = (bufs[k] for k in ("x", "y", "rs", "cs", "ws", "m", "l", "t"))
    M, N = x.shape
    tm.check(tm.tm_scale2d(x, N, y, N, M, N, 1.5, 32, 128, 1, tm.TM_VAR_VEC4))
    tm.check(tm.tm_rowsum(y, N, rs, M, N, 4, 256, 1))
    tm.check(tm.tm_colsum(y, N, cs, M, N, 64, 64, 1, tm.TM_COL_LDS, ws, ws.numel() * 4))
    tm.check(tm.tm_softmax_stats(x, N, m, l, M, N, 16, 64, 1))
    tm.check(tm.tm_transpose(y, N, 0, t, M, 0, 1, M, N, 32, 32, 1))


def test_captured_sequence_replays(dev):
    M, N = 512, 1024
    x = torch.from_numpy(inputs.scores_input(M, N, seed=41)).to(dev).view(M, N)
    wsb = tm.tm_colsum_workspace_bytes(M, N, 64, 64, tm.TM_COL_LDS)

    def fresh():
        return {"x": x, "y": torch.empty_like(x), "rs": torch.empty(M, device=dev),
                "cs": torch.empty(N, device=dev), "ws": torch.empty(wsb // 4, device=dev),
                "m": torch.empty(M, device=dev), "l": torch.empty(M, device=dev),
                "t": torch.empty(N, M, device=dev)}

    eager = fresh()
    run_sequence(eager)
    torch.cuda.synchronize()
    want = {k: v.clone() for k, v in eager.items() if k not in ("x", "ws")}

    bufs = fresh()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):          # warm the stream up before capture
        run_sequence(bufs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run_sequence(bufs)
    for replay in range(4):
        note("graph replay %d" % replay)
        for k in want:
            bufs[k].fill_(-7.0)          # clear the outputs with an eager fill kernel
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in want.items():
            assert torch.equal(bufs[k].view(torch.int32), v.view(torch.int32)), (replay, k)
        # eager library work between replays, on other buffers
        other = fresh()
        run_sequence(other)
        torch.cuda.synchronize()
        assert torch.equal(other["y"].view(torch.int32), want["y"].view(torch.int32))


def test_captured_split_rows_replay(dev):
    """The split softmax statistics (two launches sharing a workspace) captured into a graph:
    every replay reproduces the eager m and l bit for bit."""
    M, N = 8, 1 << 17
    s = torch.from_numpy(inputs.uniform(44, M * N, -10.0, -1.0)).to(dev)
    wsb = tm.tm_rows_workspace_bytes(M, N)
    assert wsb > 0
    ws = torch.empty(wsb // 4, device=dev)
    m0, l0 = torch.empty(M, device=dev), torch.empty(M, device=dev)
    tm.check(tm.tm_softmax_stats_ws(s, N, m0, l0, M, N, 1, 64, 0, ws, wsb))
    torch.cuda.synchronize()
    m, l = torch.empty(M, device=dev), torch.empty(M, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tm.check(tm.tm_softmax_stats_ws(s, N, m, l, M, N, 1, 64, 0, ws, wsb))
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        tm.check(tm.tm_softmax_stats_ws(s, N, m, l, M, N, 1, 64, 0, ws, wsb))
    for replay in range(4):
        note("split rows graph replay %d" % replay)
        m.fill_(-7.0)
        l.fill_(-7.0)
        ws.fill_(3.0)                # stale partials must be overwritten
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(m.view(torch.int32), m0.view(torch.int32)), replay
        assert torch.equal(l.view(torch.int32), l0.view(torch.int32)), replay


def test_threads_on_separate_streams(dev):
    """Four host threads, each with its own stream and buffers, run the sequence ten times at
    once; every thread's results equal the single-threaded ones (the library keeps no shared
    state, and kernels of different streams may overlap on the GPU)."""
    import threading
    M, N = 512, 1024
    x = torch.from_numpy(inputs.scores_input(M, N, seed=43)).to(dev).view(M, N)
    wsb = tm.tm_colsum_workspace_bytes(M, N, 64, 64, tm.TM_COL_LDS)

    def fresh():
        return {"x": x, "y": torch.empty_like(x), "rs": torch.empty(M, device=dev),
                "cs": torch.empty(N, device=dev), "ws": torch.empty(wsb // 4, device=dev),
                "m": torch.empty(M, device=dev), "l": torch.empty(M, device=dev),
                "t": torch.empty(N, M, device=dev)}

    ref = fresh()
    run_sequence(ref)
    torch.cuda.synchronize()
    results, errors = [None] * 4, []

    def worker(k):
        try:
            s = torch.cuda.Stream()
            b = fresh()
            with torch.cuda.stream(s):
                for _ in range(10):
                    run_sequence(b)
            s.synchronize()
            results[k] = b
        except Exception as e:  # reported below
            errors.append(e)

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
    for b in results:
        for key in ("y", "rs", "cs", "m", "l", "t"):
            assert torch.equal(b[key].view(torch.int32), ref[key].view(torch.int32)), key
