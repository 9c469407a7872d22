"""Python binding of libtilemap.so -- the same calls as include/tilemap.h, argument marshalling only.

Each function takes what the C call takes.  Pointer arguments accept a torch tensor (its
data_ptr() is passed; the tensor must live on the GPU the library runs on), a plain integer
address or None (NULL); `stream` accepts a torch stream, an integer hipStream_t, or None for
torch's current stream.  The return value is the C status code (TM_OK == 0); `check()` turns a
nonzero status into a TilemapError.  Calls that write results through host pointers in C return a
tuple starting with the status.  Nothing here computes any part of the maps or reductions: every
step runs in the HIP kernels, and importing this module fails loudly if libtilemap.so or its
extension module `_tilemap` (csrc/pyext.c, which calls the C ABI directly) has not been built.

torch is imported before the library is loaded so that both share one HIP runtime (the wheel's
libamdhip64 is then the one libtilemap.so binds to).
"""
import os

import torch  # noqa: F401  (must be loaded first: one HIP runtime per process)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtilemap.so")

TM_OK = 0
TM_E_INVAL = -1
TM_E_ALIGN = -2
TM_E_UNSUPPORTED = -3
TM_E_WORKSPACE = -4
TM_E_HIP = -5

TM_VAR_AUTO = 0
TM_VAR_SCALAR = 1
TM_VAR_VEC4_UNDERSTATED = 2
TM_VAR_VEC4 = 3

TM_COL_NAIVE = 0
TM_COL_LDS = 1
TM_COL_NAIVE_XCD = 2

TM_MAP_NONE = 0
TM_MAP_FLAT = 1
TM_MAP_SPAN = 2
TM_MAP_TILES = 3

TM_COLFORM_NONE = 0
TM_COLFORM_ONE_PASS = 1
TM_COLFORM_TILES = 2
TM_COLFORM_STRIPS = 3

if not os.path.exists(LIB_PATH):
    raise ImportError("libtilemap.so is not built (expected at %s); run "
                      "`python -c 'import __graft_entry__ as g; g.build()'` first" % LIB_PATH)
try:
    from . import _tilemap as _ext
except ImportError as e:
    raise ImportError("the _tilemap extension module is not built (%s); run "
                      "`python -c 'import __graft_entry__ as g; g.build()'` first" % e) from None


class TilemapError(RuntimeError):
    def __init__(self, status):
        self.status = status
        super().__init__("libtilemap returned %d (%s)" % (status, tm_status_string(status)))


def check(status):
    """Raise TilemapError unless status == TM_OK; returns TM_OK."""
    if status != TM_OK:
        raise TilemapError(status)
    return status


def _ptr(p):
    if isinstance(p, torch.Tensor):
        return p.data_ptr()
    if p is None or isinstance(p, int):
        return p
    raise TypeError("expected a torch tensor, an integer address or None, got %r" % type(p))


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def tm_map_affine(x, ldx, y, ldy, M, N, alpha, beta, TM, TN, aligned, variant=TM_VAR_AUTO,
                  stream=None):
    return _ext.tm_map_affine(_ptr(x), ldx, _ptr(y), ldy, M, N, alpha, beta, TM, TN, aligned,
                              variant, _stream(stream))


def tm_scale2d(x, ldx, y, ldy, M, N, alpha, TM, TN, aligned, variant=TM_VAR_AUTO, stream=None):
    return _ext.tm_scale2d(_ptr(x), ldx, _ptr(y), ldy, M, N, alpha, TM, TN, aligned, variant,
                           _stream(stream))


def tm_copy2d(x, ldx, y, ldy, M, N, TM, TN, aligned, variant=TM_VAR_AUTO, stream=None):
    return _ext.tm_copy2d(_ptr(x), ldx, _ptr(y), ldy, M, N, TM, TN, aligned, variant,
                          _stream(stream))


def tm_channel_affine(x, ldx, scale, bias, y, ldy, M, N, TM, TN, aligned, variant=TM_VAR_AUTO,
                      stream=None):
    return _ext.tm_channel_affine(_ptr(x), ldx, _ptr(scale), _ptr(bias), _ptr(y), ldy, M, N, TM, TN,
                                  aligned, variant, _stream(stream))


def tm_rowsum(x, ldx, out, M, N, TM, TN, aligned, stream=None):
    return _ext.tm_rowsum(_ptr(x), ldx, _ptr(out), M, N, TM, TN, aligned, _stream(stream))


def tm_colsum_workspace_bytes(M, N, TM, TN, walk):
    return _ext.tm_colsum_workspace_bytes(M, N, TM, TN, walk)


def tm_colsum(x, ldx, out, M, N, TM, TN, aligned, walk, ws, ws_bytes, stream=None):
    return _ext.tm_colsum(_ptr(x), ldx, _ptr(out), M, N, TM, TN, aligned, walk, _ptr(ws), ws_bytes,
                          _stream(stream))


TM_COLSUM_NOALLOC_MAX_BYTES = 16 << 20


def tm_colsum_noalloc(x, ldx, out, M, N, TM, TN, aligned, walk, stream=None):
    """tm_colsum with its partials in the library's static device array (no workspace, no
    allocation); calls overlapping on one device race."""
    return _ext.tm_colsum_noalloc(_ptr(x), ldx, _ptr(out), M, N, TM, TN, aligned, walk, _stream(stream))


def tm_rowmax_masked(s, lds, out, M, N, BR, BC, aligned, stream=None):
    return _ext.tm_rowmax_masked(_ptr(s), lds, _ptr(out), M, N, BR, BC, aligned, _stream(stream))


def tm_softmax_stats(s, lds, m, l, M, N, BR, BC, aligned, stream=None):
    return _ext.tm_softmax_stats(_ptr(s), lds, _ptr(m), _ptr(l), M, N, BR, BC, aligned,
                                 _stream(stream))


def tm_rows_workspace_bytes(M, N):
    return _ext.tm_rows_workspace_bytes(M, N)


def tm_rowsum_ws(x, ldx, out, M, N, TM, TN, aligned, ws, ws_bytes, stream=None):
    return _ext.tm_rowsum_ws(_ptr(x), ldx, _ptr(out), M, N, TM, TN, aligned, _ptr(ws), ws_bytes,
                             _stream(stream))


def tm_rowmax_masked_ws(s, lds, out, M, N, BR, BC, aligned, ws, ws_bytes, stream=None):
    return _ext.tm_rowmax_masked_ws(_ptr(s), lds, _ptr(out), M, N, BR, BC, aligned, _ptr(ws),
                                    ws_bytes, _stream(stream))


def tm_softmax_stats_ws(s, lds, m, l, M, N, BR, BC, aligned, ws, ws_bytes, stream=None):
    return _ext.tm_softmax_stats_ws(_ptr(s), lds, _ptr(m), _ptr(l), M, N, BR, BC, aligned,
                                    _ptr(ws), ws_bytes, _stream(stream))


def tm_transpose(x, ldx, bsx, y, ldy, bsy, B, M, N, TM, TN, aligned, stream=None):
    return _ext.tm_transpose(_ptr(x), ldx, bsx, _ptr(y), ldy, bsy, B, M, N, TM, TN, aligned,
                             _stream(stream))


def tm_check_promise(M, N, ld_in, ld_out, TM, TN, inp, out):
    return _ext.tm_check_promise(M, N, ld_in, ld_out, TM, TN, _ptr(inp), _ptr(out))


def tm_split(K, T):
    """Returns (status, nfull, rem)."""
    return _ext.tm_split(K, T)


def tm_plan_tiles(M, N, TM, TN):
    """Returns (status, tiles_m, tiles_n, whole)."""
    return _ext.tm_plan_tiles(M, N, TM, TN)


def tm_row_walk(M, N, ld, BR, BC, aligned, x):
    """Returns (status, bc, nfull, rem, lanes): the column walk of the one-pass row reductions.
    x is a tensor or an address (inspected, never dereferenced)."""
    return _ext.tm_row_walk(M, N, ld, BR, BC, aligned, _ptr(x))


def tm_map_walk(op, x, ldx, y, ldy, M, N, TM, TN, aligned, variant=TM_VAR_AUTO, bias=None):
    """Returns (status, walk, items): the plan an element-wise map would run (op 0 affine, 1 scale,
    2 copy, 3 channel with the vector bias).  x, y, bias: tensors or addresses (inspected, never
    dereferenced)."""
    return _ext.tm_map_walk(op, _ptr(x), ldx, _ptr(y), ldy, M, N, TM, TN, aligned, variant, _ptr(bias))


def tm_col_walk(x, ldx, out, M, N, TM, TN, aligned, walk, ws=None, ws_bytes=0):
    """Returns (status, form, slab_rows, strip_cols, slabs, strips): the plan tm_colsum would run
    (form: TM_COLFORM_*).  x, out, ws: tensors or addresses (inspected, never dereferenced)."""
    return _ext.tm_col_walk(_ptr(x), ldx, _ptr(out), M, N, TM, TN, aligned, walk, _ptr(ws), ws_bytes)


def tm_pad_extents(M, N, TM, TN):
    """Returns (status, Mp, Np, ldp)."""
    return _ext.tm_pad_extents(M, N, TM, TN)


TUNE_ROWS, TUNE_COLS = _ext.TUNE_ROWS, _ext.TUNE_COLS


def tm_autotune_map(op, x, ldx, y, ldy, M, N, alpha, beta, aligned, variant, reps, ev_start, ev_stop,
                    stream=None, table=True):
    """Returns (status, TM_best, TN_best, us_best, table) with table a 9 x 11 list of lists
    (TM = 2^i rows, TN = 2^j columns; -1 where not run), or None with table=False (the C call
    then gets a NULL table).  ev_start / ev_stop: torch.cuda.Event objects created with
    enable_timing=True, or raw hipEvent_t integers."""
    def ev(e):
        if e is None or isinstance(e, int):
            return e
        if e.cuda_event == 0:  # torch creates the event on its first record
            e.record(torch.cuda.current_stream() if stream is None else stream)
        return e.cuda_event
    st, tmb, tnb, usb, flat = _ext.tm_autotune_map(op, _ptr(x), ldx, _ptr(y), ldy, M, N, alpha, beta,
                                                   aligned, variant, reps, ev(ev_start), ev(ev_stop),
                                                   1 if table else 0, _stream(stream))
    rows = None
    if flat is not None:
        rows = [list(flat[i * TUNE_COLS:(i + 1) * TUNE_COLS]) for i in range(TUNE_ROWS)]
    return st, tmb, tnb, usb, rows


def tm_status_string(status):
    return _ext.tm_status_string(status)


def library_path():
    return LIB_PATH
