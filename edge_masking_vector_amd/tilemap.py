"""ctypes binding to libtilemap.so -- the same calls as include/tilemap.h, argument marshalling only.

Each function takes what the C call takes.  Pointer arguments accept a torch tensor (its
data_ptr() is passed; the tensor must live on the GPU the library runs on) or a plain integer
address; `stream` accepts a torch stream, an integer hipStream_t, or None for torch's current
stream.  The return value is the C status code (TM_OK == 0); `check()` turns a nonzero status into
a TilemapError.  Nothing here computes any part of the maps or reductions: every step runs in the
HIP kernels, and importing this module fails loudly if libtilemap.so has not been built.

torch is imported before the library is loaded so that both share one HIP runtime (the wheel's
libamdhip64 is then the one libtilemap.so binds to).
"""
import ctypes
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

if not os.path.exists(LIB_PATH):
    raise ImportError("libtilemap.so is not built (expected at %s); run "
                      "`python -c 'import __graft_entry__ as g; g.build()'` first" % LIB_PATH)

_lib = ctypes.CDLL(LIB_PATH)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_f32 = ctypes.c_float
_i64p = ctypes.POINTER(ctypes.c_int64)

_SIGS = {
    "tm_map_affine": (_int, [_vp, _i64, _vp, _i64, _i64, _i64, _f32, _f32, _int, _int, _int, _int, _vp]),
    "tm_scale2d": (_int, [_vp, _i64, _vp, _i64, _i64, _i64, _f32, _int, _int, _int, _int, _vp]),
    "tm_copy2d": (_int, [_vp, _i64, _vp, _i64, _i64, _i64, _int, _int, _int, _int, _vp]),
    "tm_channel_affine": (_int, [_vp, _i64, _vp, _vp, _vp, _i64, _i64, _i64, _int, _int, _int, _int, _vp]),
    "tm_rowsum": (_int, [_vp, _i64, _vp, _i64, _i64, _int, _int, _int, _vp]),
    "tm_colsum_workspace_bytes": (ctypes.c_size_t, [_i64, _i64, _int, _int, _int]),
    "tm_colsum": (_int, [_vp, _i64, _vp, _i64, _i64, _int, _int, _int, _int, _vp, ctypes.c_size_t, _vp]),
    "tm_rowmax_masked": (_int, [_vp, _i64, _vp, _i64, _i64, _int, _int, _int, _vp]),
    "tm_softmax_stats": (_int, [_vp, _i64, _vp, _vp, _i64, _i64, _int, _int, _int, _vp]),
    "tm_transpose": (_int, [_vp, _i64, _i64, _vp, _i64, _i64, _i64, _i64, _i64, _int, _int, _int, _vp]),
    "tm_check_promise": (_int, [_i64, _i64, _i64, _i64, _int, _int, _vp, _vp]),
    "tm_split": (_int, [_i64, _i64, _i64p, _i64p]),
    "tm_plan_tiles": (_int, [_i64, _i64, _int, _int, _i64p, _i64p, _i64p]),
    "tm_pad_extents": (_int, [_i64, _i64, _int, _int, _i64p, _i64p, _i64p]),
    "tm_autotune_map": (_int, [_int, _vp, _i64, _vp, _i64, _i64, _i64, _f32, _f32, _int, _int, _int,
                               _vp, _vp, ctypes.POINTER(_int), ctypes.POINTER(_int),
                               ctypes.POINTER(_f32), ctypes.POINTER(_f32), _vp]),
    "tm_status_string": (ctypes.c_char_p, [_int]),
}
for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


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
    if p is None:
        return None
    if isinstance(p, int):
        return p
    if isinstance(p, torch.Tensor):
        return p.data_ptr()
    raise TypeError("expected a torch tensor, an integer address or None, got %r" % type(p))


def _stream(s):
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def tm_map_affine(x, ldx, y, ldy, M, N, alpha, beta, TM, TN, aligned, variant=TM_VAR_AUTO,
                  stream=None):
    return _lib.tm_map_affine(_ptr(x), ldx, _ptr(y), ldy, M, N, alpha, beta, TM, TN, aligned,
                              variant, _stream(stream))


def tm_scale2d(x, ldx, y, ldy, M, N, alpha, TM, TN, aligned, variant=TM_VAR_AUTO, stream=None):
    return _lib.tm_scale2d(_ptr(x), ldx, _ptr(y), ldy, M, N, alpha, TM, TN, aligned, variant,
                           _stream(stream))


def tm_copy2d(x, ldx, y, ldy, M, N, TM, TN, aligned, variant=TM_VAR_AUTO, stream=None):
    return _lib.tm_copy2d(_ptr(x), ldx, _ptr(y), ldy, M, N, TM, TN, aligned, variant,
                          _stream(stream))


def tm_channel_affine(x, ldx, scale, bias, y, ldy, M, N, TM, TN, aligned, variant=TM_VAR_AUTO,
                      stream=None):
    return _lib.tm_channel_affine(_ptr(x), ldx, _ptr(scale), _ptr(bias), _ptr(y), ldy, M, N, TM, TN,
                                  aligned, variant, _stream(stream))


def tm_rowsum(x, ldx, out, M, N, TM, TN, aligned, stream=None):
    return _lib.tm_rowsum(_ptr(x), ldx, _ptr(out), M, N, TM, TN, aligned, _stream(stream))


def tm_colsum_workspace_bytes(M, N, TM, TN, walk):
    return _lib.tm_colsum_workspace_bytes(M, N, TM, TN, walk)


def tm_colsum(x, ldx, out, M, N, TM, TN, aligned, walk, ws, ws_bytes, stream=None):
    return _lib.tm_colsum(_ptr(x), ldx, _ptr(out), M, N, TM, TN, aligned, walk, _ptr(ws), ws_bytes,
                          _stream(stream))


def tm_rowmax_masked(s, lds, out, M, N, BR, BC, aligned, stream=None):
    return _lib.tm_rowmax_masked(_ptr(s), lds, _ptr(out), M, N, BR, BC, aligned, _stream(stream))


def tm_softmax_stats(s, lds, m, l, M, N, BR, BC, aligned, stream=None):
    return _lib.tm_softmax_stats(_ptr(s), lds, _ptr(m), _ptr(l), M, N, BR, BC, aligned,
                                 _stream(stream))


def tm_transpose(x, ldx, bsx, y, ldy, bsy, B, M, N, TM, TN, aligned, stream=None):
    return _lib.tm_transpose(_ptr(x), ldx, bsx, _ptr(y), ldy, bsy, B, M, N, TM, TN, aligned,
                             _stream(stream))


def tm_check_promise(M, N, ld_in, ld_out, TM, TN, inp, out):
    return _lib.tm_check_promise(M, N, ld_in, ld_out, TM, TN, _ptr(inp), _ptr(out))


def tm_split(K, T):
    """Returns (status, nfull, rem)."""
    nf, rm = ctypes.c_int64(-1), ctypes.c_int64(-1)
    st = _lib.tm_split(K, T, ctypes.byref(nf), ctypes.byref(rm))
    return st, nf.value, rm.value


def tm_plan_tiles(M, N, TM, TN):
    """Returns (status, tiles_m, tiles_n, whole)."""
    a, b, c = ctypes.c_int64(-1), ctypes.c_int64(-1), ctypes.c_int64(-1)
    st = _lib.tm_plan_tiles(M, N, TM, TN, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return st, a.value, b.value, c.value


def tm_pad_extents(M, N, TM, TN):
    """Returns (status, Mp, Np, ldp)."""
    a, b, c = ctypes.c_int64(-1), ctypes.c_int64(-1), ctypes.c_int64(-1)
    st = _lib.tm_pad_extents(M, N, TM, TN, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c))
    return st, a.value, b.value, c.value


TUNE_ROWS, TUNE_COLS = 9, 11


def tm_autotune_map(op, x, ldx, y, ldy, M, N, alpha, beta, aligned, variant, reps, ev_start, ev_stop,
                    stream=None):
    """Returns (status, TM_best, TN_best, us_best, table) with table a 9 x 11 list of lists
    (TM = 2^i rows, TN = 2^j columns; -1 where not run).  ev_start / ev_stop: torch.cuda.Event
    objects created with enable_timing=True (or raw hipEvent_t integers)."""
    tmb, tnb, usb = _int(0), _int(0), _f32(0.0)
    table = (_f32 * (TUNE_ROWS * TUNE_COLS))()
    def ev(e):
        if isinstance(e, int):
            return e
        if e.cuda_event == 0:  # torch creates the event on its first record
            e.record(torch.cuda.current_stream() if stream is None else stream)
        return e.cuda_event
    st = _lib.tm_autotune_map(op, _ptr(x), ldx, _ptr(y), ldy, M, N, alpha, beta, aligned, variant,
                              reps, ev(ev_start), ev(ev_stop), ctypes.byref(tmb), ctypes.byref(tnb),
                              ctypes.byref(usb), table, _stream(stream))
    rows = [[table[i * TUNE_COLS + j] for j in range(TUNE_COLS)] for i in range(TUNE_ROWS)]
    return st, tmb.value, tnb.value, usb.value, rows


def tm_status_string(status):
    return _lib.tm_status_string(status).decode()


def library_path():
    return LIB_PATH
