"""CPU oracle for the tiled f32 map / reduction path -- TEST INFRASTRUCTURE ONLY.

Only the test suite, the package's smoke check and the benchmark's CPU-baseline leg import this
module.  The product library (edge_masking_vector_amd) never imports it and shares no code with
it.  This file is argument marshalling only: every number comes from oracle.c (plain C99, see
oracle.h for the definitions and the pages each one follows).

Arrays are numpy; 2-D tensors are described exactly as in the C functions, by a flat buffer plus
(M, N, ld).  Outputs are written in place, so a caller can pre-fill sentinels and check that
nothing outside the M x N window changes.
"""
import ctypes
import os

import numpy as np

from . import _build

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i64 = ctypes.c_int64
_i64p = ctypes.POINTER(ctypes.c_int64)

_lib = None

MAX_FILL = np.float32(-1.0e30)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_build.LIB):
        _build.build()
    lib = ctypes.CDLL(_build.LIB)
    sig = {
        "orc_split": (None, [_i64, _i64, _i64p, _i64p]),
        "orc_tile_live": (_i64, [_i64, _i64, _i64, _i64, _i64, _i64]),
        "orc_promise_holds": (ctypes.c_int, [_i64, _i64, _i64, _i64, _i64, _i64,
                                             ctypes.c_uint64, ctypes.c_uint64]),
        "orc_map_affine": (None, [_f32p, _i64, _f32p, _i64, _i64, _i64, ctypes.c_float,
                                  ctypes.c_float]),
        "orc_scale2d": (None, [_f32p, _i64, _f32p, _i64, _i64, _i64, ctypes.c_float]),
        "orc_copy2d": (None, [_f32p, _i64, _f32p, _i64, _i64, _i64]),
        "orc_rowsum_f64": (None, [_f32p, _i64, _i64, _i64, _f64p]),
        "orc_colsum_f64": (None, [_f32p, _i64, _i64, _i64, _f64p]),
        "orc_rowmax": (None, [_f32p, _i64, _i64, _i64, _f32p]),
        "orc_map_affine_tiled": (None, [_f32p, _i64, _f32p, _i64, _i64, _i64, ctypes.c_float,
                                        ctypes.c_float, _i64, _i64]),
        "orc_rowsum_tiled_f64": (None, [_f32p, _i64, _i64, _i64, _i64, _f64p]),
        "orc_rowmax_tiled": (None, [_f32p, _i64, _i64, _i64, _i64, ctypes.c_float, _f32p]),
        "orc_softmax_stats": (None, [_f32p, _i64, _i64, _i64, _f32p, _f64p]),
        "orc_transpose": (None, [_f32p, _i64, _i64, _f32p, _i64, _i64, _i64, _i64, _i64]),
        "orc_channel_affine": (None, [_f32p, _i64, _f32p, _f32p, _f32p, _i64, _i64, _i64]),
        "orc_softmax_stats_tiled": (None, [_f32p, _i64, _i64, _i64, _i64, ctypes.c_float, _f32p, _f64p]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _need(a, dtype, M, N, ld, what):
    """Check that flat array `a` holds an M x N view with row stride ld."""
    if not isinstance(a, np.ndarray) or a.dtype != dtype or not a.flags.c_contiguous:
        raise TypeError("%s must be a C-contiguous numpy %s array" % (what, np.dtype(dtype).name))
    if M > 0 and N > 0:
        if ld < N:
            raise ValueError("%s: ld=%d < N=%d" % (what, ld, N))
        if a.size < (M - 1) * ld + N:
            raise ValueError("%s: buffer of %d elements is too small" % (what, a.size))


def _p(a, t):
    return a.ctypes.data_as(t)


def split(K, T):
    """(whole tiles, remainder width) of a loop over K in steps of T."""
    nf, rm = ctypes.c_int64(), ctypes.c_int64()
    _load().orc_split(K, T, ctypes.byref(nf), ctypes.byref(rm))
    return nf.value, rm.value


def tile_live(M, N, TM, TN, pm, pn):
    return _load().orc_tile_live(M, N, TM, TN, pm, pn)


def promise_holds(M, N, ld_in, ld_out, TM, TN, in_addr, out_addr):
    return bool(_load().orc_promise_holds(M, N, ld_in, ld_out, TM, TN, in_addr, out_addr))


def map_affine(x, ldx, y, ldy, M, N, alpha, beta):
    _need(x, np.float32, M, N, ldx, "x"); _need(y, np.float32, M, N, ldy, "y")
    _load().orc_map_affine(_p(x, _f32p), ldx, _p(y, _f32p), ldy, M, N, alpha, beta)


def scale2d(x, ldx, y, ldy, M, N, alpha):
    _need(x, np.float32, M, N, ldx, "x"); _need(y, np.float32, M, N, ldy, "y")
    _load().orc_scale2d(_p(x, _f32p), ldx, _p(y, _f32p), ldy, M, N, alpha)


def copy2d(x, ldx, y, ldy, M, N):
    _need(x, np.float32, M, N, ldx, "x"); _need(y, np.float32, M, N, ldy, "y")
    _load().orc_copy2d(_p(x, _f32p), ldx, _p(y, _f32p), ldy, M, N)


def rowsum_f64(x, ldx, M, N):
    _need(x, np.float32, M, N, ldx, "x")
    out = np.zeros(max(M, 0), np.float64)
    _load().orc_rowsum_f64(_p(x, _f32p), ldx, M, N, _p(out, _f64p))
    return out


def colsum_f64(x, ldx, M, N):
    _need(x, np.float32, M, N, ldx, "x")
    out = np.zeros(max(N, 0), np.float64)
    _load().orc_colsum_f64(_p(x, _f32p), ldx, M, N, _p(out, _f64p))
    return out


def rowmax(s, lds, M, N):
    _need(s, np.float32, M, N, lds, "s")
    out = np.zeros(max(M, 0), np.float32)
    _load().orc_rowmax(_p(s, _f32p), lds, M, N, _p(out, _f32p))
    return out


def map_affine_tiled(x, ldx, y, ldy, M, N, alpha, beta, TM, TN):
    _need(x, np.float32, M, N, ldx, "x"); _need(y, np.float32, M, N, ldy, "y")
    _load().orc_map_affine_tiled(_p(x, _f32p), ldx, _p(y, _f32p), ldy, M, N, alpha, beta, TM, TN)


def rowsum_tiled_f64(x, ldx, M, N, TN):
    _need(x, np.float32, M, N, ldx, "x")
    out = np.zeros(max(M, 0), np.float64)
    _load().orc_rowsum_tiled_f64(_p(x, _f32p), ldx, M, N, TN, _p(out, _f64p))
    return out


def rowmax_tiled(s, lds, M, N, BC, fill=MAX_FILL):
    _need(s, np.float32, M, N, lds, "s")
    out = np.zeros(max(M, 0), np.float32)
    _load().orc_rowmax_tiled(_p(s, _f32p), lds, M, N, BC, fill, _p(out, _f32p))
    return out


def softmax_stats(s, lds, M, N):
    """(m, l): row maxima (f32, from the -1e30 fill) and sum_j exp(s - m) in double."""
    _need(s, np.float32, M, N, lds, "s")
    m = np.zeros(max(M, 0), np.float32)
    l = np.zeros(max(M, 0), np.float64)
    _load().orc_softmax_stats(_p(s, _f32p), lds, M, N, _p(m, _f32p), _p(l, _f64p))
    return m, l


def softmax_stats_tiled(s, lds, M, N, BC, fill=MAX_FILL):
    _need(s, np.float32, M, N, lds, "s")
    m = np.zeros(max(M, 0), np.float32)
    l = np.zeros(max(M, 0), np.float64)
    _load().orc_softmax_stats_tiled(_p(s, _f32p), lds, M, N, BC, fill, _p(m, _f32p), _p(l, _f64p))
    return m, l


def transpose(x, ldx, bsx, y, ldy, bsy, B, M, N):
    """y[b][j][i] = x[b][i][j] (bit for bit), written in place into y."""
    for a, what in ((x, "x"), (y, "y")):
        if not isinstance(a, np.ndarray) or a.dtype != np.float32 or not a.flags.c_contiguous:
            raise TypeError("%s must be a C-contiguous numpy float32 array" % what)
    if B > 0 and M > 0 and N > 0:
        if x.size < (B - 1) * bsx + (M - 1) * ldx + N or y.size < (B - 1) * bsy + (N - 1) * ldy + M:
            raise ValueError("buffer too small")
    _load().orc_transpose(_p(x, _f32p), ldx, bsx, _p(y, _f32p), ldy, bsy, B, M, N)


def channel_affine(x, ldx, scale, bias, y, ldy, M, N):
    """y[i,j] = fmaf(x[i,j], scale[j], bias[j]) (or x + bias[j] when scale is None), in place."""
    _need(x, np.float32, M, N, ldx, "x"); _need(y, np.float32, M, N, ldy, "y")
    _need(bias, np.float32, 1, N, N, "bias")
    if scale is not None:
        _need(scale, np.float32, 1, N, N, "scale")
    _load().orc_channel_affine(_p(x, _f32p), ldx, None if scale is None else _p(scale, _f32p),
                               _p(bias, _f32p), _p(y, _f32p), ldy, M, N)
