/* pyext.c -- the CPython extension `_tilemap`: every call of include/tilemap.h under the same name,
 * taking device addresses as Python ints (None for NULL), sizes as ints, scalars as floats and the
 * stream as an int (a hipStream_t; 0 is the null stream).  Argument conversion only: each function
 * converts its arguments and calls the C ABI once.  Calls that write through host pointers
 * (tm_split, tm_plan_tiles, tm_map_walk, tm_row_walk, tm_col_walk, tm_pad_extents, tm_autotune_map)
 * return a tuple that starts with the status instead.  A wrong argument count or type raises
 * TypeError / OverflowError before any call.
 *
 * METH_FASTCALL keeps a call near half a microsecond; through ctypes the same call took several,
 * more than a 1M-element map takes on the GPU. */
#define PY_SSIZE_T_CLEAN
#include <Python.h>

#include <limits.h>
#include <stdint.h>

#include "tilemap.h"

static int want(Py_ssize_t nargs, Py_ssize_t n, const char *name) {
    if (nargs == n)
        return 1;
    PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (%zd given)", name, n, nargs);
    return 0;
}

static int as_i64(PyObject *o, int64_t *v) {
    const long long x = PyLong_AsLongLong(o);
    if (x == -1 && PyErr_Occurred())
        return 0;
    *v = (int64_t)x;
    return 1;
}

static int as_int(PyObject *o, int *v) {
    const long x = PyLong_AsLong(o);
    if (x == -1 && PyErr_Occurred())
        return 0;
    if (x < INT_MIN || x > INT_MAX) {
        PyErr_SetString(PyExc_OverflowError, "value does not fit a C int");
        return 0;
    }
    *v = (int)x;
    return 1;
}

/* A Python float (or int) rounded to the nearest f32, as a C float argument receives it. */
static int as_f32(PyObject *o, float *v) {
    const double d = PyFloat_AsDouble(o);
    if (d == -1.0 && PyErr_Occurred())
        return 0;
    *v = (float)d;
    return 1;
}

static int as_ptr(PyObject *o, void **p) {
    if (o == Py_None) {
        *p = NULL;
        return 1;
    }
    const unsigned long long x = PyLong_AsUnsignedLongLong(o);
    if (x == (unsigned long long)-1 && PyErr_Occurred())
        return 0;
    *p = (void *)(uintptr_t)x;
    return 1;
}

static int as_size(PyObject *o, size_t *v) {
    const size_t x = PyLong_AsSize_t(o);
    if (x == (size_t)-1 && PyErr_Occurred())
        return 0;
    *v = x;
    return 1;
}

#define ARGS PyObject *self, PyObject *const *a, Py_ssize_t n
#define OK(expr) \
    if (!(expr)) \
    return NULL

static PyObject *py_map_affine(ARGS) {
    void *x, *y, *s;
    int64_t ldx, ldy, M, N;
    float alpha, beta;
    int TM, TN, al, var;
    (void)self;
    OK(want(n, 13, "tm_map_affine"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ldx) && as_ptr(a[2], &y) && as_i64(a[3], &ldy) &&
       as_i64(a[4], &M) && as_i64(a[5], &N) && as_f32(a[6], &alpha) && as_f32(a[7], &beta) &&
       as_int(a[8], &TM) && as_int(a[9], &TN) && as_int(a[10], &al) && as_int(a[11], &var) &&
       as_ptr(a[12], &s));
    return PyLong_FromLong(tm_map_affine((const float *)x, ldx, (float *)y, ldy, M, N, alpha, beta,
                                         TM, TN, al, var, s));
}

static PyObject *py_scale2d(ARGS) {
    void *x, *y, *s;
    int64_t ldx, ldy, M, N;
    float alpha;
    int TM, TN, al, var;
    (void)self;
    OK(want(n, 12, "tm_scale2d"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ldx) && as_ptr(a[2], &y) && as_i64(a[3], &ldy) &&
       as_i64(a[4], &M) && as_i64(a[5], &N) && as_f32(a[6], &alpha) && as_int(a[7], &TM) &&
       as_int(a[8], &TN) && as_int(a[9], &al) && as_int(a[10], &var) && as_ptr(a[11], &s));
    return PyLong_FromLong(
        tm_scale2d((const float *)x, ldx, (float *)y, ldy, M, N, alpha, TM, TN, al, var, s));
}

static PyObject *py_copy2d(ARGS) {
    void *x, *y, *s;
    int64_t ldx, ldy, M, N;
    int TM, TN, al, var;
    (void)self;
    OK(want(n, 11, "tm_copy2d"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ldx) && as_ptr(a[2], &y) && as_i64(a[3], &ldy) &&
       as_i64(a[4], &M) && as_i64(a[5], &N) && as_int(a[6], &TM) && as_int(a[7], &TN) &&
       as_int(a[8], &al) && as_int(a[9], &var) && as_ptr(a[10], &s));
    return PyLong_FromLong(
        tm_copy2d((const float *)x, ldx, (float *)y, ldy, M, N, TM, TN, al, var, s));
}

static PyObject *py_channel_affine(ARGS) {
    void *x, *scale, *bias, *y, *s;
    int64_t ldx, ldy, M, N;
    int TM, TN, al, var;
    (void)self;
    OK(want(n, 13, "tm_channel_affine"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ldx) && as_ptr(a[2], &scale) && as_ptr(a[3], &bias) &&
       as_ptr(a[4], &y) && as_i64(a[5], &ldy) && as_i64(a[6], &M) && as_i64(a[7], &N) &&
       as_int(a[8], &TM) && as_int(a[9], &TN) && as_int(a[10], &al) && as_int(a[11], &var) &&
       as_ptr(a[12], &s));
    return PyLong_FromLong(tm_channel_affine((const float *)x, ldx, (const float *)scale,
                                             (const float *)bias, (float *)y, ldy, M, N, TM, TN,
                                             al, var, s));
}

static PyObject *py_rowsum(ARGS) {
    void *x, *out, *s;
    int64_t ldx, M, N;
    int TM, TN, al;
    (void)self;
    OK(want(n, 9, "tm_rowsum"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ldx) && as_ptr(a[2], &out) && as_i64(a[3], &M) &&
       as_i64(a[4], &N) && as_int(a[5], &TM) && as_int(a[6], &TN) && as_int(a[7], &al) &&
       as_ptr(a[8], &s));
    return PyLong_FromLong(tm_rowsum((const float *)x, ldx, (float *)out, M, N, TM, TN, al, s));
}

static PyObject *py_rows_workspace_bytes(ARGS) {
    int64_t M, N;
    (void)self;
    OK(want(n, 2, "tm_rows_workspace_bytes"));
    OK(as_i64(a[0], &M) && as_i64(a[1], &N));
    return PyLong_FromSize_t(tm_rows_workspace_bytes(M, N));
}

static PyObject *py_rowsum_ws(ARGS) {
    void *x, *out, *ws, *s;
    int64_t ldx, M, N;
    int TM, TN, al;
    size_t wsb;
    (void)self;
    OK(want(n, 11, "tm_rowsum_ws"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ldx) && as_ptr(a[2], &out) && as_i64(a[3], &M) &&
       as_i64(a[4], &N) && as_int(a[5], &TM) && as_int(a[6], &TN) && as_int(a[7], &al) &&
       as_ptr(a[8], &ws) && as_size(a[9], &wsb) && as_ptr(a[10], &s));
    return PyLong_FromLong(
        tm_rowsum_ws((const float *)x, ldx, (float *)out, M, N, TM, TN, al, ws, wsb, s));
}

static PyObject *py_rowmax_masked_ws(ARGS) {
    void *x, *out, *ws, *s;
    int64_t ld, M, N;
    int BR, BC, al;
    size_t wsb;
    (void)self;
    OK(want(n, 11, "tm_rowmax_masked_ws"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ld) && as_ptr(a[2], &out) && as_i64(a[3], &M) &&
       as_i64(a[4], &N) && as_int(a[5], &BR) && as_int(a[6], &BC) && as_int(a[7], &al) &&
       as_ptr(a[8], &ws) && as_size(a[9], &wsb) && as_ptr(a[10], &s));
    return PyLong_FromLong(
        tm_rowmax_masked_ws((const float *)x, ld, (float *)out, M, N, BR, BC, al, ws, wsb, s));
}

static PyObject *py_softmax_stats_ws(ARGS) {
    void *x, *m, *l, *ws, *s;
    int64_t ld, M, N;
    int BR, BC, al;
    size_t wsb;
    (void)self;
    OK(want(n, 12, "tm_softmax_stats_ws"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ld) && as_ptr(a[2], &m) && as_ptr(a[3], &l) &&
       as_i64(a[4], &M) && as_i64(a[5], &N) && as_int(a[6], &BR) && as_int(a[7], &BC) &&
       as_int(a[8], &al) && as_ptr(a[9], &ws) && as_size(a[10], &wsb) && as_ptr(a[11], &s));
    return PyLong_FromLong(tm_softmax_stats_ws((const float *)x, ld, (float *)m, (float *)l, M, N,
                                               BR, BC, al, ws, wsb, s));
}

static PyObject *py_colsum_noalloc(ARGS) {
    void *x, *out, *s;
    int64_t ldx, M, N;
    int TM, TN, al, walk;
    (void)self;
    OK(want(n, 10, "tm_colsum_noalloc"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ldx) && as_ptr(a[2], &out) && as_i64(a[3], &M) &&
       as_i64(a[4], &N) && as_int(a[5], &TM) && as_int(a[6], &TN) && as_int(a[7], &al) &&
       as_int(a[8], &walk) && as_ptr(a[9], &s));
    return PyLong_FromLong(tm_colsum_noalloc((const float *)x, ldx, (float *)out, M, N, TM, TN, al, walk, s));
}

static PyObject *py_colsum_workspace_bytes(ARGS) {
    int64_t M, N;
    int TM, TN, walk;
    (void)self;
    OK(want(n, 5, "tm_colsum_workspace_bytes"));
    OK(as_i64(a[0], &M) && as_i64(a[1], &N) && as_int(a[2], &TM) && as_int(a[3], &TN) &&
       as_int(a[4], &walk));
    return PyLong_FromSize_t(tm_colsum_workspace_bytes(M, N, TM, TN, walk));
}

static PyObject *py_colsum(ARGS) {
    void *x, *out, *ws, *s;
    int64_t ldx, M, N;
    int TM, TN, al, walk;
    size_t wsb;
    (void)self;
    OK(want(n, 12, "tm_colsum"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ldx) && as_ptr(a[2], &out) && as_i64(a[3], &M) &&
       as_i64(a[4], &N) && as_int(a[5], &TM) && as_int(a[6], &TN) && as_int(a[7], &al) &&
       as_int(a[8], &walk) && as_ptr(a[9], &ws) && as_size(a[10], &wsb) && as_ptr(a[11], &s));
    return PyLong_FromLong(
        tm_colsum((const float *)x, ldx, (float *)out, M, N, TM, TN, al, walk, ws, wsb, s));
}

static PyObject *py_rowmax_masked(ARGS) {
    void *x, *out, *s;
    int64_t ld, M, N;
    int BR, BC, al;
    (void)self;
    OK(want(n, 9, "tm_rowmax_masked"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ld) && as_ptr(a[2], &out) && as_i64(a[3], &M) &&
       as_i64(a[4], &N) && as_int(a[5], &BR) && as_int(a[6], &BC) && as_int(a[7], &al) &&
       as_ptr(a[8], &s));
    return PyLong_FromLong(
        tm_rowmax_masked((const float *)x, ld, (float *)out, M, N, BR, BC, al, s));
}

static PyObject *py_softmax_stats(ARGS) {
    void *x, *m, *l, *s;
    int64_t ld, M, N;
    int BR, BC, al;
    (void)self;
    OK(want(n, 10, "tm_softmax_stats"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ld) && as_ptr(a[2], &m) && as_ptr(a[3], &l) &&
       as_i64(a[4], &M) && as_i64(a[5], &N) && as_int(a[6], &BR) && as_int(a[7], &BC) &&
       as_int(a[8], &al) && as_ptr(a[9], &s));
    return PyLong_FromLong(
        tm_softmax_stats((const float *)x, ld, (float *)m, (float *)l, M, N, BR, BC, al, s));
}

static PyObject *py_transpose(ARGS) {
    void *x, *y, *s;
    int64_t ldx, bsx, ldy, bsy, B, M, N;
    int TM, TN, al;
    (void)self;
    OK(want(n, 13, "tm_transpose"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ldx) && as_i64(a[2], &bsx) && as_ptr(a[3], &y) &&
       as_i64(a[4], &ldy) && as_i64(a[5], &bsy) && as_i64(a[6], &B) && as_i64(a[7], &M) &&
       as_i64(a[8], &N) && as_int(a[9], &TM) && as_int(a[10], &TN) && as_int(a[11], &al) &&
       as_ptr(a[12], &s));
    return PyLong_FromLong(tm_transpose((const float *)x, ldx, bsx, (float *)y, ldy, bsy, B, M, N,
                                        TM, TN, al, s));
}

static PyObject *py_check_promise(ARGS) {
    void *in, *out;
    int64_t M, N, ldi, ldo;
    int TM, TN;
    (void)self;
    OK(want(n, 8, "tm_check_promise"));
    OK(as_i64(a[0], &M) && as_i64(a[1], &N) && as_i64(a[2], &ldi) && as_i64(a[3], &ldo) &&
       as_int(a[4], &TM) && as_int(a[5], &TN) && as_ptr(a[6], &in) && as_ptr(a[7], &out));
    return PyLong_FromLong(tm_check_promise(M, N, ldi, ldo, TM, TN, in, out));
}

static PyObject *py_split(ARGS) {
    int64_t K, T, nfull = -1, rem = -1;
    (void)self;
    OK(want(n, 2, "tm_split"));
    OK(as_i64(a[0], &K) && as_i64(a[1], &T));
    const int st = tm_split(K, T, &nfull, &rem);
    return Py_BuildValue("(iLL)", st, (long long)nfull, (long long)rem);
}

static PyObject *py_row_walk(ARGS) {
    int64_t M, N, ld, bc = -1, nfull = -1, rem = -1;
    int BR, BC, al, lanes = -1;
    void *x;
    (void)self;
    OK(want(n, 7, "tm_row_walk"));
    OK(as_i64(a[0], &M) && as_i64(a[1], &N) && as_i64(a[2], &ld) && as_int(a[3], &BR) &&
       as_int(a[4], &BC) && as_int(a[5], &al) && as_ptr(a[6], &x));
    const int st = tm_row_walk(M, N, ld, BR, BC, al, x, &bc, &nfull, &rem, &lanes);
    return Py_BuildValue("(iLLLi)", st, (long long)bc, (long long)nfull, (long long)rem, lanes);
}

static PyObject *py_map_walk(ARGS) {
    int64_t ldx, ldy, M, N, items = -1;
    int op, TM, TN, al, var, walk = -1;
    void *x, *y, *bias;
    (void)self;
    OK(want(n, 12, "tm_map_walk"));
    OK(as_int(a[0], &op) && as_ptr(a[1], &x) && as_i64(a[2], &ldx) && as_ptr(a[3], &y) && as_i64(a[4], &ldy) &&
       as_i64(a[5], &M) && as_i64(a[6], &N) && as_int(a[7], &TM) && as_int(a[8], &TN) && as_int(a[9], &al) &&
       as_int(a[10], &var) && as_ptr(a[11], &bias));
    const int st = tm_map_walk(op, x, ldx, y, ldy, M, N, TM, TN, al, var, bias, &walk, &items);
    return Py_BuildValue("(iiL)", st, walk, (long long)items);
}

static PyObject *py_col_walk(ARGS) {
    int64_t ldx, M, N, slab_rows = -1, strip_cols = -1, slabs = -1, strips = -1;
    int TM, TN, al, walk, form = -1;
    void *x, *out, *ws;
    size_t wsb;
    (void)self;
    OK(want(n, 11, "tm_col_walk"));
    OK(as_ptr(a[0], &x) && as_i64(a[1], &ldx) && as_ptr(a[2], &out) && as_i64(a[3], &M) && as_i64(a[4], &N) &&
       as_int(a[5], &TM) && as_int(a[6], &TN) && as_int(a[7], &al) && as_int(a[8], &walk) && as_ptr(a[9], &ws) &&
       as_size(a[10], &wsb));
    const int st = tm_col_walk(x, ldx, out, M, N, TM, TN, al, walk, ws, wsb, &form, &slab_rows, &strip_cols, &slabs,
                               &strips);
    return Py_BuildValue("(iiLLLL)", st, form, (long long)slab_rows, (long long)strip_cols, (long long)slabs,
                         (long long)strips);
}

static PyObject *py_plan_tiles(ARGS) {
    int64_t M, N, tm_ = -1, tn_ = -1, whole = -1;
    int TM, TN;
    (void)self;
    OK(want(n, 4, "tm_plan_tiles"));
    OK(as_i64(a[0], &M) && as_i64(a[1], &N) && as_int(a[2], &TM) && as_int(a[3], &TN));
    const int st = tm_plan_tiles(M, N, TM, TN, &tm_, &tn_, &whole);
    return Py_BuildValue("(iLLL)", st, (long long)tm_, (long long)tn_, (long long)whole);
}

static PyObject *py_pad_extents(ARGS) {
    int64_t M, N, Mp = -1, Np = -1, ldp = -1;
    int TM, TN;
    (void)self;
    OK(want(n, 4, "tm_pad_extents"));
    OK(as_i64(a[0], &M) && as_i64(a[1], &N) && as_int(a[2], &TM) && as_int(a[3], &TN));
    const int st = tm_pad_extents(M, N, TM, TN, &Mp, &Np, &ldp);
    return Py_BuildValue("(iLLL)", st, (long long)Mp, (long long)Np, (long long)ldp);
}

#define TUNE_ROWS 9
#define TUNE_COLS 11

/* Returns (status, TM_best, TN_best, us_best, table) with table a tuple of 99 floats (row-major,
 * 9 x 11), or None when want_table is false (the C call then gets a NULL table). */
static PyObject *py_autotune_map(ARGS) {
    void *x, *y, *e0, *e1, *s;
    int64_t ldx, ldy, M, N;
    float alpha, beta;
    int op, al, var, reps, want_table;
    (void)self;
    OK(want(n, 16, "tm_autotune_map"));
    OK(as_int(a[0], &op) && as_ptr(a[1], &x) && as_i64(a[2], &ldx) && as_ptr(a[3], &y) &&
       as_i64(a[4], &ldy) && as_i64(a[5], &M) && as_i64(a[6], &N) && as_f32(a[7], &alpha) &&
       as_f32(a[8], &beta) && as_int(a[9], &al) && as_int(a[10], &var) && as_int(a[11], &reps) &&
       as_ptr(a[12], &e0) && as_ptr(a[13], &e1) && as_int(a[14], &want_table) && as_ptr(a[15], &s));
    int tmb = 0, tnb = 0;
    float usb = 0.0f;
    float table[TUNE_ROWS * TUNE_COLS];
    int st;
    Py_BEGIN_ALLOW_THREADS
    st = tm_autotune_map(op, (const float *)x, ldx, (float *)y, ldy, M, N, alpha, beta, al, var,
                         reps, e0, e1, &tmb, &tnb, &usb, want_table ? table : NULL, s);
    Py_END_ALLOW_THREADS
    PyObject *tab;
    if (want_table) {
        tab = PyTuple_New(TUNE_ROWS * TUNE_COLS);
        if (tab == NULL)
            return NULL;
        for (int i = 0; i < TUNE_ROWS * TUNE_COLS; ++i) {
            PyObject *f = PyFloat_FromDouble((double)table[i]);
            if (f == NULL) {
                Py_DECREF(tab);
                return NULL;
            }
            PyTuple_SET_ITEM(tab, i, f);
        }
    } else {
        Py_INCREF(Py_None);
        tab = Py_None;
    }
    return Py_BuildValue("(iiidN)", st, tmb, tnb, (double)usb, tab);
}

static PyObject *py_status_string(ARGS) {
    int st;
    (void)self;
    OK(want(n, 1, "tm_status_string"));
    OK(as_int(a[0], &st));
    return PyUnicode_FromString(tm_status_string(st));
}

#define FAST(name, fn) {name, (PyCFunction)(void (*)(void))fn, METH_FASTCALL, NULL}

static PyMethodDef methods[] = {
    FAST("tm_map_affine", py_map_affine),
    FAST("tm_scale2d", py_scale2d),
    FAST("tm_copy2d", py_copy2d),
    FAST("tm_channel_affine", py_channel_affine),
    FAST("tm_rowsum", py_rowsum),
    FAST("tm_rows_workspace_bytes", py_rows_workspace_bytes),
    FAST("tm_rowsum_ws", py_rowsum_ws),
    FAST("tm_rowmax_masked_ws", py_rowmax_masked_ws),
    FAST("tm_softmax_stats_ws", py_softmax_stats_ws),
    FAST("tm_colsum_workspace_bytes", py_colsum_workspace_bytes),
    FAST("tm_colsum", py_colsum),
    FAST("tm_rowmax_masked", py_rowmax_masked),
    FAST("tm_softmax_stats", py_softmax_stats),
    FAST("tm_transpose", py_transpose),
    FAST("tm_check_promise", py_check_promise),
    FAST("tm_split", py_split),
    FAST("tm_plan_tiles", py_plan_tiles),
    FAST("tm_map_walk", py_map_walk),
    FAST("tm_colsum_noalloc", py_colsum_noalloc),
    FAST("tm_row_walk", py_row_walk),
    FAST("tm_col_walk", py_col_walk),
    FAST("tm_pad_extents", py_pad_extents),
    FAST("tm_autotune_map", py_autotune_map),
    FAST("tm_status_string", py_status_string),
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef module = {
    PyModuleDef_HEAD_INIT, "_tilemap",
    "The C ABI of libtilemap.so, one function per call (see tilemap.py for the documented binding).",
    -1, methods, NULL, NULL, NULL, NULL,
};

PyMODINIT_FUNC PyInit__tilemap(void) {
    PyObject *m = PyModule_Create(&module);
    if (m == NULL)
        return NULL;
    if (PyModule_AddIntConstant(m, "TUNE_ROWS", TUNE_ROWS) < 0 ||
        PyModule_AddIntConstant(m, "TUNE_COLS", TUNE_COLS) < 0) {
        Py_DECREF(m);
        return NULL;
    }
    return m;
}
