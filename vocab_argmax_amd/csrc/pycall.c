/* _vpa_call: CPython marshalling of the launch entry points of include/vpa.h.
 *
 * Each function here has the name of a C entry point and takes that entry
 * point's arguments in the same order, as Python objects:
 *   - a pointer is an int (an address, e.g. tensor.data_ptr()) or None;
 *   - a vpa_vocab is three ints in a row: vocab, shard_width, n_shards;
 *   - a vpa_epilogue pointer is None or a tuple (d2t address or None,
 *     d2t_len, scale), scale rounded to fp32 as a C float conversion does;
 *   - the stream is the HIP stream handle as an int (0 or None: the null
 *     stream);
 * and returns the vpa_status as an int.  A Python argument of the wrong type
 * or outside its C type's range raises before the library is called.
 *
 * The module holds no copy of the library: bind(name, address) installs the
 * address of an entry point from the libvpa.so the caller has loaded, and a
 * function called before it is bound raises.  The GIL is released while the
 * library runs (it validates its arguments and enqueues work; it never
 * blocks on the device).
 *
 * This module converts arguments and nothing else: all validation of the
 * values, and every step of the computation, stays in the library.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>

#include <stdarg.h>
#include <stdint.h>
#include <string.h>

#include "vpa.h"

_Static_assert(sizeof(vpa_dtype) == sizeof(int32_t), "vpa_dtype is passed as an int32");

static __typeof__(&vpa_block_stats) p_block_stats;
static __typeof__(&vpa_verify_stats) p_verify_stats;
static __typeof__(&vpa_verify_stats_rows) p_verify_stats_rows;
static __typeof__(&vpa_ragged_rows) p_ragged_rows;
static __typeof__(&vpa_combine_stats) p_combine_stats;
static __typeof__(&vpa_top_tokens) p_top_tokens;
static __typeof__(&vpa_top_tokens_noalloc) p_top_tokens_noalloc;
static __typeof__(&vpa_greedy_verify) p_greedy_verify;
static __typeof__(&vpa_greedy_verify_ragged) p_greedy_verify_ragged;

static const struct {
    const char* name;
    void** slot;
} k_entries[] = {
    {"vpa_block_stats", (void**)&p_block_stats},
    {"vpa_verify_stats", (void**)&p_verify_stats},
    {"vpa_verify_stats_rows", (void**)&p_verify_stats_rows},
    {"vpa_ragged_rows", (void**)&p_ragged_rows},
    {"vpa_combine_stats", (void**)&p_combine_stats},
    {"vpa_top_tokens", (void**)&p_top_tokens},
    {"vpa_top_tokens_noalloc", (void**)&p_top_tokens_noalloc},
    {"vpa_greedy_verify", (void**)&p_greedy_verify},
    {"vpa_greedy_verify_ragged", (void**)&p_greedy_verify_ragged},
};
#define N_ENTRIES ((int)(sizeof(k_entries) / sizeof(k_entries[0])))

static int to_i64(PyObject* o, int64_t* out) {
    long long v = PyLong_AsLongLong(o);
    if (v == -1 && PyErr_Occurred()) return 0;
    *out = (int64_t)v;
    return 1;
}

static int to_i32(PyObject* o, int32_t* out) {
    long long v = PyLong_AsLongLong(o);
    if (v == -1 && PyErr_Occurred()) return 0;
    if (v < INT32_MIN || v > INT32_MAX) {
        PyErr_Format(PyExc_OverflowError, "%lld does not fit a 32-bit argument", v);
        return 0;
    }
    *out = (int32_t)v;
    return 1;
}

static int to_size(PyObject* o, size_t* out) {
    size_t v = PyLong_AsSize_t(o);
    if (v == (size_t)-1 && PyErr_Occurred()) return 0;
    *out = v;
    return 1;
}

static int to_ptr(PyObject* o, void** out) {
    if (o == Py_None) {
        *out = NULL;
        return 1;
    }
    unsigned long long v = PyLong_AsUnsignedLongLong(o);
    if (v == (unsigned long long)-1 && PyErr_Occurred()) return 0;
    *out = (void*)(uintptr_t)v;
    return 1;
}

/* Converts args[0..nargs) by `fmt`, one character per Python argument:
 *   p pointer (void**), l int64 (int64_t*), i int32 (int32_t*), z size_t
 *   (size_t*), d dtype (vpa_dtype*, an int32 value), V vocab (vpa_vocab*, three
 *   arguments), e epilogue (vpa_epilogue* storage, then const vpa_epilogue**
 *   set to it or to NULL). */
static int parse(const char* name, PyObject* const* args, Py_ssize_t nargs, const char* fmt,
                 ...) {
    Py_ssize_t want = 0;
    for (const char* f = fmt; *f; ++f) want += (*f == 'V') ? 3 : 1;
    if (nargs != want) {
        PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (%zd given)", name, want, nargs);
        return 0;
    }
    va_list ap;
    va_start(ap, fmt);
    int ok = 1;
    Py_ssize_t a = 0;
    for (const char* f = fmt; ok && *f; ++f) {
        switch (*f) {
        case 'p':
            ok = to_ptr(args[a++], va_arg(ap, void**));
            break;
        case 'l':
            ok = to_i64(args[a++], va_arg(ap, int64_t*));
            break;
        case 'i':
            ok = to_i32(args[a++], va_arg(ap, int32_t*));
            break;
        case 'z':
            ok = to_size(args[a++], va_arg(ap, size_t*));
            break;
        case 'd': {
            int32_t v = 0;
            vpa_dtype* out = va_arg(ap, vpa_dtype*);
            ok = to_i32(args[a++], &v);
            /* the library reads the argument's bytes as an int, so any int32
             * reaches its own range check */
            if (ok) memcpy(out, &v, sizeof(v));
            break;
        }
        case 'V': {
            vpa_vocab* v = va_arg(ap, vpa_vocab*);
            ok = to_i64(args[a], &v->vocab) && to_i64(args[a + 1], &v->shard_width) &&
                 to_i32(args[a + 2], &v->n_shards);
            a += 3;
            break;
        }
        case 'e': {
            vpa_epilogue* e = va_arg(ap, vpa_epilogue*);
            const vpa_epilogue** pe = va_arg(ap, const vpa_epilogue**);
            PyObject* o = args[a++];
            if (o == Py_None) {
                *pe = NULL;
                break;
            }
            if (!PyTuple_Check(o) || PyTuple_GET_SIZE(o) != 3) {
                PyErr_SetString(PyExc_TypeError,
                                "an epilogue is None or a tuple (d2t, d2t_len, scale)");
                ok = 0;
                break;
            }
            void* d2t = NULL;
            double scale = 0.0;
            ok = to_ptr(PyTuple_GET_ITEM(o, 0), &d2t) &&
                 to_i64(PyTuple_GET_ITEM(o, 1), &e->d2t_len);
            if (ok) {
                scale = PyFloat_AsDouble(PyTuple_GET_ITEM(o, 2));
                ok = !(scale == -1.0 && PyErr_Occurred());
            }
            e->d2t = (const int64_t*)d2t;
            e->scale = (float)scale;
            *pe = e;
            break;
        }
        default:
            PyErr_Format(PyExc_SystemError, "%s: bad format character", name);
            ok = 0;
        }
    }
    va_end(ap);
    return ok;
}

static int bound(const char* name, const void* fn) {
    if (fn) return 1;
    PyErr_Format(PyExc_RuntimeError, "%s is not bound: call bind() with its address first", name);
    return 0;
}

#define RETURN_STATUS(call)                                                                     \
    do {                                                                                        \
        vpa_status st_;                                                                         \
        Py_BEGIN_ALLOW_THREADS st_ = (call);                                                    \
        Py_END_ALLOW_THREADS return PyLong_FromLong((long)st_);                                 \
    } while (0)

static PyObject* py_block_stats(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
    (void)self;
    void *logits, *rows, *stats, *stream;
    vpa_dtype dt;
    int64_t ld, n_rows, logits_rows;
    vpa_vocab v;
    int32_t first, n_local, block;
    if (!bound("vpa_block_stats", (const void*)p_block_stats) ||
        !parse("vpa_block_stats", args, nargs, "pdlViipllipp", &logits, &dt, &ld, &v, &first,
               &n_local, &rows, &n_rows, &logits_rows, &block, &stats, &stream))
        return NULL;
    RETURN_STATUS(p_block_stats(logits, dt, ld, v, first, n_local, (const int32_t*)rows, n_rows,
                                logits_rows, block, (vpa_stat*)stats, stream));
}

static PyObject* py_verify_stats(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
    (void)self;
    void *logits, *dst, *bst, *stream;
    vpa_dtype dt;
    int64_t ld, n_req;
    vpa_vocab v;
    int32_t first, n_local, k, bd, bb;
    if (!bound("vpa_verify_stats", (const void*)p_verify_stats) ||
        !parse("vpa_verify_stats", args, nargs, "pdlViiliiippp", &logits, &dt, &ld, &v, &first,
               &n_local, &n_req, &k, &bd, &bb, &dst, &bst, &stream))
        return NULL;
    RETURN_STATUS(p_verify_stats(logits, dt, ld, v, first, n_local, n_req, k, bd, bb,
                                 (vpa_stat*)dst, (vpa_stat*)bst, stream));
}

static PyObject* py_verify_stats_rows(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
    (void)self;
    void *logits, *drows, *brows, *dst, *bst, *stream;
    vpa_dtype dt;
    int64_t ld, nd, nb, logits_rows;
    vpa_vocab v;
    int32_t first, n_local, bd, bb;
    if (!bound("vpa_verify_stats_rows", (const void*)p_verify_stats_rows) ||
        !parse("vpa_verify_stats_rows", args, nargs, "pdlViiplplliippp", &logits, &dt, &ld, &v,
               &first, &n_local, &drows, &nd, &brows, &nb, &logits_rows, &bd, &bb, &dst, &bst,
               &stream))
        return NULL;
    RETURN_STATUS(p_verify_stats_rows(logits, dt, ld, v, first, n_local, (const int32_t*)drows,
                                      nd, (const int32_t*)brows, nb, logits_rows, bd, bb,
                                      (vpa_stat*)dst, (vpa_stat*)bst, stream));
}

static PyObject* py_ragged_rows(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
    (void)self;
    void *cu, *drows, *brows, *stream;
    int64_t n_req, total;
    if (!bound("vpa_ragged_rows", (const void*)p_ragged_rows) ||
        !parse("vpa_ragged_rows", args, nargs, "pllppp", &cu, &n_req, &total, &drows, &brows,
               &stream))
        return NULL;
    RETURN_STATUS(p_ragged_rows((const int32_t*)cu, n_req, total, (int32_t*)drows,
                                (int32_t*)brows, stream));
}

static PyObject* py_combine_stats(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
    (void)self;
    void *stats, *ids, *vals, *mapped, *stream;
    int32_t s, m;
    int64_t n;
    vpa_epilogue e;
    const vpa_epilogue* pe;
    if (!bound("vpa_combine_stats", (const void*)p_combine_stats) ||
        !parse("vpa_combine_stats", args, nargs, "piliepppp", &stats, &s, &n, &m, &e, &pe,
               &ids, &vals, &mapped, &stream))
        return NULL;
    RETURN_STATUS(p_combine_stats((const vpa_stat*)stats, s, n, m, pe, (int32_t*)ids,
                                  (uint32_t*)vals, (int64_t*)mapped, stream));
}

static PyObject* py_top_tokens(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
    (void)self;
    void *logits, *ws, *ids, *vals, *mapped, *stream;
    vpa_dtype dt;
    int64_t ld, n;
    vpa_vocab v;
    int32_t block;
    size_t ws_bytes;
    vpa_epilogue e;
    const vpa_epilogue* pe;
    if (!bound("vpa_top_tokens", (const void*)p_top_tokens) ||
        !parse("vpa_top_tokens", args, nargs, "pdlVlipzepppp", &logits, &dt, &ld, &v, &n, &block,
               &ws, &ws_bytes, &e, &pe, &ids, &vals, &mapped, &stream))
        return NULL;
    RETURN_STATUS(p_top_tokens(logits, dt, ld, v, n, block, ws, ws_bytes, pe, (int32_t*)ids,
                               (uint32_t*)vals, (int64_t*)mapped, stream));
}

static PyObject* py_top_tokens_noalloc(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
    (void)self;
    void *logits, *ids, *vals, *mapped, *stream;
    vpa_dtype dt;
    int64_t ld, n;
    vpa_vocab v;
    int32_t block;
    vpa_epilogue e;
    const vpa_epilogue* pe;
    if (!bound("vpa_top_tokens_noalloc", (const void*)p_top_tokens_noalloc) ||
        !parse("vpa_top_tokens_noalloc", args, nargs, "pdlVliepppp", &logits, &dt, &ld, &v, &n,
               &block, &e, &pe, &ids, &vals, &mapped, &stream))
        return NULL;
    RETURN_STATUS(p_top_tokens_noalloc(logits, dt, ld, v, n, block, pe, (int32_t*)ids,
                                       (uint32_t*)vals, (int64_t*)mapped, stream));
}

static PyObject* py_greedy_verify(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
    (void)self;
    void *dst, *bst, *drafts, *accept, *out, *ns, *nr, *tg, *stream;
    int32_t md, mb, s, k;
    int64_t n_req;
    if (!bound("vpa_greedy_verify", (const void*)p_greedy_verify) ||
        !parse("vpa_greedy_verify", args, nargs, "pipiilippppppp", &dst, &md, &bst, &mb, &s,
               &n_req, &k, &drafts, &accept, &out, &ns, &nr, &tg, &stream))
        return NULL;
    RETURN_STATUS(p_greedy_verify((const vpa_stat*)dst, md, (const vpa_stat*)bst, mb, s, n_req, k,
                                  (const int32_t*)drafts, (const int32_t*)accept, (int32_t*)out,
                                  (int32_t*)ns, (int32_t*)nr, (int32_t*)tg, stream));
}

static PyObject* py_greedy_verify_ragged(PyObject* self, PyObject* const* args,
                                         Py_ssize_t nargs) {
    (void)self;
    void *dst, *bst, *cu, *drafts, *pre, *accept, *out, *ns, *nr, *tg, *stream;
    int32_t md, mb, s;
    int64_t n_req, total;
    if (!bound("vpa_greedy_verify_ragged", (const void*)p_greedy_verify_ragged) ||
        !parse("vpa_greedy_verify_ragged", args, nargs, "pipiilplpppppppp", &dst, &md, &bst, &mb,
               &s, &n_req, &cu, &total, &drafts, &pre, &accept, &out, &ns, &nr, &tg, &stream))
        return NULL;
    RETURN_STATUS(p_greedy_verify_ragged(
        (const vpa_stat*)dst, md, (const vpa_stat*)bst, mb, s, n_req, (const int32_t*)cu, total,
        (const int32_t*)drafts, (const uint8_t*)pre, (const int32_t*)accept, (int32_t*)out,
        (int32_t*)ns, (int32_t*)nr, (int32_t*)tg, stream));
}

static PyObject* py_bind(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
    (void)self;
    if (nargs != 2 || !PyUnicode_Check(args[0])) {
        PyErr_SetString(PyExc_TypeError, "bind(name: str, address: int)");
        return NULL;
    }
    const char* name = PyUnicode_AsUTF8(args[0]);
    void* addr = NULL;
    if (!name || !to_ptr(args[1], &addr)) return NULL;
    if (!addr) {
        PyErr_Format(PyExc_ValueError, "bind(%s): null address", name);
        return NULL;
    }
    for (int i = 0; i < N_ENTRIES; ++i) {
        if (strcmp(k_entries[i].name, name) == 0) {
            *k_entries[i].slot = addr;
            Py_RETURN_NONE;
        }
    }
    PyErr_Format(PyExc_KeyError, "%s is not an entry point this module calls", name);
    return NULL;
}

static PyObject* py_entries(PyObject* self, PyObject* unused) {
    (void)self;
    (void)unused;
    PyObject* t = PyTuple_New(N_ENTRIES);
    if (!t) return NULL;
    for (int i = 0; i < N_ENTRIES; ++i) {
        PyObject* s = PyUnicode_FromString(k_entries[i].name);
        if (!s) {
            Py_DECREF(t);
            return NULL;
        }
        PyTuple_SET_ITEM(t, i, s);
    }
    return t;
}

#define FASTCALL(f) (PyCFunction)(void (*)(void))(f), METH_FASTCALL

static PyMethodDef k_methods[] = {
    {"vpa_block_stats", FASTCALL(py_block_stats), "vpa_block_stats (include/vpa.h)"},
    {"vpa_verify_stats", FASTCALL(py_verify_stats), "vpa_verify_stats (include/vpa.h)"},
    {"vpa_verify_stats_rows", FASTCALL(py_verify_stats_rows),
     "vpa_verify_stats_rows (include/vpa.h)"},
    {"vpa_ragged_rows", FASTCALL(py_ragged_rows), "vpa_ragged_rows (include/vpa.h)"},
    {"vpa_combine_stats", FASTCALL(py_combine_stats), "vpa_combine_stats (include/vpa.h)"},
    {"vpa_top_tokens", FASTCALL(py_top_tokens), "vpa_top_tokens (include/vpa.h)"},
    {"vpa_top_tokens_noalloc", FASTCALL(py_top_tokens_noalloc),
     "vpa_top_tokens_noalloc (include/vpa.h)"},
    {"vpa_greedy_verify", FASTCALL(py_greedy_verify), "vpa_greedy_verify (include/vpa.h)"},
    {"vpa_greedy_verify_ragged", FASTCALL(py_greedy_verify_ragged),
     "vpa_greedy_verify_ragged (include/vpa.h)"},
    {"bind", FASTCALL(py_bind), "bind(name, address): the entry point `name` is at `address`"},
    {"entries", py_entries, METH_NOARGS, "names of the entry points this module calls"},
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef k_module = {
    PyModuleDef_HEAD_INIT, "_vpa_call",
    "CPython marshalling of the vpa C ABI's launch entry points", -1, k_methods,
    NULL, NULL, NULL, NULL,
};

PyMODINIT_FUNC PyInit__vpa_call(void) { return PyModule_Create(&k_module); }
