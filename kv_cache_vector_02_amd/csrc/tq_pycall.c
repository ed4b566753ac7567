/*
 * Argument marshalling from Python to the C ABI of libtq (include/tq.h) for
 * the calls a decode or prefill loop makes every step: tq_encode, tq_encode_kv,
 * tq_prefill, tq_append and tq_attn_decode.  Plain integers (device addresses, sizes,
 * strides), one float and None (a NULL pointer) in, the library's return code
 * out; no arithmetic.  ctypes spends about 0.5 us more per call converting
 * their 12 to 21 arguments, 7-9 % of the host time of a small encode.
 *
 * The module does not link libtq: bind() receives the addresses of the entry
 * points of the library the Python package loaded, so both paths always call
 * the same code.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stdint.h>

#include "tq.h"

typedef __typeof__(tq_encode) encode_fn;
typedef __typeof__(tq_encode_kv) encode_kv_fn;
typedef __typeof__(tq_attn_decode) attn_decode_fn;
typedef __typeof__(tq_append) append_fn;
typedef __typeof__(tq_prefill) prefill_fn;

static encode_fn *p_encode;
static encode_kv_fn *p_encode_kv;
static attn_decode_fn *p_attn_decode;
static append_fn *p_append;
static prefill_fn *p_prefill;

/* an address argument: a Python int, or None for NULL */
static int arg_ptr(PyObject *o, void **out) {
    if (o == Py_None) {
        *out = NULL;
        return 0;
    }
    *out = PyLong_AsVoidPtr(o);
    return (*out == NULL && PyErr_Occurred()) ? -1 : 0;
}

static int arg_i64(PyObject *o, int64_t *out) {
    *out = (int64_t)PyLong_AsLongLong(o);
    return (*out == -1 && PyErr_Occurred()) ? -1 : 0;
}

static int arg_int(PyObject *o, int *out) {
    const long v = PyLong_AsLong(o);
    if (v == -1 && PyErr_Occurred()) return -1;
    if (v < INT32_MIN || v > INT32_MAX) {
        PyErr_SetString(PyExc_OverflowError, "argument does not fit a C int");
        return -1;
    }
    *out = (int)v;
    return 0;
}

static int check_nargs(Py_ssize_t nargs, Py_ssize_t want, const char *name) {
    if (nargs != want) {
        PyErr_Format(PyExc_TypeError, "%s takes %zd arguments (%zd given)", name, want, nargs);
        return -1;
    }
    return 0;
}

static PyObject *unbound(const char *name) {
    PyErr_Format(PyExc_RuntimeError, "%s: bind() has not been called", name);
    return NULL;
}

/* bind(addr_tq_encode, addr_tq_encode_kv, addr_tq_attn_decode, addr_tq_append,
 *      addr_tq_prefill) */
static PyObject *py_bind(PyObject *self, PyObject *args) {
    unsigned long long a, b, c, d, e;
    (void)self;
    if (!PyArg_ParseTuple(args, "KKKKK", &a, &b, &c, &d, &e)) return NULL;
    if (!a || !b || !c || !d || !e) {
        PyErr_SetString(PyExc_ValueError, "null entry point");
        return NULL;
    }
    p_encode = (encode_fn *)(uintptr_t)a;
    p_encode_kv = (encode_kv_fn *)(uintptr_t)b;
    p_attn_decode = (attn_decode_fn *)(uintptr_t)c;
    p_append = (append_fn *)(uintptr_t)d;
    p_prefill = (prefill_fn *)(uintptr_t)e;
    Py_RETURN_NONE;
}

/* encode(c, x, x_dtype, n, x_row_stride, codes, code_row_stride, norms,
 *        qjl_S, qjl_bits, qjl_gamma, stream): tq_encode's arguments in order */
static PyObject *py_encode(PyObject *self, PyObject *const *a, Py_ssize_t nargs) {
    void *c, *x, *codes, *norms, *S, *bits, *gamma, *stream;
    int dtype;
    int64_t n, xs, cs;
    (void)self;
    if (!p_encode) return unbound("encode");
    if (check_nargs(nargs, 12, "encode") || arg_ptr(a[0], &c) || arg_ptr(a[1], &x) || arg_int(a[2], &dtype) ||
        arg_i64(a[3], &n) || arg_i64(a[4], &xs) || arg_ptr(a[5], &codes) || arg_i64(a[6], &cs) ||
        arg_ptr(a[7], &norms) || arg_ptr(a[8], &S) || arg_ptr(a[9], &bits) || arg_ptr(a[10], &gamma) ||
        arg_ptr(a[11], &stream))
        return NULL;
    const int rc = p_encode((const tq_codec *)c, x, dtype, n, xs, (uint8_t *)codes, cs, (uint16_t *)norms,
                            (const float *)S, (uint8_t *)bits, (uint16_t *)gamma, stream);
    return PyLong_FromLong(rc);
}

/* encode_kv(kc, vc, k, v, x_dtype, n, x_row_stride, k_codes, k_code_row_stride,
 *           k_norms, v_codes, v_code_row_stride, v_norms, qjl_S, k_qjl_bits,
 *           k_qjl_gamma, stream): tq_encode_kv's arguments in order */
static PyObject *py_encode_kv(PyObject *self, PyObject *const *a, Py_ssize_t nargs) {
    void *kc, *vc, *k, *v, *kcodes, *knorms, *vcodes, *vnorms, *S, *bits, *gamma, *stream;
    int dtype;
    int64_t n, xs, kcs, vcs;
    (void)self;
    if (!p_encode_kv) return unbound("encode_kv");
    if (check_nargs(nargs, 17, "encode_kv") || arg_ptr(a[0], &kc) || arg_ptr(a[1], &vc) || arg_ptr(a[2], &k) ||
        arg_ptr(a[3], &v) || arg_int(a[4], &dtype) || arg_i64(a[5], &n) || arg_i64(a[6], &xs) ||
        arg_ptr(a[7], &kcodes) || arg_i64(a[8], &kcs) || arg_ptr(a[9], &knorms) || arg_ptr(a[10], &vcodes) ||
        arg_i64(a[11], &vcs) || arg_ptr(a[12], &vnorms) || arg_ptr(a[13], &S) || arg_ptr(a[14], &bits) ||
        arg_ptr(a[15], &gamma) || arg_ptr(a[16], &stream))
        return NULL;
    const int rc = p_encode_kv((const tq_codec *)kc, (const tq_codec *)vc, k, v, dtype, n, xs, (uint8_t *)kcodes,
                               kcs, (uint16_t *)knorms, (uint8_t *)vcodes, vcs, (uint16_t *)vnorms,
                               (const float *)S, (uint8_t *)bits, (uint16_t *)gamma, stream);
    return PyLong_FromLong(rc);
}

/* append(kc, vc, k, v, x_dtype, batch, n_heads, pos, ctx_cap, k_codes, k_norms,
 *        v_codes, v_norms, qjl_S, k_qjl_bits, k_qjl_gamma, stream):
 * tq_append's arguments in order */
static PyObject *py_append(PyObject *self, PyObject *const *a, Py_ssize_t nargs) {
    void *kc, *vc, *k, *v, *pos, *kcodes, *knorms, *vcodes, *vnorms, *S, *bits, *gamma, *stream;
    int dtype, batch, heads;
    int64_t cap;
    (void)self;
    if (!p_append) return unbound("append");
    if (check_nargs(nargs, 17, "append") || arg_ptr(a[0], &kc) || arg_ptr(a[1], &vc) || arg_ptr(a[2], &k) ||
        arg_ptr(a[3], &v) || arg_int(a[4], &dtype) || arg_int(a[5], &batch) || arg_int(a[6], &heads) ||
        arg_ptr(a[7], &pos) || arg_i64(a[8], &cap) || arg_ptr(a[9], &kcodes) || arg_ptr(a[10], &knorms) ||
        arg_ptr(a[11], &vcodes) || arg_ptr(a[12], &vnorms) || arg_ptr(a[13], &S) || arg_ptr(a[14], &bits) ||
        arg_ptr(a[15], &gamma) || arg_ptr(a[16], &stream))
        return NULL;
    const int rc = p_append((const tq_codec *)kc, (const tq_codec *)vc, k, v, dtype, batch, heads,
                            (const int32_t *)pos, cap, (uint8_t *)kcodes, (uint16_t *)knorms, (uint8_t *)vcodes,
                            (uint16_t *)vnorms, (const float *)S, (uint8_t *)bits, (uint16_t *)gamma, stream);
    return PyLong_FromLong(rc);
}

/* prefill(kc, vc, k, v, x_dtype, n_heads, tokens, t0, ctx_cap, k_codes,
 *         k_norms, v_codes, v_norms, qjl_S, k_qjl_bits, k_qjl_gamma, stream):
 * tq_prefill's arguments in order */
static PyObject *py_prefill(PyObject *self, PyObject *const *a, Py_ssize_t nargs) {
    void *kc, *vc, *k, *v, *kcodes, *knorms, *vcodes, *vnorms, *S, *bits, *gamma, *stream;
    int dtype, heads;
    int64_t tokens, t0, cap;
    (void)self;
    if (!p_prefill) return unbound("prefill");
    if (check_nargs(nargs, 17, "prefill") || arg_ptr(a[0], &kc) || arg_ptr(a[1], &vc) || arg_ptr(a[2], &k) ||
        arg_ptr(a[3], &v) || arg_int(a[4], &dtype) || arg_int(a[5], &heads) || arg_i64(a[6], &tokens) ||
        arg_i64(a[7], &t0) || arg_i64(a[8], &cap) || arg_ptr(a[9], &kcodes) || arg_ptr(a[10], &knorms) ||
        arg_ptr(a[11], &vcodes) || arg_ptr(a[12], &vnorms) || arg_ptr(a[13], &S) || arg_ptr(a[14], &bits) ||
        arg_ptr(a[15], &gamma) || arg_ptr(a[16], &stream))
        return NULL;
    const int rc = p_prefill((const tq_codec *)kc, (const tq_codec *)vc, k, v, dtype, heads, tokens, t0, cap,
                             (uint8_t *)kcodes, (uint16_t *)knorms, (uint8_t *)vcodes, (uint16_t *)vnorms,
                             (const float *)S, (uint8_t *)bits, (uint16_t *)gamma, stream);
    return PyLong_FromLong(rc);
}

/* attn_decode(kc, vc, q, q_dtype, batch, n_q_heads, n_kv_heads, ctx_len,
 *             ctx_cap, k_codes, k_norms, k_qjl, k_gamma, qjl_S, v_codes,
 *             v_norms, scale, out, workspace, workspace_bytes, stream):
 * tq_attn_decode's arguments in order */
static PyObject *py_attn_decode(PyObject *self, PyObject *const *a, Py_ssize_t nargs) {
    void *kc, *vc, *q, *ctx_len, *kcodes, *knorms, *kqjl, *kgamma, *S, *vcodes, *vnorms, *out, *ws, *stream;
    int q_dtype, batch, hq, hkv;
    int64_t cap, wsb;
    (void)self;
    if (!p_attn_decode) return unbound("attn_decode");
    if (check_nargs(nargs, 21, "attn_decode") || arg_ptr(a[0], &kc) || arg_ptr(a[1], &vc) || arg_ptr(a[2], &q) ||
        arg_int(a[3], &q_dtype) || arg_int(a[4], &batch) || arg_int(a[5], &hq) || arg_int(a[6], &hkv) ||
        arg_ptr(a[7], &ctx_len) || arg_i64(a[8], &cap) || arg_ptr(a[9], &kcodes) || arg_ptr(a[10], &knorms) ||
        arg_ptr(a[11], &kqjl) || arg_ptr(a[12], &kgamma) || arg_ptr(a[13], &S) || arg_ptr(a[14], &vcodes) ||
        arg_ptr(a[15], &vnorms) || arg_ptr(a[17], &out) || arg_ptr(a[18], &ws) || arg_i64(a[19], &wsb) ||
        arg_ptr(a[20], &stream))
        return NULL;
    const double scale = PyFloat_AsDouble(a[16]);
    if (scale == -1.0 && PyErr_Occurred()) return NULL;
    if (wsb < 0) {
        PyErr_SetString(PyExc_ValueError, "negative workspace size");
        return NULL;
    }
    const int rc = p_attn_decode((const tq_codec *)kc, (const tq_codec *)vc, q, q_dtype, batch, hq, hkv,
                                 (const int32_t *)ctx_len, cap, (const uint8_t *)kcodes, (const uint16_t *)knorms,
                                 (const uint8_t *)kqjl, (const uint16_t *)kgamma, (const float *)S,
                                 (const uint8_t *)vcodes, (const uint16_t *)vnorms, (float)scale, (float *)out, ws,
                                 (size_t)wsb, stream);
    return PyLong_FromLong(rc);
}

static PyMethodDef methods[] = {
    {"bind", py_bind, METH_VARARGS,
     "bind(tq_encode, tq_encode_kv, tq_attn_decode, tq_append, tq_prefill): entry point addresses"},
    {"encode", (PyCFunction)(void (*)(void))py_encode, METH_FASTCALL, "tq_encode with its C arguments"},
    {"encode_kv", (PyCFunction)(void (*)(void))py_encode_kv, METH_FASTCALL, "tq_encode_kv with its C arguments"},
    {"append", (PyCFunction)(void (*)(void))py_append, METH_FASTCALL, "tq_append with its C arguments"},
    {"prefill", (PyCFunction)(void (*)(void))py_prefill, METH_FASTCALL, "tq_prefill with its C arguments"},
    {"attn_decode", (PyCFunction)(void (*)(void))py_attn_decode, METH_FASTCALL,
     "tq_attn_decode with its C arguments"},
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_tqcall", NULL, -1, methods, NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__tqcall(void) { return PyModule_Create(&module); }
