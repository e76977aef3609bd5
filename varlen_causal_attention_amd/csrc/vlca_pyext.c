/* CPython trampoline for the two launch entry points of libvlca.so.
 *
 * Argument marshalling only: each function converts its Python integers and
 * float to C values and calls the entry point whose address the package passed
 * to set_entries() (taken from its ctypes handle of libvlca.so, so the library is
 * loaded once).  A ctypes foreign call converts each argument through its own
 * Python-level type objects and costs a few microseconds; a launch of a small
 * batch is in the same range, so the host would otherwise bound back-to-back
 * calls.  The GIL is released around the call (a launch may wait for room in
 * the stream's queue).
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>

#include "varlen_causal_attn.h"

static __typeof__(varlen_causal_attn_fwd)* p_fwd = NULL;
static __typeof__(varlen_causal_attn_fwd_worklist)* p_fwd_worklist = NULL;

static int as_ptr(PyObject* o, void** out) {
  *out = PyLong_AsVoidPtr(o);
  return !(*out == NULL && PyErr_Occurred());
}

static int as_int(PyObject* o, int* out) {
  const long v = PyLong_AsLong(o);
  if (v == -1 && PyErr_Occurred()) return 0;
  if (v < INT_MIN || v > INT_MAX) {
    PyErr_SetString(PyExc_OverflowError, "argument does not fit a C int");
    return 0;
  }
  *out = (int)v;
  return 1;
}

/* set_entries(fwd_address, fwd_worklist_address) */
static PyObject* set_entries(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
  void *a, *b;
  (void)self;
  if (nargs != 2) {
    PyErr_SetString(PyExc_TypeError, "set_entries takes 2 arguments");
    return NULL;
  }
  if (!as_ptr(args[0], &a) || !as_ptr(args[1], &b)) return NULL;
  p_fwd = (__typeof__(p_fwd))a;
  p_fwd_worklist = (__typeof__(p_fwd_worklist))b;
  Py_RETURN_NONE;
}

/* fwd(qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale, out, stream) -> int */
static PyObject* fwd(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
  void *qkv, *cu, *out, *stream;
  int num_users, max_seqlen, n_heads, head_dim, rc;
  double scale;
  (void)self;
  if (nargs != 9) {
    PyErr_SetString(PyExc_TypeError, "fwd takes 9 arguments");
    return NULL;
  }
  if (p_fwd == NULL) {
    PyErr_SetString(PyExc_RuntimeError, "set_entries() has not been called");
    return NULL;
  }
  if (!as_ptr(args[0], &qkv) || !as_ptr(args[1], &cu) || !as_int(args[2], &num_users) ||
      !as_int(args[3], &max_seqlen) || !as_int(args[4], &n_heads) || !as_int(args[5], &head_dim) ||
      !as_ptr(args[7], &out) || !as_ptr(args[8], &stream))
    return NULL;
  scale = PyFloat_AsDouble(args[6]);
  if (scale == -1.0 && PyErr_Occurred()) return NULL;
  Py_BEGIN_ALLOW_THREADS
  rc = p_fwd(qkv, (const int32_t*)cu, num_users, max_seqlen, n_heads, head_dim, (float)scale, out,
             (hipStream_t)stream);
  Py_END_ALLOW_THREADS
  return PyLong_FromLong(rc);
}

/* fwd_worklist(qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale,
 *              items, capacity, count, out, stream) -> int */
static PyObject* fwd_worklist(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
  void *qkv, *cu, *items, *count, *out, *stream;
  int num_users, max_seqlen, n_heads, head_dim, rc;
  long long capacity;
  double scale;
  (void)self;
  if (nargs != 12) {
    PyErr_SetString(PyExc_TypeError, "fwd_worklist takes 12 arguments");
    return NULL;
  }
  if (p_fwd_worklist == NULL) {
    PyErr_SetString(PyExc_RuntimeError, "set_entries() has not been called");
    return NULL;
  }
  if (!as_ptr(args[0], &qkv) || !as_ptr(args[1], &cu) || !as_int(args[2], &num_users) ||
      !as_int(args[3], &max_seqlen) || !as_int(args[4], &n_heads) || !as_int(args[5], &head_dim) ||
      !as_ptr(args[7], &items) || !as_ptr(args[9], &count) || !as_ptr(args[10], &out) ||
      !as_ptr(args[11], &stream))
    return NULL;
  scale = PyFloat_AsDouble(args[6]);
  if (scale == -1.0 && PyErr_Occurred()) return NULL;
  capacity = PyLong_AsLongLong(args[8]);
  if (capacity == -1 && PyErr_Occurred()) return NULL;
  Py_BEGIN_ALLOW_THREADS
  rc = p_fwd_worklist(qkv, (const int32_t*)cu, num_users, max_seqlen, n_heads, head_dim, (float)scale,
                      (const int32_t*)items, (int64_t)capacity, (const int32_t*)count, out, (hipStream_t)stream);
  Py_END_ALLOW_THREADS
  return PyLong_FromLong(rc);
}

static PyMethodDef methods[] = {
    {"set_entries", (PyCFunction)(void (*)(void))set_entries, METH_FASTCALL, "Addresses of the two entry points."},
    {"fwd", (PyCFunction)(void (*)(void))fwd, METH_FASTCALL, "varlen_causal_attn_fwd."},
    {"fwd_worklist", (PyCFunction)(void (*)(void))fwd_worklist, METH_FASTCALL, "varlen_causal_attn_fwd_worklist."},
    {NULL, NULL, 0, NULL},
};

static struct PyModuleDef module = {PyModuleDef_HEAD_INIT, "_vlca_call", NULL, -1, methods, NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__vlca_call(void) { return PyModule_Create(&module); }
