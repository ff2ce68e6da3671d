/* Argument marshalling for eager calls of lowbit_linear from Python.
 *
 * A CPython extension with two functions:
 *   bind(fn, act, packed, scales, zeros, bias, bits, group, N, K) -> capsule
 *       keeps the arguments of one layer that do not change between calls,
 *       and fn, the address of lowbit_linear in the loaded library;
 *   call(capsule, x, y, M, workspace, workspace_bytes, stream) -> status
 *       calls fn with them and the per-call arguments (device pointers and
 *       the stream handle as Python ints, 0 for NULL).
 * It does no arithmetic of the layer and holds no state beyond the capsule:
 * every argument is passed on unchanged and lowbit_linear validates them.
 * (ctypes builds and converts fifteen argument objects per call; this takes
 * seven ints through the vectorcall protocol.)
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stddef.h>
#include <stdint.h>

#include "lowbit.h"

typedef __typeof__(lowbit_linear)* linear_fn;   /* the declared signature */

typedef struct {
  linear_fn fn;
  lowbit_dtype act;
  int bits, group;
  const uint8_t* packed;
  const void *scales, *zeros, *bias;
  int64_t N, K;
} bound_layer;

static const char kCapsule[] = "lowbit.bound_layer";

static void free_bound(PyObject* cap) {
  void* p = PyCapsule_GetPointer(cap, kCapsule);
  PyMem_Free(p);
}

static void* as_ptr(PyObject* o) {
  if (o == Py_None) return NULL;
  return PyLong_AsVoidPtr(o);
}

static PyObject* bind(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
  (void)self;
  if (nargs != 10) {
    PyErr_SetString(PyExc_TypeError, "bind takes 10 arguments");
    return NULL;
  }
  bound_layer* b = (bound_layer*)PyMem_Malloc(sizeof(bound_layer));
  if (!b) return PyErr_NoMemory();
  b->fn = (linear_fn)as_ptr(args[0]);
  b->act = (lowbit_dtype)PyLong_AsLong(args[1]);
  b->packed = (const uint8_t*)as_ptr(args[2]);
  b->scales = as_ptr(args[3]);
  b->zeros = as_ptr(args[4]);
  b->bias = as_ptr(args[5]);
  b->bits = (int)PyLong_AsLong(args[6]);
  b->group = (int)PyLong_AsLong(args[7]);
  b->N = PyLong_AsLongLong(args[8]);
  b->K = PyLong_AsLongLong(args[9]);
  if (PyErr_Occurred() || !b->fn) {
    PyMem_Free(b);
    if (!PyErr_Occurred()) PyErr_SetString(PyExc_ValueError, "null function address");
    return NULL;
  }
  PyObject* cap = PyCapsule_New(b, kCapsule, free_bound);
  if (!cap) PyMem_Free(b);
  return cap;
}

static PyObject* call(PyObject* self, PyObject* const* args, Py_ssize_t nargs) {
  (void)self;
  if (nargs != 7) {
    PyErr_SetString(PyExc_TypeError, "call takes 7 arguments");
    return NULL;
  }
  const bound_layer* b = (const bound_layer*)PyCapsule_GetPointer(args[0], kCapsule);
  if (!b) return NULL;
  void* x = as_ptr(args[1]);
  void* y = as_ptr(args[2]);
  const int64_t M = PyLong_AsLongLong(args[3]);
  void* ws = as_ptr(args[4]);
  const size_t ws_bytes = (size_t)PyLong_AsSize_t(args[5]);
  void* stream = as_ptr(args[6]);
  if (PyErr_Occurred()) return NULL;
  const lowbit_status st = b->fn(x, b->act, b->packed, b->scales, b->zeros, b->bias, y, b->bits, b->group,
                       M, b->N, b->K, ws, ws_bytes, stream);
  return PyLong_FromLong((long)st);
}

static PyMethodDef kMethods[] = {
    {"bind", (PyCFunction)(void (*)(void))bind, METH_FASTCALL, "bind one layer's fixed arguments"},
    {"call", (PyCFunction)(void (*)(void))call, METH_FASTCALL, "call lowbit_linear for a bound layer"},
    {NULL, NULL, 0, NULL}};

static struct PyModuleDef kModule = {PyModuleDef_HEAD_INIT, "_lowbit_fastcall",
                                     "argument marshalling for eager lowbit_linear calls", -1,
                                     kMethods, NULL, NULL, NULL, NULL};

PyMODINIT_FUNC PyInit__lowbit_fastcall(void) { return PyModule_Create(&kModule); }
