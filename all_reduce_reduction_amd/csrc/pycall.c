/* pycall.c -- the Python object behind prepare_allreduce().
 *
 * prepare_allreduce() marshals the arguments of one sim_allreduce call
 * once; calling the object it returns makes that C call again.  Through
 * ctypes every such call converts its eight argument objects on the host
 * (measured on MI355X hosts: about a sixth of a small all-reduce's
 * per-call cost); this type holds the arguments as C values and calls the
 * entry point directly.  It adds no logic of its own: every argument is
 * checked by the library, as for any other call.  The entry point's address
 * is taken from the library the package loaded, so a variant build chosen
 * at import time is the one called.
 */
#define PY_SSIZE_T_CLEAN
#include <Python.h>
#include <stddef.h>
#include <stdint.h>

#include "simar.h"

typedef int (*allreduce_fn)(const void* const*, void* const*, int, size_t, int, int, int, void*);

typedef struct {
  PyObject_HEAD
  allreduce_fn fn;
  const void* in[SIM_MAX_RANKS];
  void* out[SIM_MAX_RANKS];
  int p;
  size_t n;
  int dtype, op, algo;
  void* stream;
} PreparedCall;

/* p device pointers (Python ints) from a sequence of exactly p items */
static int read_ptrs(PyObject* seq, int p, void** dst, const char* what) {
  PyObject* fast = PySequence_Fast(seq, what);
  if (!fast) return -1;
  if (PySequence_Fast_GET_SIZE(fast) != p) {
    PyErr_Format(PyExc_ValueError, "%s: expected %d pointers, got %zd", what, p, PySequence_Fast_GET_SIZE(fast));
    Py_DECREF(fast);
    return -1;
  }
  for (int i = 0; i < p; i++) {
    const unsigned long long v = PyLong_AsUnsignedLongLong(PySequence_Fast_GET_ITEM(fast, i));
    if (v == (unsigned long long)-1 && PyErr_Occurred()) {
      Py_DECREF(fast);
      return -1;
    }
    dst[i] = (void*)(uintptr_t)v;
  }
  Py_DECREF(fast);
  return 0;
}

/* PreparedCall(entry_address, in_ptrs, out_ptrs, p, n, dtype, op, algo, stream) */
static int PreparedCall_init(PreparedCall* self, PyObject* args, PyObject* kw) {
  unsigned long long fn = 0, n = 0, stream = 0;
  PyObject *ins = NULL, *outs = NULL;
  int p = 0, dtype = 0, op = 0, algo = 0;
  if (kw && PyDict_GET_SIZE(kw) != 0) {
    PyErr_SetString(PyExc_TypeError, "PreparedCall takes positional arguments only");
    return -1;
  }
  if (!PyArg_ParseTuple(args, "KOOiKiiiK", &fn, &ins, &outs, &p, &n, &dtype, &op, &algo, &stream)) return -1;
  if (!fn) {
    PyErr_SetString(PyExc_ValueError, "null entry point");
    return -1;
  }
  /* the pointer arrays hold SIM_MAX_RANKS entries; other p values are the
     library's to refuse, with at most that many pointers read here */
  if (p < 0 || p > SIM_MAX_RANKS) {
    PyErr_Format(PyExc_ValueError, "p = %d: at most %d ranks", p, SIM_MAX_RANKS);
    return -1;
  }
  memset(self->in, 0, sizeof self->in);
  memset(self->out, 0, sizeof self->out);
  if (read_ptrs(ins, p, (void**)self->in, "in_ptrs") || read_ptrs(outs, p, self->out, "out_ptrs")) return -1;
  self->fn = (allreduce_fn)(uintptr_t)fn;
  self->p = p;
  self->n = (size_t)n;
  self->dtype = dtype;
  self->op = op;
  self->algo = algo;
  self->stream = (void*)(uintptr_t)stream;
  return 0;
}

/* call() -> the status sim_allreduce returned */
static PyObject* PreparedCall_call(PyObject* obj, PyObject* args, PyObject* kw) {
  PreparedCall* self = (PreparedCall*)obj;
  if (PyTuple_GET_SIZE(args) != 0 || (kw && PyDict_GET_SIZE(kw) != 0)) {
    PyErr_SetString(PyExc_TypeError, "a prepared call takes no arguments");
    return NULL;
  }
  if (!self->fn) {
    PyErr_SetString(PyExc_RuntimeError, "PreparedCall was not initialised");
    return NULL;
  }
  return PyLong_FromLong(self->fn(self->in, self->out, self->p, self->n, self->dtype, self->op, self->algo,
                                  self->stream));
}

static PyTypeObject PreparedCallType = {
    PyVarObject_HEAD_INIT(NULL, 0)
    .tp_name = "_pycall.PreparedCall",
    .tp_basicsize = sizeof(PreparedCall),
    .tp_flags = Py_TPFLAGS_DEFAULT,
    .tp_doc = "one sim_allreduce call with its arguments marshalled once; call it to run it",
    .tp_new = PyType_GenericNew,
    .tp_init = (initproc)PreparedCall_init,
    .tp_call = PreparedCall_call,
};

static struct PyModuleDef pycall_module = {
    PyModuleDef_HEAD_INIT, "_pycall", "Prepared C-ABI calls for the Python binding.", -1, NULL,
};

PyMODINIT_FUNC PyInit__pycall(void) {
  if (PyType_Ready(&PreparedCallType) < 0) return NULL;
  PyObject* m = PyModule_Create(&pycall_module);
  if (!m) return NULL;
  Py_INCREF(&PreparedCallType);
  if (PyModule_AddObject(m, "PreparedCall", (PyObject*)&PreparedCallType) < 0) {
    Py_DECREF(&PreparedCallType);
    Py_DECREF(m);
    return NULL;
  }
  return m;
}
