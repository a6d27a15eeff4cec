"""Python binding of libsimar.so (argument marshalling only).

Every function named ``sim_*`` here calls the C function of the same name in
``include/simar.h`` through ctypes and raises :class:`SimError` on a
non-zero status.  All work of the all-reduce path runs in the HIP kernels of
the library; there is no Python or CPU fallback -- if the library is missing
the import fails.

The ``allreduce`` / ``reduce_scatter`` / ``all_gather`` helpers take lists of
torch device tensors (PyTorch is used for device memory and streams only)
and pass their pointers and the current HIP stream to the library.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

try:  # load torch's HIP runtime first so the library and torch share it
    import torch  # noqa: F401
except Exception:  # pragma: no cover - the host-only tests work without torch
    torch = None

_HERE = os.path.dirname(os.path.abspath(__file__))
# SIMAR_LIB selects another build of the same library (e.g. a variant
# compiled with different cache-policy flags); the default is the in-tree one.
LIBPATH = os.environ.get("SIMAR_LIB") or os.path.join(_HERE, "libsimar.so")

SIM_OK = 0
STATUS = {0: "SIM_OK", -1: "SIM_ERR_INVALID_ARG", -2: "SIM_ERR_UNSUPPORTED", -3: "SIM_ERR_ALIGN",
          -4: "SIM_ERR_ALIAS", -5: "SIM_ERR_NOMEM", -6: "SIM_ERR_HIP", -7: "SIM_ERR_TIMEOUT",
          -8: "SIM_ERR_VERIFY", -9: "SIM_ERR_NOT_INIT"}
STATUS_CODE = {v: k for k, v in STATUS.items()}
DTYPES = {"int32": 0, "fp32": 1, "fp16": 2, "bf16": 3}
OPS = {"sum": 0, "prod": 1, "min": 2, "max": 3, "avg": 4}
ALGOS = {"auto": 0, "ring": 1, "allpairs": 2, "oneshot": 3, "oneshot_ll": 4, "ring_fifo": 5,
         "tree": 6, "rexch": 7, "hier": 8, "hier_large": 9, "allpairs_persistent": 10}
TOPOLOGY_ALGOS = ("tree", "rexch", "hier", "hier_large")
ALGO_NAMES = {v: k for k, v in ALGOS.items()}
ESIZE = {"int32": 4, "fp32": 4, "fp16": 2, "bf16": 2}
XFER_KINDS = {0: "REDUCE", 1: "REDUCE_POST", 2: "COPY", 3: "GATHER_REDUCE", 4: "FANOUT", 5: "ONESHOT",
              6: "GATHER", 7: "GATHER_POST", 8: "EXCH", 9: "EXCH_POST", 10: "MCAST"}
CONFIG = {"ranks_per_node": 0, "radix": 1, "max_workgroups": 2}
DEBUG = {"epoch": 0, "spin_limit": 1, "ll_wait_skew": 2, "fill_ll": 3, "log": 4, "workgroups": 5,
         "unroll": 6, "fifo_channels": 7, "fifo_slots": 8, "fifo_withhold": 9, "fifo_vecs": 10,
         "ptr_table": 11, "ptr_sets": 12, "ring_ll_max": 13,
              "phased": 14, "phased_min": 15, "phased_expired": 16, "phased_last": 17,
         "phased_layout": 18, "phased_whole_last": 19}
MAX_RANKS = 16
LL_MAX_BYTES_PER_RANK = 1 << 20


class SimError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIBPATH):
        raise ImportError(f"{LIBPATH} is not built; run __graft_entry__.build() "
                          "(hipcc --offload-arch=gfx950) first")
    lib = ctypes.CDLL(LIBPATH)
    vp, sz, i, d = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_double
    pp = ctypes.POINTER(ctypes.c_void_p)
    sig = {
        "sim_init": ([i, i, sz], i),
        "sim_finalize": ([], i),
        "sim_allreduce": ([pp, pp, i, sz, i, i, i, vp], i),
        "sim_allreduce_noalloc": ([pp, pp, i, sz, i, i, i, vp], i),
        "sim_reduce_scatter": ([pp, pp, i, sz, i, i, i, vp], i),
        "sim_all_gather": ([pp, pp, i, sz, i, i, vp], i),
        "sim_select": ([i, sz, i, i, ctypes.POINTER(i), ctypes.POINTER(d)], i),
        "sim_last_algo": ([], i),
        "sim_model_load": ([ctypes.c_char_p], i),
        "sim_model_predict": ([i, i, i, d, ctypes.POINTER(d)], i),
        "sim_model_set": ([i, d, d, d, d], i),
        "sim_model_reset": ([], i),
        "sim_model_set_workgroup_rate": ([i, d], i),
        "sim_model_set_host_overlap": ([i, d], i),
        "sim_check_error": ([vp], i),
        "sim_copy_streams": ([pp, pp, i, sz, i, vp], i),
        "sim_config_set": ([i, i], i),
        "sim_config_get": ([i, ctypes.POINTER(i)], i),
        "sim_tree_info": ([i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(i)], i),
        "sim_schedule_info": ([i, i, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.POINTER(i)], i),
        "sim_schedule_xfers": ([i, i, i, ctypes.POINTER(i), i, ctypes.POINTER(i)], i),
        "sim_schedule_state": ([i, i, i, ctypes.POINTER(ctypes.c_uint32)], i),
        "sim_verify_schedule": ([i, i, ctypes.c_char_p, sz], i),
        "sim_verify_custom": ([i, i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i), ctypes.c_char_p, sz], i),
        "sim_debug_set": ([i, ctypes.c_uint64], i),
        "sim_debug_get": ([i, ctypes.POINTER(ctypes.c_uint64)], i),
        "sim_debug_set_epoch": ([ctypes.c_uint32], i),
        "sim_status_string": ([i], ctypes.c_char_p),
        "sim_version": ([], i),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    return lib


lib = _load()

try:  # the prepared-call object (csrc/pycall.c), built beside the library
    from . import _pycall
except ImportError:  # not built: prepare_allreduce falls back to a ctypes call of the same entry point
    _pycall = None


def _check(status: int, what: str) -> int:
    if status != SIM_OK:
        raise SimError(status, what)
    return status


def _ptr_array(ptrs: Sequence[int]):
    return (ctypes.c_void_p * len(ptrs))(*[int(p) for p in ptrs])


def _code(table, v, what):
    if isinstance(v, str):
        if v not in table:
            raise ValueError(f"unknown {what} {v!r}")
        return table[v]
    return int(v)


# The model fitted by calibrate.py on MI355X; sim_init loads it unless the
# SIM_CALIB environment variable names another file (which the C library
# then loads itself).
CALIBRATION = os.path.join(_HERE, "calib", "mi355x.json")


# ---- the C functions, one to one ------------------------------------------------
def sim_init(device: int = 0, p_max: int = MAX_RANKS, max_bytes_per_rank: int = 0) -> None:
    _check(lib.sim_init(device, p_max, max_bytes_per_rank), "sim_init")
    if not os.environ.get("SIM_CALIB") and os.path.exists(CALIBRATION):
        sim_model_load(CALIBRATION)


def sim_finalize() -> None:
    _check(lib.sim_finalize(), "sim_finalize")


def sim_allreduce(in_ptrs, out_ptrs, p, n, dtype, op, algo, stream=0) -> int:
    return lib.sim_allreduce(_ptr_array(in_ptrs), _ptr_array(out_ptrs), p, n, _code(DTYPES, dtype, "dtype"),
                             _code(OPS, op, "op"), _code(ALGOS, algo, "algo"), stream or None)


def sim_allreduce_noalloc(in_ptrs, out_ptrs, p, n, dtype, op, algo, stream=0) -> int:
    return lib.sim_allreduce_noalloc(_ptr_array(in_ptrs), _ptr_array(out_ptrs), p, n,
                                     _code(DTYPES, dtype, "dtype"), _code(OPS, op, "op"),
                                     _code(ALGOS, algo, "algo"), stream or None)


NOALLOC_SCRATCH_BYTES = 64 << 20


def prepare_allreduce(in_ptrs, out_ptrs, p, n, dtype, op, algo, stream=0):
    """The same call as sim_allreduce with its arguments marshalled once:
    returns a function of no arguments that calls the C entry point and
    returns its status (for loops that repeat one call, where Python-side
    marshalling would otherwise dominate a few-microsecond call)."""
    f = lib["sim_allreduce"]
    f.restype = ctypes.c_int
    dt, o, a = _code(DTYPES, dtype, "dtype"), _code(OPS, op, "op"), _code(ALGOS, algo, "algo")
    if _pycall is not None:
        # the arguments held as C values and the entry point called directly
        return _pycall.PreparedCall(ctypes.cast(f, ctypes.c_void_p).value, [int(q) for q in in_ptrs],
                                    [int(q) for q in out_ptrs], p, n, dt, o, a, int(stream or 0))
    # a bare function pointer (no argtypes) called with ready-made ctypes
    # objects: no per-call argument conversion
    args = (_ptr_array(in_ptrs), _ptr_array(out_ptrs), ctypes.c_int(p), ctypes.c_size_t(n),
            ctypes.c_int(dt), ctypes.c_int(o), ctypes.c_int(a), ctypes.c_void_p(stream or None))
    return lambda: f(*args)


def sim_reduce_scatter(in_ptrs, out_ptrs, p, n_out_per_rank, dtype, op, algo, stream=0) -> int:
    return lib.sim_reduce_scatter(_ptr_array(in_ptrs), _ptr_array(out_ptrs), p, n_out_per_rank,
                                  _code(DTYPES, dtype, "dtype"), _code(OPS, op, "op"),
                                  _code(ALGOS, algo, "algo"), stream or None)


def sim_all_gather(in_ptrs, out_ptrs, p, n_in_per_rank, dtype, algo, stream=0) -> int:
    return lib.sim_all_gather(_ptr_array(in_ptrs), _ptr_array(out_ptrs), p, n_in_per_rank,
                              _code(DTYPES, dtype, "dtype"), _code(ALGOS, algo, "algo"), stream or None)


def sim_select(p: int, n: int, dtype, op="sum"):
    a, us = ctypes.c_int(0), ctypes.c_double(0)
    _check(lib.sim_select(p, n, _code(DTYPES, dtype, "dtype"), _code(OPS, op, "op"), ctypes.byref(a),
                          ctypes.byref(us)), "sim_select")
    return ALGO_NAMES[a.value], us.value


def sim_last_algo() -> Optional[str]:
    return ALGO_NAMES.get(lib.sim_last_algo())


def sim_model_load(path: str) -> None:
    _check(lib.sim_model_load(path.encode()), f"sim_model_load({path})")


def sim_model_predict(algo, p: int, dtype, bytes_per_rank: float) -> float:
    us = ctypes.c_double(0)
    _check(lib.sim_model_predict(_code(ALGOS, algo, "algo"), p, _code(DTYPES, dtype, "dtype"),
                                 float(bytes_per_rank), ctypes.byref(us)), "sim_model_predict")
    return us.value


def sim_model_set(algo, alpha_us: float, steps: float, bytes_factor: float, gbps: float) -> None:
    _check(lib.sim_model_set(_code(ALGOS, algo, "algo"), alpha_us, steps, bytes_factor, gbps), "sim_model_set")


def sim_model_set_workgroup_rate(algo, gbps_per_workgroup: float) -> None:
    _check(lib.sim_model_set_workgroup_rate(_code(ALGOS, algo, "algo"), float(gbps_per_workgroup)),
           "sim_model_set_workgroup_rate")


def sim_model_set_host_overlap(algo, host_us_per_launch: float) -> None:
    _check(lib.sim_model_set_host_overlap(_code(ALGOS, algo, "algo"), float(host_us_per_launch)),
           "sim_model_set_host_overlap")


def sim_model_reset() -> None:
    _check(lib.sim_model_reset(), "sim_model_reset")


def sim_check_error(stream=0) -> int:
    """Returns the status (SIM_OK or SIM_ERR_TIMEOUT) without raising."""
    return lib.sim_check_error(stream or None)


def sim_copy_streams(src_ptrs, dst_ptrs, k: int, nbytes: int, workgroups: int = 0, stream=0) -> int:
    return lib.sim_copy_streams(_ptr_array(src_ptrs), _ptr_array(dst_ptrs), k, nbytes, workgroups,
                                stream or None)


def sim_config_set(key, value: int) -> None:
    _check(lib.sim_config_set(_code(CONFIG, key, "config key"), int(value)), "sim_config_set")


def sim_config_get(key) -> int:
    v = ctypes.c_int(0)
    _check(lib.sim_config_get(_code(CONFIG, key, "config key"), ctypes.byref(v)), "sim_config_get")
    return v.value


def sim_tree_info(tree: int, p: int, ranks_per_node: int, rank: int):
    """(parent, [children ascending]) of `rank` in tree 0 or 1."""
    par, nch = ctypes.c_int(0), ctypes.c_int(0)
    ch = (ctypes.c_int * 3)()
    _check(lib.sim_tree_info(tree, p, ranks_per_node, rank, ctypes.byref(par), ch, ctypes.byref(nch)),
           "sim_tree_info")
    return par.value, list(ch[:nch.value])


def sim_schedule_info(algo, p: int):
    """(steps, transfers, chunks) of the lowered all-reduce schedule."""
    ns, nx, nc = ctypes.c_int(0), ctypes.c_int(0), ctypes.c_int(0)
    _check(lib.sim_schedule_info(_code(ALGOS, algo, "algo"), p, ctypes.byref(ns), ctypes.byref(nx),
                                 ctypes.byref(nc)), "sim_schedule_info")
    return ns.value, nx.value, nc.value


def sim_schedule_xfers(algo, p: int, step: int):
    """The step's transfers as (kind, src, dst, chunk, rank set) tuples."""
    cap = 512
    buf = (ctypes.c_int * (5 * cap))()
    cnt = ctypes.c_int(0)
    _check(lib.sim_schedule_xfers(_code(ALGOS, algo, "algo"), p, step, buf, cap, ctypes.byref(cnt)),
           "sim_schedule_xfers")
    return [tuple(buf[5 * k:5 * k + 5]) for k in range(cnt.value)]


def sim_schedule_state(algo, p: int, after_steps: int):
    """masks[r][c] after `after_steps` steps."""
    nch = sim_schedule_info(algo, p)[2]
    m = (ctypes.c_uint32 * (p * nch))()
    _check(lib.sim_schedule_state(_code(ALGOS, algo, "algo"), p, after_steps, m), "sim_schedule_state")
    return [[m[r * nch + c] for c in range(nch)] for r in range(p)]


def sim_verify_schedule(algo, p: int):
    buf = ctypes.create_string_buffer(1024)
    st = lib.sim_verify_schedule(_code(ALGOS, algo, "algo"), p, buf, 1024)
    return st, buf.value.decode()


def sim_verify_custom(algo, p: int, steps: List[List[tuple]], nchunks: Optional[int] = None,
                      rounds: Optional[int] = None):
    """Check a caller-made all-reduce schedule.  Transfers are 5-tuples
    (kind, src, dst, chunk, rank set); 4-tuples get an empty rank set.
    nchunks defaults to p, rounds to the number of steps."""
    steps = [[tuple(x) + (0,) * (5 - len(x)) for x in s] for s in steps]
    counts = (ctypes.c_int * max(1, len(steps)))(*[len(s) for s in steps])
    flat = [v for s in steps for x in s for v in x]
    xf = (ctypes.c_int * max(1, len(flat)))(*flat)
    buf = ctypes.create_string_buffer(1024)
    st = lib.sim_verify_custom(_code(ALGOS, algo, "algo"), p, p if nchunks is None else nchunks,
                               len(steps) if rounds is None else rounds, len(steps), counts, xf, buf, 1024)
    return st, buf.value.decode()


def sim_debug_set(key, value: int) -> None:
    _check(lib.sim_debug_set(_code(DEBUG, key, "debug key"), int(value) & (2 ** 64 - 1)), "sim_debug_set")


def sim_debug_get(key) -> int:
    v = ctypes.c_uint64(0)
    _check(lib.sim_debug_get(_code(DEBUG, key, "debug key"), ctypes.byref(v)), "sim_debug_get")
    return v.value


def sim_debug_set_epoch(epoch: int) -> None:
    _check(lib.sim_debug_set_epoch(int(epoch) & 0xFFFFFFFF), "sim_debug_set_epoch")


def sim_status_string(status: int) -> str:
    return lib.sim_status_string(status).decode()


def sim_version() -> int:
    return lib.sim_version()


# ---- torch tensor helpers (marshalling only) --------------------------------------
def _dtype_name(t) -> str:
    import torch as _t
    m = {_t.int32: "int32", _t.float32: "fp32", _t.float16: "fp16", _t.bfloat16: "bf16"}
    if t.dtype not in m:
        raise ValueError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _stream(stream) -> int:
    import torch as _t
    s = stream if stream is not None else _t.cuda.current_stream()
    return int(s.cuda_stream)


def _ptrs(ts) -> List[int]:
    out = []
    for t in ts:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("tensors must be contiguous device tensors")
        out.append(t.data_ptr())
    return out


def allreduce(inputs: Sequence, outputs: Optional[Sequence] = None, op="sum", algo="auto", stream=None):
    """All-reduce p same-shaped device tensors (outputs=None: in place)."""
    outputs = list(inputs) if outputs is None else list(outputs)
    dt = _dtype_name(inputs[0])
    st = sim_allreduce(_ptrs(inputs), _ptrs(outputs), len(inputs), inputs[0].numel(), dt, op, algo,
                       _stream(stream))
    _check(st, "sim_allreduce")
    return outputs


def reduce_scatter(inputs: Sequence, outputs: Sequence, op="sum", algo="auto", stream=None):
    dt = _dtype_name(inputs[0])
    st = sim_reduce_scatter(_ptrs(inputs), _ptrs(outputs), len(inputs), outputs[0].numel(), dt, op, algo,
                            _stream(stream))
    _check(st, "sim_reduce_scatter")
    return outputs


def all_gather(inputs: Sequence, outputs: Sequence, algo="auto", stream=None):
    dt = _dtype_name(inputs[0])
    st = sim_all_gather(_ptrs(inputs), _ptrs(outputs), len(inputs), inputs[0].numel(), dt, algo,
                        _stream(stream))
    _check(st, "sim_all_gather")
    return outputs
