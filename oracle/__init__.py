"""CPU oracle for the simulated all-reduce -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's
``cpu_baseline`` leg import this package.  The product library
(``all_reduce_reduction_amd``) never imports, links or calls it, and it shares
no code with the HIP path.  The arithmetic lives in ``oracle.c`` (plain C,
gcc -O2 -ffp-contract=off); this module only builds it and marshals numpy
arrays through ctypes.

What it computes follows the pages (see the header of ``oracle.c``):
  * the all-reduce contract and worked example -- "Inside NCCL all-reduce",
    section "What all-reduce promises";
  * the ring schedule -- same page, section "The ring, exactly as the kernel
    runs it" (3-GPU state table, runRing sequence);
  * the all-pairs schedule -- "MSCCL, in depth ...", section "Writing an
    algorithm in MSCCLang"; one-shot/LL share its fold order ("MSCCL++:
    Rethinking GPU Communication Abstractions for AI Inference", section
    "The Collective Algorithm Library", 1PA/2PA);
  * the double binary tree -- "Inside NCCL all-reduce", section "The double
    binary tree"; 2PH -- the MSCCL++ page, same section, item 4; the k-ary
    recursive exchange -- the NVSHMEM analysis, Fig. 7.

Every function here is pinned by ``tests/test_oracle_*.py`` against printed
values, closed forms, brute force and library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import List, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBPATH = os.path.join(_HERE, "liboracle.so")

DTYPES = {"int32": 0, "fp32": 1, "fp16": 2, "bf16": 3}
OPS = {"sum": 0, "prod": 1, "min": 2, "max": 3, "avg": 4}
ALGOS = {"ring": 1, "allpairs": 2, "oneshot": 3, "oneshot_ll": 4, "ring_fifo": 5,
         "tree": 6, "rexch": 7, "hier": 8, "hier_large": 9, "allpairs_persistent": 10}
TOPO_ALGOS = ("tree", "rexch", "hier", "hier_large")
STORAGE = {"int32": np.int32, "fp32": np.float32, "fp16": np.uint16, "bf16": np.uint16}

CFLAGS = ["-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
          "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(source: str = SOURCE, out: str = LIBPATH) -> str:
    """Compile the oracle with gcc (never hipcc)."""
    subprocess.check_call(["gcc", *CFLAGS, "-o", out, source])
    return out


class Oracle:
    """ctypes wrapper around one compiled copy of oracle.c."""

    def __init__(self, libpath: str = LIBPATH):
        if not os.path.exists(libpath):
            build(out=libpath)
        self.lib = lib = ctypes.CDLL(libpath)
        pp = ctypes.POINTER(ctypes.c_void_p)
        i64 = ctypes.c_int64
        lib.oracle_allreduce.argtypes = [pp, pp, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_definition.argtypes = [pp, pp, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int]
        lib.oracle_reduce_scatter.argtypes = [pp, pp, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_all_gather.argtypes = [pp, pp, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int]
        lib.oracle_allreduce_at.argtypes = [pp, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p, i64, ctypes.c_void_p]
        lib.oracle_allreduce_topo.argtypes = [pp, pp, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int,
                                              ctypes.c_int, ctypes.c_int, ctypes.c_int]
        lib.oracle_allreduce_at_topo.argtypes = [pp, ctypes.c_int, i64, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                                 ctypes.c_void_p, i64, ctypes.c_void_p]
        lib.oracle_tree_parent.argtypes = [ctypes.c_int] * 4
        lib.oracle_tree_parent.restype = ctypes.c_int
        for name in ("allreduce", "definition", "reduce_scatter", "all_gather", "allreduce_at",
                     "allreduce_topo", "allreduce_at_topo"):
            getattr(lib, "oracle_" + name).restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = ctypes.c_int
        lib.oracle_chunk_lo.argtypes = [i64, ctypes.c_int, ctypes.c_int]
        lib.oracle_chunk_lo.restype = i64
        for name in ("bf16", "f16"):
            getattr(lib, f"oracle_f32_to_{name}_array").argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64]
            getattr(lib, f"oracle_{name}_to_f32_array").argtypes = [ctypes.c_void_p, ctypes.c_void_p, i64]

    # -- helpers -------------------------------------------------------
    @staticmethod
    def _ptrs(arrs: Sequence[np.ndarray]):
        for a in arrs:
            assert a.flags["C_CONTIGUOUS"], "oracle needs contiguous arrays"
        return (ctypes.c_void_p * len(arrs))(*[a.ctypes.data for a in arrs])

    @staticmethod
    def _check_inputs(xs: Sequence[np.ndarray], dtype: str) -> int:
        st = STORAGE[dtype]
        n = xs[0].size
        for x in xs:
            assert x.dtype == st and x.size == n and x.ndim == 1, (x.dtype, st, x.size, n)
        return n

    # -- collectives ---------------------------------------------------
    def allreduce(self, xs: Sequence[np.ndarray], dtype: str, op: str, algo: str,
                  inplace: bool = False, ranks_per_node: int = 1, radix: int = 2
                  ) -> Tuple[List[np.ndarray], int]:
        """Run the algorithm's schedule; returns (p outputs, steps or rounds).
        ranks_per_node and radix are the topology of the tree, recursive
        exchange and 2PH schedules (ignored by the others)."""
        n = self._check_inputs(xs, dtype)
        ys = list(xs) if inplace else [np.empty_like(x) for x in xs]
        steps = self.lib.oracle_allreduce_topo(self._ptrs(xs), self._ptrs(ys), len(xs), n,
                                               DTYPES[dtype], OPS[op], ALGOS[algo], ranks_per_node, radix)
        if steps < 0:
            raise ValueError("oracle_allreduce rejected its arguments")
        return ys, steps

    def definition(self, xs: Sequence[np.ndarray], dtype: str, op: str) -> np.ndarray:
        """Left fold in rank order 0..p-1 (the plain definition)."""
        n = self._check_inputs(xs, dtype)
        ys = [np.empty_like(xs[0]) for _ in xs]
        if self.lib.oracle_definition(self._ptrs(xs), self._ptrs(ys), len(xs), n, DTYPES[dtype], OPS[op]) < 0:
            raise ValueError("oracle_definition rejected its arguments")
        return ys[0]

    def reduce_scatter(self, xs: Sequence[np.ndarray], dtype: str, op: str, algo: str
                       ) -> Tuple[List[np.ndarray], int]:
        n = self._check_inputs(xs, dtype)
        p = len(xs)
        assert n % p == 0
        ys = [np.empty(n // p, dtype=STORAGE[dtype]) for _ in xs]
        steps = self.lib.oracle_reduce_scatter(self._ptrs(xs), self._ptrs(ys), p, n // p,
                                               DTYPES[dtype], OPS[op], ALGOS[algo])
        if steps < 0:
            raise ValueError("oracle_reduce_scatter rejected its arguments")
        return ys, steps

    def all_gather(self, xs: Sequence[np.ndarray], dtype: str, algo: str) -> Tuple[List[np.ndarray], int]:
        n = self._check_inputs(xs, dtype)
        p = len(xs)
        ys = [np.empty(n * p, dtype=STORAGE[dtype]) for _ in xs]
        steps = self.lib.oracle_all_gather(self._ptrs(xs), self._ptrs(ys), p, n, DTYPES[dtype], ALGOS[algo])
        if steps < 0:
            raise ValueError("oracle_all_gather rejected its arguments")
        return ys, steps

    def allreduce_at(self, xs: Sequence[np.ndarray], dtype: str, op: str, algo: str,
                     idx: np.ndarray, ranks_per_node: int = 1, radix: int = 2) -> np.ndarray:
        """The result at the given element indices (identical on every rank)."""
        n = self._check_inputs(xs, dtype)
        idx = np.ascontiguousarray(idx, dtype=np.int64)
        out = np.empty(idx.size, dtype=STORAGE[dtype])
        rc = self.lib.oracle_allreduce_at_topo(self._ptrs(xs), len(xs), n, DTYPES[dtype], OPS[op],
                                               ALGOS[algo], ranks_per_node, radix,
                                               idx.ctypes.data, idx.size, out.ctypes.data)
        if rc < 0:
            raise ValueError("oracle_allreduce_at rejected its arguments")
        return out

    # -- codecs --------------------------------------------------------
    def f32_to_bf16(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        y = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_f32_to_bf16_array(x.ctypes.data, y.ctypes.data, x.size)
        return y

    def f32_to_f16(self, x: np.ndarray) -> np.ndarray:
        x = np.ascontiguousarray(x, dtype=np.float32)
        y = np.empty(x.shape, dtype=np.uint16)
        self.lib.oracle_f32_to_f16_array(x.ctypes.data, y.ctypes.data, x.size)
        return y

    def bf16_to_f32(self, h: np.ndarray) -> np.ndarray:
        h = np.ascontiguousarray(h, dtype=np.uint16)
        y = np.empty(h.shape, dtype=np.float32)
        self.lib.oracle_bf16_to_f32_array(h.ctypes.data, y.ctypes.data, h.size)
        return y

    def f16_to_f32(self, h: np.ndarray) -> np.ndarray:
        h = np.ascontiguousarray(h, dtype=np.uint16)
        y = np.empty(h.shape, dtype=np.float32)
        self.lib.oracle_f16_to_f32_array(h.ctypes.data, y.ctypes.data, h.size)
        return y

    def tree_parent(self, tree: int, p: int, ranks_per_node: int, rank: int) -> int:
        """Parent of `rank` in tree 0 or 1 of the double binary tree (-1: root)."""
        v = self.lib.oracle_tree_parent(tree, p, ranks_per_node, rank)
        if v < -1:
            raise ValueError("oracle_tree_parent rejected its arguments")
        return v

    def num_threads(self) -> int:
        return self.lib.oracle_num_threads()

    def set_num_threads(self, n: int) -> int:
        """Threads for later calls (timing only); returns the count in effect."""
        return self.lib.oracle_set_num_threads(n)

    def chunk_lo(self, n: int, p: int, c: int) -> int:
        return self.lib.oracle_chunk_lo(n, p, c)


_default = None


def get() -> Oracle:
    """The oracle built from this directory's oracle.c."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default
