"""Seeded synthetic inputs shared by the tests, the oracle checks and the
benchmark.  This module holds no arithmetic of the all-reduce itself: it
only draws per-rank buffers and narrows them to their storage type with
library conversions (numpy's float16 cast, torch's CPU bfloat16 cast; both
round to nearest, ties to even).

Recipe (one numpy PCG64 stream per (workload id, rank[, repetition])):
  int-uniform     rng.integers(lo, hi, n, endpoint=True, dtype=int32)
  normal          rng.standard_normal(n, dtype=float32) * scale
  uniform         rng.uniform(lo, hi, n) as float32
16-bit values are drawn in fp32 and narrowed once, so their bits are fixed
by the seed.  The shapes follow the workloads the pages measure: p ranks on
one node, power-of-two message sizes, contiguous per-rank buffers.
"""
from __future__ import annotations

from typing import List, Optional

import numpy as np

STORAGE = {"int32": np.int32, "fp32": np.float32, "fp16": np.uint16, "bf16": np.uint16}
ESIZE = {"int32": 4, "fp32": 4, "fp16": 2, "bf16": 2}


def rng_for(workload: int, rank: int, rep: Optional[int] = None) -> np.random.Generator:
    key = [workload, rank] if rep is None else [workload, rank, rep]
    return np.random.default_rng(key)


def narrow(x32: np.ndarray, dtype: str) -> np.ndarray:
    """fp32 values -> storage array of the given dtype (uint16 bits for 16-bit)."""
    if dtype == "fp32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "fp16":
        return np.ascontiguousarray(x32.astype(np.float16)).view(np.uint16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def widen(h: np.ndarray, dtype: str) -> np.ndarray:
    """Storage array -> float32 values (library conversions)."""
    if dtype in ("fp32", "int32"):
        return h
    if dtype == "fp16":
        return h.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (h.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(dtype)


def normal(workload: int, p: int, n: int, dtype: str, scale: float = 1.0,
           rep: Optional[int] = None) -> List[np.ndarray]:
    out = []
    for r in range(p):
        x = rng_for(workload, r, rep).standard_normal(n, dtype=np.float32)
        if scale != 1.0:
            x = x * np.float32(scale)
        out.append(narrow(x, dtype))
    return out


def uniform(workload: int, p: int, n: int, lo: float, hi: float, dtype: str = "fp32",
            rep: Optional[int] = None) -> List[np.ndarray]:
    return [narrow(rng_for(workload, r, rep).uniform(lo, hi, n).astype(np.float32), dtype)
            for r in range(p)]


def int_uniform(workload: int, p: int, n: int, lo: int, hi: int,
                rep: Optional[int] = None) -> List[np.ndarray]:
    return [rng_for(workload, r, rep).integers(lo, hi, n, endpoint=True, dtype=np.int32)
            for r in range(p)]


# The five workloads: (id, description) -> generator.  Sizes are per rank.
def workload_inputs(wid: int, p: int, n: int, dtype: str, rep: Optional[int] = None) -> List[np.ndarray]:
    """Inputs of workload `wid` at (p, n, dtype), per the recipe above."""
    if wid == 1:    # int32 sum, uniform in [-1000, 1000]
        return int_uniform(1, p, n, -1000, 1000, rep)
    if wid == 2:    # fp32 N(0,1)
        return normal(2, p, n, dtype, 1.0, rep)
    if wid == 3:    # tensor-parallel activations: N(0,1) * 0.02, bf16
        return normal(3, p, n, dtype, 0.02, rep)
    if wid == 4:    # small messages, N(0,1), fp16
        return normal(4, p, n, dtype, 1.0, rep)
    if wid == 5:    # large-buffer op coverage
        if dtype == "int32":
            return int_uniform(5, p, n, -(1 << 20), 1 << 20, rep)
        return uniform(5, p, n, 0.5, 2.0, dtype, rep)
    raise ValueError(wid)
