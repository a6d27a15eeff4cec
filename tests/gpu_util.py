"""Helpers for the GPU parity tests: move seeded host arrays to device
buffers, call the library through its C-ABI binding, read back, compare
with the oracle."""
from __future__ import annotations

from typing import List, Sequence

import numpy as np
import torch

import all_reduce_reduction_amd as sim

TORCH_STORAGE = {"int32": torch.int32, "fp32": torch.float32, "fp16": torch.int16, "bf16": torch.int16}
NP_STORAGE = {"int32": np.int32, "fp32": np.float32, "fp16": np.uint16, "bf16": np.uint16}


def dev() -> torch.device:
    return torch.device("cuda:0")


def to_device(xs: Sequence[np.ndarray], dtype: str) -> List[torch.Tensor]:
    out = []
    for x in xs:
        a = x.view(np.int16) if dtype in ("fp16", "bf16") else x
        out.append(torch.from_numpy(np.ascontiguousarray(a)).to(dev()))
    return out


def empty_like_poisoned(n: int, dtype: str, count: int) -> List[torch.Tensor]:
    """Output buffers pre-filled with a sentinel so an unwritten element fails."""
    out = []
    for _ in range(count):
        t = torch.empty(max(n, 1), dtype=TORCH_STORAGE[dtype], device=dev())[:n]
        if dtype == "fp32":
            t.fill_(float("nan"))
        elif dtype == "int32":
            t.fill_(-0x5A5A5A5B)
        else:
            t.fill_(0x7E5A)  # a NaN pattern in both fp16 and bf16
        out.append(t)
    return out


def to_host(ts: Sequence[torch.Tensor], dtype: str) -> List[np.ndarray]:
    torch.cuda.synchronize()
    res = []
    for t in ts:
        a = t.cpu().numpy()
        res.append(a.view(np.uint16) if dtype in ("fp16", "bf16") else a)
    return res


def ptrs(ts: Sequence[torch.Tensor]) -> List[int]:
    return [t.data_ptr() for t in ts]


def stream() -> int:
    return int(torch.cuda.current_stream().cuda_stream)


def bits(a: np.ndarray) -> np.ndarray:
    return a.view(np.uint32) if a.dtype.itemsize == 4 else a.view(np.uint16)


def widen16(h: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp16":
        return h.view(np.float16).astype(np.float32)
    return (h.astype(np.uint32) << 16).view(np.float32)


def assert_parity(got: np.ndarray, want: np.ndarray, dtype: str, what: str = "") -> None:
    """int32/fp32: bit-exact.  fp16/bf16: the 2^-8 relative bar (zero must
    stay a signed zero, any NaN fails), and bit-exact as the schedule-order
    arithmetic is the same on both sides."""
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if dtype in ("fp16", "bf16"):
        g, w = widen16(got, dtype), widen16(want, dtype)
        assert not np.isnan(g).any(), f"{what}: NaN in output"
        inf = np.isinf(w)
        assert (g[inf] == w[inf]).all(), f"{what}: infinities differ"
        nz = (w != 0) & ~inf
        rel = np.abs(g[nz] - w[nz]) / np.abs(w[nz])
        assert rel.size == 0 or rel.max() <= 2.0 ** -8, f"{what}: max rel err {rel.max()}"
        assert (g[w == 0] == 0).all(), f"{what}: nonzero where the oracle has zero"
    diff = np.nonzero(bits(got) != bits(want))[0]
    assert diff.size == 0, f"{what}: {diff.size} elements differ, first at {diff[:5]}: got {got[diff[:5]]} want {want[diff[:5]]}"


def run_allreduce(xs: Sequence[np.ndarray], dtype: str, op: str, algo: str, inplace: bool = False,
                  fill=None):
    """The library's all-reduce of xs (host arrays, storage format) on the
    device; outputs start as the poison pattern, or as `fill` (a storage
    value) when given."""
    n = xs[0].size
    p = len(xs)
    din = to_device(xs, dtype)
    if inplace:
        dout = din
    elif fill is not None:
        dout = [torch.full((max(n, 1),), fill, dtype=TORCH_STORAGE[dtype], device=dev())[:n] for _ in range(p)]
    else:
        dout = empty_like_poisoned(n, dtype, p)
    st = sim.sim_allreduce(ptrs(din), ptrs(dout), p, n, dtype, op, algo, stream())
    if st != 0:
        raise sim.SimError(st, f"sim_allreduce({algo}, p={p}, n={n}, {dtype}, {op})")
    err = sim.sim_check_error(stream())
    assert err == 0, f"device error {err}"
    return to_host(dout, dtype)
