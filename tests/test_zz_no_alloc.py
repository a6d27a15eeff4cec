"""The allocation-free all-reduce (sim_allreduce_noalloc) through the C-ABI
against the existing entry point (sim_allreduce) with the same schedule:
bit-identical outputs (int32/fp32 bit-exact; fp16/bf16 within 2^-8 and, as
both run the same kernels, bit-exact), on two calls in a row, the second
with a smaller input; the size limit of its fixed scratch refused with
nothing enqueued."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

P = 8
# the largest n whose fp32 ring partials fit the fixed array at p = 8:
# 2 p ceil512(ceil(n/p) + 8) * 4 bytes <= SIM_NOALLOC_SCRATCH_BYTES
N_MAX_RING16 = 8_388_544


@pytest.fixture(scope="module", autouse=True)
def lib():
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, 16, 0)
    yield sim


def _inputs(p, n, dtype, seed):
    import synthdata
    if dtype == "int32":
        return synthdata.int_uniform(90 + seed, p, n, -(1 << 20), 1 << 20)
    return synthdata.normal(90 + seed, p, n, dtype, 1.0)


def _run(sim, entry, xs, dtype, op, algo, inplace=False):
    import torch
    from tests.gpu_util import empty_like_poisoned, ptrs, stream, to_device, to_host
    n = xs[0].size
    din = to_device(xs, dtype)
    dout = din if inplace else empty_like_poisoned(n, dtype, len(xs))
    st = entry(ptrs(din), ptrs(dout), len(xs), n, dtype, op, algo, stream())
    assert st == 0, (entry.__name__, algo, dtype, n, st)
    assert sim.sim_check_error(stream()) == 0
    ran = sim.sim_last_algo()
    out = to_host(dout, dtype)
    del din, dout
    torch.cuda.empty_cache()
    return out, ran


@pytest.mark.parametrize("dtype,op", [("bf16", "sum"), ("fp16", "avg"), ("fp32", "sum"), ("int32", "max"),
                                      ("fp32", "prod")])
@pytest.mark.parametrize("algo", ["ring", "allpairs", "oneshot", "auto"])
def test_matches_the_existing_entry_point_on_two_calls(lib, dtype, op, algo):
    from tests.gpu_util import assert_parity
    # the second call is smaller than the first and ragged (n not a multiple of p or of a vector)
    for k, n in enumerate((3 * 65536 + 37, 4099)):
        print(f"noalloc {algo} {dtype} {op} n={n}", flush=True)
        xs = _inputs(P, n, dtype, k)
        got, ran = _run(lib, lib.sim_allreduce_noalloc, xs, dtype, op, algo)
        want, ran2 = _run(lib, lib.sim_allreduce, xs, dtype, op, ran)
        assert ran == ran2 and (algo == "auto" or ran == algo)
        for r in range(P):
            assert_parity(got[r], want[r], dtype, f"noalloc {algo}({ran}) {dtype} {op} n={n} r{r}")


def test_ring16_at_the_limit_then_smaller_and_in_place(lib):
    """The bf16 ring at the largest size the fixed array holds, then a small
    call (the array keeps the first call's partials, which must not leak),
    then in place."""
    from tests.gpu_util import assert_parity
    for n, inplace in ((N_MAX_RING16, False), (1000, False), (65536 + 3, True)):
        print(f"noalloc ring bf16 n={n} inplace={inplace}", flush=True)
        xs = _inputs(P, n, "bf16", 7)
        got, ran = _run(lib, lib.sim_allreduce_noalloc, xs, "bf16", "sum", "ring", inplace)
        want, _ = _run(lib, lib.sim_allreduce, xs, "bf16", "sum", "ring", inplace)
        assert ran == "ring"
        for r in range(P):
            assert_parity(got[r], want[r], "bf16", f"ring16 n={n} r{r}")


def test_limits_and_refusals_enqueue_nothing(lib):
    import torch
    from tests.gpu_util import empty_like_poisoned, ptrs, stream, to_device
    n = N_MAX_RING16 + 1
    xs = [np.zeros(n, dtype=np.uint16) for _ in range(P)]
    din = to_device(xs, "bf16")
    dout = empty_like_poisoned(n, "bf16", P)
    assert lib.sim_allreduce_noalloc(ptrs(din), ptrs(dout), P, n, "bf16", "sum", "ring", stream()) == -5
    for algo in ("oneshot_ll", "ring_fifo", "allpairs_persistent", "tree"):
        assert lib.sim_allreduce_noalloc(ptrs(din), ptrs(dout), P, n, "bf16", "sum", algo, stream()) == -2
    assert lib.sim_allreduce_noalloc(ptrs(din), ptrs(dout), P, n, "bf16", "sum", 99, stream()) == -1
    torch.cuda.synchronize()
    assert all(bool((t == 0x7E5A).all()) for t in dout)
    # no scratch limit for the schedules without partials, or for 32-bit rings
    assert lib.sim_allreduce_noalloc(ptrs(din), ptrs(dout), P, n, "bf16", "sum", "oneshot", stream()) == 0
    assert lib.sim_check_error(stream()) == 0
    assert all(bool((t == 0).all()) for t in dout)
    del din, dout
    torch.cuda.empty_cache()
