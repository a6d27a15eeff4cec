"""Parity at the five workloads' real sizes, in the launch configuration
bench.py times (library defaults).

  1  all-reduce sum, p=4, 4096 int32 per rank in [-1000, 1000], every
     schedule (ring = 4 chunks, 6 steps); plus the 2-rank worked example
  2  all-reduce sum, p=8, fp32 N(0,1), 32 MiB per rank: ring, all-pairs,
     one-shot -- full comparison with the schedule-ordered oracle
  3  all-reduce sum, p=8, bf16 N(0,1)*0.02, 8192 x {1,16,256,4096} tokens:
     every legal schedule and the selector's pick -- full comparison
  4  all-reduce sum, p=8, fp16 N(0,1), 1 KiB .. 1 MiB per rank: LL packet
     path vs plain one-shot -- full comparison, and LL == one-shot bit for bit
  5  p=8, 256 MiB per rank: all-reduce prod/min/max/avg fp32 in [0.5, 2] and
     sum/min/max int32 in [-2^20, 2^20] -- every element of every schedule
     against the oracle's full run of that schedule, every rank identical,
     the exact ops also against the plain definition; reduce-scatter and
     all-gather (full comparison)
"""
import numpy as np
import pytest

import synthdata

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, 16, 0)
    yield sim


def _run(xs, dtype, op, algo):
    from tests.gpu_util import run_allreduce
    return run_allreduce(xs, dtype, op, algo)


def test_workload1_int32_p4(orc):
    from tests.gpu_util import assert_parity
    xs = synthdata.workload_inputs(1, 4, 4096, "int32")
    for algo in ("ring", "allpairs", "oneshot", "oneshot_ll", "auto"):
        got = _run(xs, "int32", "sum", algo)
        import all_reduce_reduction_amd as sim
        ran = sim.sim_last_algo()
        want, steps = orc.allreduce(xs, "int32", "sum", ran)
        if ran == "ring":
            assert steps == 6
        exact = orc.definition(xs, "int32", "sum")
        for r in range(4):
            assert_parity(got[r], want[r], "int32", f"w1 {algo} r{r}")
            assert_parity(got[r], exact, "int32", f"w1 {algo} r{r} vs definition")


def test_workload2_fp32_32MiB(orc):
    from tests.gpu_util import assert_parity
    n = 8_388_608
    xs = synthdata.workload_inputs(2, 8, n, "fp32")
    outs = {}
    for algo in ("ring", "allpairs", "oneshot", "ring_fifo", "allpairs_persistent"):
        print(f"workload 2: {algo}", flush=True)
        got = _run(xs, "fp32", "sum", algo)
        want, steps = orc.allreduce(xs, "fp32", "sum", algo)
        assert steps == (14 if algo in ("ring", "ring_fifo") else 2)
        for r in range(8):
            assert_parity(got[r], want[r], "fp32", f"w2 {algo} r{r}")
        outs[algo] = got[0]
    # one-shot and all-pairs share their order; the ring's differs
    assert (outs["oneshot"].view(np.uint32) == outs["allpairs"].view(np.uint32)).all()
    assert (outs["allpairs_persistent"].view(np.uint32) == outs["allpairs"].view(np.uint32)).all()
    assert (outs["ring"].view(np.uint32) != outs["oneshot"].view(np.uint32)).any()


@pytest.mark.parametrize("tokens", [1, 16, 256, 4096])
def test_workload3_bf16_tp(orc, tokens):
    import all_reduce_reduction_amd as sim
    from tests.gpu_util import assert_parity
    n = 8192 * tokens
    xs = synthdata.workload_inputs(3, 8, n, "bf16")
    algos = ["ring", "allpairs", "oneshot", "ring_fifo", "allpairs_persistent", "auto"]
    if n * 2 <= sim.LL_MAX_BYTES_PER_RANK:
        algos.append("oneshot_ll")
    for algo in algos:
        print(f"workload 3: T={tokens} {algo}", flush=True)
        got = _run(xs, "bf16", "sum", algo)
        ran = sim.sim_last_algo()
        want, _ = orc.allreduce(xs, "bf16", "sum", ran)
        for r in range(8):
            assert_parity(got[r], want[r], "bf16", f"w3 T={tokens} {algo}({ran}) r{r}")


@pytest.mark.parametrize("kib", [1 << k for k in range(11)])
def test_workload4_fp16_ll_vs_oneshot(orc, kib):
    from tests.gpu_util import assert_parity
    n = kib * 1024 // 2
    xs = synthdata.workload_inputs(4, 8, n, "fp16")
    want, _ = orc.allreduce(xs, "fp16", "sum", "oneshot")
    got_ll = _run(xs, "fp16", "sum", "oneshot_ll")
    got_os = _run(xs, "fp16", "sum", "oneshot")
    for r in range(8):
        assert_parity(got_ll[r], want[r], "fp16", f"w4 {kib}KiB LL r{r}")
        assert (got_ll[r] == got_os[r]).all()


@pytest.mark.parametrize("dtype,ops", [("fp32", ("prod", "min", "max", "avg")), ("int32", ("sum", "min", "max"))])
def test_workload5_allreduce_256MiB(orc, dtype, ops):
    """Every one of the 67,108,864 elements, for every op and schedule: the
    device checks that all ranks hold the same bits, then rank 0 is compared
    in full with rank 0 of the oracle's own run of the schedule that ran."""
    import torch
    import all_reduce_reduction_amd as sim
    from tests.gpu_util import assert_parity, bits, empty_like_poisoned, ptrs, stream, to_device
    n = 67_108_864
    p = 8
    xs = synthdata.workload_inputs(5, p, n, dtype)
    din = to_device(xs, dtype)
    dout = empty_like_poisoned(n, dtype, p)
    for op in ops:
        want_by_algo = {}
        full = orc.definition(xs, dtype, op) if (op in ("min", "max") or dtype == "int32") else None
        for algo in ("auto", "ring", "ring_fifo", "allpairs_persistent"):
            print(f"workload 5: {dtype} {op} {algo}", flush=True)
            for t in dout:                                 # re-poison: every call must write everything
                t.fill_(float("nan") if dtype == "fp32" else -0x5A5A5A5B)
            st = sim.sim_allreduce(ptrs(din), ptrs(dout), p, n, dtype, op, algo, stream())
            assert st == 0
            assert sim.sim_check_error(stream()) == 0
            ran = sim.sim_last_algo()
            for r in range(1, p):                          # every rank identical, in full
                assert torch.equal(dout[r].view(torch.int32), dout[0].view(torch.int32)), (op, algo, r)
            if ran not in want_by_algo:
                ys, _ = orc.allreduce(xs, dtype, op, ran)
                want_by_algo[ran] = ys[0]
                del ys
            g0 = dout[0].cpu().numpy()
            assert_parity(g0, want_by_algo[ran], dtype, f"w5 {dtype} {op} {ran} (all elements)")
            if full is not None:                           # exact ops: also the plain definition
                assert (bits(g0) == bits(full)).all(), (op, algo)
            del g0
        del want_by_algo
    del din, dout
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["fp32", "int32"])
def test_workload5_rs_ag_256MiB(orc, dtype):
    import torch
    import all_reduce_reduction_amd as sim
    from tests.gpu_util import assert_parity, empty_like_poisoned, ptrs, stream, to_device, to_host
    p, n = 8, 67_108_864
    n_out = n // p
    xs = synthdata.workload_inputs(5, p, n, dtype)
    din = to_device(xs, dtype)
    for algo in ("allpairs", "ring"):
        for op in (("sum", "max") if dtype == "int32" else ("avg", "min")):
            print(f"workload 5: reduce-scatter {dtype} {op} {algo}", flush=True)
            dout = empty_like_poisoned(n_out, dtype, p)
            assert sim.sim_reduce_scatter(ptrs(din), ptrs(dout), p, n_out, dtype, op, algo, stream()) == 0
            assert sim.sim_check_error(stream()) == 0
            got = to_host(dout, dtype)
            want, _ = orc.reduce_scatter(xs, dtype, op, algo)
            for r in range(p):
                assert_parity(got[r], want[r], dtype, f"RS {algo} {op} r{r}")
            del dout
    # all-gather of 32 MiB per rank into 256 MiB per rank
    small = [x[:n_out].copy() for x in xs]
    dsm = to_device(small, dtype)
    for algo in ("allpairs", "ring"):
        print(f"workload 5: all-gather {dtype} {algo}", flush=True)
        dout = empty_like_poisoned(n, dtype, p)
        assert sim.sim_all_gather(ptrs(dsm), ptrs(dout), p, n_out, dtype, algo, stream()) == 0
        got = to_host(dout, dtype)
        want, _ = orc.all_gather(small, dtype, algo)
        for r in range(p):
            assert (got[r] == want[r]).all(), (algo, r)
        del dout
    torch.cuda.empty_cache()
