"""Launch configurations: every bulk kernel walks its transfer with a
grid-stride loop, so results must not depend on how many workgroups run
it.  Checked against the oracle under a workgroup budget (T-CCL's
restricted mode), under forced totals far below the exact cover, and with a
calibration launch table loaded, for every schedule and both standalone
collectives, on ragged sizes."""
import json

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

ALGOS = [("oneshot", 1), ("allpairs", 1), ("ring", 1), ("ring_fifo", 1), ("allpairs_persistent", 1),
         ("oneshot_ll", 1), ("tree", 2),
         ("rexch", 1), ("hier", 4), ("hier_large", 2)]


@pytest.fixture(scope="module", autouse=True)
def lib():
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, 8, 0)
    yield sim
    sim.sim_config_set("max_workgroups", 0)
    sim.sim_config_set("ranks_per_node", 1)
    sim.sim_debug_set("workgroups", 0)
    sim.sim_debug_set("unroll", 0)
    sim.sim_model_load(sim.CALIBRATION)


def _inputs(p, n, dtype, seed, orc):
    import synthdata
    if dtype == "int32":
        return synthdata.int_uniform(seed, p, n, -1000, 1000)
    return synthdata.normal(seed, p, n, dtype)


def _check_all(orc, sim, label):
    from tests.gpu_util import assert_parity, run_allreduce
    p = 8
    for dtype, n in (("bf16", 8 * 8192 * 3 + 77), ("int32", 8 * 4096 * 2 + 5)):
        xs = _inputs(p, n, dtype, 70, orc)
        for algo, g in ALGOS:
            sim.sim_config_set("ranks_per_node", g)
            want, _ = orc.allreduce(xs, dtype, "sum", algo, ranks_per_node=g)
            print(f"{label} {algo} {dtype} n={n}", flush=True)
            got = run_allreduce(xs, dtype, "sum", algo)
            for r in range(p):
                assert_parity(got[r], want[r], dtype, f"{label} {algo} r{r}")
    sim.sim_config_set("ranks_per_node", 1)


def _check_rs_ag(orc, sim, label):
    import torch
    from tests.gpu_util import assert_parity, empty_like_poisoned, ptrs, stream, to_device, to_host
    p, n_out = 8, 4096 * 3 + 7
    xs = _inputs(p, p * n_out, "bf16", 71, orc)
    din = to_device(xs, "bf16")
    for algo in ("allpairs", "ring"):
        dout = empty_like_poisoned(n_out, "bf16", p)
        assert sim.sim_reduce_scatter(ptrs(din), ptrs(dout), p, n_out, "bf16", "sum", algo, stream()) == 0
        got = to_host(dout, "bf16")
        want, _ = orc.reduce_scatter(xs, "bf16", "sum", algo)
        for r in range(p):
            assert_parity(got[r], want[r], "bf16", f"{label} RS {algo} r{r}")
        small = [x[:n_out].copy() for x in xs]
        dsm = to_device(small, "bf16")
        dag = empty_like_poisoned(p * n_out, "bf16", p)
        assert sim.sim_all_gather(ptrs(dsm), ptrs(dag), p, n_out, "bf16", algo, stream()) == 0
        got = to_host(dag, "bf16")
        want, _ = orc.all_gather(small, "bf16", algo)
        for r in range(p):
            assert (got[r] == want[r]).all(), (label, "AG", algo, r)
    torch.cuda.synchronize()


@pytest.mark.parametrize("budget", [1, 7, 64, 1000])
def test_workgroup_budget(orc, lib, budget):
    lib.sim_config_set("max_workgroups", budget)
    try:
        _check_all(orc, lib, f"budget {budget}")
        _check_rs_ag(orc, lib, f"budget {budget}")
    finally:
        lib.sim_config_set("max_workgroups", 0)


@pytest.mark.parametrize("total", [8, 100, 3000])
def test_forced_workgroups(orc, lib, total):
    lib.sim_debug_set("workgroups", total)
    try:
        _check_all(orc, lib, f"forced {total}")
    finally:
        lib.sim_debug_set("workgroups", 0)


@pytest.mark.parametrize("unroll", [None, 1, 2, 4])
def test_launch_table(orc, lib, tmp_path, unroll):
    f = tmp_path / "table.json"
    extra = [] if unroll is None else [unroll]
    table = {a: [[1024, 16] + extra, [1 << 20, 40] + extra, [64 << 20, 0] + extra] for a, _ in ALGOS}
    f.write_text(json.dumps({"algos": {}, "workgroups": table}))
    lib.sim_model_load(str(f))
    try:
        _check_all(orc, lib, f"table unroll {unroll}")
    finally:
        lib.sim_model_load(lib.CALIBRATION)


@pytest.mark.parametrize("how", ["budget 7", "budget 64", "forced 4"])
@pytest.mark.parametrize("p", [2, 4, 8])
def test_fold_four_vectors_per_lane(orc, lib, how, p):
    """The fused fold's 4-vector form (taken where a workgroup budget below
    the CU count caps the launch -- budget 7 here; under budget 64 these
    sizes keep the table's form -- or forced with SIM_DEBUG_UNROLL = 4)
    against the oracle:
    one-shot and all-pairs for every dtype and op, in place and not, and the
    direct reduce-scatter, on a ragged size with several 4-vector spans per
    chunk and a partial last span."""
    from tests.gpu_util import (assert_parity, empty_like_poisoned, ptrs, run_allreduce, stream, to_device,
                                to_host)
    kind, val = how.split()
    if kind == "budget":
        lib.sim_config_set("max_workgroups", int(val))
    else:
        lib.sim_debug_set("unroll", int(val))
    try:
        n = p * 8192 * 3 + 77  # a 4-vector span is 256 lanes x 4 x 16 bytes = 8192 bf16 elements
        for dtype in ("int32", "fp32", "fp16", "bf16"):
            for op in ("sum", "prod", "min", "max", "avg"):
                xs = _inputs(p, n, dtype, 90 + p, orc)
                if op == "prod":
                    import synthdata
                    xs = (synthdata.int_uniform(91, p, n, -3, 3) if dtype == "int32"
                          else synthdata.uniform(91, p, n, 0.5, 2.0, dtype))
                for algo in ("oneshot", "allpairs"):
                    want, _ = orc.allreduce(xs, dtype, op, algo)
                    for inplace in (False, True):
                        print(f"{how} p={p} {algo} {dtype} {op} inplace={inplace} n={n}", flush=True)
                        got = run_allreduce(xs, dtype, op, algo, inplace=inplace)
                        for r in range(p):
                            assert_parity(got[r], want[r], dtype, f"{how} {algo} {dtype} {op} r{r}")
        n_out = 8192 * 2 + 5
        xs = _inputs(p, p * n_out, "bf16", 92, orc)
        din = to_device(xs, "bf16")
        dout = empty_like_poisoned(n_out, "bf16", p)
        assert lib.sim_reduce_scatter(ptrs(din), ptrs(dout), p, n_out, "bf16", "sum", "allpairs", stream()) == 0
        got = to_host(dout, "bf16")
        want, _ = orc.reduce_scatter(xs, "bf16", "sum", "allpairs")
        for r in range(p):
            assert_parity(got[r], want[r], "bf16", f"{how} RS r{r}")
    finally:
        lib.sim_config_set("max_workgroups", 0)
        lib.sim_debug_set("unroll", 0)
