"""Random calls against the oracle: a seeded generator draws (collective, p,
n, dtype, op, schedule, topology, in place, launch settings), sizes
log-uniform from empty to tens of thousands of elements, and every drawn
call must match the oracle element by element (the parity bar of
gpu_util.assert_parity).  The draws are fixed by the seed, so every run
makes the same calls; each test id names its call."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

DTYPES = ["int32", "fp32", "fp16", "bf16"]
OPS = ["sum", "prod", "min", "max", "avg"]
SINGLE = ["ring", "allpairs", "oneshot", "oneshot_ll", "ring_fifo", "allpairs_persistent", "auto"]
ESIZE = {"int32": 4, "fp32": 4, "fp16": 2, "bf16": 2}


def _size(rng, hi):
    """0, or log-uniform in [1, hi]."""
    if rng.random() < 0.05:
        return 0
    return int(np.exp(rng.uniform(0, np.log(hi))))


def _topology_cases():
    """(algo, p, ranks per node, radix) for which the library lowers and
    verifies a schedule (host-only queries)."""
    import all_reduce_reduction_amd as sim
    cases = []
    for algo in ("tree", "rexch", "hier", "hier_large"):
        for p in range(2, 17):
            for G in (g for g in range(1, p + 1) if p % g == 0):
                for k in ((2, 3, 4) if algo == "rexch" else (2,)):
                    sim.sim_config_set("ranks_per_node", G)
                    sim.sim_config_set("radix", k)
                    try:
                        sim.sim_schedule_info(algo, p)
                    except sim.SimError:
                        continue
                    cases.append((algo, p, G, k))
    sim.sim_config_set("ranks_per_node", 1)
    sim.sim_config_set("radix", 2)
    return cases


def _draw_calls():
    rng = np.random.default_rng(20261202)
    topo = _topology_cases()
    calls = []
    for i in range(160):  # all-reduce, single-node schedules and AUTO
        calls.append(dict(coll="ar", p=int(rng.integers(2, 17)), n=_size(rng, 40000), dtype=str(rng.choice(DTYPES)),
                          op=str(rng.choice(OPS)), algo=str(rng.choice(SINGLE)), G=1, k=2,
                          inplace=bool(rng.integers(0, 2)), table=int(rng.integers(0, 2)),
                          unroll=int(rng.integers(0, 3)), budget=int(rng.choice([0, 0, 0, 1, 7, 64, 1000])),
                          seed=int(rng.integers(0, 2 ** 31))))
    for i in range(80):  # all-reduce, topology schedules
        algo, p, G, k = topo[int(rng.integers(0, len(topo)))]
        calls.append(dict(coll="ar", p=p, n=max(1, _size(rng, 20000)), dtype=str(rng.choice(DTYPES)),
                          op=str(rng.choice(OPS)), algo=algo, G=G, k=k, inplace=bool(rng.integers(0, 2)),
                          table=1, unroll=0, budget=int(rng.choice([0, 0, 5, 300])),
                          seed=int(rng.integers(0, 2 ** 31))))
    for i in range(60):  # reduce-scatter and all-gather
        calls.append(dict(coll=str(rng.choice(["rs", "ag"])), p=int(rng.integers(2, 17)), n=max(1, _size(rng, 3000)),
                          dtype=str(rng.choice(DTYPES)), op=str(rng.choice(OPS)),
                          algo=str(rng.choice(["ring", "allpairs", "auto"])), G=1, k=2, inplace=False, table=1,
                          unroll=0, budget=int(rng.choice([0, 0, 3, 200])), seed=int(rng.integers(0, 2 ** 31))))
    return calls


CALLS = _draw_calls()


def _id(c):
    return (f"{c['coll']}-{c['algo']}-p{c['p']}-G{c['G']}-k{c['k']}-n{c['n']}-{c['dtype']}-{c['op']}"
            f"{'-ip' if c['inplace'] else ''}-t{c['table']}-u{c['unroll']}-b{c['budget']}")


@pytest.fixture(scope="module", autouse=True)
def lib():
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, 16, 0)
    yield sim
    for key, v in (("ptr_table", 1), ("unroll", 0)):
        sim.sim_debug_set(key, v)
    sim.sim_config_set("max_workgroups", 0)
    sim.sim_config_set("ranks_per_node", 1)
    sim.sim_config_set("radix", 2)


def _inputs(orc, p, n, dtype, op, seed):
    rng = np.random.default_rng(seed)
    if dtype == "int32":
        lim = 3 if op == "prod" else 1 << 20
        return [rng.integers(-lim, lim, n, endpoint=True, dtype=np.int32) for _ in range(p)]
    x32 = [(rng.uniform(0.5, 2.0, n) if op == "prod" else rng.standard_normal(n)).astype(np.float32)
           for _ in range(p)]
    if dtype == "fp32":
        return x32
    if dtype == "fp16":
        return [x.astype(np.float16).view(np.uint16) for x in x32]
    return [orc.f32_to_bf16(x) for x in x32]


@pytest.mark.parametrize("c", CALLS, ids=_id)
def test_random_call(orc, lib, c):
    from tests.gpu_util import assert_parity, empty_like_poisoned, ptrs, run_allreduce, stream, to_device, to_host
    sim = lib
    print(f"random call {_id(c)} seed={c['seed']}", flush=True)
    sim.sim_debug_set("ptr_table", c["table"])
    sim.sim_debug_set("unroll", c["unroll"])
    sim.sim_config_set("max_workgroups", c["budget"])
    sim.sim_config_set("ranks_per_node", c["G"])
    sim.sim_config_set("radix", c["k"])
    p, n, dtype, op, algo = c["p"], c["n"], c["dtype"], c["op"], c["algo"]
    if c["coll"] == "ar":
        if n == 0:  # a no-op once the scalar arguments are checked
            d = to_device([np.zeros(1, np.int32) for _ in range(p)], "int32")
            assert sim.sim_allreduce(ptrs(d), ptrs(d), p, 0, dtype, op, algo, stream()) == 0
            return
        if algo == "oneshot_ll" and n * ESIZE[dtype] > sim.LL_MAX_BYTES_PER_RANK:
            algo = "oneshot"
        xs = _inputs(orc, p, n, dtype, op, c["seed"])
        got = run_allreduce(xs, dtype, op, algo, inplace=c["inplace"])
        ran = sim.sim_last_algo()
        assert algo == "auto" or ran == algo
        want, _ = orc.allreduce(xs, dtype, op, ran, ranks_per_node=c["G"], radix=c["k"])
    elif c["coll"] == "rs":
        xs = _inputs(orc, p, p * n, dtype, op, c["seed"])
        want, _ = orc.reduce_scatter(xs, dtype, op, "allpairs" if algo == "auto" else algo)
        din, dout = to_device(xs, dtype), empty_like_poisoned(n, dtype, p)
        assert sim.sim_reduce_scatter(ptrs(din), ptrs(dout), p, n, dtype, op, algo, stream()) == 0
        assert sim.sim_check_error(stream()) == 0
        got = to_host(dout, dtype)
    else:
        xs = _inputs(orc, p, n, dtype, "sum", c["seed"])
        want, _ = orc.all_gather(xs, dtype, "allpairs" if algo == "auto" else algo)
        din, dout = to_device(xs, dtype), empty_like_poisoned(p * n, dtype, p)
        assert sim.sim_all_gather(ptrs(din), ptrs(dout), p, n, dtype, algo, stream()) == 0
        assert sim.sim_check_error(stream()) == 0
        got = to_host(dout, dtype)
    for r in range(p):
        assert_parity(got[r], want[r], dtype, f"{_id(c)} r{r}")
