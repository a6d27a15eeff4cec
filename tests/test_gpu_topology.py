"""GPU parity of the tree, recursive-exchange and 2PH schedules: the HIP
step executor through the C-ABI against the CPU oracle's independent
implementation, element by element (int32/fp32 bit-exact; fp16/bf16 within
2^-8 relative and bit-exact), on several topologies, ragged and tiny sizes,
in and out of place; and at the 64 MiB-per-rank bf16 size on every
element, with every rank identical."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

DTYPES = ["int32", "fp32", "fp16", "bf16"]
OPS = ["sum", "prod", "min", "max", "avg"]
# (algo, p, ranks_per_node, radix)
CASES = [
    ("tree", 8, 1, 2), ("tree", 7, 1, 2), ("tree", 14, 1, 2), ("tree", 8, 2, 2), ("tree", 12, 3, 2),
    ("tree", 4, 4, 2), ("tree", 16, 1, 2),
    ("rexch", 8, 1, 2), ("rexch", 16, 1, 4), ("rexch", 9, 1, 3), ("rexch", 8, 1, 8), ("rexch", 2, 1, 2),
    ("hier", 8, 2, 2), ("hier", 8, 4, 2), ("hier", 12, 3, 2), ("hier", 8, 1, 2), ("hier", 8, 8, 2),
    ("hier_large", 8, 2, 2), ("hier_large", 8, 4, 2), ("hier_large", 16, 4, 2), ("hier_large", 6, 1, 2),
]
SIZES = [1, 3, 37, 4096 + 5, 3 * 8192 + 13]


@pytest.fixture(scope="module", autouse=True)
def lib():
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, 16, 0)
    yield sim
    sim.sim_config_set("ranks_per_node", 1)
    sim.sim_config_set("radix", 2)


def _topo(sim, G, k):
    sim.sim_config_set("ranks_per_node", G)
    sim.sim_config_set("radix", k)


def _inputs(p, n, dtype, op, seed, orc):
    rng = np.random.default_rng([seed, p, n])
    if dtype == "int32":
        if op == "prod":
            return [rng.integers(-3, 4, n, dtype=np.int32) for _ in range(p)]
        return [rng.integers(-(2 ** 31), 2 ** 31 - 1, n, endpoint=True, dtype=np.int32) for _ in range(p)]
    x32 = [(rng.uniform(0.5, 2.0, n) if op == "prod" else rng.standard_normal(n)).astype(np.float32)
           for _ in range(p)]
    if dtype == "fp32":
        return x32
    if dtype == "fp16":
        return [x.astype(np.float16).view(np.uint16) for x in x32]
    return [orc.f32_to_bf16(x) for x in x32]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}-p{c[1]}-G{c[2]}-k{c[3]}")
@pytest.mark.parametrize("dtype", DTYPES)
def test_topology_schedules_match_oracle(orc, lib, case, dtype):
    from tests.gpu_util import assert_parity, run_allreduce
    algo, p, G, k = case
    _topo(lib, G, k)
    for op in OPS:
        for n in SIZES:
            xs = _inputs(p, n, dtype, op, 3, orc)
            want, _ = orc.allreduce(xs, dtype, op, algo, ranks_per_node=G, radix=k)
            for inplace in (False, True):
                print(f"{algo} p={p} G={G} k={k} {dtype} {op} n={n} inplace={inplace}", flush=True)
                got = run_allreduce([x.copy() for x in xs], dtype, op, algo, inplace=inplace)
                for r in range(p):
                    assert_parity(got[r], want[r], dtype, f"{algo} p{p} G{G} k{k} {op} n{n} ip{inplace} r{r}")


def test_topology_edge_values(orc, lib):
    """Signed zeros, infinities and ties of min/max reach every rank with the
    oracle's bits."""
    from tests.gpu_util import assert_parity, run_allreduce
    p, n = 8, 4096 + 3
    rng = np.random.default_rng(77)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 1.0, -1.0, 2.0 ** -149, 3.0e38], dtype=np.float32)
    xs = [special[rng.integers(0, special.size, n)] for _ in range(p)]
    for algo, G in (("tree", 2), ("rexch", 1), ("hier", 4), ("hier_large", 2)):
        _topo(lib, G, 2)
        for op in ("min", "max", "sum"):
            if op == "sum":  # +inf + -inf would be NaN on both sides; keep one sign of infinity
                ys = [np.where(np.isneginf(x), np.float32(np.inf), x).astype(np.float32) for x in xs]
            else:
                ys = xs
            want, _ = orc.allreduce(ys, "fp32", op, algo, ranks_per_node=G)
            got = run_allreduce(ys, "fp32", op, algo)
            for r in range(p):
                assert (got[r].view(np.uint32) == want[r].view(np.uint32)).all(), (algo, op, r)


def test_topology_nan_inputs(orc, lib):
    """NaN inputs through the step executor: fp32 min/max select inputs, so
    they match the oracle bit for bit (payloads included); sum, prod and avg
    are NaN exactly where the oracle is, bit-exact elsewhere, in fp32 and in
    the fp32 partials of the 16-bit schedules.  Outputs start as a finite
    sentinel, so an unwritten element fails where a NaN is expected too."""
    from tests.gpu_util import bits, run_allreduce, widen16
    p, n = 8, 4096 + 3
    rng = np.random.default_rng(78)
    vals = np.array([0.5, -1.25, 2.0, -3.0, 1.0, 0.0, -0.0], dtype=np.float32)
    nans = np.array([0x7FC00000, 0xFFC00000, 0x7FC12345, 0x7F800001], dtype=np.uint32).view(np.float32)
    x32 = []
    for _ in range(p):
        v = vals[rng.integers(0, vals.size, n)]
        m = rng.random(n) < 0.08
        v[m] = nans[rng.integers(0, nans.size, int(m.sum()))]
        x32.append(v)
    for algo, G, k in (("tree", 2, 2), ("rexch", 1, 2), ("hier", 4, 2), ("hier_large", 2, 2)):
        _topo(lib, G, k)
        for dtype in ("fp32", "bf16"):
            xs = x32 if dtype == "fp32" else [orc.f32_to_bf16(x) for x in x32]
            fill = -12345.0 if dtype == "fp32" else int(
                orc.f32_to_bf16(np.array([-12345.0], dtype=np.float32)).view(np.int16)[0])
            for op in OPS:
                want, _ = orc.allreduce(xs, dtype, op, algo, ranks_per_node=G, radix=k)
                got = run_allreduce(xs, dtype, op, algo, fill=fill)
                for r in range(p):
                    g = got[r] if dtype == "fp32" else widen16(got[r], dtype)
                    w = want[r] if dtype == "fp32" else widen16(want[r], dtype)
                    what = (algo, dtype, op, r)
                    assert (np.isnan(g) == np.isnan(w)).all(), what
                    ok = ~np.isnan(w)
                    assert (bits(got[r])[ok] == bits(want[r])[ok]).all(), what
                    if dtype == "fp32" and op in ("min", "max"):
                        assert (bits(got[r]) == bits(want[r])).all(), what


def test_topology_repeated_calls_reuse_scratch(orc, lib):
    """fp16 partials live in library scratch: back-to-back calls of different
    schedules and sizes on one stream stay independent."""
    from tests.gpu_util import assert_parity, run_allreduce
    p = 8
    plan = [("tree", 1, 2, 70001), ("hier_large", 4, 2, 5), ("rexch", 1, 8, 131072 + 9),
            ("hier", 2, 2, 70001), ("tree", 4, 2, 17)]
    for algo, G, k, n in plan:
        _topo(lib, G, k)
        xs = _inputs(p, n, "fp16", "sum", 9, orc)
        want, _ = orc.allreduce(xs, "fp16", "sum", algo, ranks_per_node=G, radix=k)
        got = run_allreduce(xs, "fp16", "sum", algo)
        for r in range(p):
            assert_parity(got[r], want[r], "fp16", f"{algo} n{n} r{r}")


def test_topology_unfit_is_unsupported_and_enqueues_nothing(orc, lib):
    import torch
    import all_reduce_reduction_amd as sim
    from tests.gpu_util import empty_like_poisoned, ptrs, stream, to_device
    xs = _inputs(8, 100, "fp32", "sum", 1, orc)
    din = to_device(xs, "fp32")
    dout = empty_like_poisoned(100, "fp32", 8)
    for algo, G, k in (("tree", 3, 2), ("hier", 5, 2), ("rexch", 1, 3)):
        _topo(lib, G, k)
        assert sim.sim_allreduce(ptrs(din), ptrs(dout), 8, 100, "fp32", "sum", algo, stream()) == -2
    torch.cuda.synchronize()
    assert all(torch.isnan(t).all() for t in dout)
    for algo in ("tree", "rexch", "hier", "hier_large"):  # topology schedules serve all-reduce only
        assert sim.sim_reduce_scatter(ptrs(din), ptrs(dout), 8, 12, "fp32", "sum", algo, stream()) == -2


@pytest.mark.parametrize("algo,G,k", [("tree", 1, 2), ("rexch", 1, 2), ("hier", 4, 2), ("hier_large", 2, 2)])
def test_topology_full_size_bf16(orc, lib, algo, G, k):
    """p = 8, bf16, 64 MiB per rank (the bench workload): every rank
    identical, and all 33,554,432 elements of rank 0 against rank 0 of the
    oracle's own run of the schedule at the same topology."""
    import torch
    import all_reduce_reduction_amd as sim
    import synthdata
    from tests.gpu_util import assert_parity, empty_like_poisoned, ptrs, stream, to_device
    _topo(lib, G, k)
    p, n = 8, 33_554_432
    xs = synthdata.workload_inputs(3, p, n, "bf16")
    din = to_device(xs, "bf16")
    dout = empty_like_poisoned(n, "bf16", p)
    print(f"full size {algo} G={G} k={k}", flush=True)
    assert sim.sim_allreduce(ptrs(din), ptrs(dout), p, n, "bf16", "sum", algo, stream()) == 0
    assert sim.sim_check_error(stream()) == 0
    for r in range(1, p):
        assert torch.equal(dout[r], dout[0]), r
    got = dout[0].cpu().numpy().view(np.uint16)
    ys, _ = orc.allreduce(xs, "bf16", "sum", algo, ranks_per_node=G, radix=k)
    assert_parity(got, ys[0], "bf16", f"{algo} full size, all elements")
    del din, dout, ys
    torch.cuda.empty_cache()
