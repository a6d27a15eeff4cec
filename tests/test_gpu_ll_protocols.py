"""The LL protocol of the single-launch ring (small messages): every value
that crosses between ranks is one 8-byte {payload, epoch} packet polled by
its reader.  The fold order is that of the counter protocol, so both
protocols must give the oracle's bits at the same sizes:
every dtype and op, in place, channel counts; stale packets and unrelated
flags in the buffer; the epoch count shared with the LL one-shot across a
wraparound; and a missing partner or an unsatisfiable flag ending in
SIM_ERR_TIMEOUT."""
import pytest

from tests.test_gpu_parity import inputs, prod_inputs

pytestmark = pytest.mark.gpu

OK, TIMEOUT = 0, -7
DTYPES = ["int32", "fp32", "fp16", "bf16"]
OPS = ["sum", "prod", "min", "max", "avg"]
SHAPES = [(2, 1), (3, 7), (8, 3), (8, 4096), (5, 999), (16, 257), (8, 8191), (7, 12345)]
FORCE_LL, NEVER_LL = 1 << 30, 0
DEFAULT_LIMIT = 256 << 10
# (schedule, its debug key for the LL size limit)
SCHEDULES = [("ring_fifo", "ring_ll_max")]


@pytest.fixture(autouse=True)
def lib():
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, 16, 0)
    yield sim
    for _, key in SCHEDULES:
        sim.sim_debug_set(key, DEFAULT_LIMIT)
    sim.sim_debug_set("fifo_channels", 0)
    sim.sim_debug_set("ll_wait_skew", 0)
    sim.sim_debug_set("fifo_withhold", 0)
    sim.sim_debug_set("spin_limit", 1 << 20)


def test_default_limits(lib):
    for _, key in SCHEDULES:
        assert lib.sim_debug_get(key) == DEFAULT_LIMIT


@pytest.mark.parametrize("algo,key", SCHEDULES, ids=[a for a, _ in SCHEDULES])
@pytest.mark.parametrize("op", OPS)
@pytest.mark.parametrize("dtype", DTYPES)
def test_both_protocols_match_the_oracle(orc, lib, dtype, op, algo, key):
    from tests.gpu_util import assert_parity, run_allreduce
    sim = lib
    for p, n in SHAPES:
        xs = (prod_inputs if op == "prod" else inputs)(p, n, dtype, 9, orc)
        want, _ = orc.allreduce(xs, dtype, op, algo)
        for limit in (FORCE_LL, NEVER_LL):
            sim.sim_debug_set(key, limit)
            for inplace in (False, True):
                print(f"{algo} limit={limit} p={p} n={n} {dtype} {op} inplace={inplace}", flush=True)
                got = run_allreduce([x.copy() for x in xs], dtype, op, algo, inplace=inplace)
                for r in range(p):
                    assert_parity(got[r], want[r], dtype, f"{algo} limit {limit} p={p} n={n} ip={inplace} r{r}")


@pytest.mark.parametrize("algo,key", SCHEDULES, ids=[a for a, _ in SCHEDULES])
def test_channel_counts(orc, lib, algo, key):
    import synthdata
    from tests.gpu_util import assert_parity, run_allreduce
    sim = lib
    xs = synthdata.normal(61, 8, 8 * 2048 + 5, "fp32")
    want, _ = orc.allreduce(xs, "fp32", "sum", algo)
    sim.sim_debug_set(key, FORCE_LL)
    for ch in (1, 2, 5, 16):
        sim.sim_debug_set("fifo_channels", ch)
        print(f"{algo} LL channels {ch}", flush=True)
        got = run_allreduce(xs, "fp32", "sum", algo)
        for r in range(8):
            assert_parity(got[r], want[r], "fp32", f"{algo} channels {ch} r{r}")


@pytest.mark.parametrize("algo", [a for a, _ in SCHEDULES])
def test_stale_and_foreign_packets_are_ignored(orc, lib, algo):
    import synthdata
    from tests.gpu_util import run_allreduce
    sim = lib
    xs = synthdata.normal(62, 8, 4096, "bf16")
    want, _ = orc.allreduce(xs, "bf16", "sum", algo)
    run_allreduce(xs, "bf16", "sum", algo)
    cur = sim.sim_debug_get("epoch")
    for fill in ((cur << 32) | 0xDEADBEEF, (0x13572468 << 32) | 0x0BADF00D):
        sim.sim_debug_set("fill_ll", fill)
        got = run_allreduce(xs, "bf16", "sum", algo)
        for r in range(8):
            assert (got[r] == want[r]).all()


def test_epoch_wraparound_shared_with_the_ll_oneshot(orc, lib):
    import synthdata
    from tests.gpu_util import run_allreduce
    sim = lib
    xs = synthdata.normal(63, 8, 4096 + 3, "fp16")
    algos = ["ring_fifo", "oneshot_ll"]
    want = {a: orc.allreduce(xs, "fp16", "sum", a)[0] for a in algos}
    sim.sim_debug_set("epoch", 0xFFFFFFFD)
    seen = []
    for k in range(6):
        algo = algos[k % 2]
        got = run_allreduce(xs, "fp16", "sum", algo)
        seen.append(sim.sim_debug_get("epoch"))
        for r in range(8):
            assert (got[r] == want[algo][r]).all(), (k, algo, r)
    assert seen == [0xFFFFFFFE, 0xFFFFFFFF, 1, 2, 3, 4]


@pytest.mark.parametrize("algo", [a for a, _ in SCHEDULES])
def test_missing_partner_and_unsatisfiable_flag_time_out(orc, lib, algo):
    """Rank 0's workgroups leave at once, or every reader waits for a flag
    no writer sets (both host-set test flags): the bounded polls expire,
    the kernel ends, the error word says SIM_ERR_TIMEOUT; the next call is
    correct."""
    import synthdata
    from tests.gpu_util import empty_like_poisoned, ptrs, run_allreduce, stream, to_device
    sim = lib
    xs = synthdata.normal(64, 8, 4096, "bf16")
    want, _ = orc.allreduce(xs, "bf16", "sum", algo)
    din = to_device(xs, "bf16")
    for hook in ("fifo_withhold", "ll_wait_skew"):
        sim.sim_debug_set("spin_limit", 64)
        sim.sim_debug_set(hook, 1)
        dout = empty_like_poisoned(4096, "bf16", 8)
        assert sim.sim_allreduce(ptrs(din), ptrs(dout), 8, 4096, "bf16", "sum", algo, stream()) == OK
        assert sim.sim_check_error(stream()) == TIMEOUT, hook
        sim.sim_debug_set(hook, 0)
        sim.sim_debug_set("spin_limit", 1 << 20)
        got = run_allreduce(xs, "bf16", "sum", algo)
        for r in range(8):
            assert (got[r] == want[r]).all(), (hook, r)
