"""HIP graph capture of the collectives (torch.cuda.graph on the library's
stream argument).  Each graph is replayed several times with eager work in
between (new inputs copied in, synchronisation), and every replay is
checked against the oracle on the inputs it saw.  Schedules whose kernels
carry a per-call epoch (LL, the single-launch ring) are refused under
capture, and scratch never grows during capture."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

CAPTURABLE = [("oneshot", 1), ("allpairs", 1), ("ring", 1), ("tree", 2), ("rexch", 1), ("hier_large", 4)]


@pytest.fixture(scope="module", autouse=True)
def lib():
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, 8, 0)
    yield sim
    sim.sim_config_set("ranks_per_node", 1)


def _fresh(p, n, dtype, seed, orc):
    import synthdata
    return synthdata.normal(seed, p, n, dtype)


def _capture(sim, din, dout, p, n, dtype, algo):
    import torch
    from tests.gpu_util import ptrs
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    status = []
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            s = int(torch.cuda.current_stream().cuda_stream)
            status.append(sim.sim_allreduce(ptrs(din), ptrs(dout), p, n, dtype, "sum", algo, s))
    torch.cuda.current_stream().wait_stream(side)
    return graph, status[0]


@pytest.mark.parametrize("algo,g", CAPTURABLE)
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_graph_replays_match_the_oracle(orc, lib, algo, g, dtype):
    import torch
    from tests.gpu_util import assert_parity, empty_like_poisoned, ptrs, stream, to_device, to_host
    sim = lib
    sim.sim_config_set("ranks_per_node", g)
    p, n = 8, 8 * 4096 * 3 + 29
    xs = _fresh(p, n, dtype, 60, orc)
    din = to_device(xs, dtype)
    dout = empty_like_poisoned(n, dtype, p)
    # one uncaptured call of the same shape sizes the scratch
    assert sim.sim_allreduce(ptrs(din), ptrs(dout), p, n, dtype, "sum", algo, stream()) == 0
    torch.cuda.synchronize()
    graph, st = _capture(sim, din, dout, p, n, dtype, algo)
    assert st == 0, st
    for rep in range(3):
        xr = _fresh(p, n, dtype, 61 + rep, orc)
        for t, x in zip(din, to_device(xr, dtype)):  # eager work between replays
            t.copy_(x)
        for t in dout:
            t.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = to_host(dout, dtype)
        want, _ = orc.allreduce(xr, dtype, "sum", algo, ranks_per_node=g)
        for r in range(p):
            assert_parity(got[r], want[r], dtype, f"graph {algo} replay {rep} r{r}")
    del graph


def test_epoch_schedules_are_refused_under_capture(orc, lib):
    import torch
    from tests.gpu_util import empty_like_poisoned, to_device
    sim = lib
    p, n = 8, 4096
    xs = _fresh(p, n, "fp16", 62, orc)
    din = to_device(xs, "fp16")
    dout = empty_like_poisoned(n, "fp16", p)
    for algo in ("oneshot_ll", "ring_fifo", "allpairs_persistent"):
        graph, st = _capture(sim, din, dout, p, n, "fp16", algo)
        assert st == -2, (algo, st)
        del graph
    # AUTO under capture picks a capturable schedule and the replay is right
    graph, st = _capture(sim, din, dout, p, n, "fp16", "auto")
    assert st == 0 and sim.sim_last_algo() not in ("oneshot_ll", "ring_fifo", "allpairs_persistent")
    graph.replay()
    torch.cuda.synchronize()
    want, _ = orc.allreduce(xs, "fp16", "sum", sim.sim_last_algo())
    for r in range(p):
        assert (dout[r].cpu().numpy().view(np.uint16) == want[r]).all()
    # outside capture the selector is unaffected
    assert sim.sim_select(p, n, "fp16")[0] == "oneshot"


def test_scratch_does_not_grow_under_capture_and_outgrown_scratch_is_kept(orc, lib):
    import torch
    from tests.gpu_util import assert_parity, empty_like_poisoned, ptrs, stream, to_device, to_host
    sim = lib
    sim.sim_init(0, 8, 0)  # fresh library: no scratch yet
    p, n = 8, 8 * 4096 * 2 + 3
    xs = _fresh(p, n, "bf16", 63, orc)
    din = to_device(xs, "bf16")
    dout = empty_like_poisoned(n, "bf16", p)
    graph, st = _capture(sim, din, dout, p, n, "bf16", "ring")  # 16-bit ring needs fp32 scratch
    assert st == -2, st
    del graph
    assert sim.sim_allreduce(ptrs(din), ptrs(dout), p, n, "bf16", "sum", "ring", stream()) == 0
    torch.cuda.synchronize()
    graph, st = _capture(sim, din, dout, p, n, "bf16", "ring")
    assert st == 0
    # a larger uncaptured call outgrows the scratch; the graph keeps working
    big = 4 * n
    xb = _fresh(p, big, "bf16", 64, orc)
    db = to_device(xb, "bf16")
    ob = empty_like_poisoned(big, "bf16", p)
    assert sim.sim_allreduce(ptrs(db), ptrs(ob), p, big, "bf16", "sum", "ring", stream()) == 0
    torch.cuda.synchronize()
    wantb, _ = orc.allreduce(xb, "bf16", "sum", "ring")
    gotb = to_host(ob, "bf16")
    for r in range(p):
        assert_parity(gotb[r], wantb[r], "bf16", f"large eager r{r}")
    for t in dout:
        t.fill_(0)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    want, _ = orc.allreduce(xs, "bf16", "sum", "ring")
    got = to_host(dout, "bf16")
    for r in range(p):
        assert_parity(got[r], want[r], "bf16", f"replay after growth r{r}")
    del graph
    sim.sim_init(0, 8, 0)


def test_phased_sizes_capture_the_fused_kernels(orc, lib):
    """At a size where the one-shot runs phased, a captured call takes the
    fused kernel (the phased grid's barrier counts are fixed when it is
    enqueued, which a replay would repeat); every replay matches the
    oracle, and the eager call after the replays runs phased again."""
    import torch
    from tests.gpu_util import assert_parity, ptrs, stream, to_device, to_host
    sim = lib
    p, n = 8, (64 << 20) // 2 + 8 * 3  # 64 MiB of bf16 per rank, chunks a little ragged
    xs = _fresh(p, n, "bf16", 70, orc)
    din = to_device(xs, "bf16")
    dout = [torch.empty(n, dtype=torch.int16, device="cuda:0") for _ in range(p)]
    assert sim.sim_allreduce(ptrs(din), ptrs(dout), p, n, "bf16", "sum", "oneshot", stream()) == 0
    assert sim.sim_debug_get("phased_last") == 1
    torch.cuda.synchronize()
    graph, st = _capture(sim, din, dout, p, n, "bf16", "oneshot")
    assert st == 0 and sim.sim_debug_get("phased_last") == 0
    # compare a sample of indices on every rank, and every element of rank 0
    idx = np.unique(np.concatenate([np.arange(0, n, 9973), np.arange(n - 64, n)]))
    for rep in range(2):
        xr = _fresh(p, n, "bf16", 71 + rep, orc)
        for t, x in zip(din, to_device(xr, "bf16")):
            t.copy_(x)
        for t in dout:
            t.fill_(0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = to_host(dout, "bf16")
        want = orc.allreduce_at(xr, "bf16", "sum", "oneshot", idx)
        for r in range(p):
            assert_parity(got[r][idx], want, "bf16", f"captured one-shot replay {rep} r{r}")
        want0, _ = orc.allreduce(xr, "bf16", "sum", "oneshot")
        assert_parity(got[0], want0[0], "bf16", f"captured one-shot replay {rep} rank 0 in full")
    del graph
    assert sim.sim_allreduce(ptrs(din), ptrs(dout), p, n, "bf16", "sum", "oneshot", stream()) == 0
    assert sim.sim_debug_get("phased_last") == 1
    torch.cuda.synchronize()
