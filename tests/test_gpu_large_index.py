"""Buffers past 4 GiB per rank: element indices above 2^31 and byte offsets
above 2^32 in every schedule's addressing (bf16, p = 2, n = 2^31 + 2^16 + 7,
so chunk 1 and the fp32 ring partials cross both limits too).  The oracle's
sampled entry point checks elements around the chunk edge, the 2^31 element
and the 2^32 byte boundaries, the ragged tail and random positions; the two
ranks' outputs are compared in full on the device."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

P = 2
N = (1 << 31) + (1 << 16) + 7
# "oneshot_phased": the one-shot with its phased form forced (at p = 2 the
# fused form is the default at every size)
ALGOS = [("oneshot", 1), ("oneshot_phased", 1), ("allpairs", 1), ("ring", 1), ("ring_fifo", 1),
         ("allpairs_persistent", 1), ("tree", 1), ("hier_large", 1)]


@pytest.fixture(scope="module")
def big(orc):
    import torch

    import all_reduce_reduction_amd as sim
    free, _ = torch.cuda.mem_get_info()
    # inputs and outputs 4 x 4 GiB, the 16-bit partial scratch up to 16 GiB, headroom
    if free < (48 << 30):
        pytest.skip(f"needs ~48 GiB of free device memory, {free >> 30} GiB free")
    sim.sim_init(0, 16, 0)
    rng = np.random.default_rng(2031)
    # small integers, exact in bf16: sums of two ranks stay exact
    table = orc.f32_to_bf16(np.arange(-127, 128, dtype=np.float32))
    xs = []
    for r in range(P):
        print(f"large-index inputs: rank {r} of {P}, {N} bf16 elements", flush=True)
        xs.append(np.take(table, rng.integers(0, table.size, N, dtype=np.uint8)))
    dev = torch.device("cuda:0")
    din = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs]
    dout = [torch.empty(N, dtype=torch.int16, device=dev) for _ in range(P)]
    edge = N // 2  # chunk 1 starts here
    idx = np.concatenate([
        np.array([0, 1, 7, 8, edge - 9, edge - 1, edge, edge + 1, edge + 8,
                  (1 << 31) - 9, (1 << 31) - 1, 1 << 31, (1 << 31) + 1, (1 << 31) + 8,
                  N - 17, N - 9, N - 8, N - 2, N - 1], dtype=np.int64),
        rng.integers(0, N, 4096, dtype=np.int64),
        rng.integers((1 << 31) - (1 << 20), N, 1024, dtype=np.int64),
    ])
    yield sim, xs, din, dout, idx
    del din, dout
    torch.cuda.empty_cache()
    sim.sim_config_set("ranks_per_node", 1)


@pytest.mark.parametrize("algo,G", ALGOS, ids=[a for a, _ in ALGOS])
@pytest.mark.parametrize("op", ["sum", "max"])
def test_past_4GiB_per_rank(orc, big, algo, G, op):
    import torch

    from tests.gpu_util import ptrs, stream
    sim, xs, din, dout, idx = big
    sim.sim_config_set("ranks_per_node", G)
    for t in dout:
        t.fill_(0x7E5A)  # a NaN pattern in bf16: an unwritten element fails
    print(f"large-index {algo} {op} p={P} n={N}", flush=True)
    phased = algo == "oneshot_phased"
    algo = "oneshot" if phased else algo
    sim.sim_debug_set("phased", 1 if phased else 0)
    try:
        st = sim.sim_allreduce(ptrs(din), ptrs(dout), P, N, "bf16", op, algo, stream())
    finally:
        sim.sim_debug_set("phased", 0)
    assert st == 0, st
    if phased:
        assert sim.sim_debug_get("phased_last") == 1
    assert sim.sim_check_error(stream()) == 0
    assert torch.equal(dout[0], dout[1]), "ranks differ"
    want = orc.allreduce_at(xs, "bf16", op, algo, idx)
    ti = torch.from_numpy(idx).to(dout[0].device)
    got = dout[0][ti].cpu().numpy().view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} sampled elements differ, first at index {idx[bad[:5]]}"
    # integer-valued inputs: the sum is exact, the max is one of the inputs
    x0 = orc.bf16_to_f32(xs[0][idx])
    x1 = orc.bf16_to_f32(xs[1][idx])
    exact = x0 + x1 if op == "sum" else np.maximum(x0, x1)
    assert (orc.bf16_to_f32(got) == exact).all()


def test_phased_reduce_scatter_and_all_gather_past_4GiB(orc, big):
    """The phased direct reduce-scatter (input past 2^31 elements and 2^32
    bytes per rank) and the phased direct all-gather (output past both),
    p = 2, bf16 integer values: sampled elements around every limit against
    the exact results, and the all-gather's two outputs compared in full."""
    import torch

    from tests.gpu_util import ptrs, stream
    sim, xs, din, dout, idx = big
    n_out = (1 << 30) + (1 << 15)  # whole 16-byte vectors per chunk: the phased forms run
    n_in = 2 * n_out
    dev = din[0].device
    rs = [torch.full((n_out,), 0x7E5A, dtype=torch.int16, device=dev) for _ in range(P)]
    print(f"large-index phased reduce-scatter p={P} n_in={n_in}", flush=True)
    sim.sim_debug_set("phased", 1)  # at p = 2 the reduce-scatter is not phased by default
    try:
        assert sim.sim_reduce_scatter(ptrs(din), ptrs(rs), P, n_out, "bf16", "sum", "allpairs", stream()) == 0
    finally:
        sim.sim_debug_set("phased", 0)
    assert sim.sim_debug_get("phased_last") == 1
    assert sim.sim_check_error(stream()) == 0
    sidx = np.unique(np.concatenate([
        np.array([0, 1, 7, 8, (1 << 30) - 1, 1 << 30, n_out - 9, n_out - 1], dtype=np.int64),
        np.random.default_rng(7).integers(0, n_out, 4096, dtype=np.int64)]))
    ti = torch.from_numpy(sidx).to(dev)
    for r in range(P):
        got = orc.bf16_to_f32(rs[r][ti].cpu().numpy().view(np.uint16))
        src = r * n_out + sidx  # element of the all-reduce the owner r holds
        want = orc.bf16_to_f32(xs[0][src]) + orc.bf16_to_f32(xs[1][src])
        assert (got == want).all(), f"reduce-scatter rank {r}"
    del rs
    # all-gather: rank q's first n_out elements into block q of every output
    for t in dout:
        t.fill_(0x7E5A)
    ins = [d[:n_out] for d in din]
    print(f"large-index phased all-gather p={P} n_out={P * n_out}", flush=True)
    assert sim.sim_all_gather(ptrs(ins), ptrs(dout), P, n_out, "bf16", "allpairs", stream()) == 0
    assert sim.sim_debug_get("phased_last") == 1
    assert sim.sim_check_error(stream()) == 0
    assert torch.equal(dout[0][:n_in], dout[1][:n_in]), "outputs differ"
    gidx = np.unique(np.concatenate([sidx, n_out + sidx, np.array([(1 << 31) - 1, 1 << 31, n_in - 1])]))
    got = dout[0][torch.from_numpy(gidx).to(dev)].cpu().numpy().view(np.uint16)
    q = gidx // n_out
    want = np.where(q == 0, xs[0][gidx % n_out], xs[1][gidx % n_out])
    assert (got == want).all()
    torch.cuda.synchronize()
