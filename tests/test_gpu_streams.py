"""Calls that use no library buffer may run at the same time on different
streams: one-shot, all-pairs, the 32-bit ring all-reduce and the all-pairs
reduce-scatter / all-gather, enqueued alternately on two streams over
distinct buffers, each result checked against the oracle afterwards."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, 16, 0)
    yield sim


def test_buffer_free_calls_overlap_on_two_streams(orc, lib):
    import torch

    from tests.gpu_util import assert_parity, empty_like_poisoned, ptrs, to_device, to_host
    sim = lib
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    rng = np.random.default_rng(404)
    plan = [("ar", "oneshot", "bf16"), ("ar", "allpairs", "fp16"), ("ar", "ring", "fp32"),
            ("ar", "ring", "int32"), ("rs", "allpairs", "fp32"), ("ag", "allpairs", "bf16")]
    p, m = 8, 70001 // 8 * 8  # elements per rank (a whole number of rank blocks for RS / AG)
    jobs = []
    for rep in range(4):
        for s_i, stream in enumerate(streams):
            for coll, algo, dtype in plan:
                n_in = m if coll != "ag" else m // p
                if dtype == "int32":
                    xs = [rng.integers(-1000, 1000, n_in, dtype=np.int32) for _ in range(p)]
                else:
                    x32 = [rng.standard_normal(n_in).astype(np.float32) for _ in range(p)]
                    xs = (x32 if dtype == "fp32" else [x.astype(np.float16).view(np.uint16) for x in x32]
                          if dtype == "fp16" else [orc.f32_to_bf16(x) for x in x32])
                with torch.cuda.stream(stream):
                    din = to_device(xs, dtype)
                    n_out = {"ar": m, "rs": m // p, "ag": m}[coll]
                    dout = empty_like_poisoned(n_out, dtype, p)
                h = int(stream.cuda_stream)
                if coll == "ar":
                    st = sim.sim_allreduce(ptrs(din), ptrs(dout), p, m, dtype, "sum", algo, h)
                elif coll == "rs":
                    st = sim.sim_reduce_scatter(ptrs(din), ptrs(dout), p, m // p, dtype, "sum", algo, h)
                else:
                    st = sim.sim_all_gather(ptrs(din), ptrs(dout), p, m // p, dtype, algo, h)
                assert st == 0, (rep, s_i, coll, algo, dtype, st)
                jobs.append((coll, algo, dtype, xs, din, dout))
    torch.cuda.synchronize()
    for s in streams:
        assert sim.sim_check_error(int(s.cuda_stream)) == 0
    for coll, algo, dtype, xs, din, dout in jobs:
        if coll == "ar":
            want, _ = orc.allreduce(xs, dtype, "sum", algo)
        elif coll == "rs":
            want, _ = orc.reduce_scatter(xs, dtype, "sum", algo)
        else:
            want, _ = orc.all_gather(xs, dtype, algo)
        got = to_host(dout, dtype)
        for r in range(p):
            assert_parity(got[r], want[r], dtype, f"{coll} {algo} {dtype} r{r}")
