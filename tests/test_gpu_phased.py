"""The phased one-shot (k_fold_phased): the grid folds each phase's spans
into registers, meets at a grid barrier, writes them out, and meets again
before the next phase.  It must give the fused one-shot's bits (same fold
order, same arithmetic) for every rank count it serves (2, 4, 8, 16),
dtype and op, in place or not, with ragged chunk edges, with several
phases, with no whole span at all, and when its barriers give up early (the
barrier orders the traffic; it guards no data)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def lib():
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, 16, 0)
    yield sim
    for key, v in (("phased", 0), ("workgroups", 0), ("spin_limit", 1 << 20)):
        sim.sim_debug_set(key, v)
    sim.sim_init(0, 8, 0)


def _inputs(dtype, op, p, n, seed):
    import synthdata
    if dtype == "int32":
        lo, hi = (-3, 4) if op == "prod" else (-1000, 1000)
        return synthdata.int_uniform(seed, p, n, lo, hi)
    if op == "prod":
        rng = np.random.default_rng([seed, p, n])
        x32 = [rng.uniform(0.5, 2.0, n).astype(np.float32) for _ in range(p)]
        if dtype == "fp32":
            return x32
        if dtype == "fp16":
            return [x.astype(np.float16).view(np.uint16) for x in x32]
        import oracle
        return [oracle.get().f32_to_bf16(x) for x in x32]
    return synthdata.normal(seed, p, n, dtype)


def _run(sim, xs, dtype, op, p, n, inplace=False, mode=1, wg=0):
    from tests.gpu_util import empty_like_poisoned, ptrs, stream, to_device, to_host
    din = to_device(xs, dtype)
    dout = din if inplace else empty_like_poisoned(n, dtype, p)
    sim.sim_debug_set("phased", mode)
    sim.sim_debug_set("workgroups", wg)
    try:
        assert sim.sim_allreduce(ptrs(din), ptrs(dout), p, n, dtype, op, "oneshot", stream()) == 0
        ran = sim.sim_debug_get("phased_last")
        got = to_host(dout, dtype)
    finally:
        sim.sim_debug_set("phased", 0)
        sim.sim_debug_set("workgroups", 0)
    assert sim.sim_check_error(stream()) == 0
    return got, ran


# 2 workgroups per chunk: a span is 256 lanes x 32 vectors (p <= 8) or x 16
# (p = 16), so these sizes give chunks of several whole spans plus a rest
# and phases that not every workgroup has work in
@pytest.mark.parametrize("p", [2, 4, 8, 16])
@pytest.mark.parametrize("dtype,op", [("bf16", "sum"), ("fp16", "avg"), ("fp32", "prod"), ("fp32", "min"),
                                      ("int32", "max"), ("int32", "avg"), ("int32", "sum")])
def test_phased_matches_oracle(orc, lib, p, dtype, op):
    from tests.gpu_util import assert_parity
    sim = lib
    V = 16 // (2 if dtype in ("fp16", "bf16") else 4)
    vecs = 256 * (32 if p <= 8 else 16)
    n = p * (5 * vecs * V + 3 * 256 * V) + 2 * p + 3  # 5 whole spans and a rest per chunk, ragged edges
    xs = _inputs(dtype, op, p, n, 70 + p)
    want, _ = orc.allreduce(xs, dtype, op, "oneshot")
    for inplace in (False, True):
        got, ran = _run(sim, [x.copy() for x in xs], dtype, op, p, n, inplace=inplace, wg=2 * p)
        assert ran == 1
        for r in range(p):
            assert_parity(got[r], want[r], dtype, f"phased p={p} {dtype} {op} inplace={inplace} r{r}")
    assert sim.sim_debug_get("phased_expired") == 0


@pytest.mark.parametrize("p", [2, 8, 16])
def test_phased_equals_fused_bits(orc, lib, p):
    """Same fold order, same arithmetic: the phased and fused one-shot agree
    bit for bit, at the full grid and with one workgroup per chunk."""
    from tests.gpu_util import bits
    sim = lib
    n = p * 256 * 32 * 8 * 3 + 77
    xs = _inputs("bf16", "sum", p, n, 9)
    fused, ran_f = _run(sim, xs, "bf16", "sum", p, n, mode=2)
    assert ran_f == 0
    for wg in (0, p):
        phased, ran_p = _run(sim, xs, "bf16", "sum", p, n, mode=1, wg=wg)
        assert ran_p == 1
        for r in range(p):
            assert (bits(phased[r]) == bits(fused[r])).all(), (p, wg, r)


@pytest.mark.parametrize("p", [4, 8, 16])
def test_phased_last_phase_runs(orc, lib, p):
    """A last phase holding fewer than K blocks per workgroup is dealt out
    evenly and taken as runs of K/2, K/4, ..., 1 blocks (one per bit of the
    count, fixed result registers): counts that set every bit, uneven
    dealing over 3 and 5 workgroups per chunk, a lone trailing block and a
    ragged tail, bit-identical to the fused one-shot."""
    from tests.gpu_util import bits
    sim = lib
    K = 32 if p <= 8 else 16
    blk = 256 * 8  # bf16 elements per block (256 lanes x 8)
    for tiles, left in ((1, K - 1), (3, 3 * K - 1), (3, K + 13), (5, 2 * K + 3), (3, 1)):
        chunk = (tiles * K + left) * blk + 3 * 8 + 5  # one full phase, the last one, a rest and a ragged tail
        n = p * chunk
        xs = _inputs("bf16", "sum", p, n, 31 + tiles + left)
        fused, ran_f = _run(sim, xs, "bf16", "sum", p, n, mode=2)
        phased, ran_p = _run(sim, xs, "bf16", "sum", p, n, mode=1, wg=tiles * p)
        assert ran_f == 0 and ran_p == 1
        for r in range(p):
            assert (bits(phased[r]) == bits(fused[r])).all(), (p, tiles, left, r)
    assert sim.sim_debug_get("phased_expired") == 0


def test_phased_small_and_degenerate(orc, lib):
    """No whole span at all (every vector done after the phases, no
    barrier), a chunk shorter than a vector, and n < p."""
    from tests.gpu_util import assert_parity
    sim = lib
    for p, n in ((8, 1), (8, 7), (2, 3), (8, 8 * 8 + 5), (16, 16 * 1000 + 9), (4, 4 * 256 * 8 * 32 - 1)):
        xs = _inputs("bf16", "sum", p, n, 5)
        want, _ = orc.allreduce(xs, "bf16", "sum", "oneshot")
        got, ran = _run(sim, xs, "bf16", "sum", p, n)
        assert ran == 1
        for r in range(p):
            assert_parity(got[r], want[r], "bf16", f"phased p={p} n={n} r{r}")


def test_phased_barrier_gives_up_without_changing_results(orc, lib):
    """A spin limit of one poll: waiting workgroups give up at once (and
    say so in the expired count), the grid runs unaligned, and the result
    is the same: the barrier orders traffic, it guards no data."""
    from tests.gpu_util import assert_parity
    sim = lib
    p = 8
    n = p * 256 * 32 * 8 * 4 + 11
    xs = _inputs("fp32", "sum", p, n, 21)
    want, _ = orc.allreduce(xs, "fp32", "sum", "oneshot")
    sim.sim_debug_set("phased_expired", 0)
    sim.sim_debug_set("spin_limit", 1)
    try:
        got, ran = _run(sim, xs, "fp32", "sum", p, n, wg=2 * p)
    finally:
        sim.sim_debug_set("spin_limit", 1 << 20)
    assert ran == 1
    for r in range(p):
        assert_parity(got[r], want[r], "fp32", f"phased, barrier giving up, r{r}")
    sim.sim_debug_set("phased_expired", 0)
    assert sim.sim_debug_get("phased_expired") == 0


def test_phased_selection_rules(orc, lib):
    """By default, at p = 8, the one-shot runs phased from 12 MiB per rank
    on (3/4 of the 16 MiB unit), the owner-only fold (direct reduce-scatter,
    all-pairs step 1) and the copy (direct all-gather, all-pairs step 2) from
    24 MiB; other rank counts have their own thresholds (the one-shot from
    16 MiB at p = 4 and 8 MiB at p = 16, never at p = 2); never for rank
    counts other than 2, 4, 8 and 16, under a workgroup budget or when
    switched off; the unit is settable (the thresholds follow it)."""
    import torch
    from tests.gpu_util import ptrs, stream
    sim = lib
    MIN = 16 << 20
    assert sim.sim_debug_get("phased_min") == MIN

    def ran(p, nbytes, **cfg):
        n = nbytes // 2
        xs = [torch.zeros(n, dtype=torch.int16, device="cuda:0") for _ in range(p)]
        ys = [torch.empty_like(x) for x in xs]
        try:
            for k, v in cfg.items():
                (sim.sim_config_set if k == "max_workgroups" else sim.sim_debug_set)(k, v)
            assert sim.sim_allreduce(ptrs(xs), ptrs(ys), p, n, "bf16", "sum", "oneshot", stream()) == 0
            return sim.sim_debug_get("phased_last")
        finally:
            sim.sim_config_set("max_workgroups", 0)
            sim.sim_debug_set("phased", 0)
            sim.sim_debug_set("phased_min", MIN)

    assert ran(8, MIN * 3 // 4) == 1
    assert ran(8, MIN * 3 // 4 - 16) == 0
    assert ran(4, MIN - 16) == 0
    assert ran(4, MIN) == 1
    assert ran(16, MIN // 2) == 1
    assert ran(16, MIN // 2 - 32) == 0
    assert ran(2, 4 * MIN) == 0
    assert ran(2, 4 * MIN, phased=1) == 1
    assert ran(6, 2 * MIN) == 0
    assert ran(8, 2 * MIN, max_workgroups=64) == 0
    assert ran(8, 2 * MIN, phased=2) == 0
    assert ran(8, 1 << 20, phased_min=1 << 20) == 1
    torch.cuda.synchronize()

    def ran_rs(nbytes):
        n = nbytes // 2
        xs = [torch.zeros(n, dtype=torch.int16, device="cuda:0") for _ in range(8)]
        ys = [torch.empty(n // 8, dtype=torch.int16, device="cuda:0") for _ in range(8)]
        assert sim.sim_reduce_scatter(ptrs(xs), ptrs(ys), 8, n // 8, "bf16", "sum", "allpairs", stream()) == 0
        return sim.sim_debug_get("phased_last")
    assert ran_rs(MIN * 3 // 2 - 16 * 8) == 0
    assert ran_rs(MIN * 3 // 2) == 1

    def ran_ag(out_bytes):
        n_in = out_bytes // 2 // 8
        xs = [torch.zeros(n_in, dtype=torch.int16, device="cuda:0") for _ in range(8)]
        ys = [torch.empty(8 * n_in, dtype=torch.int16, device="cuda:0") for _ in range(8)]
        assert sim.sim_all_gather(ptrs(xs), ptrs(ys), 8, n_in, "bf16", "allpairs", stream()) == 0
        return sim.sim_debug_get("phased_last")
    assert ran_ag(MIN * 3 // 2 - 16 * 8) == 0
    assert ran_ag(MIN * 3 // 2) == 1
    torch.cuda.synchronize()
    assert sim.sim_debug_get("phased_expired") == 0


def test_phased_across_streams(orc, lib):
    """A phased call on another stream while a phased launch may still run
    takes the fused kernel (two persistent grids would hold each other's
    CUs at their barriers); on the same stream, or once the earlier launch
    is done, it runs phased.  Every result matches the oracle."""
    import torch
    from tests.gpu_util import assert_parity, empty_like_poisoned, ptrs, to_device, to_host
    sim = lib
    p = 8
    n = p * 256 * 32 * 8 * 2 + 5
    xs = _inputs("bf16", "sum", p, n, 31)
    want, _ = orc.allreduce(xs, "bf16", "sum", "oneshot")
    din = to_device(xs, "bf16")
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [empty_like_poisoned(n, "bf16", p) for _ in range(4)]
    torch.cuda.synchronize()
    sim.sim_debug_set("phased", 1)
    try:
        ran = []
        for k, st in enumerate((sa, sa, sb, sa)):
            assert sim.sim_allreduce(ptrs(din), ptrs(outs[k]), p, n, "bf16", "sum", "oneshot", st.cuda_stream) == 0
            ran.append(sim.sim_debug_get("phased_last"))
        torch.cuda.synchronize()
        assert sim.sim_allreduce(ptrs(din), ptrs(outs[3]), p, n, "bf16", "sum", "oneshot", sb.cuda_stream) == 0
        ran.append(sim.sim_debug_get("phased_last"))
    finally:
        sim.sim_debug_set("phased", 0)
    torch.cuda.synchronize()
    # the first two on one stream run phased; the first call on the other
    # stream finds the phased launch before it unfinished, or already done
    assert ran[0] == 1 and ran[1] == 1 and ran[4] == 1
    assert ran[2] in (0, 1)
    for k in range(4):
        got = to_host(outs[k], "bf16")
        for r in range(p):
            assert_parity(got[r], want[r], "bf16", f"stream call {k} r{r}")
    assert sim.sim_debug_get("phased_expired") == 0


@pytest.mark.parametrize("p", [2, 4, 8, 16])
@pytest.mark.parametrize("dtype,op", [("bf16", "sum"), ("fp16", "max"), ("fp32", "avg"), ("int32", "prod")])
def test_phased_owner_only_matches_oracle(orc, lib, p, dtype, op):
    """The owner-only phased fold: all-pairs step 1 (outputs in place in
    the all-reduce layout) and the direct reduce-scatter (each owner's
    chunk written from offset 0 of its output, and in place), several
    phases and a rest per chunk; a chunk that does not fill whole 16-byte
    vectors keeps the reduce-scatter on the fused fold."""
    from tests.gpu_util import assert_parity, empty_like_poisoned, ptrs, stream, to_device, to_host
    sim = lib
    V = 16 // (2 if dtype in ("fp16", "bf16") else 4)
    vecs = 256 * (32 if p <= 8 else 16)
    # all-pairs all-reduce
    n = p * (5 * vecs * V + 3 * 256 * V) + 2 * p + 3
    xs = _inputs(dtype, op, p, n, 80 + p)
    want, _ = orc.allreduce(xs, dtype, op, "allpairs")
    din = to_device(xs, dtype)
    dout = empty_like_poisoned(n, dtype, p)
    sim.sim_debug_set("phased", 1)
    sim.sim_debug_set("workgroups", 2 * p)
    try:
        assert sim.sim_allreduce(ptrs(din), ptrs(dout), p, n, dtype, op, "allpairs", stream()) == 0
        assert sim.sim_debug_get("phased_last") == 1
        got = to_host(dout, dtype)
        for r in range(p):
            assert_parity(got[r], want[r], dtype, f"all-pairs phased p={p} {dtype} {op} r{r}")
        # direct reduce-scatter: whole vectors per chunk (phased), then a ragged chunk (fused)
        for n_out, phased in ((V * (5 * vecs + 3 * 256 + 7), 1), (V * (2 * vecs) + 1, 0)):
            xs = _inputs(dtype, op, p, p * n_out, 90 + p)
            want, _ = orc.reduce_scatter(xs, dtype, op, "allpairs")
            for inplace in (False, True):
                din = to_device(xs, dtype)
                outs = ([d[r * n_out:(r + 1) * n_out] for r, d in enumerate(din)] if inplace
                        else empty_like_poisoned(n_out, dtype, p))
                st = sim.sim_reduce_scatter(ptrs(din), ptrs(outs), p, n_out, dtype, op, "allpairs", stream())
                if inplace and (n_out * (16 // V)) % 16:
                    assert st == sim.STATUS_CODE["SIM_ERR_ALIGN"]
                    continue
                assert st == 0
                assert sim.sim_debug_get("phased_last") == phased
                got = to_host(outs, dtype)
                for r in range(p):
                    assert_parity(got[r], want[r], dtype,
                                  f"RS phased={phased} p={p} {dtype} {op} n_out={n_out} inplace={inplace} r{r}")
    finally:
        sim.sim_debug_set("phased", 0)
        sim.sim_debug_set("workgroups", 0)
    assert sim.sim_check_error(stream()) == 0
    assert sim.sim_debug_get("phased_expired") == 0


@pytest.mark.parametrize("p", [2, 4, 8, 16])
@pytest.mark.parametrize("dtype", ["int32", "fp32", "fp16", "bf16"])
def test_phased_all_gather_matches_oracle(orc, lib, p, dtype):
    """The phased direct all-gather: several phases and a rest per block, out
    of place and in place (each rank's input is its own block of its
    output); a block that does not fill whole 16-byte vectors keeps the fused
    copy.  Copies are exact: compared bit for bit."""
    from tests.gpu_util import assert_parity, empty_like_poisoned, ptrs, stream, to_device, to_host
    sim = lib
    V = 16 // (2 if dtype in ("fp16", "bf16") else 4)
    vecs = 256 * (32 if p <= 8 else 16)
    sim.sim_debug_set("phased", 1)
    sim.sim_debug_set("workgroups", 2 * p)
    try:
        for n_in, phased in ((V * (5 * vecs + 3 * 256 + 7), 1), (V * (2 * vecs) + 3, 0)):
            xs = _inputs(dtype, "sum", p, n_in, 40 + p)
            want, _ = orc.all_gather(xs, dtype, "allpairs")
            din = to_device(xs, dtype)
            dout = empty_like_poisoned(p * n_in, dtype, p)
            assert sim.sim_all_gather(ptrs(din), ptrs(dout), p, n_in, dtype, "allpairs", stream()) == 0
            assert sim.sim_debug_get("phased_last") == phased
            got = to_host(dout, dtype)
            for r in range(p):
                assert_parity(got[r], want[r], dtype, f"AG phased={phased} p={p} {dtype} n_in={n_in} r{r}")
            if phased:
                outs = empty_like_poisoned(p * n_in, dtype, p)
                for r in range(p):
                    outs[r][r * n_in:(r + 1) * n_in].copy_(din[r])
                ins = [o[r * n_in:(r + 1) * n_in] for r, o in enumerate(outs)]
                assert sim.sim_all_gather(ptrs(ins), ptrs(outs), p, n_in, dtype, "allpairs", stream()) == 0
                assert sim.sim_debug_get("phased_last") == 1
                got = to_host(outs, dtype)
                for r in range(p):
                    assert_parity(got[r], want[r], dtype, f"AG phased in place p={p} {dtype} r{r}")
    finally:
        sim.sim_debug_set("phased", 0)
        sim.sim_debug_set("workgroups", 0)
    assert sim.sim_check_error(stream()) == 0
    assert sim.sim_debug_get("phased_expired") == 0


def _run_layout(sim, xs, dtype, op, p, n, layout, wg, inplace=False, mode=1):
    """The one-shot with the phased kernel's block layout set (0: whole
    buffer where it applies, 1: per chunk); returns the outputs and whether
    the whole-buffer layout ran."""
    sim.sim_debug_set("phased_layout", layout)
    try:
        got, ran = _run(sim, [x.copy() for x in xs], dtype, op, p, n, inplace=inplace, mode=mode, wg=wg)
        whole = sim.sim_debug_get("phased_whole_last")
    finally:
        sim.sim_debug_set("phased_layout", 0)
    return got, ran, whole


@pytest.mark.parametrize("p", [2, 4, 8, 16])
@pytest.mark.parametrize("dtype,op", [("bf16", "sum"), ("fp16", "avg"), ("fp32", "prod"), ("fp32", "min"),
                                      ("int32", "max"), ("int32", "avg")])
def test_phased_whole_layout_matches_oracle(orc, lib, p, dtype, op):
    """The one-shot's whole-buffer layout: the grid takes the buffer's blocks
    in turn and folds each block in its own chunk's order.  Chunks change
    inside a workgroup's run of blocks at varying places; one phase dealt
    out unevenly, three phases with a short last one, and one workgroup per
    chunk over more than p phases.  Against the oracle, in place and not,
    and bit-identical to the per-chunk layout and to the fused kernel."""
    from tests.gpu_util import assert_parity, bits
    sim = lib
    V = 16 // (2 if dtype in ("fp16", "bf16") else 4)
    blk = 256 * V  # elements per block
    K = 32 if p <= 8 else 16
    for tiles, bpc in ((2, 4 * p + 3), (3, 3 * p * K // 4 + 5), (1, p * K + 7)):
        n = p * bpc * blk  # every chunk bpc whole blocks, bpc >= the grid's tiles * p workgroups
        xs = _inputs(dtype, op, p, n, 300 + p + tiles)
        want, _ = orc.allreduce(xs, dtype, op, "oneshot")
        fused, ran_f, _ = _run_layout(sim, xs, dtype, op, p, n, 0, 0, mode=2)
        chunked, ran_c, whole_c = _run_layout(sim, xs, dtype, op, p, n, 1, tiles * p)
        assert ran_f == 0 and ran_c == 1 and whole_c == 0
        for inplace in (False, True):
            print(f"whole layout p={p} {dtype} {op} tiles={tiles} blocks/chunk={bpc} inplace={inplace}", flush=True)
            got, ran, whole = _run_layout(sim, xs, dtype, op, p, n, 0, tiles * p, inplace=inplace)
            assert ran == 1 and whole == 1
            for r in range(p):
                assert_parity(got[r], want[r], dtype, f"whole p={p} {dtype} {op} tiles={tiles} r{r}")
                assert (bits(got[r]) == bits(fused[r])).all(), (p, dtype, op, tiles, r)
                assert (bits(got[r]) == bits(chunked[r])).all(), (p, dtype, op, tiles, r)
    assert sim.sim_debug_get("phased_expired") == 0


def test_phased_whole_layout_selection(orc, lib):
    """Where the whole-buffer layout runs: the phased one-shot only, when
    every chunk is the same whole number of blocks and no fewer blocks than
    the grid has workgroups, and not when the layout is set to per chunk."""
    from tests.gpu_util import assert_parity
    sim = lib
    p, blk = 8, 256 * 8
    cases = [(p * 64 * blk, 16, 1),        # 64 blocks per chunk, 16 workgroups
             (p * 64 * blk + 8, 16, 0),    # not whole blocks
             (p * 64 * blk + p, 16, 0),    # whole elements per chunk, not whole blocks
             (p * 15 * blk, 16, 0),        # fewer blocks per chunk than workgroups
             (p * 16 * blk, 16, 1)]        # exactly as many
    for n, wg, expect in cases:
        xs = _inputs("bf16", "sum", p, n, 41)
        want, _ = orc.allreduce(xs, "bf16", "sum", "oneshot")
        got, ran, whole = _run_layout(sim, xs, "bf16", "sum", p, n, 0, wg)
        assert ran == 1 and whole == expect, (n, wg, whole)
        for r in range(p):
            assert_parity(got[r], want[r], "bf16", f"selection n={n} r{r}")
    n = p * 64 * blk
    xs = _inputs("bf16", "sum", p, n, 42)
    _, ran, whole = _run_layout(sim, xs, "bf16", "sum", p, n, 1, 16)
    assert ran == 1 and whole == 0
    # all-pairs step 1 (the owner-only phased fold) keeps the per-chunk layout
    from tests.gpu_util import run_allreduce
    sim.sim_debug_set("phased", 1)
    sim.sim_debug_set("workgroups", 16)
    try:
        got = run_allreduce(xs, "bf16", "sum", "allpairs")
        assert sim.sim_debug_get("phased_last") == 1 and sim.sim_debug_get("phased_whole_last") == 0
    finally:
        sim.sim_debug_set("phased", 0)
        sim.sim_debug_set("workgroups", 0)
    want, _ = orc.allreduce(xs, "bf16", "sum", "allpairs")
    for r in range(p):
        assert_parity(got[r], want[r], "bf16", f"allpairs r{r}")
    with pytest.raises(sim.SimError):
        sim.sim_debug_set("phased_layout", 2)
