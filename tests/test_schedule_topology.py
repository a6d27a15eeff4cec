"""Tree, recursive-exchange and 2PH schedules in the schedule layer and the
verifier (host only): tree shapes against the page's figures, the lowered
schedules against closed forms, the verifier against mutated schedules."""
import json
import os

import pytest

import all_reduce_reduction_amd as sim

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
GATHER, GATHER_POST, EXCH, EXCH_POST, MCAST = 6, 7, 8, 9, 10


@pytest.fixture(autouse=True)
def default_topology():
    yield
    sim.sim_config_set("ranks_per_node", 1)
    sim.sim_config_set("radix", 2)


def bits(m):
    return [q for q in range(32) if (m >> q) & 1]


def lib_tree(t, p, G):
    return [sim.sim_tree_info(t, p, G, r) for r in range(p)]


def test_config_round_trip_and_errors():
    assert sim.sim_config_get("ranks_per_node") == 1 and sim.sim_config_get("radix") == 2
    sim.sim_config_set("ranks_per_node", 4)
    sim.sim_config_set("radix", 3)
    assert sim.sim_config_get("ranks_per_node") == 4 and sim.sim_config_get("radix") == 3
    for key, bad in (("ranks_per_node", 0), ("ranks_per_node", 17), ("radix", 1), ("radix", 17)):
        with pytest.raises(sim.SimError) as e:
            sim.sim_config_set(key, bad)
        assert e.value.status == -1
    assert sim.sim_config_get("ranks_per_node") == 4 and sim.sim_config_get("radix") == 3
    with pytest.raises(sim.SimError):
        sim.sim_config_set(7, 1)


def test_tree_is_the_drawn_14_rank_tree():
    g = json.load(open(os.path.join(GOLDEN, "tree14.json")))
    parent = {c: q for c, q in g["edges"]}
    for r, (par, ch) in enumerate(lib_tree(0, g["n"], 1)):
        assert par == parent.get(r, -1), r
        assert ch == sorted(c for c, q in g["edges"] if q == r), r


def test_double_tree_12_rank_figure():
    g = json.load(open(os.path.join(GOLDEN, "dtree12.json")))
    n, k = g["n"], g["interior"]
    for t, listing in ((0, g["tree_one"]), (1, g["tree_two"])):
        info = lib_tree(t, n, 1)
        assert {r for r in range(n) if info[r][1]} == set(listing[:k]), t
        assert {r for r in range(n) if not info[r][1]} == set(listing[k:]), t


@pytest.mark.parametrize("p", range(2, 17))
def test_tree_shapes_match_the_oracle(orc, p):
    for G in range(1, p + 1):
        if p % G:
            continue
        for t in (0, 1):
            info = lib_tree(t, p, G)
            assert [par for par, _ in info] == [orc.tree_parent(t, p, G, r) for r in range(p)], (p, G, t)
            for r, (par, ch) in enumerate(info):  # parent and child lists agree
                assert ch == sorted(c for c in range(p) if info[c][0] == r)
                assert len(ch) <= 3


@pytest.mark.parametrize("p", range(2, 17))
def test_verifier_proves_the_topology_lowerings(p):
    for G in range(1, p + 1):
        if p % G:
            continue
        sim.sim_config_set("ranks_per_node", G)
        for algo in ("tree", "hier", "hier_large"):
            st, diag = sim.sim_verify_schedule(algo, p)
            assert st == 0, (algo, p, G, diag)
    sim.sim_config_set("ranks_per_node", 1)
    for k in range(2, p + 1):
        sim.sim_config_set("radix", k)
        v, m = 1, 0
        while v < p:
            v, m = v * k, m + 1
        st, diag = sim.sim_verify_schedule("rexch", p)
        if v == p:
            assert st == 0, (p, k, diag)
            assert sim.sim_schedule_info("rexch", p)[0] == m
        else:
            assert st == -2, (p, k)


def test_unfit_topologies_are_unsupported():
    sim.sim_config_set("ranks_per_node", 3)
    for algo in ("tree", "hier", "hier_large"):
        with pytest.raises(sim.SimError) as e:
            sim.sim_schedule_info(algo, 8)
        assert e.value.status == -2
    sim.sim_config_set("radix", 3)
    with pytest.raises(sim.SimError):
        sim.sim_schedule_info("rexch", 8)


@pytest.mark.parametrize("p,G", [(16, 1), (8, 1), (4, 1), (2, 1), (8, 2), (16, 4), (8, 8), (12, 3)])
def test_tree_round_count_is_the_latency_formula(p, G):
    # 2((ranks per node - 1) + log2(nodes)), rounded up for a node count
    # that is not a power of two
    sim.sim_config_set("ranks_per_node", G)
    nodes = p // G
    want = 2 * ((G - 1) + (nodes - 1).bit_length())
    assert sim.sim_schedule_info("tree", p)[0] == want


def test_tree_steps_fold_children_once_complete():
    # every up step folds, at each rank, exactly its children; the root's
    # fold completes the value; the down steps hand it to the children
    p = 14
    nsteps = sim.sim_schedule_info("tree", p)[0]
    seen = {t: {r for r in range(p) if not sim.sim_tree_info(t, p, 1, r)[1]} for t in (0, 1)}  # leaves
    for st in range(nsteps):
        for kind, src, dst, chunk, m in sim.sim_schedule_xfers("tree", p, st):
            par, ch = sim.sim_tree_info(chunk, p, 1, dst if kind != MCAST else src)
            assert bits(m) == ch
            if kind in (GATHER, GATHER_POST):
                assert st < nsteps // 2
                assert (kind == GATHER_POST) == (par == -1)
                assert set(ch) <= seen[chunk]  # children finished earlier
                seen[chunk].add(dst)
            else:
                assert kind == MCAST and st >= nsteps // 2


def test_hier_phases():
    sim.sim_config_set("ranks_per_node", 4)
    p, G = 8, 4
    steps = [sim.sim_schedule_xfers("hier", p, s) for s in range(sim.sim_schedule_info("hier", p)[0])]
    assert [sorted({x[0] for x in s}) for s in steps] == [[GATHER], [EXCH_POST], [MCAST]]
    for kind, src, dst, chunk, m in steps[0]:  # local reduce-scatter into G chunks
        assert chunk == dst % G and bits(m) == [q for q in range(dst // G * G, dst // G * G + G) if q != dst]
    for kind, src, dst, chunk, m in steps[1]:  # cross-node all-pairs of the same position
        assert bits(m) == [dst % G + k * G for k in range(p // G)]
    steps = [sim.sim_schedule_xfers("hier_large", p, s)
             for s in range(sim.sim_schedule_info("hier_large", p)[0])]
    assert [sorted({x[0] for x in s}) for s in steps] == [[GATHER], [GATHER_POST], [MCAST], [MCAST]]
    assert sim.sim_schedule_info("hier_large", p)[2] == p


def _steps(algo, p):
    return [list(sim.sim_schedule_xfers(algo, p, s)) for s in range(sim.sim_schedule_info(algo, p)[0])]


def _custom(algo, p, steps):
    nch = sim.sim_schedule_info(algo, p)[2]
    return sim.sim_verify_custom(algo, p, steps, nchunks=nch, rounds=sim.sim_schedule_info(algo, p)[0])


def test_verifier_accepts_the_unmodified_topology_schedules():
    for algo, cfg in (("tree", {}), ("rexch", {}), ("hier", {"ranks_per_node": 2}),
                      ("hier_large", {"ranks_per_node": 2})):
        for k, v in cfg.items():
            sim.sim_config_set(k, v)
        assert _custom(algo, 8, _steps(algo, 8))[0] == 0, algo


def test_verifier_rejects_tree_mutations():
    p = 14
    base = _steps("tree", p)
    muts = {}
    m = [list(s) for s in base]; k, a, b, c, w = m[1][0]; m[1][0] = (k, a, b, c, w & (w - 1)); muts["child dropped"] = m
    m = [list(s) for s in base]; m[0], m[1] = m[1], m[0]; muts["parent before child"] = m
    m = [list(s) for s in base]; m[-1], m[-2] = m[-2], m[-1]; muts["broadcast before the value arrives"] = m
    m = [list(s) for s in base]; m[3] = [(GATHER,) + x[1:] for x in m[3]]; muts["root without post-op"] = m
    m = [list(s) for s in base]; k, a, b, c, w = m[0][0]; m[0][0] = (k, a, b, 1 - c, w); muts["wrong tree"] = m
    m = [list(s) for s in base]; del m[-1][0]; muts["missing broadcast"] = m
    m = [list(s) for s in base]; m[4] = m[4] + m[3]; muts["root folds twice"] = m
    for name, steps in muts.items():
        st, diag = _custom("tree", p, steps)
        assert st == -8 and diag, name


def test_verifier_rejects_exchange_mutations():
    sim.sim_config_set("radix", 2)
    p = 8
    base = _steps("rexch", p)
    muts = {}
    m = [list(s) for s in base]; m[0], m[1] = m[1], m[0]; muts["digit order"] = m
    m = [list(s) for s in base]; k, a, b, c, w = m[1][0]; m[1][0] = (k, a, b, c, w ^ (1 << 4)); muts["foreign group member"] = m
    m = [list(s) for s in base]; k, a, b, c, w = m[0][0]; m[0][0] = (k, a, b, c, w | (1 << 2)); muts["overlapping group"] = m
    m = [list(s) for s in base]; m[-1] = [(EXCH,) + x[1:] for x in m[-1]]; muts["no post-op"] = m
    m = [list(s) for s in base]; del m[-1]; muts["missing round"] = m
    for name, steps in muts.items():
        st, diag = _custom("rexch", p, steps)
        assert st == -8 and diag, name


def test_verifier_rejects_hier_mutations():
    sim.sim_config_set("ranks_per_node", 4)
    p = 8
    base = _steps("hier", p)
    muts = {}
    m = [list(s) for s in base]; m[2], m[1] = m[1], m[2]; muts["all-gather before the cross-node step"] = m
    m = [list(s) for s in base]; k, a, b, c, w = m[0][0]; m[0][0] = (k, a, b, (c + 1) % 4, w); muts["wrong local chunk"] = m
    m = [list(s) for s in base]; k, a, b, c, w = m[1][0]; m[1][0] = (k, a, b, c, w & ~(1 << 4)); muts["node left out"] = m
    m = [list(s) for s in base]; m[1] = [(GATHER_POST, -1, d, c, w & ~(1 << d)) for (_, _, d, c, w) in m[1]]; muts["node order"] = m
    for name, steps in muts.items():
        st, diag = _custom("hier", p, steps)
        assert st == -8 and diag, name


def test_exchange_groups_must_share_their_set():
    # two transfers that read each other's slot are legal only as members of
    # one exchange group; a gather reading a slot an exchange writes is a hazard
    steps = [[(EXCH_POST, -1, 0, 0, 0b11), (EXCH_POST, -1, 1, 0, 0b11)]]
    assert sim.sim_verify_custom("rexch", 2, steps, nchunks=1, rounds=1)[0] == 0
    steps = [[(EXCH_POST, -1, 0, 0, 0b11), (GATHER_POST, -1, 1, 0, 0b01)]]
    st, diag = sim.sim_verify_custom("rexch", 2, steps, nchunks=1, rounds=1)
    assert st == -8 and "read by one transfer and written by another" in diag
