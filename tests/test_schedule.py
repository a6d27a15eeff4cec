"""The schedule layer and its symbolic verifier (host only)."""
import json
import os

import pytest

import all_reduce_reduction_amd as sim

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
REDUCE, REDUCE_POST, COPY, GATHER_REDUCE, FANOUT, ONESHOT = range(6)


def mask(ranks):
    m = 0
    for r in ranks:
        m |= 1 << r
    return m


def test_ring_reproduces_the_3gpu_table():
    g = json.load(open(os.path.join(GOLDEN, "ring_3gpu_table.json")))
    for t, name in enumerate(g["steps"]):
        want = [[mask(cell) for cell in gpu] for gpu in g["cells"][name]]
        assert sim.sim_schedule_state("ring", 3, t) == want, name


@pytest.mark.parametrize("p", range(2, 17))
def test_step_counts(p):
    assert sim.sim_schedule_info("ring", p) == (2 * (p - 1), 2 * (p - 1) * p, p)
    assert sim.sim_schedule_info("allpairs", p) == (2, 2 * p, p)
    assert sim.sim_schedule_info("oneshot", p)[0] == 1


@pytest.mark.parametrize("p", range(2, 17))
def test_ring_primitive_counts_per_rank(p):
    # per rank: one send, then p-1 reduce-receives (the last with the post-op)
    # and p-1 copy-receives
    recv_reduce = {r: 0 for r in range(p)}
    recv_post = {r: 0 for r in range(p)}
    recv_copy = {r: 0 for r in range(p)}
    for st in range(2 * (p - 1)):
        xs = sim.sim_schedule_xfers("ring", p, st)
        assert len(xs) == p and sorted(x[1] for x in xs) == list(range(p))  # every rank sends once
        for kind, src, dst, chunk, _ in xs:
            assert dst == (src + 1) % p
            if kind == REDUCE:
                recv_reduce[dst] += 1
            elif kind == REDUCE_POST:
                recv_post[dst] += 1
                assert chunk == dst  # the chunk completes at its owner
            else:
                assert kind == COPY
                recv_copy[dst] += 1
    for r in range(p):
        assert recv_reduce[r] == p - 2 and recv_post[r] == 1 and recv_copy[r] == p - 1


@pytest.mark.parametrize("p", [2, 3, 4, 8, 16])
def test_bytes_sent_per_rank_is_optimal(p):
    # each rank sends 2(p-1)/p of its buffer (counted in chunks of S/p)
    sent = {r: 0 for r in range(p)}
    for st in range(2 * (p - 1)):
        for kind, src, dst, chunk, _ in sim.sim_schedule_xfers("ring", p, st):
            sent[src] += 1
    assert all(v == 2 * (p - 1) for v in sent.values())
    sent = {r: 0 for r in range(p)}
    for st in range(2):
        for kind, src, dst, chunk, _ in sim.sim_schedule_xfers("allpairs", p, st):
            if kind == GATHER_REDUCE:
                for q in range(p):
                    if q != dst:
                        sent[q] += 1
            else:
                sent[src] += p - 1
    assert all(v == 2 * (p - 1) for v in sent.values())


@pytest.mark.parametrize("algo", ["ring", "allpairs", "oneshot", "oneshot_ll", "ring_fifo", "allpairs_persistent"])
@pytest.mark.parametrize("p", range(2, 17))
def test_verifier_proves_every_lowering(algo, p):
    st, diag = sim.sim_verify_schedule(algo, p)
    assert st == 0, diag


def _ring(p):
    return [sim.sim_schedule_xfers("ring", p, s) for s in range(2 * (p - 1))]


def test_verifier_accepts_the_unmodified_copy():
    assert sim.sim_verify_custom("ring", 4, _ring(4))[0] == 0
    # a schedule that claims another round count than the closed form
    st, diag = sim.sim_verify_custom("ring", 4, _ring(4), rounds=5)
    assert st == -8 and "closed form" in diag


@pytest.mark.parametrize("p", [3, 4, 8])
def test_verifier_rejects_mutations(p):
    base = _ring(p)
    muts = {}
    m = [list(s) for s in base]; del m[1][2]; muts["dropped transfer"] = m
    m = [list(s) for s in base]; m[0].append(m[0][0]); muts["duplicated reduce"] = m
    m = [list(s) for s in base]; k, a, b, c, w = m[0][1]; m[0][1] = (k, a, b, (c + 1) % p, w); muts["swapped chunk"] = m
    m = [list(s) for s in base]; m[1], m[0] = m[0], m[1]; muts["steps reordered"] = m
    m = [list(s) for s in base]; del m[-1]; muts["missing step"] = m
    m = [list(s) for s in base]; m[p - 2] = [(REDUCE, a, b, c, w) for (_, a, b, c, w) in m[p - 2]]; muts["no post-op"] = m
    m = [list(s) for s in base]; k, a, b, c, w = m[p - 1][0]; m[p - 1][0] = (k, a, (b + 1) % p, c, w); muts["wrong copy target"] = m
    for name, steps in muts.items():
        st, diag = sim.sim_verify_custom("ring", p, steps, rounds=2 * (p - 1))
        assert st == -8, (name, diag)
        assert diag, name


def test_verifier_rejects_an_intra_step_hazard():
    # two reduces in one step: the second reads the slot the first writes
    steps = [[(REDUCE, 0, 1, 0), (REDUCE, 1, 2, 0)]]
    st, diag = sim.sim_verify_custom("ring", 3, steps, rounds=4)
    assert st == -8 and "read by one transfer and written by another" in diag


def test_verifier_checks_fold_order():
    # the all-pairs schedule is correct as an all-pairs but not in ring order
    ap = [sim.sim_schedule_xfers("allpairs", 4, s) for s in range(2)]
    assert sim.sim_verify_custom("allpairs", 4, ap)[0] == 0
    st, diag = sim.sim_verify_custom("ring", 4, ap, rounds=6)
    assert st == -8 and "another order" in diag
