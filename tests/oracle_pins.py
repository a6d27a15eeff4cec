"""Pins of the CPU oracle against facts that do not come from the oracle.

Each check_* function raises AssertionError on a mismatch.  They are run
against the real oracle by tests/test_oracle_pins.py and against planted
mistakes (compiled mutants of oracle.c) by tests/test_oracle_mutants.py,
which must make at least one of them fail.
"""
from __future__ import annotations

import itertools
import json
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
ALGOS = ("ring", "allpairs", "oneshot", "oneshot_ll", "ring_fifo", "allpairs_persistent")
TOPO_ALGOS = ("tree", "rexch", "hier", "hier_large")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def chunk_bounds(n, p):
    """Chunk c = [floor(c n / p), floor((c+1) n / p))."""
    return [(c * n // p, (c + 1) * n // p) for c in range(p)]


def documented_order(algo, p, c):
    """Fold order of chunk c: ring starts at rank c+1 and walks the ring;
    all-pairs (and one-shot, LL) starts at the owner c, then ascending."""
    if algo in ("ring", "ring_fifo"):
        return [(c + 1 + k) % p for k in range(p)]
    return [c] + [q for q in range(p) if q != c]


def f32_left_fold(vals, order, op="sum"):
    acc = np.float32(vals[order[0]])
    for q in order[1:]:
        b = np.float32(vals[q])
        acc = np.float32(acc + b) if op == "sum" else np.float32(acc * b)
    return acc


# --------------------------------------------------------------------------
def check_worked_example(orc):
    g = _golden("worked_example.json")
    xs = [np.array(v, dtype=np.int32) for v in g["inputs"]]
    for algo in ALGOS:
        ys, _ = orc.allreduce(xs, "int32", "sum", algo)
        for r, y in enumerate(ys):
            assert y.tolist() == g["outputs"][r], (algo, r, y)
        ys, _ = orc.allreduce([x.copy() for x in xs], "int32", "sum", algo, inplace=True)
        for r, y in enumerate(ys):
            assert y.tolist() == g["outputs"][r], ("inplace", algo, r, y)


def check_step_counts(orc):
    for p in range(2, 17):
        xs = [np.full(3 * p + 1, q, dtype=np.int32) for q in range(p)]
        assert orc.allreduce(xs, "int32", "sum", "ring")[1] == 2 * (p - 1), p
        assert orc.allreduce(xs, "int32", "sum", "ring_fifo")[1] == 2 * (p - 1), p
        for algo in ("allpairs", "oneshot", "oneshot_ll", "allpairs_persistent"):
            assert orc.allreduce(xs, "int32", "sum", algo)[1] == 2, (p, algo)


def check_exactly_once(orc):
    """X[q] = 2^q everywhere: each contribution counted once gives 2^p - 1."""
    for p in (2, 3, 5, 8, 13):
        for n in (p, 7 * p + 3, 64):
            xs = [np.full(n, 1 << q, dtype=np.int32) for q in range(p)]
            for algo in ALGOS:
                ys, _ = orc.allreduce(xs, "int32", "sum", algo)
                for y in ys:
                    assert (y == (1 << p) - 1).all(), (p, n, algo)
            # one-hot: only rank k contributes 1 at element e
            for k in range(p):
                xs = [np.zeros(n, dtype=np.int32) for _ in range(p)]
                xs[k][:] = np.arange(n, dtype=np.int32) + 1
                for algo in ALGOS:
                    ys, _ = orc.allreduce(xs, "int32", "sum", algo)
                    for y in ys:
                        assert (y == np.arange(n) + 1).all(), (p, n, k, algo)


def _wrap32(v):
    v &= 0xFFFFFFFF
    return v - (1 << 32) if v >= 1 << 31 else v


def check_int_brute_force(orc):
    """int32 sum/prod (mod 2^32), min, max, avg against Python integers."""
    rng = np.random.default_rng(1234)
    for p in (2, 3, 4, 7, 8):
        for n in (1, p - 1, p, 5 * p + 3, 50):
            for lo, hi in ((-1000, 1000), (-(2 ** 31), 2 ** 31 - 1)):
                xs = [rng.integers(lo, hi, n, endpoint=True, dtype=np.int32) for _ in range(p)]
                cols = [[int(x[i]) for x in xs] for i in range(n)]
                want = {
                    "sum": [_wrap32(sum(c)) for c in cols],
                    "prod": [_wrap32(int(np.prod([Fraction(v) for v in c]))) for c in cols],
                    "min": [min(c) for c in cols],
                    "max": [max(c) for c in cols],
                }
                # avg: the wrapped int32 sum divided once, truncating toward zero
                want["avg"] = [int(Fraction(s, p)) if s >= 0 else -int(Fraction(-s, p))
                               for s in want["sum"]]
                for op, w in want.items():
                    for algo in ALGOS:
                        ys, _ = orc.allreduce(xs, "int32", op, algo)
                        for r, y in enumerate(ys):
                            assert y.tolist() == w, (p, n, op, algo, r)
                    assert orc.definition(xs, "int32", op).tolist() == w, (p, n, op)


def check_fold_order_probes(orc):
    """Order-revealing fp32 probes: values from {2^24, -2^24, 1, 0.5, 3}
    make addition non-associative in visible ways; among all p! left-fold
    orders exactly the documented one (up to swapping the first two, which
    addition cannot see) must reproduce every probe."""
    vals = np.array([2.0 ** 24, -2.0 ** 24, 1.0, 0.5, 3.0], dtype=np.float32)
    rng = np.random.default_rng(99)
    for p in (2, 3, 4):
        per_chunk = 120
        n = p * per_chunk
        xs = [vals[rng.integers(0, 5, n)].astype(np.float32) for _ in range(p)]
        for algo in ALGOS:
            ys, _ = orc.allreduce(xs, "fp32", "sum", algo)
            for c, (lo, hi) in enumerate(chunk_bounds(n, p)):
                consistent = set()
                for perm in itertools.permutations(range(p)):
                    ok = all(f32_left_fold([x[i] for x in xs], perm) == ys[0][i] for i in range(lo, hi))
                    if ok:
                        consistent.add((frozenset(perm[:2]), perm[2:]))
                doc = documented_order(algo, p, c)
                assert consistent == {(frozenset(doc[:2]), tuple(doc[2:]))}, (p, algo, c, consistent)
        # the sampled entry point follows the same orders
        idx = np.arange(n, dtype=np.int64)
        for algo in ALGOS:
            ys, _ = orc.allreduce(xs, "fp32", "sum", algo)
            assert (orc.allreduce_at(xs, "fp32", "sum", algo, idx).view(np.uint32) == ys[0].view(np.uint32)).all()


def check_identical_ranks(orc):
    rng = np.random.default_rng(7)
    for dtype in ("int32", "fp32", "fp16", "bf16"):
        for p in (2, 3, 8):
            n = 11 * p + 5
            x32 = [rng.standard_normal(n).astype(np.float32) for _ in range(p)]
            if dtype == "int32":
                xs = [rng.integers(-50, 50, n, dtype=np.int32) for _ in range(p)]
            elif dtype == "fp32":
                xs = x32
            elif dtype == "fp16":
                xs = [x.astype(np.float16).view(np.uint16) for x in x32]
            else:
                xs = [orc.f32_to_bf16(x) for x in x32]
            for op in ("sum", "prod", "min", "max", "avg"):
                for algo in ALGOS:
                    ys, _ = orc.allreduce(xs, dtype, op, algo)
                    for y in ys[1:]:
                        assert y.tobytes() == ys[0].tobytes(), (dtype, p, op, algo)


def check_order_independent_fp(orc):
    """Small integers and dyadic rationals in fp32 with |partials| < 2^24:
    every schedule is exact, so all algos agree and equal the exact sum."""
    rng = np.random.default_rng(11)
    for p in (2, 4, 8, 16):
        n = 9 * p + 2
        xs = [(rng.integers(-4096, 4096, n) / np.float32(8)).astype(np.float32) for _ in range(p)]
        exact = [sum(Fraction(float(x[i])) for x in xs) for i in range(n)]
        for algo in ALGOS:
            ys, _ = orc.allreduce(xs, "fp32", "sum", algo)
            assert [Fraction(float(v)) for v in ys[0]] == exact, (p, algo)
        # prod of powers of two is exact
        xs = [np.ldexp(np.float32(1), rng.integers(-8, 8, n)).astype(np.float32) *
              np.where(rng.random(n) < 0.5, -1, 1).astype(np.float32) for _ in range(p)]
        exact = [np.prod([Fraction(float(x[i])) for x in xs]) for i in range(n)]
        for algo in ALGOS:
            ys, _ = orc.allreduce(xs, "fp32", "prod", algo)
            assert [Fraction(float(v)) for v in ys[0]] == exact, (p, algo, "prod")


def check_minmax_library(orc):
    rng = np.random.default_rng(5)
    for p in (2, 5, 8):
        n = 13 * p + 1
        x32 = [rng.standard_normal(n).astype(np.float32) for _ in range(p)]
        for op, f in (("min", np.minimum), ("max", np.maximum)):
            want = f.reduce(np.stack(x32), axis=0)
            for algo in ALGOS:
                ys, _ = orc.allreduce(x32, "fp32", op, algo)
                assert (ys[0] == want).all(), (p, op, algo)
            # 16-bit: min/max commute with the monotone RNE narrowing
            xf16 = [x.astype(np.float16) for x in x32]
            want16 = f.reduce(np.stack(xf16), axis=0)
            for algo in ALGOS:
                ys, _ = orc.allreduce([x.view(np.uint16) for x in xf16], "fp16", op, algo)
                assert (ys[0].view(np.float16) == want16).all(), (p, op, algo, "fp16")


def check_minmax_nan_and_signed_zero(orc):
    """Min/max keep the accumulator unless the new operand compares strictly
    below (min) or above (max) it; the pages leave NaN and signed-zero ties
    open, and this is the reading both the oracle and the kernels take.
    Expected values worked by hand at p = 2, n = 2 (element c is chunk c):
    the all-pairs family folds chunk c owner first (rank c, then the other),
    the ring starts chunk c at rank c + 1."""
    nan, pz, nz = np.float32("nan"), np.float32(0.0), np.float32(-0.0)
    # x0 = [NaN, NaN], x1 = [1, 1]: a NaN accumulator stays, a NaN operand is passed over
    x = [np.array([nan, nan], np.float32), np.array([1.0, 1.0], np.float32)]
    # x0 = [+0, -0], x1 = [-0, +0]: a tie keeps whichever value came first
    z = [np.array([pz, nz], np.float32), np.array([nz, pz], np.float32)]
    for algo in ALGOS:
        ring = algo in ("ring", "ring_fifo")
        # all-pairs: chunk 0 starts at rank 0 (NaN), chunk 1 at rank 1 (1.0);
        # ring: chunk 0 starts at rank 1 (1.0), chunk 1 at rank 0 (NaN)
        want_nan = [False, True] if ring else [True, False]
        # all-pairs: chunk 0 starts with +0, chunk 1 with +0; ring: -0 and -0
        want_sign = [True, True] if ring else [False, False]
        for op in ("min", "max"):
            ys, _ = orc.allreduce(x, "fp32", op, algo)
            for r in range(2):
                assert list(np.isnan(ys[r])) == want_nan, (algo, op, r, ys[r])
                assert (ys[r][~np.isnan(ys[r])] == 1.0).all(), (algo, op, r, ys[r])
            ys, _ = orc.allreduce(z, "fp32", op, algo)
            for r in range(2):
                assert (ys[r] == 0).all() and list(np.signbit(ys[r])) == want_sign, (algo, op, r, ys[r])


def check_p2_sum(orc):
    rng = np.random.default_rng(3)
    a, b = (rng.standard_normal(1001).astype(np.float32) for _ in range(2))
    for algo in ALGOS:
        ys, _ = orc.allreduce([a, b], "fp32", "sum", algo)
        assert (ys[0] == a + b).all() and (ys[1] == a + b).all(), algo
        ys, _ = orc.allreduce([a, b], "fp32", "prod", algo)
        assert (ys[0] == a * b).all(), algo


def check_avg(orc):
    rng = np.random.default_rng(8)
    p, n = 8, 8 * 40 + 3
    xs = [rng.standard_normal(n).astype(np.float32) for _ in range(p)]
    for algo in ALGOS:
        s, _ = orc.allreduce(xs, "fp32", "sum", algo)
        a, _ = orc.allreduce(xs, "fp32", "avg", algo)
        # x/8 is exact, so pre-scaling commutes with every rounding
        assert (a[0] == s[0] * np.float32(0.125)).all(), algo
    # p = 3: the scale fp32(1/3) is applied to each operand before the sum
    xs = [rng.standard_normal(30).astype(np.float32) for _ in range(3)]
    inv3 = np.float32(1) / np.float32(3)
    for algo in ALGOS:
        a, _ = orc.allreduce(xs, "fp32", "avg", algo)
        for c, (lo, hi) in enumerate(chunk_bounds(30, 3)):
            order = documented_order(algo, 3, c)
            for i in range(lo, hi):
                want = f32_left_fold([np.float32(x[i] * inv3) for x in xs], order)
                assert a[0][i] == want, (algo, i)


def check_16bit_single_rounding(orc):
    """16-bit results = RNE narrowing (library cast) of the fp32 result of
    the same schedule on the widened inputs: partials stay fp32 and are
    rounded once, at the end."""
    import torch
    rng = np.random.default_rng(21)
    for p in (2, 3, 8):
        n = 17 * p + 3
        x32 = [(rng.standard_normal(n) * 0.02).astype(np.float32) for _ in range(p)]
        for dtype in ("fp16", "bf16"):
            if dtype == "fp16":
                xs = [x.astype(np.float16).view(np.uint16) for x in x32]
                wide = [x.view(np.float16).astype(np.float32) for x in xs]
            else:
                xs = [torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                      for x in x32]
                wide = [(x.astype(np.uint32) << 16).view(np.float32) for x in xs]
            for op in ("sum", "prod", "avg", "min", "max"):
                for algo in ALGOS:
                    ys, _ = orc.allreduce(xs, dtype, op, algo)
                    ref, _ = orc.allreduce(wide, "fp32", op, algo)
                    if dtype == "fp16":
                        want = ref[0].astype(np.float16).view(np.uint16)
                    else:
                        want = torch.from_numpy(ref[0]).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
                    assert (ys[0] == want).all(), (p, dtype, op, algo)


def check_error_bound_16bit(orc):
    """bf16/fp16 results within 2^-8 relative of the exact sum wherever the
    fp32 accumulation error cannot dominate (|exact| >= 2^-12 sum|x|)."""
    rng = np.random.default_rng(31)
    p, n = 8, 8 * 64
    x32 = [(rng.standard_normal(n) * 0.02).astype(np.float32) for _ in range(p)]
    for dtype in ("fp16", "bf16"):
        xs = [x.astype(np.float16).view(np.uint16) for x in x32] if dtype == "fp16" else [orc.f32_to_bf16(x) for x in x32]
        wide = [orc.f16_to_f32(x) if dtype == "fp16" else orc.bf16_to_f32(x) for x in xs]
        exact = np.sum(np.stack(wide).astype(np.float64), axis=0)
        mag = np.sum(np.abs(np.stack(wide).astype(np.float64)), axis=0)
        keep = np.abs(exact) >= mag * 2.0 ** -12
        assert keep.sum() > n // 2
        for algo in ALGOS:
            ys, _ = orc.allreduce(xs, dtype, "sum", algo)
            got = (orc.f16_to_f32(ys[0]) if dtype == "fp16" else orc.bf16_to_f32(ys[0])).astype(np.float64)
            rel = np.abs(got - exact)[keep] / np.abs(exact)[keep]
            assert rel.max() <= 2.0 ** -8, (dtype, algo, rel.max())


def check_rs_ag(orc):
    rng = np.random.default_rng(17)
    for p in (2, 3, 8):
        n_out = 13
        n = p * n_out
        for dtype in ("int32", "fp32", "bf16"):
            x32 = [rng.standard_normal(n).astype(np.float32) for _ in range(p)]
            xs = ([rng.integers(-99, 99, n, dtype=np.int32) for _ in range(p)] if dtype == "int32"
                  else x32 if dtype == "fp32" else [orc.f32_to_bf16(x) for x in x32])
            for op in ("sum", "max", "avg"):
                ar_ring, _ = orc.allreduce(xs, dtype, op, "ring")
                ar_ap, _ = orc.allreduce(xs, dtype, op, "allpairs")
                rs_ring, s1 = orc.reduce_scatter(xs, dtype, op, "ring")
                rs_dir, s2 = orc.reduce_scatter(xs, dtype, op, "allpairs")
                assert s1 == p - 1 and s2 == 1
                for r in range(p):
                    sl = slice(r * n_out, (r + 1) * n_out)
                    assert rs_ring[r].tobytes() == ar_ring[0][sl].tobytes(), (p, dtype, op, r)
                    assert rs_dir[r].tobytes() == ar_ap[0][sl].tobytes(), (p, dtype, op, r)
            # all-gather: concatenation, for both schedules
            small = [x[:n_out].copy() for x in xs]
            want = np.concatenate(small)
            for algo, steps in (("ring", p - 1), ("allpairs", 1)):
                ys, s = orc.all_gather(small, dtype, algo)
                assert s == steps
                for y in ys:
                    assert y.tobytes() == want.tobytes(), (p, dtype, algo)


def check_sampled(orc):
    rng = np.random.default_rng(41)
    for p, n in ((3, 100), (8, 8 * 33 + 5), (5, 4)):
        xs = [rng.standard_normal(n).astype(np.float32) for _ in range(p)]
        idx = rng.integers(0, n, 40).astype(np.int64)
        for algo in ALGOS:
            for op in ("sum", "prod", "avg"):
                ys, _ = orc.allreduce(xs, "fp32", op, algo)
                got = orc.allreduce_at(xs, "fp32", op, algo, idx)
                assert got.tobytes() == ys[0][idx].tobytes(), (p, n, algo, op)


# --------------------------------------------------------------------------
# Double binary tree, recursive exchange, 2PH.
# --------------------------------------------------------------------------
def _tree_from_golden():
    g = _golden("tree14.json")
    parent = [-1] * g["n"]
    for child, par in g["edges"]:
        parent[child] = par
    return g["n"], parent


def _children(parent):
    ch = {r: [] for r in range(len(parent))}
    for r, q in enumerate(parent):
        if q >= 0:
            ch[q].append(r)
    return {r: sorted(v) for r, v in ch.items()}


def _tree_ok(parent):
    """A spanning tree: one root, every rank reaches it without a cycle."""
    n = len(parent)
    roots = [r for r in range(n) if parent[r] == -1]
    assert len(roots) == 1, roots
    for r in range(n):
        seen, q = set(), r
        while q != -1:
            assert q not in seen and 0 <= q < n, (r, q)
            seen.add(q)
            q = parent[q]
    return roots[0]


def _f32_tree_total(vals, parent):
    """Own value first, then each child's subtree total, children ascending."""
    ch = _children(parent)
    root = _tree_ok(parent)

    def total(r):
        acc = np.float32(vals[r])
        for c in ch[r]:
            acc = np.float32(acc + total(c))
        return acc
    return total(root)


def _oracle_tree(orc, t, p, G):
    return [orc.tree_parent(t, p, G, r) for r in range(p)]


def check_tree_drawing(orc):
    """Tree one over 14 ranks is the tree the page draws, edge for edge."""
    n, parent = _tree_from_golden()
    assert _oracle_tree(orc, 0, n, 1) == parent


def check_dtree_listing(orc):
    """The 12-rank figure: interior/leaf split of both trees, tree two as
    the mirror image of tree one, and tree one's interior ranks in level
    order (levels top down, ascending inside a level)."""
    g = _golden("dtree12.json")
    n, k = g["n"], g["interior"]
    for t, listing in ((0, g["tree_one"]), (1, g["tree_two"])):
        ch = _children(_oracle_tree(orc, t, n, 1))
        interior = {r for r in range(n) if ch[r]}
        assert interior == set(listing[:k]), (t, interior)
        assert {r for r in range(n) if not ch[r]} == set(listing[k:]), t
    # the figure's own mirror relation: interior lists correspond rank for rank
    assert g["tree_two"][:k] == [n - 1 - r for r in g["tree_one"][:k]]
    parent = _oracle_tree(orc, 0, n, 1)
    ch = _children(parent)
    level, order = [_tree_ok(parent)], []
    while level:
        order += [r for r in level if ch[r]]
        level = sorted(c for r in level for c in ch[r])
    assert order == g["tree_one"][:k], order


def check_tree_shapes(orc):
    """For every node count: both trees span all ranks, binary, tree one's
    leaves are the odd ranks, height ceil(log2 n); with an even count every
    rank is interior in exactly one tree, with an odd count exactly one
    rank is interior in both."""
    for n in range(2, 65):
        both = None
        for t in (0, 1):
            parent = _oracle_tree(orc, t, n, 1)
            _tree_ok(parent)
            ch = _children(parent)
            assert max(len(v) for v in ch.values()) <= 2, (n, t)
            if t == 0:
                assert {r for r in range(n) if not ch[r]} == {r for r in range(1, n, 2)}, n
                depth = 0
                for r in range(n):
                    d, q = 0, r
                    while parent[q] != -1:
                        q, d = parent[q], d + 1
                    depth = max(depth, d)
                assert depth == (n - 1).bit_length(), (n, depth)
            inner = {r for r in range(n) if ch[r]}
            both = inner if both is None else both & inner
            if t == 1:
                union = both | inner
        interior_in_both = both
        if n % 2 == 0:
            assert not interior_in_both, (n, interior_in_both)
        else:
            assert len(interior_in_both) == 1, (n, interior_in_both)


def check_tree_chains(orc):
    """G ranks per node: rank kG+i (i > 0) hangs below kG+i-1; rank kG sits
    at node k's place in the node tree."""
    for p, G in ((8, 2), (12, 3), (16, 4), (12, 12), (6, 1)):
        for t in (0, 1):
            parent = _oracle_tree(orc, t, p, G)
            node = _oracle_tree(orc, t, p // G, 1) if p // G > 1 else [-1]
            for r in range(p):
                if r % G:
                    assert parent[r] == r - 1, (p, G, t, r)
                else:
                    want = node[r // G]
                    assert parent[r] == (-1 if want == -1 else want * G), (p, G, t, r)


def check_tree_rounds(orc):
    """The page's tree latency count 2((ranks per node - 1) + log2(nodes))
    hops, and its two printed cases: 16 nodes -> 8, 128 nodes -> 14."""
    for nodes, want in ((16, 8), (128, 14)):
        xs = [np.zeros(1, dtype=np.int32) for _ in range(nodes)]
        assert orc.allreduce(xs, "int32", "sum", "tree")[1] == want, nodes
    for p in range(2, 17):
        for G in range(1, p + 1):
            nodes = p // G
            if p % G or nodes & (nodes - 1):
                continue
            xs = [np.zeros(3, dtype=np.int32) for _ in range(p)]
            rounds = orc.allreduce(xs, "int32", "sum", "tree", ranks_per_node=G)[1]
            assert rounds == 2 * ((G - 1) + nodes.bit_length() - 1), (p, G, rounds)


def check_tree_association(orc):
    """fp32 sums: each half of the buffer is the tree total (own value, then
    children ascending) on its tree -- for 14 ranks the page's drawing and
    its mirror; elsewhere the oracle's trees, whose shapes the checks above
    pin."""
    rng = np.random.default_rng(61)
    n14, drawn = _tree_from_golden()
    mirror = [-1 if drawn[n14 - 1 - r] == -1 else n14 - 1 - drawn[n14 - 1 - r] for r in range(n14)]
    cases = [(n14, 1, drawn, mirror)]
    for p, G in ((5, 1), (8, 1), (9, 1), (16, 1), (8, 2), (12, 3), (6, 6)):
        cases.append((p, G, _oracle_tree(orc, 0, p, G), _oracle_tree(orc, 1, p, G)))
    for p, G, t0, t1 in cases:
        n = 41
        xs = [rng.standard_normal(n).astype(np.float32) for _ in range(p)]
        ys, _ = orc.allreduce(xs, "fp32", "sum", "tree", ranks_per_node=G)
        for i in range(n):
            parent = t0 if i < n // 2 else t1
            want = _f32_tree_total([x[i] for x in xs], parent)
            for y in ys:
                assert y[i] == want, (p, G, i)


def check_tree_chain_closed_form(orc):
    """One node (G = p): the tree is the chain 0 <- 1 <- ... <- p-1, so the
    result is x0 + (x1 + (... + x_{p-1})), a right fold; 2(p-1) rounds."""
    rng = np.random.default_rng(62)
    for p in (2, 3, 5, 8):
        xs = [rng.standard_normal(23).astype(np.float32) for _ in range(p)]
        ys, rounds = orc.allreduce(xs, "fp32", "sum", "tree", ranks_per_node=p)
        assert rounds == 2 * (p - 1)
        acc = xs[p - 1].copy()
        for q in range(p - 2, -1, -1):
            acc = (xs[q] + acc).astype(np.float32)
        for y in ys:
            assert y.tobytes() == acc.tobytes(), p


def _kary_closed_form(xs, k):
    """Consecutive blocks of k values folded left to right, repeated: the
    k-ary tree reduction over the rank order."""
    cur = [x.astype(np.float32) for x in xs]
    while len(cur) > 1:
        nxt = []
        for b in range(0, len(cur), k):
            acc = cur[b]
            for t in range(1, k):
                acc = (acc + cur[b + t]).astype(np.float32)
            nxt.append(acc)
        cur = nxt
    return cur[0]


def check_rexch(orc):
    """Recursive exchange: log_k p rounds; fp32 sums equal the k-ary tree
    reduction over consecutive rank blocks (digit 0 first); one round
    (p = k) is the plain left fold of the definition; p must be k^m."""
    rng = np.random.default_rng(63)
    for p, k in ((2, 2), (4, 2), (8, 2), (16, 2), (16, 4), (9, 3), (8, 8), (16, 16), (27, 3)):
        xs = [rng.standard_normal(37).astype(np.float32) for _ in range(p)]
        ys, rounds = orc.allreduce(xs, "fp32", "sum", "rexch", radix=k)
        m, v = 0, 1
        while v < p:
            v, m = v * k, m + 1
        assert rounds == m, (p, k, rounds)
        want = _kary_closed_form(xs, k)
        for y in ys:
            assert y.tobytes() == want.tobytes(), (p, k)
        if p == k:
            assert ys[0].tobytes() == orc.definition(xs, "fp32", "sum").tobytes()
    for p, k in ((6, 2), (8, 3), (12, 4)):
        xs = [np.zeros(4, dtype=np.int32) for _ in range(p)]
        try:
            orc.allreduce(xs, "int32", "sum", "rexch", radix=k)
        except ValueError:
            continue
        raise AssertionError(("accepted a rank count that is not a power of the radix", p, k))


def _hier_closed_form(xs, G, large):
    p = len(xs)
    nodes = p // G
    n = xs[0].size
    nch = p if large else G
    out = np.empty(n, dtype=np.float32)

    def partial(K, pos, i):
        acc = np.float32(xs[K * G + pos][i])
        for j in range(G):
            if j != pos:
                acc = np.float32(acc + xs[K * G + j][i])
        return acc
    for c, (lo, hi) in enumerate(chunk_bounds(n, nch)):
        for i in range(lo, hi):
            if large:
                K0, pos = divmod(c, G)
                order = [K0] + [K for K in range(nodes) if K != K0]
            else:
                pos, order = c, list(range(nodes))
            acc = partial(order[0], pos, i)
            for K in order[1:]:
                acc = np.float32(acc + partial(K, pos, i))
            out[i] = acc
    return out


def check_hier(orc):
    """2PH: one rank per node, small form = the plain definition (all-pairs
    across nodes, ascending), large form = the 2PA all-pairs; one node = the
    2PA all-pairs (the local reduce-scatter + all-gather); in between, the
    node partials of the page's description; round counts per phase."""
    rng = np.random.default_rng(64)
    for p in (2, 4, 6, 8):
        xs = [rng.standard_normal(29).astype(np.float32) for _ in range(p)]
        ap = orc.allreduce(xs, "fp32", "sum", "allpairs")[0][0]
        df = orc.definition(xs, "fp32", "sum")
        ys, r = orc.allreduce(xs, "fp32", "sum", "hier", ranks_per_node=1)
        assert r == 1 and all(y.tobytes() == df.tobytes() for y in ys), p
        ys, r = orc.allreduce(xs, "fp32", "sum", "hier_large", ranks_per_node=1)
        assert r == 2 and all(y.tobytes() == ap.tobytes() for y in ys), p
        for algo in ("hier", "hier_large"):
            ys, r = orc.allreduce(xs, "fp32", "sum", algo, ranks_per_node=p)
            assert r == 2 and all(y.tobytes() == ap.tobytes() for y in ys), (p, algo)
    for p, G in ((4, 2), (8, 2), (8, 4), (12, 3), (16, 4)):
        xs = [rng.standard_normal(3 * p + 5).astype(np.float32) for _ in range(p)]
        for algo, large, rounds in (("hier", False, 3), ("hier_large", True, 4)):
            ys, r = orc.allreduce(xs, "fp32", "sum", algo, ranks_per_node=G)
            assert r == rounds, (p, G, algo, r)
            want = _hier_closed_form(xs, G, large)
            for y in ys:
                assert y.tobytes() == want.tobytes(), (p, G, algo)


def check_topology_exact(orc):
    """Exactly-once and the exact integer ops (Python integers) for every
    topology schedule and several topologies, all ranks identical, in and
    out of place; the sampled entry point agrees."""
    rng = np.random.default_rng(65)
    for algo, p, topo in (("tree", 8, dict(ranks_per_node=1)), ("tree", 12, dict(ranks_per_node=3)),
                          ("tree", 7, dict(ranks_per_node=1)), ("rexch", 8, dict(radix=2)),
                          ("rexch", 9, dict(radix=3)), ("hier", 8, dict(ranks_per_node=2)),
                          ("hier", 12, dict(ranks_per_node=4)), ("hier_large", 8, dict(ranks_per_node=4)),
                          ("hier_large", 6, dict(ranks_per_node=3))):
        n = 5 * p + 3
        xs = [np.full(n, 1 << q, dtype=np.int32) for q in range(p)]
        for y in orc.allreduce(xs, "int32", "sum", algo, **topo)[0]:
            assert (y == (1 << p) - 1).all(), (algo, p, topo)
        xs = [rng.integers(-(2 ** 31), 2 ** 31 - 1, n, endpoint=True, dtype=np.int32) for _ in range(p)]
        cols = [[int(x[i]) for x in xs] for i in range(n)]
        want = {"sum": [_wrap32(sum(c)) for c in cols], "min": [min(c) for c in cols],
                "max": [max(c) for c in cols],
                "prod": [_wrap32(int(np.prod([Fraction(v) for v in c]))) for c in cols]}
        for op, w in want.items():
            ys, _ = orc.allreduce(xs, "int32", op, algo, **topo)
            for y in ys:
                assert y.tolist() == w, (algo, p, topo, op)
            ys2, _ = orc.allreduce([x.copy() for x in xs], "int32", op, algo, inplace=True, **topo)
            assert all(y.tolist() == w for y in ys2), (algo, p, topo, op, "inplace")
        x32 = [rng.standard_normal(n).astype(np.float32) for _ in range(p)]
        idx = rng.integers(0, n, 30).astype(np.int64)
        for op in ("sum", "avg", "prod"):
            ys, _ = orc.allreduce(x32, "fp32", op, algo, **topo)
            for y in ys[1:]:
                assert y.tobytes() == ys[0].tobytes(), (algo, op)
            assert orc.allreduce_at(x32, "fp32", op, algo, idx, **topo).tobytes() == ys[0][idx].tobytes()


ALL_CHECKS = [
    check_worked_example, check_step_counts, check_exactly_once, check_int_brute_force,
    check_fold_order_probes, check_identical_ranks, check_order_independent_fp,
    check_minmax_library, check_minmax_nan_and_signed_zero, check_p2_sum, check_avg, check_16bit_single_rounding,
    check_error_bound_16bit, check_rs_ag, check_sampled,
    check_tree_drawing, check_dtree_listing, check_tree_shapes, check_tree_chains, check_tree_rounds,
    check_tree_association, check_tree_chain_closed_form, check_rexch, check_hier, check_topology_exact,
]
