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
ALGOS = ("ring", "allpairs", "oneshot", "oneshot_ll", "ring_fifo")


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
        for algo in ("allpairs", "oneshot", "oneshot_ll"):
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


ALL_CHECKS = [
    check_worked_example, check_step_counts, check_exactly_once, check_int_brute_force,
    check_fold_order_probes, check_identical_ranks, check_order_independent_fp,
    check_minmax_library, check_p2_sum, check_avg, check_16bit_single_rounding,
    check_error_bound_16bit, check_rs_ag, check_sampled,
]
