"""Planted mistakes in the oracle must be caught by its pins.

Each mutant is a copy of oracle/oracle.c with one plausible mistake (a wrong
chunk index, a dropped term, a transposed operand, a wrong rounding rule),
compiled with the same gcc flags into a temporary directory and run against
every pin in tests/oracle_pins.py in a child process.  The child must report
a failing pin (or die); a mutant that passes every pin would mean the pins
cannot see that mistake.  Everything runs on the CPU.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = open(os.path.join(ROOT, "oracle", "oracle.c")).read()

MUTANTS = {
    "ring_send_chunk": ("const int ch = ((r - 1 - s) % p + p) % p;    /* chunk rank r sends */",
                        "const int ch = ((r - s) % p + p) % p;    /* chunk rank r sends */"),
    "ring_local_operand": ("acc_t v = combine(c, a, pre(c, X[d], i));",
                           "acc_t v = combine(c, a, pre(c, X[r], i));"),
    "ring_post_step": ("if (s == p - 2) {\n          /* the chunk", "if (s == 0) {\n          /* the chunk"),
    "ring_first_operand": ("acc_t a = (s == 0) ? pre(c, X[r], i) : Pr[i];",
                           "acc_t a = (s == 0) ? pre(c, X[d], i) : Pr[i];"),
    "ag_forward_chunk": ("const int ch = ((r - s) % p + p) % p;\n      const int d = (r + 1) % p;\n      const int64_t lo = chunk_lo(n, p, ch), hi = chunk_lo(n, p, ch + 1);\n      memcpy",
                         "const int ch = ((r - 1 - s) % p + p) % p;\n      const int d = (r + 1) % p;\n      const int64_t lo = chunk_lo(n, p, ch), hi = chunk_lo(n, p, ch + 1);\n      memcpy"),
    "allpairs_drop_last_rank": ("if (q == j) continue;\n      v = combine", "if (q == j || q == p - 1) continue;\n      v = combine"),
    "allpairs_start_rank0": ("acc_t v = pre(c, X[j], i);\n    for (int q = 0; q < p; q++) {\n      if (q == j) continue;",
                             "acc_t v = pre(c, X[0], i);\n    for (int q = 0; q < p; q++) {\n      if (q == 0) continue;"),
    "allpairs_fanout_missing": ("if (r == j) continue;\n      memcpy", "if (r != (j + 1) % p) continue;\n      memcpy"),
    "min_operands_swapped": ("case OR_MIN: r.i = (b.i < a.i) ? b.i : a.i; break;",
                             "case OR_MIN: r.i = (b.i < a.i) ? a.i : b.i; break;"),
    "fp_max_is_min": ("default:     r.f = (b.f > a.f) ? b.f : a.f; break;",
                      "default:     r.f = (b.f < a.f) ? b.f : a.f; break;"),
    "fp_min_ties_take_operand": ("case OR_MIN: r.f = (b.f < a.f) ? b.f : a.f; break;",
                                 "case OR_MIN: r.f = (b.f <= a.f) ? b.f : a.f; break;"),
    "fp_min_replaces_nan_accumulator": ("case OR_MIN: r.f = (b.f < a.f) ? b.f : a.f; break;",
                                        "case OR_MIN: r.f = (b.f < a.f || a.f != a.f) ? b.f : a.f; break;"),
    "int_prod_is_sum": ("case OR_PROD: r.u = a.u * b.u; break;", "case OR_PROD: r.u = a.u + b.u; break;"),
    "int_avg_no_divide": ("(c->op == OR_AVG) ? (int32_t)(v.i / c->p) : v.i", "v.i"),
    "fp_avg_not_scaled": ("a.f = scaled;", "(void)scaled;"),
    "fp_avg_scaled_twice": ("a.f = scaled;", "a.f = scaled * c->inv_p;"),
    "bf16_truncates": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;", ""),
    "bf16_ties_away": ("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)"),
    "f16_subnormal_shift": ("int shift = 14 - e16;", "int shift = 13 - e16;"),
    "f16_decode_subnormal_scale": ("float v = (float)m * u2f(0x33800000u);", "float v = (float)m * u2f(0x34000000u);"),
    "f16_exponent_bias": ("int e16 = (int)exp - 127 + 15;", "int e16 = (int)exp - 127 + 16;"),
    "sampled_ring_start": ("v = pre(&c, X[(ch + 1) % p], i);", "v = pre(&c, X[ch], i);"),
    "tree_children_descending": ("for (int q = 0; q < c->p; q++)\n    if (q != r && T->parent[t][q] == r)",
                                 "for (int q = c->p - 1; q >= 0; q--)\n    if (q != r && T->parent[t][q] == r)"),
    "tree_children_before_own": ("acc_t v = pre(c, X[r], i);\n  for (int q = 0; q < c->p; q++)\n    if (q != r && T->parent[t][q] == r) v = combine(c, v, subtree(c, T, X, t, q, i));\n  return v;",
                                 "acc_t v = pre(c, X[r], i);\n  int first = 1; acc_t w = v;\n  for (int q = 0; q < c->p; q++)\n    if (q != r && T->parent[t][q] == r) { w = first ? subtree(c, T, X, t, q, i) : combine(c, w, subtree(c, T, X, t, q, i)); first = 0; }\n  return first ? v : combine(c, w, v);"),
    "tree_no_range_fallback": ("if (up >= n) up = x & ~b;", "if (up >= n) up = 0;"),
    "tree_mirror_as_shift": ("if (n % 2 == 0) {\n    int q = bittree_parent(n, n - 1 - x);",
                             "if (n % 2 == 2) {\n    int q = bittree_parent(n, n - 1 - x);"),
    "tree_chain_reversed": ("if (r % G != 0) { T->parent[t][r] = r - 1; continue; }",
                            "if (r % G != G - 1) { T->parent[t][r] = r + 1; continue; }"),
    "tree_one_tree_only": ("return subtree(c, T, X, ch, root, i);", "return subtree(c, T, X, 0, 0, i);"),
    "rexch_high_digit_first": ("for (int stride = 1; stride < p; stride *= T->k) {",
                               "for (int stride = p / T->k; stride >= 1; stride /= T->k) {"),
    "rexch_group_descending": ("acc_t a = v[first];\n          for (int m = 1; m < T->k; m++) a = combine(c, a, v[first + m * stride]);",
                               "acc_t a = v[first + (T->k - 1) * stride];\n          for (int m = T->k - 2; m >= 0; m--) a = combine(c, a, v[first + m * stride]);"),
    "hier_nodes_descending": ("acc_t a = node_partial(c, T->G, X, 0, ch, i);\n      for (int K = 1; K < p / T->G; K++)",
                              "acc_t a = node_partial(c, T->G, X, p / T->G - 1, ch, i);\n      for (int K = p / T->G - 2; K >= 0; K--)"),
    "hier_node_partial_from_node_start": ("acc_t v = pre(c, X[K * G + pos], i);\n  for (int j = 0; j < G; j++)\n    if (j != pos)",
                                          "acc_t v = pre(c, X[K * G], i);\n  for (int j = 0; j < G; j++)\n    if (j != 0)"),
    "hier_large_owner_not_first": ("acc_t a = node_partial(c, T->G, X, K0, pos, i);\n      for (int K = 0; K < p / T->G; K++)\n        if (K != K0)",
                                   "acc_t a = node_partial(c, T->G, X, 0, pos, i);\n      for (int K = 0; K < p / T->G; K++)\n        if (K != 0)"),
    "hier_rounds_no_local_ag": ("return (T->algo == OR_HIER) ? 2 * local + cross : 2 * local + 2 * cross;",
                                "return (T->algo == OR_HIER) ? local + cross : 2 * local + 2 * cross;"),
    "rs_direct_offset": ("allpairs_fold_chunk(&c, X, Y[j], n, j, chunk_lo(n, p, j));",
                         "allpairs_fold_chunk(&c, X, Y[j], n, (j + 1) % p, chunk_lo(n, p, (j + 1) % p));"),
}

RUNNER = r"""
import sys
sys.path.insert(0, {root!r})
from oracle import Oracle
from tests import oracle_pins
orc = Oracle({lib!r})
for check in oracle_pins.ALL_CHECKS:
    try:
        check(orc)
    except AssertionError:
        print("caught by", check.__name__)
        sys.exit(1)
print("NOT CAUGHT")
sys.exit(0)
"""


def _run_mutant(name, tmp):
    old, new = MUTANTS[name]
    assert SRC.count(old) >= 1, f"mutation site for {name} not found in oracle.c"
    src = SRC.replace(old, new, 1)
    d = os.path.join(tmp, name)
    os.makedirs(d, exist_ok=True)
    cpath, lib = os.path.join(d, "oracle.c"), os.path.join(d, "liboracle.so")
    open(cpath, "w").write(src)
    sys.path.insert(0, ROOT)
    import oracle
    oracle.build(cpath, lib)
    r = subprocess.run([sys.executable, "-c", RUNNER.format(root=ROOT, lib=lib)],
                       capture_output=True, text=True, timeout=300,
                       env={**os.environ, "OMP_NUM_THREADS": "1"})
    return r.returncode, r.stdout + r.stderr[-2000:]


@pytest.fixture(scope="module")
def mutant_results(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("mutants"))
    with ThreadPoolExecutor(max_workers=6) as ex:
        futs = {name: ex.submit(_run_mutant, name, tmp) for name in MUTANTS}
        return {name: f.result() for name, f in futs.items()}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(mutant_results, name):
    rc, out = mutant_results[name]
    assert rc != 0, f"mutant {name} passed every pin:\n{out}"
