"""The written-out alpha-beta model against the printed worked example."""
import json
import os

from oracle import model

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "alpha_beta_example.json")))


def test_allpairs_wins_at_64KB():
    ta, tr = model.worked_example(65536, p=G["p"], link_Bps=G["link_GBps"] * 1e9, alpha_s=G["alpha_us"] * 1e-6)
    assert round(tr / ta, 2) == G["printed"]["allpairs_speedup_at_64KB"]


def test_crossover_near_4_2_MB():
    x = model.crossover_bytes(p=G["p"], link_Bps=G["link_GBps"] * 1e9, alpha_s=G["alpha_us"] * 1e-6)
    assert round(x / 2 ** 20, 1) == G["printed"]["crossover_MB_near"]
    ta, tr = model.worked_example(x)
    assert abs(ta - tr) / ta < 1e-12


def test_ring_wins_at_64MB():
    ta, tr = model.worked_example(64 * 2 ** 20)
    assert round(ta / tr, 1) == G["printed"]["ring_speedup_at_64MB_about"]


def test_step_terms():
    # with B -> infinity only the latency terms remain: 14 alphas vs 2 at p = 8
    assert model.t_ring(8, 0, 1.0, 1.0) == 14 and model.t_allpairs(8, 0, 1.0, 1.0) == 2
    # the bandwidth terms are identical
    assert model.t_ring(8, 1e6, 0, 1.0) == model.t_allpairs(8, 1e6, 0, 1.0) == 2 * 7 / 8 * 1e6
