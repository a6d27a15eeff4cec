"""The alpha-beta selector of the library (host only), against the
written-out model in oracle/model.py and the printed worked example."""
import json
import os

import pytest

import all_reduce_reduction_amd as sim
from oracle import model

G = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "alpha_beta_example.json")))


@pytest.fixture
def example_model():
    p = G["p"]
    k = 2 * (p - 1) / p
    # all-pairs with LL (half the link rate), ring with LL128 (120/128)
    sim.sim_model_set("allpairs", G["alpha_us"], 2, k, G["link_GBps"] * model.LL_EFFICIENCY)
    sim.sim_model_set("ring", G["alpha_us"], 2 * (p - 1), k, G["link_GBps"] * model.LL128_EFFICIENCY)
    yield
    sim.sim_model_reset()


@pytest.mark.parametrize("nbytes", [1024, 65536, 1 << 20, 4 << 20, 64 << 20, 1 << 30])
def test_predictions_match_the_written_out_model(example_model, nbytes):
    ta, tr = model.worked_example(nbytes)
    # sim_model_predict takes bytes per rank; fp32 elements
    assert sim.sim_model_predict("allpairs", 8, "fp32", nbytes) == pytest.approx(ta * 1e6, rel=1e-12)
    assert sim.sim_model_predict("ring", 8, "fp32", nbytes) == pytest.approx(tr * 1e6, rel=1e-12)


def test_printed_ratios(example_model):
    r64k = sim.sim_model_predict("ring", 8, "fp32", 65536) / sim.sim_model_predict("allpairs", 8, "fp32", 65536)
    assert round(r64k, 2) == G["printed"]["allpairs_speedup_at_64KB"]
    r64m = sim.sim_model_predict("allpairs", 8, "fp32", 64 << 20) / sim.sim_model_predict("ring", 8, "fp32", 64 << 20)
    assert round(r64m, 1) == G["printed"]["ring_speedup_at_64MB_about"]


def test_argmin_switches_at_the_crossover(example_model):
    # make the other schedules unattractive so the choice is ring vs all-pairs
    for other in ("oneshot", "oneshot_ll", "ring_fifo", "allpairs_persistent"):
        sim.sim_model_set(other, 1e9, -1, -1, 1.0)
    x = model.crossover_bytes()
    below = int(x * 0.98) // 4 * 4
    above = int(x * 1.02) // 4 * 4
    assert sim.sim_select(8, below // 4, "fp32")[0] == "allpairs"
    assert sim.sim_select(8, above // 4, "fp32")[0] == "ring"
    algo, us = sim.sim_select(8, (64 << 20) // 4, "fp32")
    assert algo == "ring" and us == pytest.approx(model.worked_example(64 << 20)[1] * 1e6)


def test_ll_is_never_picked_above_its_buffer():
    sim.sim_model_reset()
    sim.sim_model_set("oneshot_ll", 0.0, -1, -1, 1e9)   # LL would win everything
    try:
        assert sim.sim_select(8, 4096, "fp16")[0] == "oneshot_ll"
        assert sim.sim_select(8, (1 << 20) // 2, "fp16")[0] == "oneshot_ll"
        assert sim.sim_select(8, (1 << 20) // 2 + 1, "fp16")[0] != "oneshot_ll"
    finally:
        sim.sim_model_reset()


def test_builtin_traffic_laws():
    sim.sim_model_reset()
    for algo in ("ring", "allpairs", "oneshot", "oneshot_ll", "ring_fifo", "allpairs_persistent"):
        sim.sim_model_set(algo, 0.0, -1, -1, 1e-3)   # 1 MB/s: time in us == bytes
    S = 1 << 20
    n = S // 2
    assert sim.sim_model_predict("oneshot", 8, "bf16", S) == pytest.approx(2 * 8 * S)
    assert sim.sim_model_predict("allpairs", 8, "bf16", S) == pytest.approx(17 * S)
    assert sim.sim_model_predict("oneshot_ll", 8, "bf16", S) == pytest.approx(48 * S)
    # ring, 16-bit with fp32 partials: 94 bytes per element at p = 8
    assert sim.sim_model_predict("ring", 8, "bf16", S) == pytest.approx(94 * n)
    # ring, 32-bit: 5 (p-1) S
    assert sim.sim_model_predict("ring", 8, "fp32", S) == pytest.approx(35 * S)
    # the single-launch ring: inputs read and outputs written once (2pS), fp32
    # partials through the FIFOs (written and read, (p-1) n 8 bytes), finished
    # slices read from the predecessor's output ((p-1) n e bytes): 51 S at p = 8
    assert sim.sim_model_predict("ring_fifo", 8, "bf16", S) == pytest.approx(16 * S + 7 * n * 8 + 7 * n * 2)
    assert sim.sim_model_predict("ring_fifo", 8, "fp32", S) == pytest.approx(16 * S + 7 * (S // 4) * 12)
    # the single-launch all-pairs: step 1 reads pS and writes S; step 2 every
    # rank reads the p-1 other finished chunks and writes them: 23 S at p = 8
    assert sim.sim_model_predict("allpairs_persistent", 8, "bf16", S) == pytest.approx(23 * S)
    sim.sim_model_reset()


def test_model_json_roundtrip(tmp_path):
    f = tmp_path / "m.json"
    f.write_text(json.dumps({"device": "x", "algos": {"oneshot": {"alpha_us": 1.5, "gbps": 1000.0},
                                                       "ring": {"alpha_us": 2.0, "gbps": 2000.0}}}))
    sim.sim_model_load(str(f))
    try:
        assert sim.sim_model_predict("oneshot", 2, "fp32", 1000) == pytest.approx(1.5 + 4000 / 1e6)
        bad = tmp_path / "bad.json"
        bad.write_text('{"algos": {"ring": {"alpha_us": "x"}}}')
        with pytest.raises(sim.SimError):
            sim.sim_model_load(str(bad))
        with pytest.raises(sim.SimError):
            sim.sim_model_load(str(tmp_path / "missing.json"))
        good = '{"algos": {"ring": {"alpha_us": 2.0, "gbps": %s}}}'
        for text in (good % "Infinity", good % "inf", good % "nan", good % "-1e999", good % "0x10",
                     good % "1e999", good % "2000" + " x", good % "2000" + "{}"):
            bad.write_text(text)
            with pytest.raises(sim.SimError):
                sim.sim_model_load(str(bad))
        bad.write_text(good % "2.5e3" + "\n")
        sim.sim_model_load(str(bad))
        assert sim.sim_model_predict("ring", 2, "fp32", 1000) > 0
    finally:
        sim.sim_model_reset()


def test_packaged_calibration_loads_and_picks_oneshot():
    """The MI355X fit: on one HBM the fused one-shot moves the fewest bytes in
    one launch, so it is the model's pick at every evaluation size."""
    sim.sim_model_load(sim.CALIBRATION)
    try:
        for dtype, n in [("bf16", 8192 * t) for t in (1, 16, 256, 4096)] + [("fp16", (1 << k) // 2) for k in range(10, 21)]:
            assert sim.sim_select(8, n, dtype)[0] == "oneshot"
        rep = json.load(open(os.path.join(os.path.dirname(sim.CALIBRATION), "selector_check_mi355x.json")))
        assert rep["strict_matches"] == rep["cases"]
        # the committed check, under every workgroup budget it ran: the pick
        # is the measured fastest or within the measurement's tolerance of
        # it (under a budget, at 64 MiB per rank the fused one-shot and the
        # all-pairs come within 1-3% of each other), and the model orders at
        # least 90% of the pairs of schedules as measured
        assert set(rep["budgets"]) == {"none", "128", "32"}
        assert rep["budgets"]["none"]["strict_matches"] == rep["budgets"]["none"]["cases"]
        for b in rep["budgets"].values():
            assert b["tolerant_matches"] == b["cases"] == len(b["rows"])
            assert b["strict_matches"] >= b["cases"] - 2
            for r in b["rows"]:
                assert r["tolerant"]
            assert b["pairs_agree"] >= 0.9 * b["pairs"]
            # the model's pick among the schedules left once the measured
            # fastest is removed, against the measured one
            assert b["runner_up_strict"] >= 0.9 * b["cases"]
            assert all(r["runner_up_pick"] != r["measured_best"] for r in b["rows"])
        # unbudgeted, the pick's predicted time is within 5% of measured in the median case
        assert rep["budgets"]["none"]["pick_rel_error_median"] <= 0.05
        # the fitted per-workgroup rates are there, and a budget slows the one-shot's prediction
        model = json.load(open(sim.CALIBRATION))
        assert model["algos"]["oneshot"]["wg_gbps"] > 0
        t0 = sim.sim_model_predict("oneshot", 8, "bf16", 64 << 20)
        sim.sim_config_set("max_workgroups", 32)
        t32 = sim.sim_model_predict("oneshot", 8, "bf16", 64 << 20)
        sim.sim_config_set("max_workgroups", 0)
        assert t32 > 2 * t0
    finally:
        sim.sim_model_reset()


def test_launch_table_json(tmp_path):
    """The calibration's launch table ("workgroups") loads with the model;
    malformed tables are refused and leave the model as it was."""
    good = tmp_path / "wg.json"
    good.write_text(json.dumps({"algos": {"oneshot": {"alpha_us": 3.0, "gbps": 5000.0}},
                                "workgroups": {"oneshot": [[1048576, 0], [67108864, 4096, 2]],
                                               "ring": [[4096, 64, 1]]}}))
    try:
        sim.sim_model_load(str(good))
        assert sim.sim_model_predict("oneshot", 8, "bf16", 1 << 20) == pytest.approx(
            3.0 + 16 * (1 << 20) / 5000.0e3)
        for table in ('{"oneshot": [[0, 10]]}', '{"oneshot": [[4096, -1]]}', '{"oneshot": [4096, 16]}',
                      '{"oneshot": {"4096": 16}}', '[1, 2]', '{"oneshot": [[4096, 16, 3]]}',
                      '{"oneshot": [[4096, 16, 0]]}', '{"oneshot": [[4096, 16, "2"]]}',
                      '{"oneshot": [[4096, 16, 2, 1]]}'):
            bad = tmp_path / "bad.json"
            bad.write_text('{"algos": {"oneshot": {"alpha_us": 9.0, "gbps": 1.0}}, "workgroups": %s}' % table)
            with pytest.raises(sim.SimError):
                sim.sim_model_load(str(bad))
            # the refused file changed nothing
            assert sim.sim_model_predict("oneshot", 8, "bf16", 1 << 20) == pytest.approx(
                3.0 + 16 * (1 << 20) / 5000.0e3)
        # the rank count the table was measured at: an integer in 2..16
        for pv in ('1', '17', '2.5', '"8"', '[8]', '-8'):
            bad = tmp_path / "bad.json"
            bad.write_text('{"p": %s, "algos": {"oneshot": {"alpha_us": 9.0, "gbps": 1.0}}}' % pv)
            with pytest.raises(sim.SimError):
                sim.sim_model_load(str(bad))
            assert sim.sim_model_predict("oneshot", 8, "bf16", 1 << 20) == pytest.approx(
                3.0 + 16 * (1 << 20) / 5000.0e3)
        ok = tmp_path / "ok.json"
        ok.write_text('{"p": 8, "algos": {"oneshot": {"alpha_us": 9.0, "gbps": 1.0}}}')
        sim.sim_model_load(str(ok))
        assert sim.sim_model_predict("oneshot", 8, "bf16", 1 << 20) == pytest.approx(9.0 + 16 * (1 << 20) / 1e3)
    finally:
        sim.sim_model_reset()


def test_unroll_debug_hook_range():
    assert sim.sim_debug_get("unroll") == 0  # default: the launch table decides
    for v in (1, 2, 4, 0):
        sim.sim_debug_set("unroll", v)
        assert sim.sim_debug_get("unroll") == v
    for v in (3, 5):
        with pytest.raises(sim.SimError):
            sim.sim_debug_set("unroll", v)


def test_workgroup_budget_config():
    assert sim.sim_config_get("max_workgroups") == 0
    try:
        sim.sim_config_set("max_workgroups", 64)
        assert sim.sim_config_get("max_workgroups") == 64
        with pytest.raises(sim.SimError):
            sim.sim_config_set("max_workgroups", -1)
        assert sim.sim_config_get("max_workgroups") == 64
    finally:
        sim.sim_config_set("max_workgroups", 0)


def _smooth_min(b, w, rate):
    # written out independently of the library: 1 / B_eff^3 = 1 / B^3 + 1 / (W b)^3
    return 1.0 / ((1.0 / b ** 3 + 1.0 / (w * rate) ** 3) ** (1.0 / 3.0))


def test_budget_term_prices_and_flips_the_argmin():
    """Under a workgroup budget an algo with a per-workgroup rate is priced
    with the smooth minimum of B and W b; without one (or with rate 0) the
    budget changes nothing.  A schedule that needs fewer bytes but sustains
    little per workgroup loses to one that streams faster per workgroup once
    the budget is tight."""
    sim.sim_model_reset()
    S = 64 << 20
    try:
        for other in ("ring", "oneshot_ll", "ring_fifo", "allpairs_persistent"):
            sim.sim_model_set(other, 1e9, -1, -1, 1.0)
        sim.sim_model_set("oneshot", 3.0, -1, -1, 6000.0)
        sim.sim_model_set("allpairs", 3.0, -1, -1, 5000.0)
        sim.sim_model_set_workgroup_rate("oneshot", 40.0)
        sim.sim_model_set_workgroup_rate("allpairs", 120.0)
        assert sim.sim_select(8, S // 2, "bf16")[0] == "oneshot"
        assert sim.sim_model_predict("oneshot", 8, "bf16", S) == pytest.approx(3.0 + 16 * S / 6000e3)
        sim.sim_config_set("max_workgroups", 32)
        t1 = sim.sim_model_predict("oneshot", 8, "bf16", S)
        t2 = sim.sim_model_predict("allpairs", 8, "bf16", S)
        assert t1 == pytest.approx(3.0 + 16 * S / (_smooth_min(6000.0, 32, 40.0) * 1e3), rel=1e-12)
        assert t2 == pytest.approx(2 * 3.0 + 17 * S / (_smooth_min(5000.0, 32, 120.0) * 1e3), rel=1e-12)
        algo, us = sim.sim_select(8, S // 2, "bf16")
        assert algo == "allpairs" and us == pytest.approx(t2)
        # a generous budget hardly matters: 4096 workgroups sustain far more than B
        sim.sim_config_set("max_workgroups", 4096)
        assert sim.sim_select(8, S // 2, "bf16")[0] == "oneshot"
        # rate 0 removes the term
        sim.sim_config_set("max_workgroups", 32)
        sim.sim_model_set_workgroup_rate("oneshot", 0.0)
        assert sim.sim_model_predict("oneshot", 8, "bf16", S) == pytest.approx(3.0 + 16 * S / 6000e3)
        # the single-launch schedules keep one workgroup per rank: W = max(budget, p)
        sim.sim_model_set("allpairs_persistent", 6.0, -1, -1, 6500.0)
        sim.sim_model_set_workgroup_rate("allpairs_persistent", 50.0)
        sim.sim_config_set("max_workgroups", 2)
        assert sim.sim_model_predict("allpairs_persistent", 8, "bf16", S) == pytest.approx(
            6.0 + 23 * S / (_smooth_min(6500.0, 8, 50.0) * 1e3), rel=1e-12)
        with pytest.raises(sim.SimError):
            sim.sim_model_set_workgroup_rate("oneshot", -1.0)
        with pytest.raises(sim.SimError):
            sim.sim_model_set_workgroup_rate("auto", 1.0)
    finally:
        sim.sim_config_set("max_workgroups", 0)
        sim.sim_model_reset()


def test_budget_rate_json(tmp_path):
    f = tmp_path / "m.json"
    f.write_text(json.dumps({"algos": {"oneshot": {"alpha_us": 3.0, "gbps": 6000.0, "wg_gbps": 40.0}}}))
    try:
        sim.sim_model_load(str(f))
        S = 1 << 26
        sim.sim_config_set("max_workgroups", 64)
        assert sim.sim_model_predict("oneshot", 8, "bf16", S) == pytest.approx(
            3.0 + 16 * S / (_smooth_min(6000.0, 64, 40.0) * 1e3), rel=1e-12)
        for bad in ('"x"', "-1", "null"):
            f.write_text('{"algos": {"oneshot": {"alpha_us": 1.0, "gbps": 1.0, "wg_gbps": %s}}}' % bad)
            with pytest.raises(sim.SimError):
                sim.sim_model_load(str(f))
        # the refused files changed nothing
        assert sim.sim_model_predict("oneshot", 8, "bf16", S) == pytest.approx(
            3.0 + 16 * S / (_smooth_min(6000.0, 64, 40.0) * 1e3), rel=1e-12)
    finally:
        sim.sim_config_set("max_workgroups", 0)
        sim.sim_model_reset()


def test_host_overlap_term():
    """With a host enqueue cost H per launch a call costs max(H L, alpha L +
    bytes / B); sim_model_set restores the additive form; the file's
    host_us loads and is validated."""
    sim.sim_model_reset()
    try:
        sim.sim_model_set("oneshot", 1.0, -1, -1, 5000.0)
        sim.sim_model_set_host_overlap("oneshot", 3.0)
        small, large = 4096, 64 << 20
        assert sim.sim_model_predict("oneshot", 8, "bf16", small) == pytest.approx(3.0)
        assert sim.sim_model_predict("oneshot", 8, "bf16", large) == pytest.approx(1.0 + 16 * large / 5000e3)
        sim.sim_model_set("ring", 1.0, -1, -1, 5000.0)
        sim.sim_model_set_host_overlap("ring", 2.5)   # 14 launches at p = 8
        assert sim.sim_model_predict("ring", 8, "bf16", small) == pytest.approx(14 * 2.5)
        sim.sim_model_set("oneshot", 1.0, -1, -1, 5000.0)   # clears the host term
        assert sim.sim_model_predict("oneshot", 8, "bf16", small) == pytest.approx(1.0 + 16 * small / 5000e3)
        with pytest.raises(sim.SimError):
            sim.sim_model_set_host_overlap("oneshot", -1.0)
    finally:
        sim.sim_model_reset()


def test_host_overlap_json(tmp_path):
    f = tmp_path / "m.json"
    f.write_text(json.dumps({"algos": {"oneshot": {"alpha_us": 1.0, "gbps": 5000.0, "host_us": 3.0}}}))
    try:
        sim.sim_model_load(str(f))
        assert sim.sim_model_predict("oneshot", 8, "bf16", 4096) == pytest.approx(3.0)
        for bad in ('"x"', "-2", "null"):
            f.write_text('{"algos": {"oneshot": {"alpha_us": 1.0, "gbps": 1.0, "host_us": %s}}}' % bad)
            with pytest.raises(sim.SimError):
                sim.sim_model_load(str(f))
        assert sim.sim_model_predict("oneshot", 8, "bf16", 4096) == pytest.approx(3.0)
    finally:
        sim.sim_model_reset()


def test_second_regime_prices_from_the_switch(tmp_path):
    """An "algos_hi" entry prices the one-shot from the size where it runs
    phased (per rank count; never under a budget or when switched off) and
    the single-launch ring above its LL limit; sim_model_set and a file
    entry without "algos_hi" go back to one entry for every size."""
    f = tmp_path / "m.json"
    lo_os, hi_os = {"alpha_us": 2.0, "gbps": 5000.0}, {"alpha_us": 4.0, "gbps": 6400.0}
    lo_rf, hi_rf = {"alpha_us": 10.0, "gbps": 3000.0}, {"alpha_us": 20.0, "gbps": 6000.0}
    f.write_text(json.dumps({"algos": {"oneshot": lo_os, "ring_fifo": lo_rf},
                             "algos_hi": {"oneshot": hi_os, "ring_fifo": hi_rf}}))

    def t(e, p, S, law):  # one launch, law bytes per message byte
        return e["alpha_us"] + law * S / (e["gbps"] * 1e3)

    try:
        sim.sim_model_load(str(f))
        MIN = sim.sim_debug_get("phased_min")
        pr = lambda algo, p, S: sim.sim_model_predict(algo, p, "bf16", S)
        # phased from 3/4 of the unit at p = 8, 1 at p = 4, 1/2 at p = 16, never at p = 2
        T8 = MIN * 3 // 4
        assert pr("oneshot", 8, T8 - 2) == pytest.approx(t(lo_os, 8, T8 - 2, 16))
        assert pr("oneshot", 8, T8) == pytest.approx(t(hi_os, 8, T8, 16))
        assert pr("oneshot", 4, MIN - 2) == pytest.approx(t(lo_os, 4, MIN - 2, 8))
        assert pr("oneshot", 4, MIN) == pytest.approx(t(hi_os, 4, MIN, 8))
        assert pr("oneshot", 2, 8 * MIN) == pytest.approx(t(lo_os, 2, 8 * MIN, 4))
        assert pr("oneshot", 16, MIN // 2) == pytest.approx(t(hi_os, 16, MIN // 2, 32))
        try:
            sim.sim_config_set("max_workgroups", 64)  # no per-workgroup rate: B as it is
            assert pr("oneshot", 8, 4 * MIN) == pytest.approx(t(lo_os, 8, 4 * MIN, 16))
        finally:
            sim.sim_config_set("max_workgroups", 0)
        for mode, S, e in ((2, 4 * MIN, lo_os), (1, 4096, hi_os)):
            try:
                sim.sim_debug_set("phased", mode)
                assert pr("oneshot", 8, S) == pytest.approx(t(e, 8, S, 16))
            finally:
                sim.sim_debug_set("phased", 0)
        # the single-launch ring moves 51 S at p = 8 in bf16 (2pS + (p-1) 8 n + (p-1) 2 n, n = S / 2)
        LL = sim.sim_debug_get("ring_ll_max")
        assert pr("ring_fifo", 8, LL) == pytest.approx(t(lo_rf, 8, LL, 51))
        assert pr("ring_fifo", 8, LL + 16) == pytest.approx(t(hi_rf, 8, LL + 16, 51))
        # one entry for every size again
        sim.sim_model_set("oneshot", 2.0, -1, -1, 5000.0)
        assert pr("oneshot", 8, 4 * MIN) == pytest.approx(t(lo_os, 8, 4 * MIN, 16))
        assert pr("ring_fifo", 8, LL + 16) == pytest.approx(t(hi_rf, 8, LL + 16, 51))
        f.write_text(json.dumps({"algos": {"ring_fifo": lo_rf}}))
        sim.sim_model_load(str(f))
        assert pr("ring_fifo", 8, LL + 16) == pytest.approx(t(lo_rf, 8, LL + 16, 51))
        # a bad second entry is refused and changes nothing
        for bad in ('[]', '{"oneshot": {"alpha_us": 1.0}}', '{"oneshot": {"alpha_us": -1.0, "gbps": 1.0}}'):
            f.write_text('{"algos": {"oneshot": {"alpha_us": 9.0, "gbps": 9.0}}, "algos_hi": %s}' % bad)
            with pytest.raises(sim.SimError):
                sim.sim_model_load(str(f))
        assert pr("ring_fifo", 8, LL + 16) == pytest.approx(t(lo_rf, 8, LL + 16, 51))
    finally:
        sim.sim_model_reset()
