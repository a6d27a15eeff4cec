"""Host logic of the calibration and the bench (no GPU): the fits recover
the parameters of synthetic timings generated from known models, and the
bench's traffic laws equal the library's own."""

import pytest

import all_reduce_reduction_amd as sim
from all_reduce_reduction_amd import calibrate as cal

SIZES = [int(1.5 * (1 << k)) // 16 * 16 for k in range(10, 28)]


def _points(launches, alpha, gbps, host=0.0, per_byte=16.0):
    """(launches, traffic bytes, us) of T = max(H L, alpha L + bytes / B)."""
    pts = []
    for nb in SIZES:
        tb = per_byte * nb
        pts.append((launches, tb, max(host * launches, alpha * launches + tb / (gbps * 1e3))))
    return pts


def test_additive_fit_recovers_alpha_and_b():
    alpha, gbps = cal.fit(_points(2, 2.5, 5700.0), "x")
    assert alpha == pytest.approx(2.5, rel=0.02)
    assert gbps == pytest.approx(5700.0, rel=0.02)


def test_pipelined_fit_recovers_the_host_term():
    h, alpha, gbps = cal.fit_host(_points(1, 1.2, 5700.0, host=3.1), "x")
    assert h == pytest.approx(3.1, rel=1e-6)
    assert gbps == pytest.approx(5700.0, rel=0.03)
    assert alpha == pytest.approx(1.2, abs=0.3)


def test_pipelined_form_is_dropped_when_the_floor_is_the_kernel():
    # a schedule whose small-size floor is its own kernel time: additive data
    h, alpha, gbps = cal.fit_host(_points(1, 8.6, 13000.0, per_byte=48.0), "x")
    assert h == 0.0
    assert alpha == pytest.approx(8.6, rel=0.02)


def test_budget_rate_inverts_the_smooth_minimum():
    b, rate = 5700.0, 49.0
    obs = [(w, (b ** -3 + (w * rate) ** -3) ** (-1 / 3)) for w in (16, 32, 64, 128)]
    assert cal.fit_wg_rate(obs, b) == pytest.approx(rate, rel=1e-9)
    # no budget binds: no term
    assert cal.fit_wg_rate([(4096, b), (8192, b)], b) == 0.0


def test_pairs_agree_counts_ties_and_inversions():
    meas = {"a": 1.0, "b": 2.0, "c": 2.01}
    assert cal._pairs_agree({"a": 1.0, "b": 2.0, "c": 3.0}, meas, 0.03) == (3, 3)
    # b and c tie within 3%, so only the inverted (a, b) and (a, c) pairs disagree
    assert cal._pairs_agree({"a": 5.0, "b": 2.0, "c": 1.0}, meas, 0.03) == (1, 3)


@pytest.mark.parametrize("algo", ["oneshot", "allpairs", "ring", "ring_fifo", "allpairs_persistent"])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_bench_laws_equal_the_library_laws(algo, dtype):
    import bench
    e = 2 if dtype == "bf16" else 4
    n = 33_554_432
    sim.sim_model_set(algo, 0.0, -1, -1, 1e-3)  # 1 MB/s: predicted us == bytes
    try:
        lib = sim.sim_model_predict(algo, 8, dtype, n * e)
    finally:
        sim.sim_model_reset()
    assert bench.algorithmic_bytes_at(algo, n, e) == pytest.approx(lib, rel=1e-12)
    if dtype == "bf16":
        assert bench.algorithmic_bytes(algo) == pytest.approx(lib, rel=1e-12)
