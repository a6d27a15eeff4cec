"""Calibrate the alpha-beta model on this GPU and check the selector.

The cost model ("MSCCL, in depth ...", section "Why generic collectives
leave time on the table"; "Inside NCCL all-reduce", section "How NCCL
picks: a cost model, not a threshold") prices a schedule as
    T_a = alpha_a * launches_a(p) + traffic_a(p, n, dtype) / B_a,
linear in (alpha_a, 1/B_a).  This sweep times every schedule on a grid of
message sizes that sits BETWEEN the evaluation sizes (powers of two times
1.5, 1 KiB .. 192 MiB per rank, p = 8, bf16), fits alpha_a and B_a by least
squares with relative weights (so microsecond and millisecond points count
alike), and writes the JSON file sim_model_load() reads.

The fit is a two-regime estimate (see fit()).  The one-shot and the
single-launch ring change kernels with the size (phased form, FIFO
protocol); each of them gets a second entry ("algos_hi") fitted on the
sizes of its second regime.  A launch-configuration sweep
(sweep_workgroups) then stores the best (total workgroups, 16-byte vectors
per lane) per size for the bulk schedules.  --check then times every legal schedule at the evaluation sizes (8192 x
{1, 16, 256, 4096} tokens bf16, and 1 KiB .. 1 MiB fp16) and compares the
selector's pick with the measured fastest: a strict match, and a tolerant
match when the pick is within max(3%, the measured spread) of the best.

Workgroup budgets (T-CCL's restricted mode, "T-CCL ...", sections III-C3
and IV-B): sweep_budget() times each schedule at a bandwidth-bound size
under budgets of 16 .. 128 workgroups and fits the rate one workgroup
sustains (wg_gbps), which the model uses under a budget (see sim_select in
include/simar.h).  The check runs at budgets none, 128 and 32.  Besides the
argmin it reports, per case, every schedule's predicted and measured time,
the relative error of each prediction, how many pairs of schedules the
model ranks in the measured order (pairs measured within the tolerance of
each other count as ties), and the runner-up: the model's argmin over the
schedules left once the measured fastest is removed, against the measured
one.  On one HBM the one-shot is expected to be the fastest at every size,
so the argmin alone could not tell a working model from a constant pick;
the pairwise ranking and the errors can.  (On MI355X the measured runner-up
is the two-launch all-pairs at every checked size and budget, so it adds one
ordering, not a test of its own.)

Buffers: every measurement rotates over up to 8 sets of rank buffers, as
many as keep the working set of consecutive calls at 512 MiB or more
(above the 256 MB Infinity Cache) while the sets fit, so sizes from 4 MiB
per rank up are timed from HBM as calls that touch fresh data would be;
below that the whole rotation still fits the cache.

Run on the GPU:  python -m all_reduce_reduction_amd.calibrate [--check]
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
DEFAULT_OUT = os.path.join(HERE, "calib", "mi355x.json")
ALGOS = ("ring", "allpairs", "oneshot", "oneshot_ll", "ring_fifo", "allpairs_persistent")
# Schedules whose kernels change with the size, fitted as two regimes
# ("algos" below the switch, "algos_hi" from it): the one-shot's fused and
# phased forms, the single-launch ring's LL and FIFO protocols.
REGIMES = ("oneshot", "ring_fifo")
# The topology schedules are fitted too (sim_model_predict prices them),
# each at the topology stated here; AUTO does not weigh them.
TOPOLOGY = {"tree": (1, 2), "rexch": (1, 2), "hier": (4, 2), "hier_large": (4, 2)}  # (ranks per node, radix)
P = 8


def set_topology(sim, algo):
    g, k = TOPOLOGY.get(algo, (1, 2))
    sim.sim_config_set("ranks_per_node", g)
    sim.sim_config_set("radix", k)


def _timer():
    import torch

    def run(fn, steps, warmup, reps=5):
        for _ in range(warmup):
            fn()
        out = []
        for _ in range(reps):
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(steps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            out.append(e0.elapsed_time(e1) * 1e3 / steps)  # microseconds
        return statistics.median(out), (max(out) - min(out)) / statistics.median(out)
    return run


class Bench:
    """Device buffers for p ranks: set 0 holds the largest size, sets 1..7
    up to ROT_SET_BYTES per rank; calls rotate over the sets (see the module
    docstring)."""

    ROT_BYTES = 512 << 20      # working set the rotation aims for
    ROT_SET_BYTES = 32 << 20   # bytes per rank of the extra sets
    MAX_SETS = 8

    def __init__(self, max_bytes: int, steps_scale: float = 1.0):
        import torch
        import all_reduce_reduction_amd as sim
        self.sim = sim
        dev = torch.device("cuda:0")
        self.sets = []
        for k in range(self.MAX_SETS):
            cap = max_bytes if k == 0 else min(max_bytes, self.ROT_SET_BYTES)
            ins = [torch.randint(-3000, 3000, (cap // 2,), dtype=torch.int16, device=dev) for _ in range(P)]
            outs = [torch.empty_like(ins[0]) for _ in range(P)]
            self.sets.append((cap, ins, outs))
        self.stream = int(torch.cuda.current_stream().cuda_stream)
        self.time = _timer()
        self.steps_scale = steps_scale

    def legal(self, algo, nbytes):
        return algo != "oneshot_ll" or nbytes <= self.sim.LL_MAX_BYTES_PER_RANK

    def nsets(self, nbytes: int) -> int:
        want = -(-self.ROT_BYTES // (2 * P * max(nbytes, 1)))
        fit = sum(1 for cap, _, _ in self.sets if cap >= nbytes)
        return max(1, min(self.MAX_SETS, want, fit))

    def measure(self, algo, dtype, n, reps=5):
        sim = self.sim
        nbytes = n * sim.ESIZE[dtype]
        steps = max(5, min(2000, int(2e5 / max(1.0, nbytes / 4e3) * self.steps_scale)))
        calls = []
        for cap, ins, outs in self.sets[:self.nsets(nbytes)]:
            c = sim.prepare_allreduce([t.data_ptr() for t in ins], [t.data_ptr() for t in outs], P, n, dtype,
                                      "sum", algo, self.stream)
            st = c()
            if st:
                raise sim.SimError(st, f"sim_allreduce({algo})")
            calls.append(c)
        if len(calls) == 1:
            fn = calls[0]
        else:
            it = [0]

            def fn():
                calls[it[0]]()
                it[0] = (it[0] + 1) % len(calls)
        us, spread = self.time(fn, steps, max(2, steps // 10), reps)
        if sim.sim_check_error(self.stream) != 0:
            raise RuntimeError("device error during calibration")
        self.last_phased = sim.sim_debug_get("phased_last")
        return us, spread


def fit(points, algo):
    """Fit t = alpha * L + bytes / B over the points [(launches, bytes, t_us)].

    A start from weighted least squares (weights 1/t, i.e. relative error),
    then each parameter re-estimated from the regime it governs: B from the
    points where the bytes term is at least 80% of the predicted time
    (total bytes over total time left after the launches), alpha from the
    points where the launch term is at least 80% (median of the time left
    after the bytes, per launch).  A joint line across the bend between the
    latency-flat small sizes and the bandwidth-bound large ones otherwise
    under-estimates B and mis-ranks schedules at large sizes."""
    import numpy as np
    A = np.array([[L / t, b / t] for (L, b, t) in points])
    y = np.ones(len(points))
    sol, *_ = np.linalg.lstsq(A, y, rcond=None)
    alpha = max(float(sol[0]), 0.0)
    inv_b = max(float(sol[1]), 1e-9)
    for _ in range(3):
        pred = [(alpha * L, b * inv_b) for (L, b, t) in points]
        bw = [(L, b, t) for (L, b, t), (pa, pb) in zip(points, pred) if pb >= 0.8 * (pa + pb)]
        lat = [(L, b, t) for (L, b, t), (pa, pb) in zip(points, pred) if pa >= 0.8 * (pa + pb)]
        if bw:
            left = sum(max(t - alpha * L, 1e-3) for (L, b, t) in bw)
            inv_b = left / sum(b for (L, b, t) in bw)
        if lat:
            alpha = max(0.0, float(np.median([(t - b * inv_b) / L for (L, b, t) in lat])))
    return alpha, 1.0 / inv_b / 1e3  # bytes/us -> GB/s


def fit_host(points, algo):
    """(H, alpha, B) of T = max(H L, alpha L + bytes / B): calls timed back
    to back overlap the host's enqueue of one call with the GPU's execution
    of the previous one.  H = the latency floor per launch (median of t / L
    over the three smallest sizes); alpha and B are fitted (fit()) on the
    points the GPU side bounds, t >= 1.25 H L.  The form is kept only when
    it fits every point better (mean squared relative error) than the
    additive one fitted on all points; otherwise, and with fewer than three
    GPU-bound points, H = 0: schedules whose floor is their own kernel's
    time (the persistent and LL kernels) are additive."""
    def mse(h, a, b):
        return statistics.fmean(((max(h * L, a * L + tb / b / 1e3) - t) / t) ** 2 for (L, tb, t) in points)
    a0, b0 = fit(points, algo)
    pts = sorted(points, key=lambda x: x[1])
    h = float(statistics.median(t / L for (L, b, t) in pts[:3]))
    gpu = [(L, b, t) for (L, b, t) in pts if t >= 1.25 * h * L]
    if len(gpu) >= 3:
        a1, b1 = fit(gpu, algo)
        if mse(h, a1, b1) < mse(0.0, a0, b0):
            return h, a1, b1
    return 0.0, a0, b0


# Launch-configuration sweep (after T-CCL's offline ranking of CTA
# configurations per collective and size, section III-C3): the bulk
# schedules at each grid size with a range of total workgroups and one or
# two 16-byte vectors per lane (also four for the one-shot, whose fused fold
# has that form); (0, 1) is the library's default (one vector
# per lane, one workgroup per kBlock vectors, covering the transfer).  The
# best pair per size goes into the calibration file; a pair within 1% of the
# default's time keeps the default.
WG_ALGOS = ("oneshot", "allpairs", "ring")
WG_TOTALS = (0, 256, 512, 1024, 2048, 4096, 8192, 16384)
WG_UNROLLS = {"oneshot": (1, 2, 4), "allpairs": (1, 2), "ring": (1, 2)}  # 16-byte vectors per lane per pass


def sweep_workgroups(sim, b, sizes):
    table = {}
    raw = {}
    for algo in WG_ALGOS:
        rows = []
        for nbytes in sizes:
            if nbytes < (96 << 10):
                continue
            n = nbytes // 2
            times = {}
            for unroll in WG_UNROLLS[algo]:
                sim.sim_debug_set("unroll", unroll)
                for total in WG_TOTALS:
                    sim.sim_debug_set("workgroups", total)
                    times[(total, unroll)] = b.measure(algo, "bf16", n)[0]
            sim.sim_debug_set("workgroups", 0)
            sim.sim_debug_set("unroll", 0)
            best = min(times, key=times.get)
            if times[best] >= times[(0, 1)] * 0.99:  # keep the default unless it gains >= 1%
                best = (0, 1)
            rows.append([nbytes, best[0], best[1]])
            raw.setdefault(algo, []).append({"bytes_per_rank": nbytes,
                                             "us": {f"{t}x{u}": round(v, 3) for (t, u), v in times.items()}})
            print(f"workgroups {algo:9s} {nbytes:>10d} B/rank best {best[0]:6d} x{best[1]} "
                  + " ".join(f"{t}x{u}={v:.1f}" for (t, u), v in times.items()), flush=True)
        table[algo] = rows
    return table, raw


# Workgroup budgets of the sweep and the size it runs at (bandwidth-bound:
# the bytes term is > 90% of every schedule's time there); LL only up to its
# buffer, at its largest grid size.
BUDGETS = (16, 32, 64, 128)
BUDGET_BYTES = 48 << 20
BUDGET_BYTES_LL = 768 << 10


def fit_wg_rate(points, gbps):
    """Per-workgroup rate b from [(W, B_obs)]: each point where the budget
    binds (B_obs < 0.97 B) gives W b = (B_obs^-3 - B^-3)^(-1/3), the
    inverse of the model's smooth minimum; b is their median over W.  0
    when no budget bound (the algo then keeps B under every budget)."""
    est = []
    for w, bo in points:
        if 0 < bo < 0.97 * gbps:
            est.append((bo ** -3 - gbps ** -3) ** (-1.0 / 3.0) / w)
    return float(statistics.median(est)) if est else 0.0


def sweep_budget(sim, b, fits):
    rates, raw = {}, {}
    for algo in ALGOS:
        nbytes = BUDGET_BYTES_LL if algo == "oneshot_ll" else BUDGET_BYTES
        n = nbytes // 2
        alpha, gbps = fits[algo]["alpha_us"], fits[algo]["gbps"]
        sim.sim_model_set(algo, 1.0, -1, -1, 1e300)
        launches = sim.sim_model_predict(algo, P, "bf16", nbytes)
        sim.sim_model_set(algo, 0.0, -1, -1, 1.0)
        traffic = sim.sim_model_predict(algo, P, "bf16", nbytes) * 1e3  # bytes
        sim.sim_model_reset()
        pts = []
        for w in BUDGETS:
            sim.sim_config_set("max_workgroups", w)
            us = b.measure(algo, "bf16", n)[0]
            # persistent schedules keep at least one workgroup per rank
            weff = max(w, P) if algo in ("ring_fifo", "allpairs_persistent") else w
            left = max(us - alpha * launches, 1e-3)
            pts.append((weff, traffic / left / 1e3))
            raw.setdefault(algo, []).append({"budget": w, "bytes_per_rank": nbytes, "us": round(us, 3),
                                             "gbps_observed": round(traffic / left / 1e3, 1)})
            print(f"budget {algo:20s} {w:4d} workgroups {us:10.2f} us", flush=True)
        sim.sim_config_set("max_workgroups", 0)
        rates[algo] = fit_wg_rate(pts, gbps)
    return rates, raw


def calibrate(out_path: str):
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, P, 0)
    sizes = [int(1.5 * (1 << k)) // 16 * 16 for k in range(10, 28)]   # 1.5 KiB .. 192 MiB
    b = Bench(max(sizes))
    raw = {}
    # warm-up: the first schedule measured otherwise ran its smallest sizes
    # while host and GPU clocks were still ramping (a run measured the ring
    # at 59.7 us for 1.5 and 3 KiB per rank and 39.1 us from 6 KiB on)
    for algo in ALGOS:
        set_topology(sim, algo)
        for nbytes in sizes[:6]:
            if b.legal(algo, nbytes):
                b.measure(algo, "bf16", nbytes // 2)
    ll_max = sim.sim_debug_get("ring_ll_max")
    for algo in ALGOS + tuple(TOPOLOGY):
        set_topology(sim, algo)
        pts, regime = [], []
        for nbytes in sizes:
            if not b.legal(algo, nbytes):
                continue
            n = nbytes // 2
            us, spread = b.measure(algo, "bf16", n)
            # the second regime (see REGIMES): the one-shot's phased calls,
            # the single-launch ring's FIFO protocol
            regime.append(b.last_phased == 1 if algo == "oneshot" else
                          nbytes > ll_max if algo == "ring_fifo" else False)
            # the laws (launch count, traffic) of this algo, with unit alpha / B
            sim.sim_model_set(algo, 1.0, -1, -1, 1e300)
            launches = sim.sim_model_predict(algo, P, "bf16", nbytes)
            sim.sim_model_set(algo, 0.0, -1, -1, 1.0)
            tb = sim.sim_model_predict(algo, P, "bf16", nbytes) * 1e3
            pts.append((launches, tb, us))
            raw.setdefault(algo, []).append({"bytes_per_rank": nbytes, "us": round(us, 3),
                                             "spread": round(spread, 4)})
            print(f"calibrate {algo:10s} {nbytes:>10d} B/rank {us:10.2f} us", flush=True)
        raw[algo + "_fit_points"] = len(pts)
        lo = [x for x, r in zip(pts, regime) if not r]
        hi = [x for x, r in zip(pts, regime) if r]
        if algo in REGIMES and len(lo) >= 3 and len(hi) >= 3:
            for key, part in (("fit", lo), ("fit_hi", hi)):
                host, alpha, gbps = fit_host(part, algo)
                raw.setdefault(key, {})[algo] = {"alpha_us": alpha, "gbps": gbps, "host_us": host}
        else:
            host, alpha, gbps = fit_host(pts, algo)
            raw.setdefault("fit", {})[algo] = {"alpha_us": alpha, "gbps": gbps, "host_us": host}
    set_topology(sim, "ring")
    sim.sim_model_reset()
    # the budget sweep's size runs the one-shot fused (no phased form under a
    # budget) and the single-launch ring with FIFOs: each is fitted against
    # the regime it runs in, and the rate goes into both entries
    hi_fits = raw.get("fit_hi", {})
    budget_fits = {a: (hi_fits[a] if a == "ring_fifo" and a in hi_fits else f) for a, f in raw["fit"].items()}
    rates, budget_raw = sweep_budget(sim, b, budget_fits)
    for algo, r in rates.items():
        raw["fit"][algo]["wg_gbps"] = r
        if algo in hi_fits:
            hi_fits[algo]["wg_gbps"] = r
    wg_table, wg_raw = sweep_workgroups(sim, b, sizes)
    model = {"device": "MI355X (gfx950)", "p": P, "dtype": "bf16",
             "grid": "1.5 x 2^k bytes per rank, k = 10..27",
             "form": "T = max(host_us * launches, alpha_us * launches + traffic / B_eff); B_eff = gbps, or "
                     "(gbps^-3 + (W wg_gbps)^-3)^(-1/3) under a budget of W workgroups",
             "topology": {a: {"ranks_per_node": g, "radix": k} for a, (g, k) in TOPOLOGY.items()},
             "algos": raw["fit"], "algos_hi": raw.get("fit_hi", {}),
             "regimes": {"oneshot": "algos_hi from the size where it runs phased (at this p)",
                         "ring_fifo": f"algos_hi above {ll_max} bytes per rank (FIFO protocol)"},
             "workgroups": wg_table,
             "measurements": {a: raw[a] for a in ALGOS + tuple(TOPOLOGY) if a in raw},
             "budget_measurements": budget_raw,
             "rotation": f"up to {Bench.MAX_SETS} buffer sets, >= {Bench.ROT_BYTES >> 20} MiB per rotation "
                         f"where they fit",
             "workgroup_measurements": wg_raw}
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        json.dump(model, f, indent=1)
    print(json.dumps({"calibration": out_path, "algos": raw["fit"], "algos_hi": raw.get("fit_hi", {})}), flush=True)
    return out_path


CHECK_BUDGETS = (0, 128, 32)


def _pairs_agree(pred, meas, tol):
    """(agreeing pairs, pairs): a pair of schedules agrees when the model
    orders it as measured, or when the two measured times are within `tol`
    of each other (a tie either way)."""
    names = sorted(meas)
    agree = total = 0
    for i, a in enumerate(names):
        for c in names[i + 1:]:
            total += 1
            if abs(meas[a] - meas[c]) <= tol * min(meas[a], meas[c]):
                agree += 1
            elif (pred[a] < pred[c]) == (meas[a] < meas[c]):
                agree += 1
    return agree, total


def check(model_path: str, steps_scale: float = 1.0, budgets=CHECK_BUDGETS, reps: int = 5):
    """The selector against measurement at the evaluation sizes, under each
    workgroup budget; returns the report (see the module docstring)."""
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, P, 0)
    sim.sim_model_load(model_path)
    cases = [("bf16", 8192 * t) for t in (1, 16, 256, 4096)] + [("fp16", (1 << k) // 2) for k in range(10, 21)]
    b = Bench(64 << 20, steps_scale)
    by_budget = {}
    for budget in budgets:
        sim.sim_config_set("max_workgroups", budget)
        rows = []
        strict = tolerant = agree = pairs = ru_strict = ru_tolerant = 0
        errs = []
        for dtype, n in cases:
            nbytes = n * sim.ESIZE[dtype]
            meas, spreads, pred = {}, {}, {}
            for algo in ALGOS:
                if b.legal(algo, nbytes):
                    meas[algo], spreads[algo] = b.measure(algo, dtype, n, reps)
                    pred[algo] = sim.sim_model_predict(algo, P, dtype, nbytes)
            pick, pick_us = sim.sim_select(P, n, dtype)
            best = min(meas, key=meas.get)
            tol = max(0.03, spreads[best], spreads[pick])
            s_ok = pick == best
            t_ok = meas[pick] <= meas[best] * (1 + tol)
            ag, pt = _pairs_agree(pred, meas, max(0.03, max(spreads.values())))
            # the runner-up: the model's argmin over the schedules left once the
            # measured fastest is taken out, against the measured one
            rest = [a for a in meas if a != best]
            ru_pick = min(rest, key=lambda a: pred[a])
            ru_best = min(rest, key=lambda a: meas[a])
            ru_tol = max(0.03, spreads[ru_best], spreads[ru_pick])
            ru_strict += ru_pick == ru_best
            ru_tolerant += meas[ru_pick] <= meas[ru_best] * (1 + ru_tol)
            strict += s_ok
            tolerant += t_ok
            agree += ag
            pairs += pt
            err = {a: round((pred[a] - meas[a]) / meas[a], 4) for a in meas}
            errs.append(abs(err[pick]))
            rows.append({"dtype": dtype, "bytes_per_rank": nbytes, "pick": pick, "predicted_us": round(pick_us, 2),
                         "measured_best": best, "measured_us": {a: round(v, 2) for a, v in meas.items()},
                         "predicted_us_all": {a: round(v, 2) for a, v in pred.items()},
                         "rel_error": err, "strict": s_ok, "tolerant": t_ok,
                         "runner_up_pick": ru_pick, "runner_up_measured": ru_best,
                         "pairs_agree": ag, "pairs": pt})
            print(f"check budget {budget or 'none':>4} {dtype} {nbytes:>9d} B/rank pick {pick:10s} "
                  f"best {best:10s} err(pick) {err[pick]:+.3f} pairs {ag}/{pt} "
                  + " ".join(f"{a}={v:.1f}" for a, v in meas.items()), flush=True)
        by_budget["none" if budget == 0 else str(budget)] = {
            "cases": len(cases), "strict_matches": strict, "tolerant_matches": tolerant,
            "runner_up_strict": ru_strict, "runner_up_tolerant": ru_tolerant,
            "pairs_agree": agree, "pairs": pairs,
            "pick_rel_error_median": round(float(statistics.median(errs)), 4),
            "pick_rel_error_max": round(max(errs), 4), "rows": rows}
    sim.sim_config_set("max_workgroups", 0)
    report = {"model": os.path.basename(model_path), "cases": len(cases),
              "strict_matches": by_budget["none"]["strict_matches"] if "none" in by_budget else None,
              "tolerant_matches": by_budget["none"]["tolerant_matches"] if "none" in by_budget else None,
              "budgets": by_budget}
    print(json.dumps({"selector_check": {k: {kk: v[kk] for kk in ("cases", "strict_matches", "tolerant_matches",
                                                                    "runner_up_strict", "runner_up_tolerant",
                                                                    "pairs_agree", "pairs", "pick_rel_error_median",
                                                                    "pick_rel_error_max")}
                                         for k, v in by_budget.items()}}), flush=True)
    return report


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", default=DEFAULT_OUT)
    ap.add_argument("--check", action="store_true", help="also run the selector check with the fitted model")
    ap.add_argument("--check-only", action="store_true")
    ap.add_argument("--report", default="", help="write the check report (JSON) here")
    a = ap.parse_args(argv)
    if not a.check_only:
        calibrate(a.out)
    if a.check or a.check_only:
        rep = check(a.out)
        if a.report:
            with open(a.report, "w") as f:
                json.dump(rep, f, indent=1)


if __name__ == "__main__":
    sys.exit(main())
