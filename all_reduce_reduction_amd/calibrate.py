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

The fit is a two-regime estimate (see fit()).  A launch-configuration sweep
(sweep_workgroups) then stores the best (total workgroups, 16-byte vectors
per lane) per size for the bulk schedules.  --check then times every legal schedule at the evaluation sizes (8192 x
{1, 16, 256, 4096} tokens bf16, and 1 KiB .. 1 MiB fp16) and compares the
selector's pick with the measured fastest: a strict match, and a tolerant
match when the pick is within max(3%, the measured spread) of the best.

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
    """Device buffers for p ranks, reused across sizes (largest first)."""

    def __init__(self, max_bytes: int):
        import torch
        import all_reduce_reduction_amd as sim
        self.sim = sim
        dev = torch.device("cuda:0")
        self.ins = [torch.randint(-3000, 3000, (max_bytes // 2,), dtype=torch.int16, device=dev) for _ in range(P)]
        self.outs = [torch.empty_like(self.ins[0]) for _ in range(P)]
        self.ip = [t.data_ptr() for t in self.ins]
        self.op = [t.data_ptr() for t in self.outs]
        self.stream = int(torch.cuda.current_stream().cuda_stream)
        self.time = _timer()

    def legal(self, algo, nbytes):
        return algo != "oneshot_ll" or nbytes <= self.sim.LL_MAX_BYTES_PER_RANK

    def measure(self, algo, dtype, n):
        sim = self.sim
        nbytes = n * sim.ESIZE[dtype]
        steps = max(5, min(2000, int(2e5 / max(1.0, nbytes / 4e3))))

        call = sim.prepare_allreduce(self.ip, self.op, P, n, dtype, "sum", algo, self.stream)
        st = call()
        if st:
            raise sim.SimError(st, f"sim_allreduce({algo})")
        us, spread = self.time(call, steps, max(2, steps // 10))
        if sim.sim_check_error(self.stream) != 0:
            raise RuntimeError("device error during calibration")
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


# Launch-configuration sweep (after T-CCL's offline ranking of CTA
# configurations per collective and size, section III-C3): the bulk
# schedules at each grid size with a range of total workgroups and one or
# two 16-byte vectors per lane; (0, 1) is the library's default (one vector
# per lane, one workgroup per kBlock vectors, covering the transfer).  The
# best pair per size goes into the calibration file; a pair within 1% of the
# default's time keeps the default.
WG_ALGOS = ("oneshot", "allpairs", "ring")
WG_TOTALS = (0, 256, 512, 1024, 2048, 4096, 8192, 16384)
WG_UNROLLS = (1, 2)  # 16-byte vectors per lane per pass


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
            for unroll in WG_UNROLLS:
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
    for algo in ALGOS + tuple(TOPOLOGY):
        set_topology(sim, algo)
        pts = []
        for nbytes in sizes:
            if not b.legal(algo, nbytes):
                continue
            n = nbytes // 2
            us, spread = b.measure(algo, "bf16", n)
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
        alpha, gbps = fit(pts, algo)
        raw.setdefault("fit", {})[algo] = {"alpha_us": alpha, "gbps": gbps}
    set_topology(sim, "ring")
    sim.sim_model_reset()
    wg_table, wg_raw = sweep_workgroups(sim, b, sizes)
    model = {"device": "MI355X (gfx950)", "p": P, "dtype": "bf16",
             "grid": "1.5 x 2^k bytes per rank, k = 10..27",
             "topology": {a: {"ranks_per_node": g, "radix": k} for a, (g, k) in TOPOLOGY.items()},
             "algos": raw["fit"], "workgroups": wg_table,
             "measurements": {a: raw[a] for a in ALGOS + tuple(TOPOLOGY) if a in raw},
             "workgroup_measurements": wg_raw}
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as f:
        json.dump(model, f, indent=1)
    print(json.dumps({"calibration": out_path, "algos": raw["fit"]}), flush=True)
    return out_path


def check(model_path: str):
    import all_reduce_reduction_amd as sim
    sim.sim_init(0, P, 0)
    sim.sim_model_load(model_path)
    cases = [("bf16", 8192 * t) for t in (1, 16, 256, 4096)] + [("fp16", (1 << k) // 2) for k in range(10, 21)]
    b = Bench(64 << 20)
    rows = []
    strict = tolerant = 0
    for dtype, n in cases:
        nbytes = n * sim.ESIZE[dtype]
        meas = {}
        spreads = {}
        for algo in ALGOS:
            if b.legal(algo, nbytes):
                meas[algo], spreads[algo] = b.measure(algo, dtype, n)
        pick, pred = sim.sim_select(P, n, dtype)
        best = min(meas, key=meas.get)
        tol = max(0.03, spreads[best], spreads[pick])
        s_ok = pick == best
        t_ok = meas[pick] <= meas[best] * (1 + tol)
        strict += s_ok
        tolerant += t_ok
        rows.append({"dtype": dtype, "bytes_per_rank": nbytes, "pick": pick, "predicted_us": round(pred, 2),
                     "measured_best": best, "measured_us": {a: round(v, 2) for a, v in meas.items()},
                     "strict": s_ok, "tolerant": t_ok})
        print(f"check {dtype} {nbytes:>9d} B/rank pick {pick:10s} best {best:10s} "
              + " ".join(f"{a}={v:.1f}" for a, v in meas.items()), flush=True)
    report = {"model": os.path.basename(model_path), "cases": len(cases), "strict_matches": strict, "tolerant_matches": tolerant,
              "rows": rows}
    print(json.dumps({"selector_check": {k: report[k] for k in ("cases", "strict_matches", "tolerant_matches")}}),
          flush=True)
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
