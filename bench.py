#!/usr/bin/env python3
"""Benchmark of the simulated all-reduce on one MI355X.

Workload (one "step" = one all-reduce call through the C-ABI, selector
included): p = 8 simulated ranks, bf16 in/out with fp32 accumulation,
8192 hidden x 4096 tokens = 33,554,432 elements = 64 MiB per rank, values
N(0,1) * 0.02 from the seeded generator -- a tensor-parallel activation
all-reduce.  Inputs are resident in HBM before the timed region starts.

Printed JSON line:
  value          NCCL-style bus bandwidth 2(p-1)/p * S / t  (GB/s)
  roofline       the dominant kernel's algorithmic bytes per launch over its
                 average launch time (HIP events on the launch stream), vs
                 MI355X's 8 TB/s HBM peak; `traffic` = rocprofv3 FETCH_SIZE +
                 WRITE_SIZE per launch when a matching counter summary is
                 committed under profiles/, else null
  per_algo       the same workload forced to each legal schedule (the tree,
                 recursive-exchange and 2PH ones at a stated topology)
  latency_8KiB   per-call microseconds at 8 KiB per rank (p = 8, fp16):
                 plain one-shot vs the LL packet path vs the selector's pick
                 (and, as latency_8KiB_graph_us, calls replayed from a
                 captured HIP graph)
  cpu_baseline   the CPU oracle on the same host arrays (all host threads)
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
METRIC = "all-reduce busBW & HBM GB/s vs peak, p=8 bf16 64 MiB; 8 KiB latency (us)"
P = 8
HIDDEN, TOKENS = 8192, 4096
N = HIDDEN * TOKENS          # elements per rank
ESIZE = 2
S = N * ESIZE                # bytes per rank
LAT_N = 4096                 # 8 KiB of fp16 per rank


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--algo", default="auto", help="auto|ring|allpairs|oneshot")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip per-algo and latency figures")
    ap.add_argument("--profile-only", action="store_true",
                    help="only the timed steps of the headline workload (for rocprofv3 runs)")
    ap.add_argument("--profile-large", action="store_true",
                    help="only the 256 MiB-per-rank fp32 avg one-shot (workload 5's 4 GiB working set)")
    ap.add_argument("--profile-copy", action="store_true",
                    help="only a plain 512 MiB -> 512 MiB device copy (the counter scale reference)")
    return ap.parse_args()


def algorithmic_bytes(algo: str) -> float:
    """HBM bytes of one call over all ranks (the schedules' traffic laws)."""
    if algo == "oneshot":
        return 2.0 * P * S
    if algo == "allpairs":
        return (2.0 * P + 1.0) * S
    if algo == "ring":  # bf16 with fp32 partials
        n, e = N, ESIZE
        rs = n * (e + e + 4) + (P - 3) * n * (4 + e + 4) + n * (4 + e + e)
        return rs + (P - 1) * n * (e + e)
    if algo == "ring_fifo":  # inputs and outputs once; fp32 partials through FIFOs; peer reads
        return 2.0 * P * S + (P - 1) * N * 8.0 + (P - 1) * N * ESIZE
    if algo == "allpairs_persistent":  # step 1 pS + S; step 2 each rank pulls p-1 chunks: 2(p-1)S
        return (3.0 * P - 1.0) * S
    raise ValueError(algo)


# The tree, recursive-exchange and 2PH schedules, each at the topology it is
# timed with: (name, algo, ranks per node, radix).
TOPOLOGY_RUNS = [("tree", "tree", 1, 2), ("rexch_k2", "rexch", 1, 2), ("hier_G4", "hier", 4, 2),
                 ("hier_large_G4", "hier_large", 4, 2)]


def schedule_bytes(sim, algo: str, n: int, esize: int) -> float:
    """Algorithmic HBM bytes of one call of a lowered tree / exchange / 2PH
    schedule as the step executor runs it: a fold reads each operand once
    (inputs at storage width, partials as 4-byte fp32) and writes each
    receiver once (finished values at storage width, partials at 4 bytes);
    an exchange group shares one fold; a broadcast reads once and writes
    each receiver."""
    nsteps, _, nch = sim.sim_schedule_info(algo, P)
    part = set()
    total = 0.0
    for st in range(nsteps):
        groups, nxt = set(), set(part)
        for kind, src, dst, chunk, mask in sim.sim_schedule_xfers(algo, P, st):
            ln = n / nch
            members = [q for q in range(P) if (mask >> q) & 1]
            width = lambda q: 4 if (q, chunk) in part else esize  # noqa: E731
            if kind in (6, 7, 8, 9):
                post = kind in (7, 9)
                if kind in (6, 7):
                    total += ln * (width(dst) + sum(width(q) for q in members))
                elif (chunk, mask) not in groups:
                    groups.add((chunk, mask))
                    total += ln * sum(width(q) for q in members)
                total += ln * (esize if post else 4)
                (nxt.discard if post else nxt.add)((dst, chunk))
            elif kind == 10:
                total += ln * esize * (1 + len(members))
        part = nxt
    return total


def time_calls(fn, steps: int, warmup: int) -> float:
    """Seconds per call: HIP events on torch's current stream, which is the
    stream every call here launches on."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / steps


KERNEL_SOURCES = ["all_reduce_reduction_amd/csrc/k_fold.hip", "all_reduce_reduction_amd/csrc/k_step.hip",
                  "all_reduce_reduction_amd/csrc/device_common.h", "all_reduce_reduction_amd/csrc/kernels.h"]


def kernel_source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]


def load_traffic(algo: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    or None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic_bf16_p8_64MiB.json")
    if not os.path.exists(path):
        return None
    try:
        d = json.load(open(path))
    except Exception:
        return None
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    ent = d.get("algos", {}).get(algo)
    return None if not ent else ent.get("hbm_bytes_per_launch_scaled")


N5 = 67_108_864  # workload 5: 256 MiB of fp32 per rank


def large_workload(sim, synthdata, torch, np, dev, stream, steps, warmup) -> float:
    """Microseconds per one-shot fp32 avg all-reduce at 256 MiB per rank
    (inputs 2 GiB + outputs 2 GiB: far past the 256 MB Infinity Cache)."""
    xs5 = synthdata.workload_inputs(5, P, N5, "fp32")
    d5 = [torch.from_numpy(x).to(dev) for x in xs5]
    del xs5
    o5 = [torch.empty(N5, dtype=torch.float32, device=dev) for _ in range(P)]
    i5, p5 = [t.data_ptr() for t in d5], [t.data_ptr() for t in o5]

    def call():
        if sim.sim_allreduce(i5, p5, P, N5, "fp32", "avg", "oneshot", stream):
            raise sim.SimError(-1, "sim_allreduce (workload 5)")
    t5 = time_calls(call, steps, warmup)
    assert sim.sim_check_error(stream) == 0
    del d5, o5
    torch.cuda.empty_cache()
    return t5 * 1e6


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: the p simulated ranks all live in one GPU's HBM "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {world}).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import all_reduce_reduction_amd as sim
    import synthdata

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    if args.profile_copy:
        # Counter scale references of known size: (1) the library's own copy
        # kernel (the ring all-gather step, same 16-byte streaming loads/stores
        # as k_fold) in a p = 2 fp32 ring all-reduce of 256 MiB per rank: each
        # such launch reads 256 MiB and writes 256 MiB; (2) torch's
        # device-to-device copy of 512 MiB.
        sim.sim_init(0, 2, 0)
        n2 = (256 << 20) // 4
        bufs = [torch.empty(n2, dtype=torch.float32, device=dev).fill_(1.0) for _ in range(4)]
        ptr = [b.data_ptr() for b in bufs]
        s2 = int(torch.cuda.current_stream().cuda_stream)
        t1 = time_calls(lambda: sim.sim_allreduce(ptr[:2], ptr[2:], 2, n2, "fp32", "sum", "ring", s2),
                        args.steps, args.warmup)
        src = torch.empty(S * P // 2 // 4, dtype=torch.int32, device=dev).fill_(7)
        dst = torch.empty_like(src)
        t2 = time_calls(lambda: dst.copy_(src), args.steps, args.warmup)
        print(json.dumps({"k_copy_bytes_read": 2 * n2 * 4 // 2 * 1, "k_copy_bytes_written": n2 * 4,
                          "us_per_ring_call": t1 * 1e6, "torch_copy_bytes": src.numel() * 4,
                          "us_per_torch_copy": t2 * 1e6}), flush=True)
        return
    sim.sim_init(0, P, S)
    stream = int(torch.cuda.current_stream().cuda_stream)
    if args.profile_large:
        us5 = large_workload(sim, synthdata, torch, np, dev, stream, args.steps, args.warmup)
        print(json.dumps({"workload": "fp32 avg, p=8, 256 MiB per rank", "us_per_step": us5}), flush=True)
        return

    xs = synthdata.workload_inputs(3, P, N, "bf16")
    din = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs]
    dout = [torch.empty(N, dtype=torch.int16, device=dev) for _ in range(P)]
    ip = [t.data_ptr() for t in din]
    op_ = [t.data_ptr() for t in dout]

    def step(algo=args.algo):
        st = sim.sim_allreduce(ip, op_, P, N, "bf16", "sum", algo, stream)
        if st:
            raise sim.SimError(st, "sim_allreduce")

    t = time_calls(step, args.steps, args.warmup)
    assert sim.sim_check_error(stream) == 0
    ran = sim.sim_last_algo()
    if args.profile_only:
        print(json.dumps({"algo": ran, "us_per_step": t * 1e6}), flush=True)
        return
    # the same step repeated in 5 further batches (spread of the timed figure)
    reps = [time_calls(step, max(10, args.steps // 5), 2) for _ in range(5)]
    busbw = 2 * (P - 1) / P * S / t / 1e9
    kernel = {"oneshot": "k_fold (one-shot, all outputs)", "allpairs": "k_fold + k_copy",
              "ring": "k_ring_reduce + k_copy", "ring_fifo": "k_ring_fifo",
              "allpairs_persistent": "k_allpairs_persistent"}[ran]
    achieved = algorithmic_bytes(ran) / t / 1e9
    traffic = load_traffic(ran)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic, "kernel": kernel,
                "algorithmic_bytes_per_launch": algorithmic_bytes(ran)}

    extras = {}
    if not args.no_extras:
        per_algo = {}
        for a in ("oneshot", "allpairs", "ring", "ring_fifo", "allpairs_persistent"):
            ta = time_calls(lambda a=a: step(a), max(10, args.steps // 4), 5)
            per_algo[a] = {"us": round(ta * 1e6, 2), "busbw_GBps": round(2 * (P - 1) / P * S / ta / 1e9, 1),
                           "hbm_algorithmic_GBps": round(algorithmic_bytes(a) / ta / 1e9, 1)}
        for name, a, G, k in TOPOLOGY_RUNS:
            sim.sim_config_set("ranks_per_node", G)
            sim.sim_config_set("radix", k)
            ta = time_calls(lambda a=a: step(a), max(10, args.steps // 4), 5)
            per_algo[name] = {"us": round(ta * 1e6, 2), "busbw_GBps": round(2 * (P - 1) / P * S / ta / 1e9, 1),
                              "hbm_algorithmic_GBps": round(schedule_bytes(sim, a, N, ESIZE) / ta / 1e9, 1),
                              "steps": sim.sim_schedule_info(a, P)[0]}
        sim.sim_config_set("ranks_per_node", 1)
        sim.sim_config_set("radix", 2)
        extras["per_algo"] = per_algo
        # reduce-scatter then all-gather vs the all-reduce of the same schedule
        # (the ring all-reduce is exactly these two halves back to back)
        n_out = N // P
        rs_out = [torch.empty(n_out, dtype=torch.int16, device=dev) for _ in range(P)]
        rs_p = [t_.data_ptr() for t_ in rs_out]
        rs_ag = {}
        for a in ("ring", "allpairs"):
            def rs_then_ag(a=a):
                if sim.sim_reduce_scatter(ip, rs_p, P, n_out, "bf16", "sum", a, stream):
                    raise sim.SimError(-1, "sim_reduce_scatter")
                if sim.sim_all_gather(rs_p, op_, P, n_out, "bf16", a, stream):
                    raise sim.SimError(-1, "sim_all_gather")
            tr = time_calls(rs_then_ag, max(10, args.steps // 4), 5)
            rs_ag[a] = {"rs_plus_ag_us": round(tr * 1e6, 2), "allreduce_us": per_algo[a]["us"],
                        "ratio": round(tr * 1e6 / per_algo[a]["us"], 3)}
        extras["rs_then_ag_vs_allreduce"] = rs_ag
        # T-CCL's restricted mode: the one-shot with a workgroup budget
        budget = {}
        for b in (32, 128, 512, 2048, 0):
            sim.sim_config_set("max_workgroups", b)
            tb = time_calls(lambda: step("oneshot"), max(10, args.steps // 4), 5)
            budget[str(b) if b else "none"] = round(2 * (P - 1) / P * S / tb / 1e9, 1)
        sim.sim_config_set("max_workgroups", 0)
        extras["oneshot_busbw_by_workgroup_budget"] = budget
        us5 = large_workload(sim, synthdata, torch, np, dev, stream, max(10, args.steps // 10), 3)
        extras["workload5_fp32_avg_256MiB_oneshot"] = {
            "us": round(us5, 2), "busbw_GBps": round(2 * (P - 1) / P * N5 * 4 / us5 / 1e3, 1),
            "hbm_algorithmic_GBps": round(2 * P * N5 * 4 / us5 / 1e3, 1),
            "frac_of_peak": round(2 * P * N5 * 4 / us5 / 1e3 / HBM_PEAK_GBPS, 4)}
        # small-message latency: 8 KiB per rank, fp16
        lx = synthdata.workload_inputs(4, P, LAT_N, "fp16")
        lin = [torch.from_numpy(x.view(np.int16)).to(dev) for x in lx]
        lout = [torch.empty(LAT_N, dtype=torch.int16, device=dev) for _ in range(P)]
        lip, lop = [t_.data_ptr() for t_ in lin], [t_.data_ptr() for t_ in lout]
        lat = {}
        for a in ("oneshot", "oneshot_ll", "allpairs", "ring", "ring_fifo", "allpairs_persistent", "auto"):
            call = sim.prepare_allreduce(lip, lop, P, LAT_N, "fp16", "sum", a, stream)
            if call() != 0:
                raise sim.SimError(call(), f"sim_allreduce({a})")
            lat[a] = round(time_calls(call, 2000, 200) * 1e6, 2)
            if a == "auto":
                lat["auto_pick"] = sim.sim_last_algo()
        # the single-launch ring runs its LL protocol at this size; its FIFO
        # protocol for comparison
        sim.sim_debug_set("ring_ll_max", 0)
        call = sim.prepare_allreduce(lip, lop, P, LAT_N, "fp16", "sum", "ring_fifo", stream)
        if call() != 0:
            raise sim.SimError(call(), "sim_allreduce(ring_fifo, FIFO protocol)")
        lat["ring_fifo_fifo_protocol"] = round(time_calls(call, 2000, 200) * 1e6, 2)
        sim.sim_debug_set("ring_ll_max", 256 << 10)
        for name, a, G, k in TOPOLOGY_RUNS:
            sim.sim_config_set("ranks_per_node", G)
            sim.sim_config_set("radix", k)
            call = sim.prepare_allreduce(lip, lop, P, LAT_N, "fp16", "sum", a, stream)
            if call() != 0:
                raise sim.SimError(call(), f"sim_allreduce({a})")
            lat[name] = round(time_calls(call, 2000, 200) * 1e6, 2)
        sim.sim_config_set("ranks_per_node", 1)
        sim.sim_config_set("radix", 2)
        assert sim.sim_check_error(stream) == 0
        extras["latency_8KiB_us"] = lat
        # the same calls replayed from a captured graph (20 calls per graph):
        # no host work per call; multi-launch schedules keep their launches
        glat = {}
        for a in ("oneshot", "allpairs", "ring", "tree"):
            graph = torch.cuda.CUDAGraph()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                with torch.cuda.graph(graph, stream=side):
                    cs = int(torch.cuda.current_stream().cuda_stream)
                    for _ in range(20):
                        if sim.sim_allreduce(lip, lop, P, LAT_N, "fp16", "sum", a, cs):
                            raise sim.SimError(-1, f"captured sim_allreduce({a})")
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            glat[a] = round(time_calls(graph.replay, 100, 10) * 1e6 / 20, 2)
            del graph
        extras["latency_8KiB_graph_us"] = glat

    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        orc = oracle.get()
        runs = []
        t_end = time.perf_counter() + 10.0
        while len(runs) < 3 or (time.perf_counter() < t_end and len(runs) < 20):
            t0 = time.perf_counter()
            orc.allreduce(xs, "bf16", "sum", ran)
            runs.append(time.perf_counter() - t0)
        tc = float(np.median(runs))
        cpu = {"value": round(2 * (P - 1) / P * S / tc / 1e9, 4), "unit": "GB/s", "cores": orc.num_threads(),
               "kind": "oracle",
               "sample": f"the full workload (8 ranks x 64 MiB bf16, schedule '{ran}'), median of {len(runs)} runs",
               "seconds_per_call": round(tc, 3)}
        # one thread, on the first 1/16 of every rank's buffer (the oracle's cost per element does not
        # depend on n): a rate scaled to the same unit
        threads = orc.num_threads()
        orc.set_num_threads(1)
        sub = [x[: N // 16].copy() for x in xs]
        runs1 = []
        t_end = time.perf_counter() + 10.0
        while len(runs1) < 3 or (time.perf_counter() < t_end and len(runs1) < 10):
            t0 = time.perf_counter()
            orc.allreduce(sub, "bf16", "sum", ran)
            runs1.append(time.perf_counter() - t0)
        orc.set_num_threads(threads)
        t1 = float(np.median(runs1)) * 16
        cpu["single_thread"] = {"value": round(2 * (P - 1) / P * S / t1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                                "sample": f"first 1/16 of each rank's buffer, median of {len(runs1)} runs, "
                                          "scaled to the full buffer"}

    out = {
        "metric": METRIC, "value": round(busbw, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t * 1e3, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "all-reduce sum, p=8 simulated ranks, bf16 (fp32 accumulate), 8192 hidden x 4096 "
                               "tokens = 64 MiB per rank, N(0,1)*0.02", "p": P, "n_per_rank": N,
                   "bytes_per_rank": S, "algo": ran, "parallelism": "1 GPU (p simulated ranks in one HBM)"},
        "roofline": roofline, "cpu_baseline": cpu,
        "repeat_batches_us": {"values": [round(v * 1e6, 2) for v in reps],
                              "median": round(float(np.median(reps)) * 1e6, 2)},
        **extras,
    }
    print(json.dumps(out), flush=True)
    sim.sim_finalize()


if __name__ == "__main__":
    main()
