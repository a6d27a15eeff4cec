#!/usr/bin/env python3
"""Benchmark of the simulated all-reduce on one MI355X.

Workload (one "step" = one all-reduce call through the C-ABI, selector
included): p = 8 simulated ranks, bf16 in/out with fp32 accumulation,
8192 hidden x 4096 tokens = 33,554,432 elements = 64 MiB per rank, values
N(0,1) * 0.02 from the seeded generator -- a tensor-parallel activation
all-reduce.  Inputs are resident in HBM before the timed region starts;
consecutive steps alternate between two buffer sets (2 GiB per pair).

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
  ceiling        what the one-shot's access pattern can reach on this GPU in the
                 same run: the library's k-stream copy (sim_copy_streams) with
                 8 inputs and 8 outputs of 64 MiB (the one-shot's streams and
                 bytes, no arithmetic) and with 1 input and 1 output of 1 GiB,
                 and hipMemcpyAsync device-to-device of 1 GiB (torch's copy_);
                 and the one-shot next to that copy at p = 2, 4, 8, 16
  workload2_fp32_32MiB, workload5_256MiB
                 the parity workloads' timed figures next to the CPU oracle's
                 time for the same call (all host threads, and one thread on a
                 stated sample): busBW, algorithmic HBM GB/s per schedule; the
                 standalone reduce-scatter and all-gather with their own laws
  phased_layout_ab_us
                 the headline's phased one-shot in its per-chunk block layout
                 and in the whole-buffer layout, alternating batches
  workload4_latency_us
                 per-call microseconds of the LL packet path vs the plain
                 one-shot (and the selector's pick) from 1 KiB to 1 MiB per rank
  selector_check the selector's pick vs the measured fastest schedule at the
                 evaluation sizes, under workgroup budgets none / 128 / 32, with
                 per-case model error and pairwise ranking agreement
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
                    help="only the k-stream copy kernel at k = 1 (512 MiB) and k = 8 (64 MiB each), the counter "
                         "scale references")
    ap.add_argument("--profile-size", type=int, default=0,
                    help="only the schedules of --profile-algos at this many bytes per rank (p = 8, fp16, "
                         "workload 4's inputs), --steps calls each (for rocprofv3 kernel traces and counters)")
    ap.add_argument("--profile-algos", default="oneshot,oneshot_ll,allpairs,allpairs_persistent,ring_fifo,ring")
    ap.add_argument("--profile-rsag", action="store_true",
                    help="only workload 5's standalone reduce-scatter (fp32 avg) and all-gather, direct then ring, "
                         "256 MiB per rank, --steps calls each")
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


KERNEL_SOURCES = ["all_reduce_reduction_amd/csrc/k_phased.hip", "all_reduce_reduction_amd/csrc/phased_impl.h",
                  "all_reduce_reduction_amd/csrc/k_phased_whole.hip",
                  "all_reduce_reduction_amd/csrc/k_phased_owner.hip", "all_reduce_reduction_amd/csrc/k_phased_gather.hip",
                  "all_reduce_reduction_amd/csrc/k_fold.hip",
                  "all_reduce_reduction_amd/csrc/fold_impl.h",
                  "all_reduce_reduction_amd/csrc/fold.h", "all_reduce_reduction_amd/csrc/k_step.hip",
                  "all_reduce_reduction_amd/csrc/k_streams.hip",
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


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def time_cpu(fn, runs: int, warm: int = 0) -> float:
    """Median seconds of `runs` calls of fn after `warm` untimed ones."""
    import numpy as np
    for _ in range(warm):
        fn()
    ts = []
    for _ in range(runs):
        t0 = time.perf_counter()
        fn()
        ts.append(time.perf_counter() - t0)
    return float(np.median(ts))


def ceiling(sim, torch, dev, stream, steps: int, head_sets) -> dict:
    """The same-run bandwidth ceiling of the one-shot's access pattern:
    k independent streaming copies through the library (best over a few grid
    sizes) and the runtime's device-to-device copy, all moving random bits as
    the all-reduce does (and the copies once more with constant data)."""
    out = {}
    total = 1 << 30

    def best_copy(k, per, const=False):
        # random bits, like the all-reduce's inputs (the bus toggles as it does
        # for real data); `const`: every word the same, for comparison
        g = torch.Generator(device=dev)
        g.manual_seed(k)
        ins = [torch.randint(-2 ** 31, 2 ** 31 - 1, (per // 4,), dtype=torch.int32, device=dev, generator=g)
               for _ in range(k)]
        if const:
            for q, t in enumerate(ins):
                t.fill_(q + 1)
        outs = [torch.empty_like(ins[0]) for _ in range(k)]
        ip, op_ = [t.data_ptr() for t in ins], [t.data_ptr() for t in outs]
        res = {}
        for wg in (1024, 2048, 4096, 0):
            def call(wg=wg):
                if sim.sim_copy_streams(ip, op_, k, per, wg, stream):
                    raise sim.SimError(-1, "sim_copy_streams")
            res[wg] = time_calls(call, steps, 3)
        torch.cuda.synchronize()
        assert all(torch.equal(o, i) for i, o in zip(ins, outs)), "copy check failed"
        wg = min(res, key=res.get)
        gbs = 2 * k * per / res[wg] / 1e9
        del ins, outs
        torch.cuda.empty_cache()
        return {"GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBPS, 4),
                "us": round(res[wg] * 1e6, 2), "workgroups": wg or "cover",
                "GBps_by_workgroups": {str(w or "cover"): round(2 * k * per / t / 1e9, 1) for w, t in res.items()}}
    # the headline's own buffers and data, alternating between its two buffer
    # sets as the headline does: input q copied to output q
    res = {}
    for wg in (1024, 2048, 4096, 0):
        turn = [0]

        def call(wg=wg):
            hi, ho = head_sets[turn[0]]
            turn[0] = (turn[0] + 1) % len(head_sets)
            if sim.sim_copy_streams(hi, ho, P, S, wg, stream):
                raise sim.SimError(-1, "sim_copy_streams")
        res[wg] = time_calls(call, steps, 3)
    wg = min(res, key=res.get)
    gbs = 2 * P * S / res[wg] / 1e9
    out["copy_headline_buffers"] = {
        "GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBPS, 4), "us": round(res[wg] * 1e6, 2),
        "workgroups": wg or "cover", "what": "the 8 headline inputs copied to the 8 headline outputs (64 MiB each)",
        "GBps_by_workgroups": {str(w or "cover"): round(2 * P * S / t / 1e9, 1) for w, t in res.items()}}
    out["copy_8in_8out_64MiB_each"] = best_copy(8, S)
    out["copy_8in_8out_256MiB_each"] = best_copy(8, 256 << 20)  # workload 5's streams (4 GiB working set)
    out["copy_1in_1out_1GiB"] = best_copy(1, total)
    out["constant_data"] = {"copy_8in_8out_64MiB_each": best_copy(8, S, True),
                            "copy_1in_1out_1GiB": best_copy(1, total, True)}
    src = torch.randint(-2 ** 31, 2 ** 31 - 1, (total // 4,), dtype=torch.int32, device=dev)
    dst = torch.empty_like(src)
    t = time_calls(lambda: dst.copy_(src), steps, 3)
    gbs = 2 * total / t / 1e9
    out["hipMemcpyDtoD_1GiB"] = {"GBps": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBPS, 4),
                                 "us": round(t * 1e6, 2), "via": "torch copy_ (hipMemcpyAsync device to device)"}
    del src, dst
    torch.cuda.empty_cache()
    return out


def workload2(sim, synthdata, oracle, torch, np, dev, stream, steps: int, cpu: bool) -> dict:
    """p = 8, fp32 N(0,1), 32 MiB per rank: ring (14 steps), all-pairs (2),
    one-shot, and the single-launch forms; the CPU oracle of the same calls."""
    n2 = 8_388_608
    s2 = n2 * 4
    xs = synthdata.workload_inputs(2, P, n2, "fp32")
    din = [torch.from_numpy(x).to(dev) for x in xs]
    dout = [torch.empty(n2, dtype=torch.float32, device=dev) for _ in range(P)]
    ip, op_ = [t.data_ptr() for t in din], [t.data_ptr() for t in dout]
    laws = {"oneshot": 2 * P * s2, "allpairs": (2 * P + 1) * s2, "ring": 5 * (P - 1) * s2,
            "ring_fifo": 2 * P * s2 + (P - 1) * n2 * 12, "allpairs_persistent": (3 * P - 1) * s2}
    res = {}
    for a in ("ring", "allpairs", "oneshot", "ring_fifo", "allpairs_persistent"):
        def call(a=a):
            if sim.sim_allreduce(ip, op_, P, n2, "fp32", "sum", a, stream):
                raise sim.SimError(-1, f"sim_allreduce({a})")
        t = time_calls(call, steps, 3)
        res[a] = {"us": round(t * 1e6, 2), "busbw_GBps": round(2 * (P - 1) / P * s2 / t / 1e9, 1),
                  "hbm_algorithmic_GBps": round(laws[a] / t / 1e9, 1),
                  "algorithmic_bytes": laws[a]}
    assert sim.sim_check_error(stream) == 0
    del din, dout
    torch.cuda.empty_cache()
    if cpu:
        orc = oracle.get()
        threads = orc.num_threads()
        for a in ("ring", "allpairs", "oneshot"):
            tc = time_cpu(lambda a=a: orc.allreduce(xs, "fp32", "sum", a), 3, 1)
            res[a]["cpu_oracle"] = {"seconds": round(tc, 4), "busbw_GBps": round(2 * (P - 1) / P * s2 / tc / 1e9, 3),
                                    "cores": threads}
        orc.set_num_threads(1)
        sub = [x[: n2 // 8].copy() for x in xs]
        for a in ("ring", "oneshot"):
            t1 = time_cpu(lambda a=a: orc.allreduce(sub, "fp32", "sum", a), 3, 1) * 8
            res[a]["cpu_oracle"]["single_thread"] = {
                "seconds": round(t1, 3), "busbw_GBps": round(2 * (P - 1) / P * s2 / t1 / 1e9, 4), "cores": 1,
                "sample": "first 1/8 of each rank's buffer, median of 3, scaled to the full buffer"}
        orc.set_num_threads(threads)
    return res


def workload5(sim, synthdata, oracle, torch, np, dev, stream, steps: int, cpu: bool) -> dict:
    """p = 8, 256 MiB per rank: the all-reduce of every op of the workload
    (selector's pick), the standalone reduce-scatter (32 MiB out per rank)
    and all-gather (32 MiB in per rank), direct and ring; the CPU oracle of
    the same calls (median of 2)."""
    res = {"allreduce": {}, "reduce_scatter": {}, "all_gather": {}}
    n_out = N5 // P
    s_full = N5 * 4
    orc = oracle.get() if cpu else None
    for dtype, ops in (("fp32", ("prod", "min", "max", "avg")), ("int32", ("sum", "min", "max"))):
        xs = synthdata.workload_inputs(5, P, N5, dtype)
        tdt = torch.float32 if dtype == "fp32" else torch.int32
        din = [torch.from_numpy(x).to(dev) for x in xs]
        dout = [torch.empty(N5, dtype=tdt, device=dev) for _ in range(P)]
        ip, op_ = [t.data_ptr() for t in din], [t.data_ptr() for t in dout]
        for op in ops:
            def call(op=op):
                if sim.sim_allreduce(ip, op_, P, N5, dtype, op, "auto", stream):
                    raise sim.SimError(-1, "sim_allreduce (workload 5)")
            t = time_calls(call, steps, 2)
            ran = sim.sim_last_algo()
            law = algorithmic_bytes_at(ran, N5, 4)
            ent = {"algo": ran, "us": round(t * 1e6, 2), "busbw_GBps": round(2 * (P - 1) / P * s_full / t / 1e9, 1),
                   "hbm_algorithmic_GBps": round(law / t / 1e9, 1),
                   "frac_of_peak": round(law / t / 1e9 / HBM_PEAK_GBPS, 4)}
            if orc is not None:
                tc = time_cpu(lambda op=op: orc.allreduce(xs, dtype, op, ran), 2)
                ent["cpu_oracle"] = {"seconds": round(tc, 3), "cores": orc.num_threads(),
                                     "busbw_GBps": round(2 * (P - 1) / P * s_full / tc / 1e9, 3)}
            res["allreduce"][f"{dtype} {op}"] = ent
        # standalone reduce-scatter and all-gather: direct (p+1) S_full; the ring
        # reduce-scatter 3 (p-1) S_full (32-bit partials through scratch), the
        # ring all-gather (2p-1) S_full
        rs_out = [torch.empty(n_out, dtype=tdt, device=dev) for _ in range(P)]
        rp = [t.data_ptr() for t in rs_out]
        op_rs = "sum" if dtype == "int32" else "avg"
        for a, law in (("allpairs", (P + 1) * s_full), ("ring", 3 * (P - 1) * s_full)):
            def rs(a=a):
                if sim.sim_reduce_scatter(ip, rp, P, n_out, dtype, op_rs, a, stream):
                    raise sim.SimError(-1, "sim_reduce_scatter")
            t = time_calls(rs, steps, 2)
            ent = {"op": op_rs, "us": round(t * 1e6, 2),
                   "busbw_GBps": round((P - 1) / P * s_full / t / 1e9, 1),
                   "hbm_algorithmic_GBps": round(law / t / 1e9, 1), "algorithmic_bytes": law,
                   "frac_of_peak": round(law / t / 1e9 / HBM_PEAK_GBPS, 4)}
            if orc is not None:
                tc = time_cpu(lambda a=a: orc.reduce_scatter(xs, dtype, op_rs, a), 2)
                ent["cpu_oracle"] = {"seconds": round(tc, 3), "cores": orc.num_threads(),
                                     "busbw_GBps": round((P - 1) / P * s_full / tc / 1e9, 3)}
            res["reduce_scatter"][f"{dtype} {'direct' if a == 'allpairs' else 'ring'}"] = ent
        small = [x[:n_out].copy() for x in xs] if orc is not None else None
        for a, law in (("allpairs", (P + 1) * s_full), ("ring", (2 * P - 1) * s_full)):
            def ag(a=a):
                if sim.sim_all_gather(rp, op_, P, n_out, dtype, a, stream):
                    raise sim.SimError(-1, "sim_all_gather")
            t = time_calls(ag, steps, 2)
            ent = {"us": round(t * 1e6, 2), "busbw_GBps": round((P - 1) / P * s_full / t / 1e9, 1),
                   "hbm_algorithmic_GBps": round(law / t / 1e9, 1), "algorithmic_bytes": law,
                   "frac_of_peak": round(law / t / 1e9 / HBM_PEAK_GBPS, 4)}
            if orc is not None:
                tc = time_cpu(lambda a=a: orc.all_gather(small, dtype, a), 2)
                ent["cpu_oracle"] = {"seconds": round(tc, 3), "cores": orc.num_threads(),
                                     "busbw_GBps": round((P - 1) / P * s_full / tc / 1e9, 3)}
            res["all_gather"][f"{dtype} {'direct' if a == 'allpairs' else 'ring'}"] = ent
        assert sim.sim_check_error(stream) == 0
        if orc is not None:  # one thread, on 1/16 of every buffer (cost per element does not depend on n)
            threads = orc.num_threads()
            orc.set_num_threads(1)
            sub = [x[: N5 // 16].copy() for x in xs]
            op1 = "avg" if dtype == "fp32" else "sum"
            t1 = time_cpu(lambda: orc.allreduce(sub, dtype, op1, "oneshot"), 2) * 16
            orc.set_num_threads(threads)
            res["allreduce"][f"{dtype} {op1}"]["cpu_oracle"]["single_thread"] = {
                "seconds": round(t1, 3), "busbw_GBps": round(2 * (P - 1) / P * s_full / t1 / 1e9, 4), "cores": 1,
                "sample": "first 1/16 of each rank's buffer, median of 2, scaled to the full buffer"}
            del sub, small
        del din, dout, rs_out, xs
        torch.cuda.empty_cache()
    return res


def oneshot_by_p(sim, torch, dev, stream, steps: int) -> dict:
    """The one-shot at 64 MiB per rank, bf16, for p = 2, 4, 8, 16 (workload
    3's values), each next to the k-stream copy of the same p input and p
    output buffers (its access pattern without the fold)."""
    out = {}
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    for p in (2, 4, 8, 16):
        ins = [(torch.randn(N, device=dev, generator=g) * 0.02).to(torch.bfloat16).view(torch.int16)
               for _ in range(p)]
        outs = [torch.empty_like(ins[0]) for _ in range(p)]
        ip, op_ = [t.data_ptr() for t in ins], [t.data_ptr() for t in outs]

        def ar():
            if sim.sim_allreduce(ip, op_, p, N, "bf16", "sum", "oneshot", stream):
                raise sim.SimError(-1, "sim_allreduce")

        def cp():
            if sim.sim_copy_streams(ip, op_, p, S, 0, stream):
                raise sim.SimError(-1, "sim_copy_streams")
        t_ar, t_cp = time_calls(ar, steps, 3), time_calls(cp, steps, 3)
        law = 2.0 * p * S
        out[str(p)] = {"oneshot_us": round(t_ar * 1e6, 2), "oneshot_frac": round(law / t_ar / 1e9 / HBM_PEAK_GBPS, 4),
                       "copy_us": round(t_cp * 1e6, 2), "copy_frac": round(law / t_cp / 1e9 / HBM_PEAK_GBPS, 4),
                       "oneshot_over_copy": round(t_cp / t_ar, 4)}
        del ins, outs
        torch.cuda.empty_cache()
    assert sim.sim_check_error(stream) == 0
    return out


def workload4(sim, synthdata, torch, np, dev, stream) -> dict:
    """Per-call microseconds, p = 8, fp16 N(0,1), 1 KiB .. 1 MiB per rank:
    the LL packet path vs the plain one-shot, and the selector's pick.  The
    buffers are re-used (at these sizes the working set sits in the cache
    either way)."""
    out = {}
    for k in range(10, 21):
        n = (1 << k) // 2
        xs = synthdata.workload_inputs(4, P, n, "fp16")
        din = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs]
        dout = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(P)]
        ip, op_ = [t.data_ptr() for t in din], [t.data_ptr() for t in dout]
        row = {}
        for a in ("oneshot", "oneshot_ll", "auto"):
            call = sim.prepare_allreduce(ip, op_, P, n, "fp16", "sum", a, stream)
            if call() != 0:
                raise sim.SimError(call(), f"sim_allreduce({a})")
            row[a] = round(time_calls(call, 1000, 100) * 1e6, 2)
            if a == "auto":
                row["auto_pick"] = sim.sim_last_algo()
        out[f"{1 << k >> 10}KiB"] = row
    assert sim.sim_check_error(stream) == 0
    return out


def algorithmic_bytes_at(algo: str, n: int, esize: int) -> float:
    """All-reduce traffic laws at n elements per rank of `esize` bytes."""
    s_ = n * esize
    if algo == "oneshot":
        return 2.0 * P * s_
    if algo == "allpairs":
        return (2.0 * P + 1.0) * s_
    if algo == "allpairs_persistent":
        return (3.0 * P - 1.0) * s_
    if algo == "ring":
        if esize == 4:
            return 5.0 * (P - 1) * s_
        return n * (esize + esize + 4) + (P - 3) * n * (4 + esize + 4) + n * (4 + esize + esize) \
            + (P - 1) * n * (esize + esize)
    if algo == "ring_fifo":
        return 2.0 * P * s_ + (P - 1) * n * 8.0 + (P - 1) * n * esize
    raise ValueError(algo)


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
        # Counter scale references of known size: the library's k-stream copy
        # (sim_copy_streams) with k = 1, 512 MiB read and 512 MiB written per
        # launch, and with k = 8, 64 MiB per stream (the one-shot's 16
        # streams: 512 MiB read, 512 MiB written); torch's device-to-device
        # copy of 512 MiB for comparison.
        sim.sim_init(0, 2, 0)
        s2 = int(torch.cuda.current_stream().cuda_stream)
        res = {}
        for k, per in ((1, 512 << 20), (8, 64 << 20)):
            src = [torch.randint(-2 ** 31, 2 ** 31 - 1, (per // 4,), dtype=torch.int32, device=dev) for _ in range(k)]
            dst = [torch.empty_like(src[0]) for _ in range(k)]
            sp, dp = [t.data_ptr() for t in src], [t.data_ptr() for t in dst]
            res[f"k_copy_streams<{k}> us"] = round(time_calls(
                lambda: sim.sim_copy_streams(sp, dp, k, per, 0, s2), args.steps, args.warmup) * 1e6, 2)
            res[f"k_copy_streams<{k}> bytes read / written per launch"] = k * per
            del src, dst
        src = torch.randint(-2 ** 31, 2 ** 31 - 1, ((512 << 20) // 4,), dtype=torch.int32, device=dev)
        dst = torch.empty_like(src)
        res["torch copy of 512 MiB us"] = round(time_calls(lambda: dst.copy_(src), args.steps, args.warmup) * 1e6, 2)
        print(json.dumps(res), flush=True)
        return
    sim.sim_init(0, 16, S)  # p up to 16 for the one-shot-by-p figures
    stream = int(torch.cuda.current_stream().cuda_stream)
    if args.profile_size:
        n = args.profile_size // 2
        xs = synthdata.workload_inputs(4, P, n, "fp16")
        din = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs]
        dout = [torch.empty(n, dtype=torch.int16, device=dev) for _ in range(P)]
        ip, op_ = [t.data_ptr() for t in din], [t.data_ptr() for t in dout]
        res = {}
        for a in args.profile_algos.split(","):
            call = sim.prepare_allreduce(ip, op_, P, n, "fp16", "sum", a, stream)
            if call() != 0:
                raise sim.SimError(call(), f"sim_allreduce({a})")
            res[a] = round(time_calls(call, args.steps, args.warmup) * 1e6, 3)
        assert sim.sim_check_error(stream) == 0
        print(json.dumps({"bytes_per_rank": args.profile_size, "us_per_call": res}), flush=True)
        return
    if args.profile_rsag:
        n_out = N5 // P
        xs5 = synthdata.workload_inputs(5, P, N5, "fp32")
        d5 = [torch.from_numpy(x).to(dev) for x in xs5]
        del xs5
        o5 = [torch.empty(N5, dtype=torch.float32, device=dev) for _ in range(P)]
        r5 = [torch.empty(n_out, dtype=torch.float32, device=dev) for _ in range(P)]
        i5, p5, q5 = [t.data_ptr() for t in d5], [t.data_ptr() for t in o5], [t.data_ptr() for t in r5]
        res = {}
        for a in ("allpairs", "ring"):
            def rs(a=a):
                if sim.sim_reduce_scatter(i5, q5, P, n_out, "fp32", "avg", a, stream):
                    raise sim.SimError(-1, "sim_reduce_scatter")
            res[f"reduce_scatter {a}"] = round(time_calls(rs, args.steps, args.warmup) * 1e6, 2)
        for a in ("allpairs", "ring"):
            def ag(a=a):
                if sim.sim_all_gather(q5, p5, P, n_out, "fp32", a, stream):
                    raise sim.SimError(-1, "sim_all_gather")
            res[f"all_gather {a}"] = round(time_calls(ag, args.steps, args.warmup) * 1e6, 2)
        assert sim.sim_check_error(stream) == 0
        print(json.dumps({"workload": "fp32, p=8, 256 MiB per rank", "us_per_call": res}), flush=True)
        return
    if args.profile_large:
        us5 = large_workload(sim, synthdata, torch, np, dev, stream, args.steps, args.warmup)
        print(json.dumps({"workload": "fp32 avg, p=8, 256 MiB per rank", "us_per_step": us5}), flush=True)
        return

    xs = synthdata.workload_inputs(3, P, N, "bf16")
    din = [torch.from_numpy(x.view(np.int16)).to(dev) for x in xs]
    dout = [torch.empty(N, dtype=torch.int16, device=dev) for _ in range(P)]
    ip = [t.data_ptr() for t in din]
    op_ = [t.data_ptr() for t in dout]
    # consecutive timed calls alternate between two buffer sets (the second
    # set's inputs are the same seeded values), so no call finds its
    # predecessor's data in the 256 MB Infinity Cache: 2 GiB touched per pair
    din2 = [t.clone() for t in din]
    dout2 = [torch.empty_like(t) for t in dout]
    sets = [(ip, op_), ([t.data_ptr() for t in din2], [t.data_ptr() for t in dout2])]
    turn = [0]

    def step(algo=args.algo):
        i_, o_ = sets[turn[0]]
        turn[0] ^= 1
        st = sim.sim_allreduce(i_, o_, P, N, "bf16", "sum", algo, stream)
        if st:
            raise sim.SimError(st, "sim_allreduce")

    t = time_calls(step, args.steps, args.warmup)
    assert sim.sim_check_error(stream) == 0
    ran = sim.sim_last_algo()
    phased = ran == "oneshot" and sim.sim_debug_get("phased_last") == 1
    if args.profile_only:
        print(json.dumps({"algo": ran, "us_per_step": t * 1e6}), flush=True)
        return
    # the same step repeated in 5 further batches (spread of the timed figure)
    reps = [time_calls(step, max(10, args.steps // 5), 2) for _ in range(5)]
    busbw = 2 * (P - 1) / P * S / t / 1e9
    kernel = {"oneshot": "k_fold_phased (one-shot, phased)" if phased else "k_fold (one-shot, all outputs)",
              "allpairs": "k_fold + k_copy",
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
        # the phased one-shot's block layouts side by side on the headline:
        # per chunk against the whole-buffer layout the library picks here
        # (SIM_DEBUG_PHASED_LAYOUT), alternating, three batches each
        lay = {"per_chunk_us": [], "whole_buffer_us": []}
        for _ in range(3):
            for key, v in (("per_chunk_us", 1), ("whole_buffer_us", 0)):
                sim.sim_debug_set("phased_layout", v)
                lay[key].append(round(time_calls(lambda: step("oneshot"), max(10, args.steps // 4), 5) * 1e6, 2))
                if v == 0:
                    lay["whole_buffer_ran"] = sim.sim_debug_get("phased_whole_last")
        sim.sim_debug_set("phased_layout", 0)
        lay["ratio_of_medians"] = round(float(np.median(lay["whole_buffer_us"]) / np.median(lay["per_chunk_us"])), 4)
        extras["phased_layout_ab_us"] = lay
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
        extras["workload4_latency_us"] = workload4(sim, synthdata, torch, np, dev, stream)
        import oracle
        ext_steps = max(10, args.steps // 4)
        extras["workload2_fp32_32MiB"] = workload2(sim, synthdata, oracle, torch, np, dev, stream, ext_steps,
                                                   not args.no_cpu_baseline)
        extras["workload5_256MiB"] = workload5(sim, synthdata, oracle, torch, np, dev, stream,
                                               max(5, args.steps // 10), not args.no_cpu_baseline)
        extras["ceiling"] = ceiling(sim, torch, dev, stream, max(10, args.steps // 2), sets)
        extras["ceiling"]["oneshot_vs_copy_by_p"] = oneshot_by_p(sim, torch, dev, stream, max(10, args.steps // 2))
        cf = max(extras["ceiling"]["copy_8in_8out_64MiB_each"]["GBps"],
                 extras["ceiling"]["copy_headline_buffers"]["GBps"])
        extras["ceiling"]["oneshot_over_8x8_copy"] = round(achieved / cf, 4) if ran == "oneshot" else None
        w5 = extras["workload5_256MiB"]["allreduce"]["fp32 avg"]
        extras["ceiling"]["workload5_oneshot_over_its_8x8_copy"] = round(
            w5["hbm_algorithmic_GBps"] / extras["ceiling"]["copy_8in_8out_256MiB_each"]["GBps"], 4)

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
               "kind": "oracle", "cpu_model": cpu_model(),
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
    if not args.no_extras:
        # the selector against measurement (this re-initialises the library
        # and loads the packaged calibration)
        from all_reduce_reduction_amd import calibrate
        del din, dout, din2, dout2, sets
        torch.cuda.empty_cache()
        rep = calibrate.check(sim.CALIBRATION, steps_scale=0.1, reps=3)
        out["selector_check"] = {
            b: {k: v[k] for k in ("cases", "strict_matches", "tolerant_matches", "runner_up_strict",
                                  "runner_up_tolerant", "pairs_agree", "pairs",
                                  "pick_rel_error_median", "pick_rel_error_max")}
            | {"picks": sorted({r["pick"] for r in v["rows"]}), "fastest": sorted({r["measured_best"] for r in v["rows"]})}
            for b, v in rep["budgets"].items()}
    print(json.dumps(out), flush=True)
    sim.sim_finalize()


if __name__ == "__main__":
    main()
