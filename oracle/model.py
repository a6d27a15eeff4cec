"""Alpha-beta cost model, written out -- TEST INFRASTRUCTURE ONLY.

"MSCCL, in depth ...", section "Why generic collectives leave time on the
table", prices a schedule as a per-step latency alpha times its number of
synchronised steps, plus the bytes it moves over the bandwidth B.  Over p
ranks the ring all-reduce has 2(p-1) steps and the all-pairs schedule 2,
and each moves 2(p-1)/p of the buffer:

    T_ring(n)     = 2(p-1) alpha + 2(p-1)/p * n / B
    T_allpairs(n) = 2      alpha + 2(p-1)/p * n / B

The same page's section "Worked example: all-pairs versus ring on 8 GPUs"
prices all-pairs with the LL protocol (4 data bytes per 8-byte word, so half
the link rate) and the ring with LL128 (120 of 128 bytes carry data).
"Inside NCCL all-reduce", section "How NCCL picks: a cost model, not a
threshold", states the same form (latency x hop count + bytes / bandwidth)
and takes the argmin over the legal candidates.
"""
from __future__ import annotations

LL_EFFICIENCY = 4.0 / 8.0        # 4 data bytes per 8-byte LL word
LL128_EFFICIENCY = 120.0 / 128.0  # 120 data bytes per 128-byte LL128 line


def t_ring(p: int, nbytes: float, alpha_s: float, bw_Bps: float) -> float:
    return 2 * (p - 1) * alpha_s + 2 * (p - 1) / p * nbytes / bw_Bps


def t_allpairs(p: int, nbytes: float, alpha_s: float, bw_Bps: float) -> float:
    return 2 * alpha_s + 2 * (p - 1) / p * nbytes / bw_Bps


def worked_example(nbytes: float, p: int = 8, link_Bps: float = 300e9, alpha_s: float = 2e-6):
    """(T_allpairs with LL, T_ring with LL128) for the 8-GPU example."""
    return (t_allpairs(p, nbytes, alpha_s, link_Bps * LL_EFFICIENCY),
            t_ring(p, nbytes, alpha_s, link_Bps * LL128_EFFICIENCY))


def crossover_bytes(p: int = 8, link_Bps: float = 300e9, alpha_s: float = 2e-6) -> float:
    """Size where the two example lines cross (solved in closed form)."""
    # 2(p-1) a + k n / B128 = 2 a + k n / BLL, with k = 2(p-1)/p
    k = 2 * (p - 1) / p
    lat_gap = (2 * (p - 1) - 2) * alpha_s
    per_byte_gap = k / (link_Bps * LL_EFFICIENCY) - k / (link_Bps * LL128_EFFICIENCY)
    return lat_gap / per_byte_gap


def argmin(costs: dict) -> str:
    """The cheapest legal candidate (ties: the first in insertion order)."""
    best = None
    for name, t in costs.items():
        if best is None or t < costs[best]:
            best = name
    return best
