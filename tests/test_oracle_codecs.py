"""The oracle's own bf16/fp16 codecs against library conversions
(torch CPU bfloat16 casts, numpy float16 casts; both round to nearest,
ties to even)."""
import numpy as np
import torch


def _same_or_both_nan(a32, b32):
    a = a32.view(np.float32)
    b = b32.view(np.float32)
    both_nan = np.isnan(a) & np.isnan(b)
    return both_nan | (a32.view(np.uint32) == b32.view(np.uint32))


def _torch_bf16_bits(x32):
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_widen_all_patterns(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.bf16_to_f32(h)
    want = torch.from_numpy(h.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    assert _same_or_both_nan(got, want).all()


def test_f16_widen_all_patterns(orc):
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.f16_to_f32(h)
    want = h.view(np.float16).astype(np.float32)
    assert _same_or_both_nan(got, want).all()


def _bf16_probe_patterns():
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x4000, 0xC000], dtype=np.uint32)
    pats = (hi[:, None] | lows[None, :]).ravel()
    rnd = np.random.default_rng(0).integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32)
    return np.concatenate([pats, rnd]).view(np.float32)


def test_bf16_narrow_ties_and_random(orc):
    x = _bf16_probe_patterns()
    got = orc.f32_to_bf16(x)
    want = _torch_bf16_bits(x)
    nan = np.isnan(x)
    assert (got[~nan] == want[~nan]).all()
    # NaN stays NaN (exponent all ones, nonzero fraction)
    assert (((got[nan] & 0x7F80) == 0x7F80) & ((got[nan] & 0x7F) != 0)).all()


def _f16_probe_patterns():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    v = h.view(np.float16).astype(np.float32)
    fin = np.isfinite(v)
    v = v[fin]
    with np.errstate(over="ignore"):
        nxt = np.nextafter(h[fin].view(np.float16), np.float16(np.inf)).astype(np.float32)
    mid = ((v.astype(np.float64) + nxt.astype(np.float64)) / 2).astype(np.float32)  # exact ties
    around = np.concatenate([mid, np.nextafter(mid, np.float32(np.inf)), np.nextafter(mid, np.float32(-np.inf))])
    big = np.array([65504, 65519.996, 65520, 65536, 1e9, -65520, 2.0 ** -24, 2.0 ** -25, 2.0 ** -26,
                    3 * 2.0 ** -26, 1e-30, -1e-30, 0.0, -0.0], dtype=np.float32)
    rnd = np.random.default_rng(1).integers(0, 1 << 32, 1 << 22, dtype=np.uint64).astype(np.uint32).view(np.float32)
    return np.concatenate([v, around[np.isfinite(around)], big, rnd])


def test_f16_narrow_ties_and_random(orc):
    x = _f16_probe_patterns()
    got = orc.f32_to_f16(x)
    with np.errstate(over="ignore", invalid="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert (got[~nan] == want[~nan]).all()
    assert (((got[nan] & 0x7C00) == 0x7C00) & ((got[nan] & 0x3FF) != 0)).all()
