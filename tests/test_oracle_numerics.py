"""Pins for the oracle's bit-level conversions (exact rational rounding as the reference)."""

from fractions import Fraction

import numpy as np

from oracle.numerics import bf16_to_f32, f32_to_f16_bits, f16_bits_to_f64


def _f16_values():
    """All finite fp16 values as (bits, Fraction), sorted by value."""
    bits = np.arange(0, 0x10000, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    ok = np.isfinite(vals)
    out = sorted({(float(v), int(b)) for v, b in zip(vals[ok], bits[ok]) if not (v == 0 and b == 0x8000)})
    return out


_F16 = _f16_values()
_F16_VALS = np.array([v for v, _ in _F16])


def _rne_f16_exact(x: float) -> float:
    """Round a float to fp16 exactly (nearest, ties to the even mantissa)."""
    fx = Fraction(x)
    i = int(np.searchsorted(_F16_VALS, x))
    cands = []
    for j in (i - 1, i, i + 1):
        if 0 <= j < len(_F16_VALS):
            cands.append((abs(Fraction(_F16_VALS[j]) - fx), _F16[j][1], _F16_VALS[j]))
    cands.sort(key=lambda c: c[0])
    best = cands[0]
    ties = [c for c in cands if c[0] == best[0]]
    if len(ties) > 1:
        best = min(ties, key=lambda c: c[1] & 1)   # even mantissa
    return float(best[2])


def test_f32_to_f16_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    xs = np.concatenate([
        rng.standard_normal(3000).astype(np.float32) * 3,
        rng.standard_normal(500).astype(np.float32) * 1e-5,      # subnormal fp16 range
        np.clip(rng.standard_normal(500) * 3e4, -65000, 65000).astype(np.float32),
    ])  # fp16 overflow is outside the quantizer's contract
    # exact midpoints between neighbouring fp16 values (ties), representable in fp32
    mids = []
    for a, b in zip(_F16_VALS[1000:1100], _F16_VALS[1001:1101]):
        m = np.float32((a + b) / 2)
        if float(m) == (a + b) / 2:
            mids.append(m)
    xs = np.concatenate([xs, np.array(mids, dtype=np.float32)])
    got = f16_bits_to_f64(f32_to_f16_bits(xs))
    for x, g in zip(xs, got):
        assert g == _rne_f16_exact(float(x)), (x, g)


def test_bf16_to_f32_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0001, 0x7F7F], dtype=np.uint16)
    want = [1.0, -1.0, 3.140625, float(np.uint32(1 << 16).view(np.float32)),
            float(np.uint32(0x7F7F0000).view(np.float32))]
    assert list(bf16_to_f32(bits).astype(np.float64)) == want
