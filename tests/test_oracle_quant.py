"""Pins for the oracle's per-token asymmetric quantizer."""

import json
import os

import numpy as np
import pytest

from oracle.hadamard import fwht_f32
from oracle.numerics import f16_bits_to_f64
from oracle.quant import (INT2_QMAX, INT3_QMAX, INT4_QMAX, INT8_QMAX, bytes_per_token_head, dequantize,
                          pack_int2, pack_int3, pack_int4, qmax_of, quantize, tie_flags, tie_near, unpack_int2, unpack_int3,
                          unpack_int4)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _vectors(n, seed, outliers=True):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128))
    if outliers:
        x[:, rng.choice(128, 4, replace=False)] *= 20
    return x.astype(np.float32)


def _brute_nearest(y, scale_h, zero_h, qmax):
    """Exhaustive nearest grid level zero + c*scale over all qmax+1 codes (fp64,
    exact for these magnitudes), ties to the even code."""
    s = f16_bits_to_f64(scale_h)[:, None, None]
    z = f16_bits_to_f64(zero_h)[:, None, None]
    levels = z + s * np.arange(qmax + 1)[None, None, :]
    dist = np.abs(y.astype(np.float64)[:, :, None] - levels)
    cand = dist == dist.min(axis=-1, keepdims=True)
    even = cand & (np.arange(qmax + 1) % 2 == 0)
    code = np.where(even.any(axis=-1), np.argmax(even, axis=-1), np.argmax(cand, axis=-1))
    return code


@pytest.mark.parametrize("qmax", [INT2_QMAX, INT3_QMAX, INT4_QMAX, INT8_QMAX])
def test_codes_are_nearest_levels(qmax):
    y = fwht_f32(_vectors(3000, 1), 128)
    c, sb, zb = quantize(y, qmax)
    nonzero = f16_bits_to_f64(sb) > 0
    brute = _brute_nearest(y[nonzero], sb[nonzero], zb[nonzero], qmax)
    # levels outside [0, qmax] are clamped in both; compare inside the grid
    mism = brute != c[nonzero]
    ties = tie_near(y, qmax)[nonzero]
    assert not np.any(mism & ~ties), int((mism & ~ties).sum())


@pytest.mark.parametrize("qmax", [INT2_QMAX, INT3_QMAX, INT4_QMAX, INT8_QMAX])
def test_scale_and_zero_are_fp16_of_range_and_min(qmax):
    y = _vectors(2000, 2)
    c, sb, zb = quantize(y, qmax)
    mn = y.min(axis=1).astype(np.float64)
    mx = y.max(axis=1).astype(np.float64)
    s = f16_bits_to_f64(sb)
    z = f16_bits_to_f64(zb)
    exact = (mx - mn) / qmax
    assert np.all(np.abs(s - exact) <= 2.0 ** -11 * exact * 1.0001 + 1e-12)
    assert np.all(np.abs(z - mn) <= 2.0 ** -11 * np.abs(mn) * 1.0001 + 2.0 ** -25)


@pytest.mark.parametrize("qmax", [INT2_QMAX, INT3_QMAX, INT4_QMAX, INT8_QMAX])
def test_round_trip_bound(qmax):
    y = fwht_f32(_vectors(3000, 3), 64)
    c, sb, zb = quantize(y, qmax)
    xh = dequantize(c, sb, zb)
    s = f16_bits_to_f64(sb)
    z = f16_bits_to_f64(zb)
    mn = y.min(axis=1).astype(np.float64)
    mx = y.max(axis=1).astype(np.float64)
    slack = np.maximum.reduce([np.zeros_like(s), z - mn, mx - z - qmax * s])
    bound = s / 2 + slack
    err = np.abs(y.astype(np.float64) - xh).max(axis=1)
    assert np.all(err <= bound * (1 + 1e-6) + 1e-7)
    # and in exact arithmetic (fp64 scale/zero, no fp16 rounding) the bound is scale/2
    assert np.all(err <= s * 0.5 + slack + 1e-6 * np.abs(y).max(axis=1))


@pytest.mark.parametrize("qmax", [INT2_QMAX, INT3_QMAX, INT4_QMAX, INT8_QMAX])
def test_grid_vectors_round_trip_exactly(qmax):
    rng = np.random.default_rng(4)
    n = 200
    s = (rng.integers(1, 64, n) * 2.0 ** -8).astype(np.float16).astype(np.float32)
    z = (rng.integers(-64, 64, n) * 2.0 ** -4).astype(np.float16).astype(np.float32)
    codes = rng.integers(0, qmax + 1, (n, 128))
    codes[:, 0] = 0
    codes[:, 1] = qmax
    y = (z[:, None] + codes * s[:, None]).astype(np.float32)
    assert np.array_equal(y.astype(np.float64), z[:, None].astype(np.float64) + codes * s[:, None].astype(np.float64))
    c, sb, zb = quantize(y, qmax)
    assert np.array_equal(c, codes)
    assert np.array_equal(f16_bits_to_f64(sb), s.astype(np.float64))
    assert np.array_equal(f16_bits_to_f64(zb), z.astype(np.float64))
    assert np.array_equal(dequantize(c, sb, zb), y.astype(np.float64))


@pytest.mark.parametrize("qmax", [INT2_QMAX, INT3_QMAX, INT4_QMAX, INT8_QMAX])
def test_zero_range_guard(qmax):
    y = np.stack([np.full(128, 0.3, np.float32), np.zeros(128, np.float32),
                  np.full(128, -7.25, np.float32)])
    c, sb, zb = quantize(y, qmax)
    assert np.all(c == 0)
    assert np.all(f16_bits_to_f64(sb) == 0)
    assert np.array_equal(f16_bits_to_f64(zb), np.array([0.3, 0.0, -7.25], np.float32).astype(np.float16).astype(np.float64))
    assert np.all(np.isfinite(dequantize(c, sb, zb)))


def test_tiny_range_underflowing_fp16_scale_is_guarded():
    y = np.full((1, 128), 1.0, np.float32)
    y[0, 5] = np.nextafter(np.float32(1.0), np.float32(2.0))   # range 1.2e-7: fp16 scale underflows to 0
    c, sb, zb = quantize(y, INT4_QMAX)
    assert f16_bits_to_f64(sb)[0] == 0 and np.all(c == 0)


def test_rotation_reduces_error_on_outlier_keys():
    """SAW-INT4 section 2: rotating blocks before 4-bit quantization spreads outlier
    channels and lowers the quantization error (checked on outlier-heavy vectors)."""
    x = _vectors(2000, 5)
    errs = {}
    for h in (1, 128):
        y = fwht_f32(x, h)
        c, sb, zb = quantize(y, INT4_QMAX)
        errs[h] = np.mean((dequantize(c, sb, zb) - y) ** 2)
    assert errs[128] < 0.25 * errs[1]


def test_pack_unpack_round_trip():
    rng = np.random.default_rng(6)
    c = rng.integers(0, 16, (50, 128)).astype(np.uint8)
    p = pack_int4(c)
    assert p.shape == (50, 64)
    assert np.array_equal(p[:, 0], c[:, 0] | (c[:, 1] << 4))
    assert np.array_equal(unpack_int4(p), c)


def test_storage_accounting_matches_pages():
    g = json.load(open(os.path.join(GOLDEN, "storage_accounting.json")))
    d = g["group_dims"]
    per_elem_bits = bytes_per_token_head(d, 4) * 8 / (2 * d)
    assert per_elem_bits == g["bits_per_element"] == g["code_bits"] + g["param_bits_per_group"] / d
    assert bytes_per_token_head(128, 4) == 136
    assert bytes_per_token_head(128, 8) == 264


def test_pack_int2_round_trip_and_bit_order():
    rng = np.random.default_rng(7)
    c = rng.integers(0, 4, (40, 128)).astype(np.uint8)
    p = pack_int2(c)
    assert p.shape == (40, 32)
    assert np.array_equal(p[:, 0], c[:, 0] | (c[:, 1] << 2) | (c[:, 2] << 4) | (c[:, 3] << 6))
    assert np.array_equal(unpack_int2(p), c)
    # a worked byte: codes 3, 0, 2, 1 -> 0b01_10_00_11
    assert pack_int2(np.array([3, 0, 2, 1], np.uint8))[0] == 0x63


def test_code_widths():
    assert [qmax_of(b) for b in (2, 3, 4, 8)] == [3, 7, 15, 255]
    for bad in (1, 5, 6):
        with pytest.raises(ValueError):
            qmax_of(bad)
    # K+V bytes per (token, head) at 2 bits: 2 * (32 + 4) = 72, i.e. 2.25 bits per element;
    # at 3 bits: 2 * (48 + 4) = 104, 3.25 bits per element
    assert bytes_per_token_head(128, 2) == 72
    assert bytes_per_token_head(128, 2) * 8 / 256 == 2.25
    assert bytes_per_token_head(128, 3) == 104
    assert bytes_per_token_head(128, 3) * 8 / 256 == 3.25
    assert pack_int3(np.zeros((1, 128), np.uint8)).shape == (1, 48)


def test_pack_int3_round_trip_and_bit_order():
    rng = np.random.default_rng(17)
    c = rng.integers(0, 8, (40, 128)).astype(np.uint8)
    p = pack_int3(c)
    assert p.shape == (40, 48)
    assert np.array_equal(unpack_int3(p), c)
    # the low plane is the 2-bit packing of the low bits, the high plane bit i of
    # byte j is element 8 j + i's bit 2
    assert np.array_equal(p[:, :32], pack_int2(c & 3))
    assert np.array_equal((p[:, 32] >> 3) & 1, (c[:, 3] >> 2) & 1)
    # a worked vector: codes 7, 0, 5, 2, 4, 1, 6, 3 -> low plane bytes 0b10_01_00_11,
    # 0b11_10_01_00; high plane byte 0b0101_0101
    w = np.zeros(128, np.uint8)
    w[:8] = [7, 0, 5, 2, 4, 1, 6, 3]
    pw = pack_int3(w)
    assert pw[0] == 0x93 and pw[1] == 0xE4 and pw[32] == 0x55 and not pw[2:32].any() and not pw[33:].any()


def test_int3_cache_keeps_the_int8_protection():
    """A 3-bit main cache: main codes in [0, 7], the INT8 region's copies unchanged."""
    import torch
    from oracle.cache import quantize_sequence
    from workloads import bf16_bits
    rng = np.random.default_rng(18)
    k = bf16_bits(torch.from_numpy(rng.standard_normal((50, 2, 128)) * 3).to(torch.bfloat16))
    v = bf16_bits(torch.from_numpy(rng.standard_normal((50, 2, 128))).to(torch.bfloat16))
    c4 = quantize_sequence(k, v, 64, 4, 16)
    c3 = quantize_sequence(k, v, 64, 4, 16, main_bits=3)
    assert c3.k4.max() <= 7 and c3.v4.max() <= 7 and c4.k4.max() > 7
    assert np.array_equal(c3.pos8, c4.pos8) and np.array_equal(c3.k8, c4.k8) and np.array_equal(c3.v8, c4.v8)


def test_int2_cache_keeps_the_int8_protection():
    """A 2-bit main cache: main codes in [0, 3], the INT8 region's copies unchanged."""
    import torch
    from oracle.cache import quantize_sequence
    from workloads import bf16_bits
    rng = np.random.default_rng(8)
    k = bf16_bits(torch.from_numpy(rng.standard_normal((50, 2, 128)) * 3).to(torch.bfloat16))
    v = bf16_bits(torch.from_numpy(rng.standard_normal((50, 2, 128))).to(torch.bfloat16))
    c4 = quantize_sequence(k, v, 64, 4, 16)
    c2 = quantize_sequence(k, v, 64, 4, 16, main_bits=2)
    assert c2.k4.max() <= 3 and c2.v4.max() <= 3 and c4.k4.max() > 3
    assert np.array_equal(c2.pos8, c4.pos8) and np.array_equal(c2.k8, c4.k8) and np.array_equal(c2.v8, c4.v8)


# --- the tie gate: which GPU / oracle differences a parity test may forgive ----

def _f32(x):
    return np.asarray(x, np.float32)


def test_tie_flags_mark_an_exact_half_and_not_a_thousandth_away():
    """A quotient t exactly at k + 1/2 is a rounding tie; 1e-3 away it is not.
    The vector [0, 15, ...] has scale_f = 1 and zero 0 exactly (both fp16
    values), so t_i = y_i."""
    y = np.zeros((3, 128), np.float32)
    y[:, 1] = 15.0
    y[0, 2] = 7.5                  # exact tie
    y[1, 2] = 7.501                # 1e-3 away
    y[2, 2] = 7.4990               # 1e-3 away below
    el, vec = tie_flags(y, INT4_QMAX)
    assert not vec.any()
    assert el[0, 2] and not el[1, 2] and not el[2, 2]
    # grid points (t integral) are never ties
    assert not el[:, :2].any() and not el[:, 3:].any()
    # the codes themselves: 7.5 rounds to the even 8
    c, _, _ = quantize(y, INT4_QMAX)
    assert c[0, 2] == 8 and c[1, 2] == 8 and c[2, 2] == 7


@pytest.mark.parametrize("qmax", [INT2_QMAX, INT3_QMAX, INT4_QMAX, INT8_QMAX])
def test_tie_flags_every_half_integer_of_the_grid(qmax):
    """All half-integers k + 1/2 (k < qmax) are flagged, all integers are not."""
    y = np.zeros((1, 128), np.float32)
    y[0, 1] = qmax                               # scale 1, zero 0
    k = np.arange(min(qmax, 126))
    y[0, 2:2 + len(k)] = k + 0.5
    el, vec = tie_flags(y, qmax)
    assert not vec.any()
    assert el[0, 2:2 + len(k)].all()
    assert not el[0, :2].any() and not el[0, 2 + len(k):].any()


def test_tie_flags_mark_an_fp16_midpoint_scale_and_not_a_thousandth_away():
    """scale_f exactly at the midpoint 1 + 2^-11 of the fp16 neighbours 1 and
    1 + 2^-10 is a vector tie; a scale 1e-3 (relative) away is not."""
    mid = 1.0 + 2.0 ** -11
    y = np.zeros((2, 128), np.float32)
    y[0, 1] = np.float32(15 * mid)                # exact in fp32, scale_f = mid exactly
    assert np.float32(y[0, 1]) / np.float32(15) == np.float32(mid)
    y[1, 1] = np.float32(15 * mid * (1 + 1e-3))
    el, vec = tie_flags(y, INT4_QMAX)
    assert vec[0] and not vec[1]


def test_tie_flags_mark_an_fp16_midpoint_min_and_not_a_thousandth_away():
    """The offset is fp16(min): a min at an fp16 midpoint is a vector tie."""
    mid = -(1.0 + 2.0 ** -11)
    y = np.zeros((2, 128), np.float32)
    y[:, 1] = 15.0
    y[0, 0] = np.float32(mid)
    y[1, 0] = np.float32(mid * (1 + 1e-3))
    el, vec = tie_flags(y, INT4_QMAX)
    assert vec[0] and not vec[1]
    # a vector tie flags every element of the vector in tie_near
    near = tie_near(y, INT4_QMAX)
    assert near[0].all()
    assert near[1].sum() == el[1].sum()


def test_tie_flags_guarded_vectors_have_no_element_ties():
    """With the zero-range guard every code is 0: no quotient decides a code."""
    y = np.full((2, 128), 0.5, np.float32)       # 0.5 would sit at t = k + 1/2 with scale 1
    el, vec = tie_flags(y, INT4_QMAX)
    assert not el.any()


@pytest.mark.parametrize("qmax", [INT2_QMAX, INT3_QMAX, INT4_QMAX, INT8_QMAX])
def test_tie_flags_are_rare_on_random_vectors(qmax):
    """On the workloads' value distribution the gate forgives little: an element's
    t lies within 1e-6 |t| of a half-integer with probability about 2e-6 |t|
    (mean |t| about qmax / 2), and a vector's two fp16 roundings each fall within
    1e-6 of a midpoint with probability about 2e-6 / 2^-10.  Bounds: 3e-6 (qmax + 1)
    of the elements, 2% of the vectors."""
    y = fwht_f32(_vectors(20000, 8), 128)
    el, vec = tie_flags(y, qmax)
    assert el.mean() < 3e-6 * (qmax + 1), el.mean()
    assert vec.mean() < 0.02, vec.mean()
    assert tie_near(y, qmax).mean() < 0.03


def test_input_domain_edge_of_the_fp16_params():
    """The stored params are fp16: at |min| = 65504 and range / qmax = 65504 they
    are finite (the largest fp16 value); just past either the offset or the
    scale rounds to infinity and the dequantized vector is no longer finite,
    which is why the library states this input domain."""
    inside = np.zeros((2, 128), np.float32)
    inside[0, 0] = -65504.0                         # |min| at the fp16 maximum
    inside[1, 1] = np.float32(15 * 65504.0)         # range / 15 at the fp16 maximum
    c, sb, zb = quantize(inside, INT4_QMAX)
    assert np.all(np.isfinite(dequantize(c, sb, zb)))
    outside = np.zeros((2, 128), np.float32)
    outside[0, 0] = -65536.0                        # rounds past the fp16 maximum
    outside[1, 1] = np.float32(15 * 65536.0)
    c, sb, zb = quantize(outside, INT4_QMAX)
    assert not np.isfinite(dequantize(c, sb, zb)[0]).all()
    assert not np.isfinite(dequantize(c, sb, zb)[1]).all()
