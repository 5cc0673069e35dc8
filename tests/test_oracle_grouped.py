"""Pins for the oracle's keys with a bit width per RoPE-block group.

RoPE-Aware Bit Allocation for KV-Cache Quantization (Block-GTQ), Abstract:
integer bit widths per RoPE frequency block, served from a packed cache.  The
allocation is an input here (packing only); these tests pin the grouping, the
quantizer and its storage cost.
"""

import numpy as np
import pytest

from oracle.attention import attend
from oracle.cache import dequantized_kv, quantize_sequence
from oracle.hadamard import fwht_f32
from oracle.numerics import f16_bits_to_f64
from oracle.quant import (INT4_QMAX, dequantize_grouped, group_widths_per_dim, grouped_key_bytes_per_token,
                          grouped_tie_flags, quantize, quantize_grouped, rope_group_of_dim)

WIDTHS = [(4, 3, 3, 2), (2, 2, 2, 2), (3, 4, 2, 3), (3, 3, 3, 3), (2, 4, 4, 2)]


def _keys(n, seed, h=8):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, 128))
    x[:, rng.choice(128, 4, replace=False)] *= 20
    return fwht_f32(x.astype(np.float32), h)


def test_every_rope_block_lies_in_one_group_of_sixteen():
    """Rotate-half RoPE pairs dims f and f + 64 (f < 64): both must carry the same
    width; each group holds 16 such blocks (32 dims), and with h <= 8 a block of
    the Hadamard rotation stays inside one group too."""
    f = np.arange(64)
    assert np.array_equal(rope_group_of_dim(f), rope_group_of_dim(f + 64))
    g = rope_group_of_dim(np.arange(128))
    assert [int((g == j).sum()) for j in range(4)] == [32, 32, 32, 32]
    for h in (1, 2, 4, 8):
        blocks = g.reshape(-1, h)
        assert np.all(blocks == blocks[:, :1])
    assert not np.all(g.reshape(-1, 16) == g.reshape(-1, 16)[:, :1])    # h = 16 would mix two groups
    # group j holds frequencies 8j .. 8j + 7 and 32 + 8j .. 32 + 8j + 7
    for j in range(4):
        assert sorted(set(f[rope_group_of_dim(f) == j].tolist())) == list(range(8 * j, 8 * j + 8)) + \
            list(range(32 + 8 * j, 40 + 8 * j))


def test_all_widths_four_is_the_four_bit_quantizer():
    y = _keys(3000, 1)
    c, u, z = quantize_grouped(y, (4, 4, 4, 4))
    c4, u4, z4 = quantize(y, INT4_QMAX)
    assert np.array_equal(c, c4) and np.array_equal(u, u4) and np.array_equal(z, z4)


@pytest.mark.parametrize("kb", WIDTHS)
def test_round_trip_within_half_a_group_step(kb):
    """|y - y^| <= m_b U / 2 plus what the fp16 rounding of U and Z moves the
    span [Z, Z + 15 U] off [min, max]."""
    y = _keys(3000, 2)
    c, u, z = quantize_grouped(y, kb)
    b = group_widths_per_dim(kb)
    assert np.all(c <= (1 << b) - 1)
    xh = dequantize_grouped(c, u, z, kb)
    U = f16_bits_to_f64(u)[:, None]
    Z = f16_bits_to_f64(z)[:, None]
    mn = y.min(axis=1, keepdims=True).astype(np.float64)
    mx = y.max(axis=1, keepdims=True).astype(np.float64)
    slack = np.maximum.reduce([np.zeros_like(U), Z - mn, mx - Z - 15 * U])
    bound = (2.0 ** (4 - b)) * U / 2 + slack
    err = np.abs(y.astype(np.float64) - xh)
    assert np.all(err <= bound * (1 + 1e-6) + 1e-7)


@pytest.mark.parametrize("kb", WIDTHS)
def test_codes_are_the_nearest_level_of_their_group(kb):
    """Brute force over every level Z + U (o_b + m_b c), c < 2^b, in fp64."""
    y = _keys(500, 3)
    c, u, z = quantize_grouped(y, kb)
    b = group_widths_per_dim(kb)
    U = f16_bits_to_f64(u)[:, None]
    Z = f16_bits_to_f64(z)[:, None]
    el, vec = grouped_tie_flags(y, kb)
    bad = 0
    for d in range(128):
        m = 2.0 ** (4 - b[d])
        levels = Z + U * ((m - 1) / 2 + m * np.arange(1 << b[d])[None, :])
        dist = np.abs(y[:, d:d + 1].astype(np.float64) - levels)
        best = np.argmin(dist, axis=1)
        tie = el[:, d] | vec
        bad += int(np.sum((best != c[:, d]) & ~tie & (U[:, 0] > 0)))
    assert bad == 0


@pytest.mark.parametrize("kb", WIDTHS)
def test_grid_vectors_round_trip_exactly(kb):
    """Vectors built on each group's own levels (min and max of the vector fixed
    at a 4-bit span of 15 U) come back exactly."""
    rng = np.random.default_rng(4)
    b = group_widths_per_dim(kb)
    m = 2.0 ** (4 - b)
    n = 100
    U = (rng.integers(1, 64, n) * 2.0 ** -6)[:, None]
    Z = (rng.integers(-64, 64, n) * 2.0 ** -4)[:, None]
    c = rng.integers(0, 1 << b, (n, 128))
    y = Z + U * ((m - 1) / 2 + m * c)
    # pin the span: one dim at Z, one at Z + 15 U (widths 4 only reach both)
    y = np.concatenate([y, Z, Z + 15 * U], axis=1)[:, :128]
    wide = np.nonzero(b == 4)[0]
    if len(wide) < 2:
        pytest.skip("the span needs two width-4 dims")
    y[:, wide[0]] = Z[:, 0]
    y[:, wide[1]] = (Z + 15 * U)[:, 0]
    c[:, wide[0]] = 0
    c[:, wide[1]] = 15
    y = y.astype(np.float32)
    assert np.array_equal(y.astype(np.float64), Z + U * ((m - 1) / 2 + m * c))
    cg, ug, zg = quantize_grouped(y, kb)
    assert np.array_equal(cg, c)
    assert np.array_equal(dequantize_grouped(cg, ug, zg, kb), y.astype(np.float64))


def test_constant_keys_take_the_zero_range_guard():
    y = np.stack([np.full(128, 0.3, np.float32), np.zeros(128, np.float32)])
    c, u, z = quantize_grouped(y, (4, 3, 3, 2))
    assert np.all(c == 0) and np.all(f16_bits_to_f64(u) == 0)
    assert np.all(np.isfinite(dequantize_grouped(c, u, z, (4, 3, 3, 2))))


def test_storage_cost_closed_form():
    """32 dims of each group at its width plus an fp16 scale and offset: widths
    (4, 3, 3, 2) with 3-bit values cost the 104 bytes per (token, KV head) of a
    uniform K3V3 cache; (4, 4, 4, 4) with 4-bit values the 136 of the 4-bit one
    (4 + 32 / 128 bits per element, KV4-RL, Methodology in Plain English)."""
    assert grouped_key_bytes_per_token((4, 3, 3, 2)) == 52
    assert grouped_key_bytes_per_token((4, 3, 3, 2)) + (128 * 3 // 8 + 4) == 104
    assert grouped_key_bytes_per_token((4, 4, 4, 4)) + (128 * 4 // 8 + 4) == 136
    assert grouped_key_bytes_per_token((2, 2, 2, 2)) == 36
    for kb in WIDTHS:
        assert grouped_key_bytes_per_token(kb) == 4 * sum(kb) + 4


def test_grouped_cache_attention_equals_brute_force():
    """attend over a cache with grouped keys = a pure-Python softmax over the
    dequantized keys (each dim by its group's levels) with scipy's rotation."""
    import torch
    from scipy.linalg import hadamard

    from workloads import bf16_bits
    from test_oracle_attention import _brute
    L, Hkv, g, d, h = 23, 2, 2, 128, 8
    rng = np.random.default_rng(44)
    bf = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    kb = bf16_bits(bf(rng.standard_normal((L, Hkv, d))))
    vb = bf16_bits(bf(rng.standard_normal((L, Hkv, d))))
    q = bf(rng.standard_normal((Hkv * g, d)))
    oc = quantize_sequence(kb, vb, h, 2, 5, main_bits=3, key_bits=(4, 3, 3, 2))
    out, _ = attend(bf16_bits(q), oc)
    Hm = np.kron(np.eye(d // h), hadamard(h)) / np.sqrt(h)
    qt = q.to(torch.float64).numpy() @ Hm.T
    K, V = dequantized_kv(oc)
    ref = _brute(qt.tolist(), K.tolist(), V.tolist())
    assert np.abs(out - ref).max() < 1e-12
    # the main-cache keys of the INT4 region are the grouped ones
    c, u, z = quantize_grouped(fwht_f32(
        np.asarray(torch.from_numpy(kb.astype(np.int16)).view(torch.bfloat16).float().numpy()), h), (4, 3, 3, 2))
    assert np.array_equal(oc.k4, c)
