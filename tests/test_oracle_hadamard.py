"""Pins for the oracle's block-diagonal Hadamard rotation."""

from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg

from oracle.hadamard import (block_rotation_f64, fwht_f32, inv_sqrt_f32, rotate_f64,
                             sylvester)

HS = [1, 2, 4, 8, 16, 32, 64, 128]


@pytest.mark.parametrize("h", HS)
def test_sylvester_matches_scipy_and_is_orthogonal(h):
    H = sylvester(h)
    assert np.array_equal(H, scipy.linalg.hadamard(h))
    assert np.array_equal(H @ H.T, h * np.eye(h, dtype=np.int64))


def test_sylvester_small_closed_form():
    assert np.array_equal(sylvester(2), [[1, 1], [1, -1]])
    assert np.array_equal(sylvester(4), [[1, 1, 1, 1], [1, -1, 1, -1],
                                         [1, 1, -1, -1], [1, -1, -1, 1]])


@pytest.mark.parametrize("h", HS)
def test_block_rotation_structure(h):
    d = 128
    M = block_rotation_f64(d, h)
    want = scipy.linalg.block_diag(*([scipy.linalg.hadamard(h) / np.sqrt(h)] * (d // h)))
    assert np.allclose(M, want, atol=0, rtol=1e-15)
    assert np.allclose(M @ M.T, np.eye(d), atol=1e-13)


@pytest.mark.parametrize("h", HS)
def test_rotation_preserves_dot_products(h):
    rng = np.random.default_rng(h)
    q = rng.standard_normal((5, 128))
    k = rng.standard_normal((7, 128)) * 20
    lhs = rotate_f64(q, h) @ rotate_f64(k, h).T
    rhs = q @ k.T
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-10)


def test_h1_is_identity():
    x = np.random.default_rng(1).standard_normal((3, 128)).astype(np.float32)
    assert np.array_equal(fwht_f32(x, 1), x)
    assert np.array_equal(rotate_f64(x, 1), x.astype(np.float64))


@pytest.mark.parametrize("h", HS)
def test_inv_sqrt_is_nearest_fp32(h):
    """c_h is the fp32 value nearest to 1/sqrt(h) (exact rational bisection)."""
    lo, hi = Fraction(0), Fraction(2)
    for _ in range(200):
        mid = (lo + hi) / 2
        if mid * mid * h > 1:
            hi = mid
        else:
            lo = mid
    r = (lo + hi) / 2
    c = inv_sqrt_f32(h)
    up = np.nextafter(c, np.float32(1))
    dn = np.nextafter(c, np.float32(0))
    dc = abs(Fraction(float(c)) - r)
    assert dc <= abs(Fraction(float(up)) - r) and dc <= abs(Fraction(float(dn)) - r)


@pytest.mark.parametrize("h", HS)
def test_fwht_exact_on_integer_inputs(h):
    """Small-integer inputs keep every butterfly exact, so the result must be
    exactly fp32(H x) * c_h with H x computed in integers by a matmul."""
    rng = np.random.default_rng(10 + h)
    x = rng.integers(-8, 9, size=(20, 128))
    Hx = x @ block_rotation_f64(128, h).T * np.sqrt(h)   # integer valued
    Hx = np.rint(Hx).astype(np.int64)
    got = fwht_f32(x.astype(np.float32), h)
    want = Hx.astype(np.float32) * inv_sqrt_f32(h)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("h", HS)
def test_fwht_unit_vectors_are_scaled_columns(h):
    d = 128
    E = np.eye(d, dtype=np.float32)
    got = fwht_f32(E, h)
    M = scipy.linalg.block_diag(*([scipy.linalg.hadamard(h)] * (d // h))).astype(np.float32)
    assert np.array_equal(got, M.T * inv_sqrt_f32(h))


@pytest.mark.parametrize("h", [64, 128])
def test_fwht_f32_close_to_f64_definition(h):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((2000, 128)) * np.where(rng.random(128) < 0.03, 20, 1)).astype(np.float32)
    y32 = fwht_f32(x, h).astype(np.float64)
    y64 = rotate_f64(x.astype(np.float64), h)
    bound = 1e-5 * np.maximum(1.0, np.linalg.norm(x.astype(np.float64), axis=1))
    assert np.all(np.abs(y32 - y64).max(axis=1) <= bound)
