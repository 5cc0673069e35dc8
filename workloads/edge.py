"""Crafted key / value rows for the quantizer's edge cases (inputs only).

Each position of a row takes one kind of vector, cycling through the kinds, so
that a short row reaches every kind in both the INT4 region and the INT8
window.  The kinds are the cases a per-token min / max quantizer treats
specially:

* ``const``:     every element the same value (positive, negative, +0, -0);
* ``underflow``: all elements equal but one, which is one bf16 ulp above the
                 rest at 2^-20, so the range (2^-27) over qmax rounds to an
                 fp16 zero;
* ``subnormal``: a range of 2^-17 around 2^-10: the fp16 scale is subnormal;
* ``grid``:      values -1 + c / 8 with integer c in [0, qmax], c = 0 and
                 c = qmax both present (so min = -1, max = -1 + qmax / 8);
* ``tie``:       the same frame, the other elements half-way between two
                 consecutive levels: -1 + (c + 1/2) / 8;
* ``large``:     N(0, 1) * 8000 clipped to [-60000, 60000] and rounded to
                 bf16 (inside the fp16 range that the stored scale and offset
                 need);
* ``gauss``:     N(0, 1);
* ``big``:       N(0, 1) * 16 (keys only: keys of the ``large`` kind would put
                 the scores, and so the log-sum-exp, near 1e4, where an fp32
                 ulp alone exceeds the attention tolerance).

Keys go through a block-diagonal Hadamard rotation before they are quantized,
so a key row only keeps its kind when the rotation preserves it.  With block
size h > 1 the key kinds are built in the rotated domain where that is exact:
``const`` and ``underflow`` keys put their value at the first element of every
h-block (and zeros elsewhere), which the rotation spreads into a constant (or,
for ``underflow``, a constant plus a rotated 2^-27 step that still underflows);
the grid, tie and large kinds are left to the unrotated values and to h = 1.
"""

from __future__ import annotations

import numpy as np
import torch

VALUE_KINDS = ("const+", "const-", "zero", "negzero", "underflow", "subnormal", "grid", "tie", "large", "gauss")
KEY_KINDS = ("const+", "const-", "zero", "negzero", "underflow", "subnormal", "grid", "tie", "big", "gauss")
ROTATED_KEY_KINDS = ("const+", "const-", "zero", "negzero", "underflow", "gauss")


def _bf16_from_f32(x: np.ndarray) -> torch.Tensor:
    """bf16 tensor of fp32 values that are exactly representable in bf16."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    b = t.to(torch.bfloat16)
    assert torch.equal(b.to(torch.float32), t), "crafted value not exact in bf16"
    return b


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16 (ties to even)."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _vector(kind: str, rng: np.random.Generator, qmax: int, d: int = 128) -> np.ndarray:
    if kind == "const+":
        return np.full(d, 0.3125, np.float32)
    if kind == "const-":
        return np.full(d, -7.25, np.float32)
    if kind == "zero":
        return np.zeros(d, np.float32)
    if kind == "negzero":
        return np.full(d, -0.0, np.float32)
    if kind == "underflow":
        x = np.full(d, 2.0 ** -20, np.float32)
        x[rng.integers(d)] = np.float32(2.0 ** -20 + 2.0 ** -27)
        return x
    if kind == "subnormal":
        x = np.full(d, 2.0 ** -10, np.float32)
        x[rng.integers(d, size=d // 2)] = np.float32(2.0 ** -10 + 2.0 ** -17)
        return x
    if kind in ("grid", "tie"):
        if kind == "grid":
            c = rng.integers(0, qmax + 1, d).astype(np.float64)
        else:
            c = rng.integers(0, qmax, d) + 0.5
        perm = rng.permutation(d)
        c[perm[0]] = 0
        c[perm[1]] = qmax
        return (-1.0 + c / 8.0).astype(np.float32)
    if kind == "large":
        return _round_bf16(np.clip(rng.standard_normal(d) * 8000.0, -60000, 60000))
    if kind == "gauss":
        return _round_bf16(rng.standard_normal(d))
    if kind == "big":
        return _round_bf16(rng.standard_normal(d) * 16.0)
    raise ValueError(kind)


def _rotated_key(kind: str, rng: np.random.Generator, h: int, d: int = 128) -> np.ndarray:
    """A key whose block rotation keeps its kind (see the module docstring)."""
    if kind == "gauss":
        return _round_bf16(rng.standard_normal(d))
    x = np.zeros(d, np.float32)
    base = {"const+": 0.3125, "const-": -7.25, "zero": 0.0, "negzero": -0.0, "underflow": 2.0 ** -20}[kind]
    x[::h] = np.float32(base)
    if kind == "underflow":
        x[1] = np.float32(2.0 ** -27)
    return x


def edge_kv(L: int, H: int, h: int, qmax: int, seed: int, offset: int = 0):
    """Keys and values [L, H, 128] bf16 for one row, kinds cycling by position.

    Key and value kinds cycle with different strides (and per KV head), so that
    every pair of kinds meets.  `qmax` is the main cache's largest code; the
    grid and tie kinds are built on its grid.
    """
    rng = np.random.default_rng(seed)
    d = 128
    k = np.empty((L, H, d), np.float32)
    v = np.empty((L, H, d), np.float32)
    kinds_k = KEY_KINDS if h == 1 else ROTATED_KEY_KINDS
    for p in range(L):
        for hk in range(H):
            kk = kinds_k[(p + offset + 3 * hk) % len(kinds_k)]
            vk = VALUE_KINDS[(3 * p + offset + 1 + hk) % len(VALUE_KINDS)]
            k[p, hk] = _vector(kk, rng, qmax) if h == 1 else _rotated_key(kk, rng, h)
            v[p, hk] = _vector(vk, rng, qmax)
    return _bf16_from_f32(k), _bf16_from_f32(v)
