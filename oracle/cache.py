"""The oracle's own quantized cache of one sequence.

Built directly from the raw bf16 keys and values: every position gets INT4 codes
(keys rotated, values not), and the positions of the INT8 region get INT8
codes of the same rotated keys / raw values (KV4-RL, "Methodology in Plain
English"; SAW-INT4, section 2).  Nothing here depends on how a GPU lays the
cache out in memory.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .hadamard import fwht_f32
from .numerics import bf16_to_f32
from .quant import quantize, dequantize, qmax_of, INT8_QMAX, quantize_grouped, dequantize_grouped
from .regions import int8_region, ring_entry


@dataclass
class SeqCache:
    L: int
    s: int
    w: int
    h: int
    # INT4, every position: codes [L, H, d] uint8, scale/zero fp16 bits [L, H]
    k4: np.ndarray
    k4_scale: np.ndarray
    k4_zero: np.ndarray
    v4: np.ndarray
    v4_scale: np.ndarray
    v4_zero: np.ndarray
    # INT8, region positions only: positions [n8], codes [n8, H, d], bits [n8, H]
    pos8: np.ndarray
    k8: np.ndarray
    k8_scale: np.ndarray
    k8_zero: np.ndarray
    v8: np.ndarray
    v8_scale: np.ndarray
    v8_zero: np.ndarray
    # main-cache keys with a width per RoPE-block group (None: every key code
    # has the main width)
    key_bits: tuple = None

    def ring(self) -> np.ndarray:
        """Side-cache entry of each INT8 position."""
        return np.array([ring_entry(int(p), self.s, self.w) for p in self.pos8], dtype=np.int64)


def rotated_keys_f32(k_bits, h: int) -> np.ndarray:
    """fp32 rotated keys (the quantizer's input) from bf16 key patterns [..., d]."""
    return fwht_f32(bf16_to_f32(k_bits), h)


def quantize_sequence(k_bits, v_bits, h: int, s: int, w: int, main_bits: int = 4, key_bits=None) -> SeqCache:
    """Quantize a whole sequence's keys/values [L, H, d] (bf16 patterns).

    main_bits is the width of the main cache's codes: 4, or 3 or 2 for the
    sub-4-bit caches under the same INT8 sink / recent protection (KV4-RL,
    "Future Directions"); the fields k4 / v4 then hold the 3- or 2-bit codes.
    key_bits (four widths) gives the main-cache keys a width per RoPE-block
    group instead (quant.quantize_grouped, Block-GTQ Abstract); the values keep
    main_bits.  The INT8 copies do not change.
    """
    k_bits = np.asarray(k_bits, dtype=np.uint16)
    v_bits = np.asarray(v_bits, dtype=np.uint16)
    L = k_bits.shape[0]
    yk = rotated_keys_f32(k_bits, h)
    yv = bf16_to_f32(v_bits)
    qm = qmax_of(main_bits)
    if key_bits is not None:
        k4, k4s, k4z = quantize_grouped(yk, key_bits)
    else:
        k4, k4s, k4z = quantize(yk, qm)
    v4, v4s, v4z = quantize(yv, qm)
    pos8 = np.array(int8_region(L, s, w), dtype=np.int64)
    k8, k8s, k8z = quantize(yk[pos8], INT8_QMAX)
    v8, v8s, v8z = quantize(yv[pos8], INT8_QMAX)
    return SeqCache(L, s, w, h, k4, k4s, k4z, v4, v4s, v4z, pos8, k8, k8s, k8z, v8, v8s, v8z,
                    tuple(int(x) for x in key_bits) if key_bits is not None else None)


def dequantized_kv(c: SeqCache):
    """fp64 keys (rotated basis) and values the attention sees, [L, H, d] each.

    Positions of the INT8 region take the INT8 values, all others the INT4 ones.
    """
    if c.key_bits is not None:
        K = dequantize_grouped(c.k4, c.k4_scale, c.k4_zero, c.key_bits)
    else:
        K = dequantize(c.k4, c.k4_scale, c.k4_zero)
    V = dequantize(c.v4, c.v4_scale, c.v4_zero)
    if len(c.pos8):
        K[c.pos8] = dequantize(c.k8, c.k8_scale, c.k8_zero)
        V[c.pos8] = dequantize(c.v8, c.v8_scale, c.v8_zero)
    return K, V
