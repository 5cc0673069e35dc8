"""Decode attention over the quantized cache, in fp64.

KV4-RL ("Methodology in Plain English"): attention reads the quantized cache
with the rotated query; the INT4 and INT8 regions are attended as disjoint
sets and merged with regional softmax statistics.  Because the merge is exact
in real arithmetic, the oracle's primary definition is plain single-pass
softmax attention over every position (``attend``), and the regional form
(``attend_regions`` + ``merge``) is checked against it.

Readings: softmax scale 1/sqrt(head_dim), no soft-cap, every position < L is
visible; query head j uses KV head j // g (contiguous GQA groups); the output
is the fp64 value, compared to the GPU's fp32 output; lse is the natural-log
sum of exp over the scaled scores.
"""

from __future__ import annotations

import numpy as np

from .cache import SeqCache, dequantized_kv, quantize_sequence
from .hadamard import rotate_f64
from .numerics import bf16_to_f32
from .regions import int4_region


def softmax_attention(q, K, V):
    """Single-head-group attention. q [Hq, d], K/V [L, Hkv, d] (fp64).

    Returns (out [Hq, d], lse [Hq]); an empty context gives out = 0, lse = -inf.
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape
    L, Hkv, _ = K.shape
    g = Hq // Hkv
    out = np.zeros((Hq, d), dtype=np.float64)
    lse = np.full(Hq, -np.inf, dtype=np.float64)
    if L == 0:
        return out, lse
    for j in range(Hq):
        kv = j // g
        z = K[:, kv, :] @ q[j] / np.sqrt(d)
        m = z.max()
        e = np.exp(z - m)
        l = e.sum()
        out[j] = (e @ V[:, kv, :]) / l
        lse[j] = m + np.log(l)
    return out, lse


def region_stats(q, K, V, positions):
    """Softmax statistics of one region: (m [Hq], l [Hq], o [Hq, d]) with o normalised.

    An empty region gives (-inf, 0, 0).
    """
    q = np.asarray(q, dtype=np.float64)
    Hq, d = q.shape
    Hkv = K.shape[1]
    g = Hq // Hkv
    idx = np.asarray(list(positions), dtype=np.int64)
    m = np.full(Hq, -np.inf)
    l = np.zeros(Hq)
    o = np.zeros((Hq, d))
    if idx.size == 0:
        return m, l, o
    for j in range(Hq):
        kv = j // g
        z = K[idx, kv, :] @ q[j] / np.sqrt(d)
        m[j] = z.max()
        e = np.exp(z - m[j])
        l[j] = e.sum()
        o[j] = (e @ V[idx, kv, :]) / l[j]
    return m, l, o


def merge(stats):
    """Log-sum-exp combine of regional (m, l, o) triples -> (out, lse)."""
    ms = np.stack([s[0] for s in stats])          # [R, Hq]
    M = ms.max(axis=0)
    Hq = M.shape[0]
    d = stats[0][2].shape[1]
    out = np.zeros((Hq, d))
    lse = np.full(Hq, -np.inf)
    for j in range(Hq):
        if not np.isfinite(M[j]):
            continue
        wts = [s[1][j] * np.exp(s[0][j] - M[j]) if np.isfinite(s[0][j]) else 0.0 for s in stats]
        tot = sum(wts)
        out[j] = sum(wt * s[2][j] for wt, s in zip(wts, stats)) / tot
        lse[j] = M[j] + np.log(tot)
    return out, lse


def rotated_query(q_bits, h: int) -> np.ndarray:
    """fp64 rotated query from bf16 patterns [Hq, d]."""
    return rotate_f64(bf16_to_f32(q_bits).astype(np.float64), h)


def attend(q_bits, cache: SeqCache):
    """Decode attention of one sequence: rotated query against the dequantized cache."""
    qr = rotated_query(q_bits, cache.h)
    K, V = dequantized_kv(cache)
    return softmax_attention(qr, K, V)


def attend_regions(q_bits, cache: SeqCache):
    """Same result through the two disjoint regions and the regional merge."""
    qr = rotated_query(q_bits, cache.h)
    K, V = dequantized_kv(cache)
    s8 = region_stats(qr, K, V, cache.pos8)
    s4 = region_stats(qr, K, V, int4_region(cache.L, cache.s, cache.w))
    return merge([s4, s8])


def prefill_attend(q_rows_bits, cache: SeqCache):
    """Causal attention of the last T positions of a sequence over its quantized cache.

    KV4-RL, "Future Directions": rollouts are re-prefilled after each policy
    update; "Methodology in Plain English": attention reads the quantized
    cache with the rotated query.  Reading: query row t of q_rows_bits [T, Hq, d]
    sits at position p = L - T + t and attends positions [0, p], each key and
    value taken as the cache holds it at length L (the INT8 copy for the
    positions of the INT8 region at length L, the INT4 codes elsewhere).  The
    last row is decode attention at length L.

    Returns (out [T, Hq, d], lse [T, Hq]).
    """
    q_rows_bits = np.asarray(q_rows_bits, dtype=np.uint16)
    T = q_rows_bits.shape[0]
    if not 1 <= T <= cache.L:
        raise ValueError(f"T = {T} rows do not fit a context of {cache.L}")
    K, V = dequantized_kv(cache)
    Hq, d = q_rows_bits.shape[1], q_rows_bits.shape[2]
    out = np.zeros((T, Hq, d))
    lse = np.zeros((T, Hq))
    for t in range(T):
        p = cache.L - T + t
        out[t], lse[t] = softmax_attention(rotated_query(q_rows_bits[t], cache.h), K[:p + 1], V[:p + 1])
    return out, lse


def decode_reference(q_bits, k_bits, v_bits, h: int, s: int, w: int):
    """Quantize a sequence from raw bf16 K/V and attend with one query row."""
    return attend(q_bits, quantize_sequence(k_bits, v_bits, h, s, w))


def unquantized_attention(q_bits, k_bits, v_bits):
    """softmax(q.k / sqrt(d)) v in fp64 from the raw bf16 tensors (no rotation, no quantization)."""
    q = bf16_to_f32(q_bits).astype(np.float64)
    K = bf16_to_f32(k_bits).astype(np.float64)
    V = bf16_to_f32(v_bits).astype(np.float64)
    return softmax_attention(q, K, V)
