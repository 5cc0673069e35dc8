"""Per-token asymmetric quantization of one 128-dim token-head vector.

KV4-RL ("Methodology in Plain English"): every new K/V vector is quantized on
the fly into one affine group per 128-dimensional token-head vector with an
FP16 scale and an FP16 offset; the INT8 side cache uses the same scheme with
256 levels (reading: the pages do not describe the INT8 format beyond its
width).  SAW-INT4 (section 2) calls this token-wise INT4 quantization.

Steps, all in fp32 because they decide integer codes (the pages fix only the
FP16 storage of scale and offset):

1. mn = min_i y_i, mx = max_i y_i (exact);
2. scale_f = fp32(fp32(mx - mn) / qmax)   (IEEE division; qmax = 15 or 255);
3. scale_h = fp16(scale_f), zero_h = fp16(mn)   (round to nearest even);
4. if scale_h == 0 every code is 0 (constant or nearly constant vector);
   otherwise t_i = fp32(fp32(y_i - zero_h) / scale_h) and
   c_i = clamp(rint(t_i), 0, qmax) with ties to even;
5. dequantized value = scale_h * c_i + zero_h, evaluated in fp64.

The codes are taken against the stored fp16 scale and offset, so that the
dequantized value is the one attention actually sees.
"""

from __future__ import annotations

import numpy as np

from .numerics import f32_to_f16_bits, f16_bits_to_f32, f16_bits_to_f64

INT4_QMAX = 15
INT8_QMAX = 255
# Sub-4-bit main caches (KV4-RL, "Future Directions": 3- or 2-bit caches under the
# same sink / recent protection): the same affine scheme with 2^bits levels.
INT2_QMAX = 3
INT3_QMAX = 7


def qmax_of(bits: int) -> int:
    """Largest code of a `bits`-bit affine code."""
    if bits not in (2, 3, 4, 8):
        raise ValueError(f"unsupported code width {bits}")
    return (1 << bits) - 1


def quantize(y, qmax: int):
    """Quantize fp32 vectors y[..., n] along the last axis.

    Returns (codes uint8 [..., n], scale_bits uint16 [...], zero_bits uint16 [...]).
    """
    y = np.asarray(y, dtype=np.float32)
    mn = y.min(axis=-1)
    mx = y.max(axis=-1)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        scale_f = (mx - mn) / np.float32(qmax)
    scale_bits = f32_to_f16_bits(scale_f)
    zero_bits = f32_to_f16_bits(mn)
    sf = f16_bits_to_f32(scale_bits)
    zf = f16_bits_to_f32(zero_bits)
    guard = sf == 0
    safe_sf = np.where(guard, np.float32(1.0), sf).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        t = (y - zf[..., None]) / safe_sf[..., None]
    c = np.clip(np.rint(t), 0, qmax)
    c = np.where(guard[..., None], 0, c)
    return c.astype(np.uint8), scale_bits, zero_bits


def dequantize(codes, scale_bits, zero_bits) -> np.ndarray:
    """scale_h * c + zero_h in fp64."""
    s = f16_bits_to_f64(scale_bits)[..., None]
    z = f16_bits_to_f64(zero_bits)[..., None]
    return s * np.asarray(codes, dtype=np.float64) + z


def tie_flags(y, qmax: int, rel: float = 1e-6):
    """Where a rounding decision of the quantizer sits within `rel` (relative) of a tie.

    Returns (el_flag [..., n], vec_flag [...]):

    * el_flag: the element's quotient t_i lies within rel of a half-integer, so
      its code (rint of t_i) may round either way under another evaluation
      order of the same arithmetic;
    * vec_flag: the vector's fp32 scale_f or its min lies within rel of the
      midpoint between two fp16 neighbours, so its stored fp16 scale or offset
      (and then every code of the vector) may round either way.

    A code mismatch can come from either flag, a scale / offset mismatch only
    from the vector flag.  With the zero-range guard (fp16 scale 0) no code is
    decided by a quotient, so el_flag is False there.
    """
    y = np.asarray(y, dtype=np.float32)
    mn = y.min(axis=-1)
    mx = y.max(axis=-1)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        scale_f = (mx - mn) / np.float32(qmax)
    vec_flag = _near_f16_midpoint(scale_f, rel) | _near_f16_midpoint(mn, rel)
    sb = f32_to_f16_bits(scale_f)
    zb = f32_to_f16_bits(mn)
    sf = f16_bits_to_f32(sb)
    zf = f16_bits_to_f32(zb)
    safe = np.where(sf == 0, np.float32(1.0), sf).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore"):
        t = ((y - zf[..., None]) / safe[..., None]).astype(np.float64)
    frac = t - np.floor(t)
    el_flag = np.abs(frac - 0.5) <= rel * np.maximum(np.abs(t), 1.0)
    el_flag &= (sf != 0)[..., None]
    return el_flag, vec_flag


def tie_near(y, qmax: int, rel: float = 1e-6):
    """Per-element flags of codes that may round either way: the element's own
    tie flag or its vector's (see tie_flags)."""
    el, vec = tie_flags(y, qmax, rel)
    return el | vec[..., None]


def _near_f16_midpoint(x, rel):
    """True where fp32 x lies within rel of the midpoint between two fp16 neighbours."""
    x = np.asarray(x, dtype=np.float64)
    h = np.asarray(x, dtype=np.float32).astype(np.float16).astype(np.float64)
    # the two fp16 neighbours around x
    up = np.nextafter(h.astype(np.float16), np.float16(np.inf)).astype(np.float64)
    dn = np.nextafter(h.astype(np.float16), np.float16(-np.inf)).astype(np.float64)
    other = np.where(x >= h, up, dn)
    mid = 0.5 * (h + other)
    with np.errstate(invalid="ignore"):
        return np.abs(x - mid) <= rel * np.maximum(np.abs(x), 1e-30)


def pack_int4(codes) -> np.ndarray:
    """Two codes per byte, low nibble = even index (canonical byte form of a vector)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0x0F
    out[..., 1::2] = p >> 4
    return out


def pack_int2(codes) -> np.ndarray:
    """Four codes per byte, element 4j + f in bits 2f .. 2f + 1 (canonical byte form)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::4] | (c[..., 1::4] << 2) | (c[..., 2::4] << 4) | (c[..., 3::4] << 6)).astype(np.uint8)


def unpack_int2(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (4 * p.shape[-1],), dtype=np.uint8)
    for f in range(4):
        out[..., f::4] = (p >> (2 * f)) & 0x3
    return out


def pack_int3(codes) -> np.ndarray:
    """Canonical byte form of 3-bit codes, as two bit planes: the low two bits of
    every code packed like pack_int2, then the high bits eight to a byte
    (element 8j + i in bit i of byte j).  A vector of n codes takes n / 4 + n / 8
    bytes."""
    c = np.asarray(codes, dtype=np.uint8)
    lo = pack_int2(c & 0x3)
    hi = np.zeros(c.shape[:-1] + (c.shape[-1] // 8,), dtype=np.uint8)
    for i in range(8):
        hi |= ((c[..., i::8] >> 2) & 0x1) << i
    return np.concatenate([lo, hi], axis=-1).astype(np.uint8)


def unpack_int3(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    n = p.shape[-1] * 8 // 3
    lo = unpack_int2(p[..., : n // 4])
    hi = p[..., n // 4:]
    out = lo.copy()
    for i in range(8):
        out[..., i::8] |= ((hi >> i) & 0x1) << 2
    return out


def bytes_per_token_head(head_dim: int, bits: int) -> int:
    """K+V bytes of one (token, KV head): codes plus an fp16 scale and offset each."""
    return 2 * (head_dim * bits // 8 + 4)


# --- keys with a bit width per RoPE-block group ----------------------------------
#
# RoPE-Aware Bit Allocation for KV-Cache Quantization (Block-GTQ), Abstract: a
# key's logit contribution splits over two-dimensional RoPE frequency blocks,
# so integer bit widths are allocated per block.  Reading (packing only; the
# allocation itself is an input): the 64 rotate-half RoPE blocks (f, f + 64)
# form four groups of 16, group j holding frequencies 8 j .. 8 j + 7 and
# 32 + 8 j .. 32 + 8 j + 7, i.e. the dims d with (d mod 32) // 8 == j; each
# group has a width b_j in {2, 3, 4}.  One per-token affine pair is kept, as
# in the 4-bit cache: U = fp16(fp32(mx - mn) / 15), Z = fp16(mn).  A group of
# width b uses the step 2^(4 - b) U and the offset ((2^(4 - b) - 1) / 2) U, so
# its 2^b levels sit centred in the 4-bit span [Z, Z + 15 U]; with every width
# 4 this is the 4-bit quantizer exactly.
ROPE_GROUPS = 4


def rope_group_of_dim(d):
    """Group (0-3) of rotated key dim d (numpy array or int)."""
    return (np.asarray(d) % 32) // 8


def group_widths_per_dim(key_bits, n=128):
    """Width of each of the n dims for the four group widths key_bits."""
    kb = np.asarray(key_bits, dtype=np.int64)
    if kb.shape != (ROPE_GROUPS,) or not np.all((kb >= 2) & (kb <= 4)):
        raise ValueError(f"key_bits must be four widths in {{2, 3, 4}}, got {key_bits}")
    return kb[rope_group_of_dim(np.arange(n))]


def quantize_grouped(y, key_bits):
    """Quantize fp32 keys y[..., 128] with the group widths key_bits.

    Returns (codes uint8 [..., 128], scale_bits uint16 [...] (U), zero_bits
    uint16 [...] (Z)).  Decisions in fp32: Z_b = fp32(Z + fp32(o_b U)),
    t = fp32(fp32(y - Z_b) / fp32(m_b U)), c = clamp(rint(t), 0, 2^b - 1) with
    m_b = 2^(4 - b), o_b = (m_b - 1) / 2; every code is 0 when U is 0.
    """
    y = np.asarray(y, dtype=np.float32)
    b = group_widths_per_dim(key_bits, y.shape[-1])
    mn = y.min(axis=-1)
    mx = y.max(axis=-1)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        scale_f = (mx - mn) / np.float32(15)
    ub = f32_to_f16_bits(scale_f)
    zb = f32_to_f16_bits(mn)
    U = f16_bits_to_f32(ub)[..., None]
    Z = f16_bits_to_f32(zb)[..., None]
    m = (2.0 ** (4 - b)).astype(np.float32)
    o = ((m - 1) / 2).astype(np.float32)
    step = (m * U).astype(np.float32)                    # exact: U times a power of two
    zb_ = (Z + (o * U).astype(np.float32)).astype(np.float32)
    guard = U == 0
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        t = ((y - zb_).astype(np.float32) / np.where(guard, np.float32(1), step)).astype(np.float32)
    c = np.clip(np.rint(t), 0, (1 << b) - 1)
    c = np.where(guard, 0, c)
    return c.astype(np.uint8), ub, zb


def dequantize_grouped(codes, scale_bits, zero_bits, key_bits) -> np.ndarray:
    """Z + U (o_b + m_b c) in fp64."""
    c = np.asarray(codes, dtype=np.float64)
    b = group_widths_per_dim(key_bits, c.shape[-1])
    m = 2.0 ** (4 - b)
    U = f16_bits_to_f64(scale_bits)[..., None]
    Z = f16_bits_to_f64(zero_bits)[..., None]
    return Z + U * ((m - 1) / 2 + m * c)


def grouped_tie_flags(y, key_bits, rel: float = 1e-6):
    """tie_flags for the grouped quantizer: an element whose quotient t lies within
    rel of a half-integer, and vectors whose fp32 range / 15 or min lies within
    rel of an fp16 midpoint."""
    y = np.asarray(y, dtype=np.float32)
    b = group_widths_per_dim(key_bits, y.shape[-1])
    mn = y.min(axis=-1)
    mx = y.max(axis=-1)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        scale_f = (mx - mn) / np.float32(15)
    vec = _near_f16_midpoint(scale_f, rel) | _near_f16_midpoint(mn, rel)
    U = f16_bits_to_f32(f32_to_f16_bits(scale_f))[..., None]
    Z = f16_bits_to_f32(f32_to_f16_bits(mn))[..., None]
    m = (2.0 ** (4 - b)).astype(np.float32)
    o = ((m - 1) / 2).astype(np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        t = ((y - (Z + (o * U).astype(np.float32)).astype(np.float32)) /
             np.where(U == 0, np.float32(1), (m * U).astype(np.float32))).astype(np.float64)
    el = (np.abs(t - np.floor(t) - 0.5) <= rel * np.maximum(np.abs(t), 1.0)) & (U != 0)
    return el, vec


def grouped_key_bytes_per_token(key_bits, head_dim: int = 128) -> int:
    """Key bytes of one (token, KV head) with group widths key_bits: 32 dims of
    each group at its width, plus the fp16 scale and offset."""
    b = group_widths_per_dim(key_bits, head_dim)
    return int(b.sum()) // 8 + 4
