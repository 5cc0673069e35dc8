"""Host-side readers of the INT4 / INT8 cache layouts documented in include/kvq.h.

Used to inspect what the GPU wrote (tests, debugging); nothing here runs on the
decode path.
"""

from __future__ import annotations

import numpy as np

SUB = 16
SUB4_BYTES = 2176
SUB2_BYTES = 1152
SUB3_BYTES = 1664
SUB8_BYTES = 4224


def sub4_index(page, kv_head, row, num_kv_heads: int, page_size: int):
    """Index of the INT4 subblock holding (page, kv_head, row) in units of SUB4_BYTES."""
    page = np.asarray(page, dtype=np.int64)
    return (page * num_kv_heads + np.asarray(kv_head, np.int64)) * (page_size // SUB) + np.asarray(row, np.int64) // SUB


def sub8_index(slot, kv_head, entry, num_kv_heads: int, nr8: int):
    slot = np.asarray(slot, dtype=np.int64)
    return (slot * num_kv_heads + np.asarray(kv_head, np.int64)) * nr8 + np.asarray(entry, np.int64) // SUB


def decode_sub4(blocks: np.ndarray, tok) -> dict:
    """Codes and fp16 params of token `tok` (0..15) of each INT4 subblock [N, 2176]."""
    blocks = np.asarray(blocks, dtype=np.uint8).reshape(-1, SUB4_BYTES)
    t = np.asarray(tok, dtype=np.int64).reshape(-1)
    N = blocks.shape[0]
    rows = np.arange(N)[:, None]
    kb = blocks[rows, 64 * t[:, None] + np.arange(64)[None, :]]
    kc = np.empty((N, 128), np.uint8)
    kc[:, 0::2] = kb & 0x0F
    kc[:, 1::2] = kb >> 4
    G, r = t // 4, t % 4
    n = np.arange(16)
    vc = np.empty((N, 128), np.uint8)
    for c in range(4):
        off = 1024 + 4 * ((G[:, None] * 16 + n[None, :]) * 4 + c) + r[:, None]
        byte = blocks[rows, off]
        vc[:, 32 * c + n] = byte & 0x0F
        vc[:, 32 * c + 16 + n] = byte >> 4
    kp = blocks[rows, 2048 + 4 * t[:, None] + np.arange(4)[None, :]].copy().view(np.uint16)
    vp = blocks[rows, 2112 + 4 * t[:, None] + np.arange(4)[None, :]].copy().view(np.uint16)
    return dict(k=kc, v=vc, k_scale=kp[:, 0], k_zero=kp[:, 1], v_scale=vp[:, 0], v_zero=vp[:, 1])


def _nibbles_k(blocks, rows, base, e):
    raw = blocks[rows, base + 64 * e[:, None] + np.arange(64)[None, :]]
    out = np.empty((raw.shape[0], 128), np.uint8)
    out[:, 0::2] = raw & 0x0F
    out[:, 1::2] = raw >> 4
    return out


def _nibbles_v(blocks, rows, base, e):
    G, r = e // 4, e % 4
    n = np.arange(16)
    out = np.empty((e.shape[0], 128), np.uint8)
    for c in range(4):
        byte = blocks[rows, base + 4 * ((G[:, None] * 16 + n[None, :]) * 4 + c) + r[:, None]]
        out[:, 32 * c + n] = byte & 0x0F
        out[:, 32 * c + 16 + n] = byte >> 4
    return out


def decode_sub8(blocks: np.ndarray, ent) -> dict:
    """Codes and fp16 params of entry `ent` (0..15) of each INT8 subblock [N, 4224]
    (codes stored as a low-nibble and a high-nibble plane)."""
    blocks = np.asarray(blocks, dtype=np.uint8).reshape(-1, SUB8_BYTES)
    e = np.asarray(ent, dtype=np.int64).reshape(-1)
    N = blocks.shape[0]
    rows = np.arange(N)[:, None]
    kc = _nibbles_k(blocks, rows, 0, e) | (_nibbles_k(blocks, rows, 1024, e) << 4)
    vc = _nibbles_v(blocks, rows, 2048, e) | (_nibbles_v(blocks, rows, 3072, e) << 4)
    kp = blocks[rows, 4096 + 4 * e[:, None] + np.arange(4)[None, :]].copy().view(np.uint16)
    vp = blocks[rows, 4160 + 4 * e[:, None] + np.arange(4)[None, :]].copy().view(np.uint16)
    return dict(k=kc, v=vc, k_scale=kp[:, 0], k_zero=kp[:, 1], v_scale=vp[:, 0], v_zero=vp[:, 1])


def _int2_codes(blocks, t, kbase, vbase):
    """Key and value codes [N, 128] of token t in the 2-bit layouts at kbase / vbase."""
    rows = np.arange(blocks.shape[0])
    kc = np.empty((blocks.shape[0], 128), np.uint8)
    for d in range(128):
        G, rem = d // 32, d % 32
        w, i = rem // 16, rem % 16
        byte = kbase + (G * 16 + t) * 8 + 4 * w + (0, 2, 1, 3)[i // 4]
        kc[:, d] = (blocks[rows, byte] >> (2 * (i % 4))) & 3
    G, r = t // 4, t % 4
    vc = np.empty((blocks.shape[0], 128), np.uint8)
    for d in range(128):
        n, f, cc = d % 16, (d // 16) % 4, d // 64
        byte = vbase + ((G * 16 + n) * 2 + cc) * 4 + r
        vc[:, d] = (blocks[rows, byte] >> (2 * f)) & 3
    return kc, vc


def _params(blocks, t, kp_off, vp_off):
    rows = np.arange(blocks.shape[0])[:, None]
    kp = blocks[rows, kp_off + 4 * t[:, None] + np.arange(4)[None, :]].copy().view(np.uint16)
    vp = blocks[rows, vp_off + 4 * t[:, None] + np.arange(4)[None, :]].copy().view(np.uint16)
    return dict(k_scale=kp[:, 0], k_zero=kp[:, 1], v_scale=vp[:, 0], v_zero=vp[:, 1])


def decode_sub2(blocks: np.ndarray, tok) -> dict:
    """Codes and fp16 params of token `tok` (0..15) of each 2-bit subblock [N, 1152]."""
    blocks = np.asarray(blocks, dtype=np.uint8).reshape(-1, SUB2_BYTES)
    t = np.asarray(tok, dtype=np.int64).reshape(-1)
    kc, vc = _int2_codes(blocks, t, 0, 512)
    return dict(k=kc, v=vc, **_params(blocks, t, 1024, 1088))


def decode_sub3(blocks: np.ndarray, tok) -> dict:
    """Codes and fp16 params of token `tok` (0..15) of each 3-bit subblock [N, 1664]:
    low two bits in the 2-bit layouts at 0 / 512, high bits in the key plane at
    1024 (dword G 16 + t; dim in 2-bit dword w, byte b, field f at bit
    16 (b / 2) + 4 f + (2 if w == 0 else 0) + b % 2) and the value plane at 1280
    (dword G 16 + n, byte t % 4; dim n + 16 f + 64 cc at bit {2, 6, 3, 7}[f] or
    {0, 4, 1, 5}[f] for cc = 0 / 1), params at 1536 / 1600."""
    blocks = np.asarray(blocks, dtype=np.uint8).reshape(-1, SUB3_BYTES)
    t = np.asarray(tok, dtype=np.int64).reshape(-1)
    rows = np.arange(blocks.shape[0])
    kc, vc = _int2_codes(blocks, t, 0, 512)
    for d in range(128):
        G, rem = d // 32, d % 32
        w, i = rem // 16, rem % 16
        b, f = (0, 2, 1, 3)[i // 4], i % 4
        bit = 16 * (b // 2) + 4 * f + (2 if w == 0 else 0) + b % 2
        off = 1024 + 4 * (G * 16 + t) + bit // 8
        kc[:, d] |= ((blocks[rows, off] >> (bit % 8)) & 1) << 2
    G, r = t // 4, t % 4
    for d in range(128):
        n, f, cc = d % 16, (d // 16) % 4, d // 64
        bit = ((2, 6, 3, 7) if cc == 0 else (0, 4, 1, 5))[f]
        off = 1280 + 4 * (G * 16 + n) + r
        vc[:, d] |= ((blocks[rows, off] >> bit) & 1) << 2
    return dict(k=kc, v=vc, **_params(blocks, t, 1536, 1600))


# --- keys with a width per RoPE-block group ----------------------------------


def subg_bytes(key_bits, vbits: int) -> int:
    """Bytes of a grouped-key subblock: key areas, value area, params."""
    return 64 * int(sum(key_bits)) + {2: 512, 3: 768}.get(vbits, 1024) + 128


def decode_subg(blocks: np.ndarray, tok, key_bits, vbits: int) -> dict:
    """Codes and fp16 params of token `tok` (0..15) of each grouped-key subblock:
    group j's key area at 64 (key_bits[0] + .. + key_bits[j-1]), slot 16 G + t
    holding dims 32 G + 8 j + e (width 4: a nibble dword; width 2: two bytes,
    dim 4 k + f at bits 2 f of byte k; width 3: those low bits, then a byte at
    +128 with bit 2 of dim e at bit e), then the value area in the value
    width's layout and the key / value params."""
    nb = subg_bytes(key_bits, vbits)
    blocks = np.asarray(blocks, dtype=np.uint8).reshape(-1, nb)
    t = np.asarray(tok, dtype=np.int64).reshape(-1)
    rows = np.arange(blocks.shape[0])
    N = blocks.shape[0]
    kc = np.zeros((N, 128), np.uint8)
    off = 0
    for j, b in enumerate(key_bits):
        for G in range(4):
            s_ = 16 * G + t
            for e in range(8):
                d = 32 * G + 8 * j + e
                if b == 4:
                    byte = blocks[rows, off + 4 * s_ + e // 2]
                    kc[:, d] = (byte >> (4 * (e % 2))) & 0xF
                else:
                    byte = blocks[rows, off + 2 * s_ + e // 4]
                    c = (byte >> (2 * (e % 4))) & 3
                    if b == 3:
                        c = c | (((blocks[rows, off + 128 + s_] >> e) & 1) << 2)
                    kc[:, d] = c
        off += 64 * b
    ka = off
    va_bytes = {2: 512, 3: 768}.get(vbits, 1024)
    if vbits == 4:
        vc = _nibbles_v(blocks, rows[:, None], ka, t)
    else:
        _, vc = _int2_codes(blocks, t, 0, ka)
        if vbits == 3:
            G, r = t // 4, t % 4
            for d in range(128):
                n, f, cc = d % 16, (d // 16) % 4, d // 64
                bit = ((2, 6, 3, 7) if cc == 0 else (0, 4, 1, 5))[f]
                o = ka + 512 + 4 * (G * 16 + n) + r
                vc[:, d] |= ((blocks[rows, o] >> bit) & 1) << 2
    return dict(k=kc, v=vc, **_params(blocks, t, ka + va_bytes, ka + va_bytes + 64))
