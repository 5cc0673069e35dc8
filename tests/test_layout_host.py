"""Host check of the subblock readers in decode_attention_int4_block_amd/layout.py
against the byte layouts documented in include/kvq.h.

Each encoder below places codes and params by the header's formulas, one byte at
a time; the reader used by the GPU parity tests must give the codes back.  This
pins the readers to the documented layouts (the GPU tests then pin the kernels
to the readers).  No GPU needed.
"""

import numpy as np
import pytest

from decode_attention_int4_block_amd.layout import decode_sub2, decode_sub3, decode_sub4


def _params(blk, t, kp_off, vp_off, ks, kz, vs, vz):
    blk[kp_off + 4 * t: kp_off + 4 * t + 4] = np.array([ks, kz], np.uint16).view(np.uint8)
    blk[vp_off + 4 * t: vp_off + 4 * t + 4] = np.array([vs, vz], np.uint16).view(np.uint8)


def _encode_low2(blk, t, k, v, kbase, vbase):
    """The 2-bit key and value layouts (low two bits of the given codes)."""
    for G in range(4):
        for w in range(2):
            for i in range(16):
                d = 32 * G + 16 * w + i
                byte = kbase + (G * 16 + t) * 8 + 4 * w + (0, 2, 1, 3)[i // 4]
                blk[byte] |= (int(k[d]) & 3) << (2 * (i % 4))
    _encode_low2_values(blk, t, v, vbase)


def _encode_low2_values(blk, t, v, vbase):
    """The 2-bit value layout (low two bits of the given codes)."""
    G, r = t // 4, t % 4
    for n in range(16):
        for cc in range(2):
            for f in range(4):
                d = n + 16 * f + 64 * cc
                blk[vbase + ((G * 16 + n) * 2 + cc) * 4 + r] |= (int(v[d]) & 3) << (2 * f)


def _encode_sub4(blk, t, k, v):
    for j in range(64):                          # key byte 64 t + j: dims 2 j, 2 j + 1
        blk[64 * t + j] = int(k[2 * j]) | (int(k[2 * j + 1]) << 4)
    G, r = t // 4, t % 4
    for n in range(16):
        for c in range(4):                       # value dword (G 16 + n) 4 + c, byte r
            blk[1024 + 4 * ((G * 16 + n) * 4 + c) + r] = int(v[32 * c + n]) | (int(v[32 * c + 16 + n]) << 4)


def _encode_sub3(blk, t, k, v):
    _encode_low2(blk, t, k, v, 0, 512)
    for G in range(4):
        hh = 0
        for w in range(2):
            for i in range(16):
                d = 32 * G + 16 * w + i
                b, f = (0, 2, 1, 3)[i // 4], i % 4
                bit = 16 * (b // 2) + 4 * f + (2 if w == 0 else 0) + b % 2
                hh |= ((int(k[d]) >> 2) & 1) << bit
        blk[1024 + 4 * (G * 16 + t): 1024 + 4 * (G * 16 + t) + 4] = np.array([hh], np.uint32).view(np.uint8)
    G, r = t // 4, t % 4
    for n in range(16):
        byte = 0
        for cc in range(2):
            for f in range(4):
                d = n + 16 * f + 64 * cc
                bit = ((2, 6, 3, 7) if cc == 0 else (0, 4, 1, 5))[f]
                byte |= ((int(v[d]) >> 2) & 1) << bit
        blk[1280 + 4 * (G * 16 + n) + r] = byte


def _round_trip(nbytes, bits, encode, kp_off, vp_off, decode):
    rng = np.random.default_rng(bits)
    K = rng.integers(0, 1 << bits, (16, 128))
    V = rng.integers(0, 1 << bits, (16, 128))
    prm = rng.integers(0, 1 << 16, (16, 4))
    blk = np.zeros(nbytes, np.uint8)
    for t in range(16):
        encode(blk, t, K[t], V[t])
        _params(blk, t, kp_off, vp_off, *prm[t])
    got = decode(np.tile(blk, (16, 1)), np.arange(16))
    assert np.array_equal(got["k"], K) and np.array_equal(got["v"], V)
    for j, name in enumerate(("k_scale", "k_zero", "v_scale", "v_zero")):
        assert np.array_equal(got[name], prm[:, j])
    assert blk.size * 8 / (16 * 256) == bits + 0.25     # codes plus fp16 scale / zero per 128 elements


def test_sub4_reader_matches_header_layout():
    _round_trip(2176, 4, _encode_sub4, 2048, 2112, decode_sub4)


def test_sub3_reader_matches_header_layout():
    _round_trip(1664, 3, _encode_sub3, 1536, 1600, decode_sub3)


def test_sub2_reader_matches_header_layout():
    _round_trip(1152, 2, lambda blk, t, k, v: _encode_low2(blk, t, k, v, 0, 512), 1024, 1088, decode_sub2)


def _encode_subg(blk, t, k, v, key_bits, vbits):
    """Grouped keys as include/kvq.h states them: group j's area at
    64 (b_0 + .. + b_{j-1}), slot 16 G + t for dims 32 G + 8 j + e."""
    off = 0
    for j, b in enumerate(key_bits):
        for G in range(4):
            s = 16 * G + t
            for e in range(8):
                c = int(k[32 * G + 8 * j + e])
                if b == 4:
                    blk[off + 4 * s + e // 2] |= c << (4 * (e % 2))
                else:
                    blk[off + 2 * s + e // 4] |= (c & 3) << (2 * (e % 4))
                    if b == 3:
                        blk[off + 128 + s] |= ((c >> 2) & 1) << e
        off += 64 * b
    ka = off
    if vbits == 4:
        G, r = t // 4, t % 4
        for n in range(16):
            for c in range(4):
                blk[ka + 4 * ((G * 16 + n) * 4 + c) + r] = int(v[32 * c + n]) | (int(v[32 * c + 16 + n]) << 4)
    else:
        _encode_low2_values(blk, t, v, ka)
        if vbits == 3:
            G, r = t // 4, t % 4
            for n in range(16):
                byte = 0
                for cc in range(2):
                    for f in range(4):
                        d = n + 16 * f + 64 * cc
                        bit = ((2, 6, 3, 7) if cc == 0 else (0, 4, 1, 5))[f]
                        byte |= ((int(v[d]) >> 2) & 1) << bit
                blk[ka + 512 + 4 * (G * 16 + n) + r] = byte


@pytest.mark.parametrize("key_bits,vbits", [((4, 3, 3, 2), 3), ((2, 2, 2, 2), 2), ((3, 4, 2, 3), 4),
                                            ((4, 4, 4, 4), 4), ((2, 3, 4, 2), 2)])
def test_grouped_reader_matches_header_layout(key_bits, vbits):
    from decode_attention_int4_block_amd.layout import decode_subg, subg_bytes
    from oracle.quant import group_widths_per_dim
    rng = np.random.default_rng(sum(key_bits) + vbits)
    kb = group_widths_per_dim(key_bits)
    K = (rng.integers(0, 1 << 16, (16, 128)) % (1 << kb)[None, :]).astype(np.int64)
    V = rng.integers(0, 1 << vbits, (16, 128))
    prm = rng.integers(0, 1 << 16, (16, 4))
    nb = subg_bytes(key_bits, vbits)
    assert nb == 64 * sum(key_bits) + {2: 512, 3: 768, 4: 1024}[vbits] + 128
    blk = np.zeros(nb, np.uint8)
    ka = 64 * sum(key_bits)
    va = {2: 512, 3: 768, 4: 1024}[vbits]
    for t in range(16):
        _encode_subg(blk, t, K[t], V[t], key_bits, vbits)
        _params(blk, t, ka + va, ka + va + 64, *prm[t])
    got = decode_subg(np.tile(blk, (16, 1)), np.arange(16), key_bits, vbits)
    assert np.array_equal(got["k"], K) and np.array_equal(got["v"], V)
    for j, name in enumerate(("k_scale", "k_zero", "v_scale", "v_zero")):
        assert np.array_equal(got[name], prm[:, j])
    # bytes per (token, KV head): the oracle's closed form
    from oracle.quant import grouped_key_bytes_per_token
    assert nb // 16 == grouped_key_bytes_per_token(key_bits) + 128 * vbits // 8 + 4
