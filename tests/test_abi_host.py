"""The C ABI library loads without a GPU, exports every symbol include/kvq.h
declares, and rejects bad arguments on the host before enqueuing anything."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_][a-z0-9_]*)\s*\(", text)) - {"if", "sizeof", "defined"})


@pytest.fixture(scope="module")
def lib():
    from decode_attention_int4_block_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libkvq.so not built")
    return _lib.load()


def test_header_declares_the_two_entry_points():
    names = _declared_functions()
    assert "kv_quant_append" in names and "kv_decode_attn" in names


def test_every_declared_symbol_is_exported(lib):
    from decode_attention_int4_block_amd import _lib
    names = _declared_functions()
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.SIGNATURES)


def _desc(**kw):
    from decode_attention_int4_block_amd._lib import KvqCache
    d = dict(num_kv_heads=8, head_dim=128, page_size=16, num_pages=100, num_slots=4,
             had_block=128, sink=4, recent=128, int4_pool=None, int8_pool=None)
    d.update(kw)
    return KvqCache(**d)


def test_pool_sizes_follow_the_documented_layout(lib):
    d = _desc()
    assert lib.kvq_int4_pool_bytes(ctypes.byref(d)) == 100 * 8 * 1 * 2176
    assert lib.kvq_int8_pool_bytes(ctypes.byref(d)) == 4 * 8 * 9 * 4224
    d64 = _desc(page_size=64)
    assert lib.kvq_int4_pool_bytes(ctypes.byref(d64)) == 100 * 8 * 4 * 2176
    # 4.25 bits per element: 2176 bytes hold 16 tokens x 256 K+V elements
    assert 2176 * 8 / (16 * 256) == 4.25


@pytest.mark.parametrize("field,value", [("head_dim", 64), ("page_size", 24), ("page_size", 0), ("page_size", 48),
                                         ("had_block", 3), ("had_block", 256), ("sink", -1),
                                         ("num_kv_heads", 0)])
def test_bad_descriptors_are_rejected(lib, field, value):
    d = _desc(**{field: value})
    assert lib.kvq_int4_pool_bytes(ctypes.byref(d)) == 0
    st = lib.kv_quant_append(ctypes.byref(d), None, None, None, None, 1, None, 1, None, None)
    assert st in (2, 3)
    assert lib.kvq_last_error()


def test_append_argument_checks(lib):
    d = _desc(int4_pool=0x1000, int8_pool=0x2000)
    assert lib.kv_quant_append(ctypes.byref(d), None, None, None, None, 0, None, 1, None, None) == 0
    assert lib.kv_quant_append(ctypes.byref(d), None, None, None, None, -1, None, 1, None, None) == 2
    assert lib.kv_quant_append(ctypes.byref(d), None, None, None, None, 5, None, 1, None, None) == 1
    p = ctypes.c_void_p(0x3000)
    assert lib.kv_quant_append(ctypes.byref(d), p, p, p, p, 5, p, 0, p, None) == 2
    d0 = _desc(int4_pool=0x1000, int8_pool=None)
    assert lib.kv_quant_append(ctypes.byref(d0), p, p, p, p, 5, p, 4, p, None) == 1
    assert lib.kv_quant_append(None, p, p, p, p, 5, p, 4, p, None) == 1


def test_decode_argument_checks(lib):
    d = _desc(int4_pool=0x1000, int8_pool=0x2000)
    p = ctypes.c_void_p(0x3000)
    # group 32 > 16 is unsupported; query heads not a multiple of KV heads
    assert lib.kv_decode_attn(ctypes.byref(d), p, 256, p, p, 4, p, 2, p, None, p, 1 << 30, None) == 3
    assert lib.kv_decode_attn(ctypes.byref(d), p, 12, p, p, 4, p, 2, p, None, p, 1 << 30, None) == 2
    assert lib.kv_decode_attn(ctypes.byref(d), p, 32, p, p, 4, p, -1, p, None, p, 1 << 30, None) == 2
    assert lib.kv_decode_attn(ctypes.byref(d), p, 32, p, p, 4, p, 0, p, None, p, 1 << 30, None) == 0
    assert lib.kv_decode_attn(ctypes.byref(d), None, 32, p, p, 4, p, 2, p, None, p, 1 << 30, None) == 1
    assert lib.kv_decode_attn(ctypes.byref(d), p, 32, p, p, 4, p, 2, p, None, None, 1 << 30, None) == 4


def test_noalloc_argument_checks(lib):
    """The no-allocation entry point rejects bad arguments on the host, before
    it looks up its scratch or touches a device."""
    d = _desc(int4_pool=0x1000, int8_pool=0x2000)
    p = ctypes.c_void_p(0x3000)
    f = lib.kv_decode_attn_noalloc
    assert f(ctypes.byref(d), p, 256, p, p, 4, p, 2, p, None, None) == 3
    assert f(ctypes.byref(d), p, 12, p, p, 4, p, 2, p, None, None) == 2
    assert f(ctypes.byref(d), p, 32, p, p, 4, p, -1, p, None, None) == 2
    assert f(ctypes.byref(d), p, 32, p, p, 4, p, 0, p, None, None) == 0
    assert f(ctypes.byref(d), None, 32, p, p, 4, p, 2, p, None, None) == 1
    assert f(ctypes.byref(d), p, 32, p, p, 4, p, 2, None, None, None) == 1
    assert f(None, p, 32, p, p, 4, p, 2, p, None, None) == 1


def test_fused_argument_checks(lib):
    d = _desc(int4_pool=0x1000, int8_pool=0x2000)
    p = ctypes.c_void_p(0x3000)
    f = lib.kv_append_decode_attn
    assert f(ctypes.byref(d), p, p, p, 32, p, p, 4, p, 0, p, None, p, 1 << 30, None) == 0
    assert f(ctypes.byref(d), p, p, p, 256, p, p, 4, p, 2, p, None, p, 1 << 30, None) == 3
    assert f(ctypes.byref(d), None, p, p, 32, p, p, 4, p, 2, p, None, p, 1 << 30, None) == 1
    assert f(ctypes.byref(d), p, None, p, 32, p, p, 4, p, 2, p, None, p, 1 << 30, None) == 1
    assert f(ctypes.byref(d), p, p, p, 32, p, p, 4, p, 2, p, None, None, 1 << 30, None) == 4
    assert f(None, p, p, p, 32, p, p, 4, p, 2, p, None, p, 1 << 30, None) == 1


def test_prefill_argument_checks(lib):
    d = _desc(int4_pool=0x1000, int8_pool=0x2000)
    p = ctypes.c_void_p(0x3000)
    f = lib.kv_prefill_attn
    assert f(ctypes.byref(d), p, 32, p, 0, p, p, 4, p, 2, p, None, None) == 0      # max_rows 0: nothing to do
    assert f(ctypes.byref(d), p, 32, p, 8, p, p, 4, p, 0, p, None, None) == 0      # B 0
    assert f(ctypes.byref(d), p, 32, p, -1, p, p, 4, p, 2, p, None, None) == 2
    assert f(ctypes.byref(d), p, 256, p, 8, p, p, 4, p, 2, p, None, None) == 3
    assert f(ctypes.byref(d), p, 12, p, 8, p, p, 4, p, 2, p, None, None) == 2
    assert f(ctypes.byref(d), p, 32, None, 8, p, p, 4, p, 2, p, None, None) == 1
    assert f(ctypes.byref(d), p, 32, p, 8, p, p, 0, p, 2, p, None, None) == 2
    assert f(ctypes.byref(d), p, 32, p, 8, p, p, 4, p, 70000, p, None, None) == 2
    assert f(None, p, 32, p, 8, p, p, 4, p, 2, p, None, None) == 1


def test_sub4bit_cache_sizes_and_limits(lib):
    d = _desc(code_bits=2)
    assert lib.kvq_int4_pool_bytes(ctypes.byref(d)) == 100 * 8 * 1 * 1152
    assert lib.kvq_int8_pool_bytes(ctypes.byref(d)) == 4 * 8 * 9 * 4224       # the INT8 side cache is unchanged
    # 1152 bytes hold 16 tokens x 256 K+V elements: 2.25 bits per element
    assert 1152 * 8 / (16 * 256) == 2.25
    # 3 bits: 1664 bytes (two low planes of 512, two high planes of 256, params)
    # hold 16 tokens x 256 K+V elements: 3.25 bits per element
    assert lib.kvq_int4_pool_bytes(ctypes.byref(_desc(code_bits=3))) == 100 * 8 * 1 * 1664
    assert 1664 * 8 / (16 * 256) == 3.25
    for bad in (1, 5, 8):
        assert lib.kvq_int4_pool_bytes(ctypes.byref(_desc(code_bits=bad))) == 0
    assert lib.kvq_int4_pool_bytes(ctypes.byref(_desc(code_bits=0))) == 100 * 8 * 2176   # 0 means 4
    p = ctypes.c_void_p(0x3000)
    for bits in (2, 3):
        d2 = _desc(int4_pool=0x1000, int8_pool=0x2000, code_bits=bits)
        # the prefill attention serves these widths: its argument checks apply as
        # for 4 bits (a launch needs a GPU, so only the rejections are called here)
        assert lib.kv_prefill_attn(ctypes.byref(d2), p, 32, p, 8, p, p, 0, p, 2, p, None, None) == 2
        assert lib.kv_prefill_attn(ctypes.byref(d2), p, 256, p, 8, p, p, 4, p, 2, p, None, None) == 3


def test_grouped_key_cache_sizes_and_limits(lib):
    """Keys with a width per RoPE-block group: subblock bytes 64 sum(key_bits) +
    the value area + 128 (include/kvq.h), widths in {2, 3, 4}, rotation blocks
    inside a group, and the entry points that do not serve such caches."""
    import ctypes as C
    kb = lambda *w: (C.c_int32 * 4)(*w)
    d = _desc(code_bits=3, key_bits=kb(4, 3, 3, 2), had_block=8)
    assert lib.kvq_int4_pool_bytes(C.byref(d)) == 100 * 8 * (64 * 12 + 768 + 128)
    # 104 bytes per (token, KV head), the cost of a uniform 3-bit cache
    assert (64 * 12 + 768 + 128) // 16 == 104
    assert lib.kvq_int4_pool_bytes(C.byref(_desc(code_bits=4, key_bits=kb(4, 4, 4, 4)))) == 100 * 8 * 2176
    assert lib.kvq_int4_pool_bytes(C.byref(_desc(code_bits=2, key_bits=kb(2, 2, 2, 2)))) == 100 * 8 * (512 + 512 + 128)
    for bad in ((1, 4, 4, 4), (4, 5, 4, 4), (4, 4, 4, 0)):
        assert lib.kvq_int4_pool_bytes(C.byref(_desc(key_bits=kb(*bad), had_block=8))) == 0
    # different widths need had_block <= 8; equal widths take any
    assert lib.kvq_int4_pool_bytes(C.byref(_desc(key_bits=kb(4, 3, 3, 2), had_block=16))) == 0
    assert lib.kvq_int4_pool_bytes(C.byref(_desc(key_bits=kb(3, 3, 3, 3), had_block=128))) > 0
    p = C.c_void_p(0x3000)
    dg = _desc(int4_pool=0x1000, int8_pool=0x2000, code_bits=3, key_bits=kb(4, 3, 3, 2), had_block=8)
    assert lib.kv_prefill_attn(C.byref(dg), p, 32, p, 8, p, p, 4, p, 2, p, None, None) == 3
    assert lib.kv_append_decode_attn(C.byref(dg), p, p, p, 32, p, p, 4, p, 2, p, None, p, 1 << 30, None) == 3
    assert lib.kv_decode_read_ceiling(C.byref(dg), p, 32, p, p, 4, p, 2, p, 1 << 30, None) == 3
    # query groups above 8 are not served
    assert lib.kv_decode_attn(C.byref(dg), p, 128, p, p, 4, p, 2, p, None, p, 1 << 30, None) == 3


def test_status_strings(lib):
    for s in range(6):
        assert lib.kvq_status_string(s)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    from decode_attention_int4_block_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "missing.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError):
        _lib.load()
