"""GPU parity for keys with a bit width per RoPE-block group.

RoPE-Aware Bit Allocation for KV-Cache Quantization (Block-GTQ), Abstract:
integer key bit widths per RoPE frequency block, served from a packed cache
(packing only: the width vector is an input).  The main-cache keys carry
key_bits[j] bits in RoPE-block group j, the values code_bits; the INT8 side
cache is unchanged.  Through the C ABI (kv_quant_append, kv_decode_attn):
codes, scales and offsets bit-exact against the oracle's quantize_grouped
(ties counted and bounded), attention within 2e-3 of its fp64 attention.
"""

import numpy as np
import pytest
import torch

from gpu_common import (ATOL, add_stats, assert_cache_exact, attention_error_scaled, compare_attention,
                        compare_cache, make_device_workload, small_config)
from workloads import get_config

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _report(name, **kw):
    print(f"[grouped] {name}: " + ", ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _check(cfg, name, poison=False, kv_fn=None, scaled=False):
    rows = [b for b in range(cfg.batch) if cfg.length_args[b] > 0]
    print(f"[grouped] case {name}", flush=True)
    dw = make_device_workload(cfg, keep=rows, poison=poison, kv_fn=kv_fn)
    tot = {}
    for b in rows:
        add_stats(tot, compare_cache(dw, b))
    assert_cache_exact(tot)
    dw.decode_step()
    torch.cuda.synchronize()
    if scaled:
        err = err_lse = attention_error_scaled(dw, rows)
    else:
        err, err_lse, _ = compare_attention(dw, list(range(cfg.batch)))
    _report(name, max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}", codes=tot["codes"], forgiven=tot["int4_ties"])
    assert err <= ATOL and err_lse <= ATOL


EDGE = [1, 3, 4, 5, 16, 17, 31, 32, 33, 36, 37, 64, 100, 129, 200, 515]
WIDTHS = [((4, 3, 3, 2), 3), ((2, 2, 2, 2), 2), ((3, 4, 2, 3), 4), ((4, 4, 4, 4), 4), ((2, 3, 4, 2), 2),
          ((3, 3, 3, 3), 3)]


@pytest.mark.parametrize("key_bits,vbits", WIDTHS)
@pytest.mark.parametrize("h", [1, 8])
def test_grouped_edge_lengths(key_bits, vbits, h):
    cfg = small_config(EDGE, h=h, s=4, w=32, seed=5100 + h + 7 * sum(key_bits) + vbits, bits=vbits,
                       key_bits=key_bits)
    _check(cfg, f"K{key_bits} V{vbits} h={h}")


def test_grouped_equal_widths_take_any_rotation():
    cfg = small_config([7, 90, 333], h=128, s=4, w=32, seed=5200, bits=3, key_bits=(3, 3, 3, 3))
    _check(cfg, "K3333 V3 h=128")


@pytest.mark.parametrize("s,w", [(0, 0), (0, 16), (16, 0), (16, 128), (4, 4000)])
def test_grouped_protection_budgets(s, w):
    cfg = small_config([2, 50, 333, 1200], h=8, s=s, w=w, seed=5300 + s + w, bits=3, key_bits=(4, 3, 3, 2))
    _check(cfg, f"budget s={s} w={w}")


@pytest.mark.parametrize("g,Hkv", [(1, 4), (3, 2), (4, 2), (6, 2), (8, 2)])
def test_grouped_query_groups(g, Hkv):
    cfg = small_config([1, 40, 300, 777], Hq=g * Hkv, Hkv=Hkv, h=8, s=4, w=64, seed=5400 + g, bits=2,
                       key_bits=(4, 2, 3, 2))
    _check(cfg, f"g={g}")


def test_grouped_page_sizes_empty_rows_and_poisoned_pools():
    for P in (16, 64, 1024):
        cfg = small_config([0, 1, 70, 1500, 0, 2049], P=P, h=4, s=4, w=128, seed=5500 + P, bits=4,
                           key_bits=(2, 4, 3, 4))
        _check(cfg, f"P={P}", poison=True)


def test_grouped_crafted_rows():
    """The quantizer's edge cases (constant, +-0, underflowing range, subnormal
    scale, grid, half-way and large vectors) with grouped keys, h = 1; the
    attention bound is relative to the values' magnitude, as for the uniform
    widths (rows with values near 6e4)."""
    from workloads.edge import edge_kv
    lengths = [1, 5, 37, 200]
    cfg = small_config(lengths, h=1, s=4, w=32, seed=5600, bits=3, key_bits=(4, 3, 3, 2))

    def kv_fn(b):
        return edge_kv(lengths[b], cfg.num_kv_heads, 1, 15, seed=5601 + b, offset=b)

    _check(cfg, "crafted rows (error relative to max(1, v_max / 256))", kv_fn=kv_fn, scaled=True)


def test_grouped_full_size_sampled_rows():
    """The 256-row Qwen3-8B batch with keys (4, 3, 3, 2) and 3-bit values (the
    bytes of a uniform K3V3 cache), h = 8, sampled rows."""
    from workloads import build_workload
    cfg = get_config("qwen3_8b_async_256").scaled(code_bits=3, key_bits=(4, 3, 3, 2), had_block=8)
    wl = build_workload(cfg)
    L = wl.lengths
    rng = np.random.default_rng(17)
    rows = sorted({int(np.argmin(L)), int(np.argmax(L))} |
                  set(int(x) for x in rng.choice(cfg.batch, size=3, replace=False)))
    print("[grouped] case full size", flush=True)
    dw = make_device_workload(cfg, keep=rows, gen_device="cuda")
    tot = {}
    for b in rows:
        Lb = int(L[b])
        positions = np.unique(np.concatenate([np.arange(min(Lb, 40)), np.arange(max(0, Lb - 200), Lb),
                                              rng.integers(0, Lb, size=min(Lb, 300))]))
        add_stats(tot, compare_cache(dw, b, positions))
    assert_cache_exact(tot)
    dw.decode_step()
    torch.cuda.synchronize()
    err, err_lse, unq = compare_attention(dw, rows, report_unquantized=True)
    _report("qwen3_8b_async_256 K(4,3,3,2) V3 h=8", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}",
            vs_unquantized_bf16=f"{unq:.3f}")
    assert err <= ATOL and err_lse <= ATOL
