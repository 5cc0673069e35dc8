"""GPU parity of the fused append + attention entry point (kv_append_decode_attn).

It must write the same cache bytes as kv_quant_append of each row's token at
position L - 1 and give the same attention as kv_decode_attn afterwards.  Both
paths start from pools pre-filled with the same 0xFF bytes, so whole pools are
compared byte for byte; the output is compared with the two-launch path
(bit-identical when both kernels split the work over the same number of
workers) and with the oracle (2e-3, as for kv_decode_attn).
"""

import numpy as np
import pytest
import torch

from gpu_common import ATOL, assert_cache_exact, compare_attention, compare_cache, make_device_workload, small_config
from workloads import get_config

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _report(name, **kw):
    print(f"[fused] {name}: " + ", ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _pair(cfg, keep=(), gen_device="cpu"):
    """Two copies of a workload, prefilled to L - 1 positions: one takes the
    step as append + decode, the other as the fused launch."""
    sep = make_device_workload(cfg, keep=keep, poison=True, prefill=False, gen_device=gen_device)
    fus = make_device_workload(cfg, keep=keep, poison=True, prefill=False, gen_device=gen_device)
    sep.prefill()
    fus.prefill()
    sep.append_step()
    sep.decode_step()
    fus.fused_step()
    torch.cuda.synchronize()
    return sep, fus


def _workers(dw):
    # the workspace header's first word is the worker count of the last launch
    return dw.workspace[:4].view(torch.int32).item()


def _check_pair(sep, fus, rows, name):
    assert torch.equal(sep.cache.int4_pool, fus.cache.int4_pool), f"{name}: INT4 pool differs"
    assert torch.equal(sep.cache.int8_pool, fus.cache.int8_pool), f"{name}: INT8 pool differs"
    same_split = _workers(sep) == _workers(fus)
    d_out = float((sep.out - fus.out).abs().max()) if sep.out.numel() else 0.0
    if same_split:
        assert torch.equal(sep.out, fus.out) and torch.equal(sep.lse, fus.lse), f"{name}: outputs differ"
    else:
        assert d_out <= 1e-5, f"{name}: outputs differ by {d_out}"
    for b in rows:
        if int(fus.wl.lengths[b]) > 0:
            assert_cache_exact(compare_cache(fus, b))
    err, err_lse, _ = compare_attention(fus, rows)
    _report(name, same_split=same_split, d_two_launch=f"{d_out:.1e}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


# lengths around the subblock (16), INT4 step (32) and ring boundaries
EDGE = [1, 2, 3, 4, 5, 15, 16, 17, 31, 32, 33, 36, 37, 47, 48, 49, 64, 100, 129, 200, 515]


@pytest.mark.parametrize("h", [1, 64, 128])
def test_fused_edge_lengths(h):
    cfg = small_config(EDGE, h=h, s=4, w=32, seed=1100 + h)
    rows = list(range(cfg.batch))
    sep, fus = _pair(cfg, keep=rows)
    _check_pair(sep, fus, rows, f"edge lengths h={h}")


@pytest.mark.parametrize("s,w", [(0, 0), (0, 16), (16, 0), (4, 1), (16, 128), (4, 4000)])
def test_fused_protection_budgets(s, w):
    """INT4 only, recent only, sinks only (the new token lands in INT4), a
    one-entry window, the default split, and INT8 everywhere."""
    cfg = small_config([1, 3, 17, 40, 129, 300, 1000], h=128, s=s, w=w, seed=1200 + s + w)
    rows = list(range(cfg.batch))
    sep, fus = _pair(cfg, keep=rows)
    _check_pair(sep, fus, rows, f"budget s={s} w={w}")


@pytest.mark.parametrize("g,Hkv", [(1, 4), (3, 2), (4, 2), (6, 2), (8, 2), (11, 1), (16, 1)])
def test_fused_query_groups(g, Hkv):
    cfg = small_config([1, 20, 77, 160, 700], Hq=g * Hkv, Hkv=Hkv, h=128, s=4, w=64, seed=1300 + g)
    rows = list(range(cfg.batch))
    sep, fus = _pair(cfg, keep=rows)
    _check_pair(sep, fus, rows, f"g={g} Hkv={Hkv}")


def test_fused_page_sizes_and_empty_rows():
    for P in (16, 64, 1024):
        cfg = small_config([0, 1, 70, 1500, 0, 2049], P=P, h=64, s=4, w=128, seed=1400 + P)
        rows = list(range(cfg.batch))
        sep, fus = _pair(cfg, keep=[b for b in rows if cfg.length_args[b] > 0])
        _check_pair(sep, fus, rows, f"P={P} with empty rows")


@pytest.mark.parametrize("s,w,bits", [(4, 32, 4), (4, 0, 4), (0, 16, 4), (4, 32, 3), (0, 16, 2)])
def test_fused_consecutive_steps(s, w, bits):
    """Forty steps in a row, one new token per row each: the recent ring wraps
    and positions move from the INT8 window into the INT4 region."""
    from decode_attention_int4_block_amd import kv_append_decode_attn, kv_decode_attn, kv_quant_append
    from workloads import seq_kv
    n = 40
    final = [41, 60, 77, 100, 140, 300]
    cfg = small_config(final, h=128, s=s, w=w, seed=1500 + s + w + bits, bits=bits)
    rows = list(range(cfg.batch))
    sep = make_device_workload(cfg, keep=rows, poison=True, prefill=False)
    fus = make_device_workload(cfg, keep=rows, poison=True, prefill=False)
    wl = sep.wl
    kv = [seq_kv(wl, b) for b in rows]
    for dw in (sep, fus):
        dw.host_kv = {b: kv[b] for b in rows}
    slots = sep.slots
    L0 = np.array(final) - n
    # prefill positions [0, L0) with one bulk append per cache
    k0 = torch.cat([kv[b][0][:L0[b]] for b in rows]).cuda().contiguous()
    v0 = torch.cat([kv[b][1][:L0[b]] for b in rows]).cuda().contiguous()
    sl0 = torch.from_numpy(np.concatenate([np.full(L0[b], wl.slots[b]) for b in rows]).astype(np.int32)).cuda()
    ps0 = torch.from_numpy(np.concatenate([np.arange(L0[b]) for b in rows]).astype(np.int32)).cuda()
    la = np.zeros(wl.num_slots, dtype=np.int32)
    la[wl.slots] = L0
    for dw in (sep, fus):
        kv_quant_append(dw.cache, k0, v0, sl0, ps0, dw.block_table, torch.from_numpy(la).cuda())
    for j in range(n):
        ctx = L0 + j + 1
        kn = torch.stack([kv[b][0][ctx[b] - 1] for b in rows]).cuda().contiguous()
        vn = torch.stack([kv[b][1][ctx[b] - 1] for b in rows]).cuda().contiguous()
        ctx_t = torch.from_numpy(ctx.astype(np.int32)).cuda()
        la = np.zeros(wl.num_slots, dtype=np.int32)
        la[wl.slots] = ctx
        kv_quant_append(sep.cache, kn, vn, slots, ctx_t - 1, sep.block_table, torch.from_numpy(la).cuda())
        kv_decode_attn(sep.cache, sep.q, slots, sep.block_table, ctx_t, out=sep.out, lse=sep.lse,
                       workspace=sep.workspace)
        kv_append_decode_attn(fus.cache, kn, vn, fus.q, slots, fus.block_table, ctx_t, out=fus.out, lse=fus.lse,
                              workspace=fus.workspace)
        torch.cuda.synchronize()
        assert torch.equal(sep.cache.int4_pool, fus.cache.int4_pool), f"step {j}: INT4 pool differs"
        assert torch.equal(sep.cache.int8_pool, fus.cache.int8_pool), f"step {j}: INT8 pool differs"
        assert torch.equal(sep.out, fus.out) and torch.equal(sep.lse, fus.lse), f"step {j}: outputs differ"
    _check_pair(sep, fus, rows, f"{n} consecutive steps s={s} w={w} {bits}-bit")


# 2- and 3-bit main caches: the fused kernel stores the token in the 2-bit
# layouts (plus the high planes at 3 bits) and patches its stage copy of them
@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("g,Hkv", [(4, 2), (7, 1), (16, 1)])
def test_fused_sub4bit_edge_lengths(bits, g, Hkv):
    cfg = small_config(EDGE, Hq=g * Hkv, Hkv=Hkv, h=128, s=4, w=32, seed=1600 + 20 * bits + g, bits=bits)
    rows = list(range(cfg.batch))
    sep, fus = _pair(cfg, keep=rows)
    _check_pair(sep, fus, rows, f"{bits}-bit g={g} edge lengths")


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("s,w", [(0, 0), (16, 0), (0, 16), (4, 4000)])
def test_fused_sub4bit_protection_budgets(bits, s, w):
    cfg = small_config([1, 17, 33, 160, 700], h=128, s=s, w=w, seed=1700 + s + w + bits, bits=bits)
    rows = list(range(cfg.batch))
    sep, fus = _pair(cfg, keep=rows)
    _check_pair(sep, fus, rows, f"{bits}-bit s={s} w={w}")


@pytest.mark.parametrize("bits", [2, 3])
def test_fused_sub4bit_page_sizes_and_empty_rows(bits):
    for P in (16, 64):
        cfg = small_config([0, 1, 70, 1500, 0, 2049], P=P, h=64, s=4, w=128, seed=1800 + P + bits, bits=bits)
        rows = list(range(cfg.batch))
        sep, fus = _pair(cfg, keep=[b for b in rows if cfg.length_args[b] > 0])
        _check_pair(sep, fus, rows, f"{bits}-bit P={P} with empty rows")


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_fused_full_size_step(bits):
    """The 256-row Qwen3-8B batch in the benchmark's launch configuration
    (and the same batch over the 3- and 2-bit main caches)."""
    import dataclasses
    cfg = dataclasses.replace(get_config("qwen3_8b_async_256"), code_bits=bits)
    from workloads import build_workload
    wl = build_workload(cfg)
    L = wl.lengths
    rng = np.random.default_rng(11)
    rows = sorted({int(np.argmin(L)), int(np.argmax(L))} |
                  set(int(x) for x in rng.choice(cfg.batch, size=3, replace=False)))
    sep, fus = _pair(cfg, keep=rows, gen_device="cuda")
    assert torch.equal(sep.cache.int4_pool, fus.cache.int4_pool)
    assert torch.equal(sep.cache.int8_pool, fus.cache.int8_pool)
    if _workers(sep) == _workers(fus):
        assert torch.equal(sep.out, fus.out) and torch.equal(sep.lse, fus.lse)
    else:
        assert float((sep.out - fus.out).abs().max()) <= 1e-5
    err, err_lse, _ = compare_attention(fus, rows)
    _report(f"qwen3_8b_async_256 {bits}-bit", rows=rows, max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


def test_fused_full_size_long_row():
    """The 128K-position row (query group 8) in the benchmark's launch
    configuration: the fused kernel of that group size holds one worker per
    workgroup (its stage ring and append slots fill a worker's LDS share), and
    the row is split over many workers and folded by the combine's helpers."""
    cfg = get_config("long_128k")
    sep, fus = _pair(cfg, keep=[0], gen_device="cuda")
    assert torch.equal(sep.cache.int4_pool, fus.cache.int4_pool)
    assert torch.equal(sep.cache.int8_pool, fus.cache.int8_pool)
    d_out = float((sep.out - fus.out).abs().max())
    if _workers(sep) == _workers(fus):
        assert torch.equal(sep.out, fus.out) and torch.equal(sep.lse, fus.lse)
    else:
        assert d_out <= 1e-5, d_out
    err, err_lse, _ = compare_attention(fus, [0])
    _report("long_128k", workers=(_workers(sep), _workers(fus)), d_two_launch=f"{d_out:.1e}",
            max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL
