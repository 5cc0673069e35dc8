"""GPU parity of causal multi-row attention over the quantized cache (kv_prefill_attn).

Each sequence's cache holds all L positions (bulk kv_quant_append); a chunk of
T query rows per sequence attends causally.  Every row is compared with the
oracle (oracle.attention.prefill_attend over the oracle's own quantization of
the same bf16 inputs) within 2e-3, lse included; the last row of each chunk is
also compared with kv_decode_attn.
"""

import numpy as np
import pytest
import torch

from gpu_common import ATOL, make_device_workload, small_config
from oracle.attention import prefill_attend, rotated_query, softmax_attention
from oracle.cache import dequantized_kv, quantize_sequence
from workloads import bf16_bits

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _report(name, **kw):
    print(f"[prefill] {name}: " + ", ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _query_rows(T, Hq, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn((int(sum(T)), Hq, 128), generator=g).to(torch.bfloat16)


def _seq_tolerance(qb_rows, cache, cfg):
    """Bound for crafted rows whose values reach 6e4: ATOL max(1, v_max / 256)
    (fp32 sums of values that large) plus 2^-22 |t|_max (v_max - v_min), where
    |t|_max is the largest |score| (natural-log units, from the oracle's fp64
    scores) the rows see: the kernel holds scores to a few fp32 ulps, a score
    error d moves the softmax weights by a relative d, and so the output by up
    to d times the values' range."""
    K, V = dequantized_kv(cache)
    g = cfg.num_q_heads // cfg.num_kv_heads
    T = qb_rows.shape[0]
    tmax = 0.0
    for t in range(T):
        p = cache.L - T + t
        qt = rotated_query(qb_rows[t], cache.h)                 # [Hq, d]
        Kg = np.repeat(K[:p + 1], g, axis=1)                    # [P, Hq, d]
        tmax = max(tmax, float(np.abs((Kg * qt[None]).sum(-1)).max()) / np.sqrt(128.0))
    vmax = float(np.abs(V).max())
    return ATOL * max(1.0, vmax / 256.0) + 2.0 ** -22 * tmax * float(V.max() - V.min())


def _run(cfg, T, seed, check_decode=True, kv_fn=None, scaled=False):
    """Fill the cache with every row's L positions, attend chunks of T[b] rows, compare.
    scaled=True: each sequence's errors relative to its _seq_tolerance, in ATOL
    units (crafted rows)."""
    from decode_attention_int4_block_amd import kv_prefill_attn
    lengths = np.asarray(cfg.length_args, np.int64)
    T = np.minimum(np.asarray(T, np.int64), lengths)
    rows = list(range(cfg.batch))
    dw = make_device_workload(cfg, keep=[b for b in rows if lengths[b] > 0], prefill=False, poison=True,
                              kv_fn=kv_fn)
    dw.prefill(include_step_token=True)
    q = _query_rows(T, cfg.num_q_heads, seed)
    q_start = torch.from_numpy(np.concatenate([[0], np.cumsum(T)]).astype(np.int32)).cuda()
    out, lse = kv_prefill_attn(dw.cache, q.cuda(), q_start, dw.slots, dw.block_table, dw.ctx_len,
                               max_rows=int(T.max()) if len(T) else 0)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    lse = lse.cpu().numpy()
    qb = bf16_bits(q)
    worst, worst_lse, r0 = 0.0, 0.0, 0
    scales = {}
    for b in rows:
        Tb = int(T[b])
        if Tb == 0:
            continue
        k, v = dw.host_kv[b]
        cache = quantize_sequence(bf16_bits(k), bf16_bits(v), cfg.had_block, cfg.sink, cfg.recent,
                                  main_bits=cfg.code_bits)
        ref, ref_lse = prefill_attend(qb[r0:r0 + Tb], cache)
        got = out[r0:r0 + Tb]
        assert np.isfinite(got).all(), f"non-finite output in sequence {b}"
        scale = _seq_tolerance(qb[r0:r0 + Tb], cache, cfg) / ATOL if scaled else 1.0
        scales[b] = scale
        worst = max(worst, float(np.abs(got - ref).max()) / scale)
        worst_lse = max(worst_lse, float(np.abs(lse[r0:r0 + Tb] - ref_lse).max()))
        r0 += Tb
    if check_decode:
        # the last row of every chunk is the decode step at length L
        last = np.cumsum(T) - 1
        sel = [b for b in rows if T[b] > 0]
        dq = q[torch.from_numpy(last[sel])].cuda().contiguous()
        from decode_attention_int4_block_amd import kv_decode_attn
        d_out, _ = kv_decode_attn(dw.cache, dq, dw.slots[sel].contiguous(), dw.block_table,
                                  dw.ctx_len[sel].contiguous())
        torch.cuda.synchronize()
        gaps = np.abs(d_out.cpu().numpy() - out[last[sel]]).reshape(len(sel), -1).max(axis=1)
        gap = max(float(gaps[i]) / scales[b] for i, b in enumerate(sel))
        assert gap <= 2 * ATOL, gap
    return worst, worst_lse


EDGE = [1, 2, 3, 5, 16, 17, 31, 33, 40, 64, 100, 129, 300]


@pytest.mark.parametrize("h", [1, 64, 128])
def test_prefill_edge_lengths_and_chunks(h):
    Ts = [1, 2, 3, 4, 5, 16, 17, 18, 33, 7, 64, 100, 300]
    cfg = small_config(EDGE, h=h, s=4, w=32, seed=2100 + h)
    err, err_lse = _run(cfg, Ts, seed=h)
    _report(f"edge lengths h={h}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


@pytest.mark.parametrize("bits", [4, 3, 2])
def test_prefill_crafted_rows(bits):
    """The quantizer's edge cases (constant, +-0, underflowing range, subnormal
    scale, grid, half-way and large vectors, values near 6e4) through the
    prefill: p * s_v reaches the f16 range's top, which the unit-scale hi / lo
    split of p * s_v relies on p <= 1 to stay inside; outputs finite.  Error
    in units of the bound _seq_tolerance derives: nearly tied scores near 2800
    (an fp32 ulp ~2.4e-4) of keys whose values differ by ~5e4 move the output by
    ~0.3 (relative 1e-4) at 3 and 2 bits, as they did before the two-tile
    kernel."""
    from workloads.edge import edge_kv
    lengths = [1, 5, 37, 200, 300]
    qmax = (1 << bits) - 1
    cfg = small_config(lengths, h=1, s=4, w=32, seed=2500 + bits, bits=bits)

    def kv_fn(b):
        return edge_kv(lengths[b], cfg.num_kv_heads, 1, qmax, seed=2510 + 10 * bits + b, offset=b)

    err, err_lse = _run(cfg, [1, 5, 20, 64, 300], seed=bits, kv_fn=kv_fn, scaled=True)
    _report(f"{bits}-bit crafted rows", max_abs_scaled=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


@pytest.mark.parametrize("s,w", [(0, 0), (0, 16), (16, 0), (4, 1), (16, 128), (4, 4000)])
def test_prefill_protection_budgets(s, w):
    lengths = [3, 17, 40, 129, 300, 700]
    cfg = small_config(lengths, h=128, s=s, w=w, seed=2200 + s + w)
    err, err_lse = _run(cfg, [3, 9, 40, 70, 150, 64], seed=s + w)
    _report(f"budget s={s} w={w}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


@pytest.mark.parametrize("g,Hkv", [(1, 4), (2, 2), (3, 2), (4, 2), (8, 2), (16, 1)])
def test_prefill_query_groups(g, Hkv):
    """R = floor(16 / g) rows per tile: 16, 8, 5 (15 of 16 columns), 4, 2, 1."""
    cfg = small_config([20, 77, 160, 333], Hq=g * Hkv, Hkv=Hkv, h=128, s=4, w=64, seed=2300 + g)
    err, err_lse = _run(cfg, [20, 19, 37, 50], seed=g)
    _report(f"g={g}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


def test_prefill_page_sizes_empty_rows_and_whole_sequences():
    for P in (16, 64, 1024):
        lengths = [0, 1, 70, 1500, 0, 600]
        cfg = small_config(lengths, P=P, h=64, s=4, w=128, seed=2400 + P)
        # T = L: a whole-sequence prefill, row 0 at position 0
        err, err_lse = _run(cfg, [0, 1, 70, 48, 0, 600], seed=P)
        _report(f"P={P}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
        assert err <= ATOL and err_lse <= ATOL


@pytest.mark.parametrize("B", [64, 70])
def test_prefill_many_sequences(B):
    """Launches of up to 64 sequences hand the waves out longest causal prefix
    first over all sequences; larger ones keep the per-sequence order.  Both
    sides of the limit, with empty chunks and chunks of every size up to a few
    waves."""
    rng = np.random.default_rng(2600 + B)
    lengths = [int(x) for x in rng.integers(1, 260, size=B)]
    lengths[3] = 0
    Ts = [min(L, int(t)) for L, t in zip(lengths, rng.integers(0, 40, size=B))]
    cfg = small_config(lengths, h=64, s=4, w=32, seed=2600 + B)
    err, err_lse = _run(cfg, Ts, seed=B, check_decode=False)
    _report(f"{B} sequences", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


def test_prefill_long_chunk_sampled_rows():
    """A 4096-token sequence with a 1024-row chunk, Qwen3-8B heads; rows sampled
    for the oracle (the first, the last, the window boundary, random)."""
    from decode_attention_int4_block_amd import kv_prefill_attn
    L, T = 4096, 1024
    cfg = small_config([L, 2000], Hq=32, Hkv=8, h=128, s=4, w=128, seed=2500)
    dw = make_device_workload(cfg, keep=[0, 1], prefill=False)
    dw.prefill(include_step_token=True)
    Ts = np.array([T, 300])
    q = _query_rows(Ts, 32, 77)
    q_start = torch.tensor([0, T, T + 300], dtype=torch.int32, device="cuda")
    out, lse = kv_prefill_attn(dw.cache, q.cuda(), q_start, dw.slots, dw.block_table, dw.ctx_len, max_rows=T)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    qb = bf16_bits(q)
    k, v = dw.host_kv[0]
    cache = quantize_sequence(bf16_bits(k), bf16_bits(v), 128, 4, 128)
    K, V = dequantized_kv(cache)
    rng = np.random.default_rng(5)
    pick = sorted({0, T - 1, T - 128, T - 129} | set(int(x) for x in rng.integers(0, T, 12)))
    worst = 0.0
    for t in pick:
        p = L - T + t
        ref, _ = softmax_attention(rotated_query(qb[t], 128), K[:p + 1], V[:p + 1])
        worst = max(worst, float(np.abs(out[t] - ref).max()))
    _report("4096 x 1024 chunk", rows=len(pick), max_abs=f"{worst:.2e}")
    assert worst <= ATOL and np.isfinite(out).all()


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("h", [1, 128])
def test_prefill_sub4bit_edge_lengths_and_chunks(bits, h):
    """The 3- and 2-bit main caches (KV4-RL, "Future Directions"): every row
    against the oracle's prefill attention over its own 3- / 2-bit
    quantization, the last row against kv_decode_attn."""
    Ts = [1, 2, 3, 4, 5, 16, 17, 18, 33, 7, 64, 100, 300]
    cfg = small_config(EDGE, h=h, s=4, w=32, seed=2600 + 10 * h + bits, bits=bits)
    err, err_lse = _run(cfg, Ts, seed=100 + h + bits)
    _report(f"{bits}-bit edge lengths h={h}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


@pytest.mark.parametrize("bits", [3, 2])
@pytest.mark.parametrize("s,w,g,Hkv,P", [(0, 0, 4, 2, 16), (16, 128, 8, 2, 64), (4, 64, 16, 1, 16),
                                         (4, 4000, 3, 2, 1024)])
def test_prefill_sub4bit_budgets_groups_pages(bits, s, w, g, Hkv, P):
    lengths = [0, 3, 17, 40, 129, 300, 700]
    cfg = small_config(lengths, Hq=g * Hkv, Hkv=Hkv, P=P, h=64, s=s, w=w, seed=2700 + s + w + g + bits, bits=bits)
    err, err_lse = _run(cfg, [0, 3, 9, 40, 70, 150, 64], seed=s + w + g)
    _report(f"{bits}-bit s={s} w={w} g={g} P={P}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


@pytest.mark.parametrize("bits", [3, 2])
def test_prefill_sub4bit_long_chunk_sampled_rows(bits):
    """A 4096-token sequence, 1024-row chunk, Qwen3-8B heads, 3- / 2-bit main
    cache; rows sampled for the oracle."""
    from decode_attention_int4_block_amd import kv_prefill_attn
    L, T = 4096, 1024
    cfg = small_config([L], Hq=32, Hkv=8, h=128, s=4, w=128, seed=2800 + bits, bits=bits)
    dw = make_device_workload(cfg, keep=[0], prefill=False)
    dw.prefill(include_step_token=True)
    q = _query_rows(np.array([T]), 32, 78 + bits)
    q_start = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    out, _ = kv_prefill_attn(dw.cache, q.cuda(), q_start, dw.slots, dw.block_table, dw.ctx_len, max_rows=T)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    qb = bf16_bits(q)
    k, v = dw.host_kv[0]
    cache = quantize_sequence(bf16_bits(k), bf16_bits(v), 128, 4, 128, main_bits=bits)
    K, V = dequantized_kv(cache)
    rng = np.random.default_rng(6)
    pick = sorted({0, T - 1, T - 128, T - 129} | set(int(x) for x in rng.integers(0, T, 12)))
    worst = 0.0
    for t in pick:
        p = L - T + t
        ref, _ = softmax_attention(rotated_query(qb[t], 128), K[:p + 1], V[:p + 1])
        worst = max(worst, float(np.abs(out[t] - ref).max()))
    _report(f"{bits}-bit 4096 x 1024 chunk", rows=len(pick), max_abs=f"{worst:.2e}")
    assert worst <= ATOL and np.isfinite(out).all()
