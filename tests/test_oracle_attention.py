"""Pins for the oracle's fp64 decode attention and the regional log-sum-exp merge."""

import math

import numpy as np
import pytest
import torch

from oracle.attention import (attend, attend_regions, merge, prefill_attend, region_stats,
                              rotated_query, softmax_attention, unquantized_attention)
from oracle.cache import dequantized_kv, quantize_sequence
from oracle.hadamard import rotate_f64
from oracle.numerics import f16_bits_to_f64
from workloads import build_workload, get_config, seq_kv, seq_query, bf16_bits


def _brute(q, K, V):
    """Pure-Python loops: out[j] = sum_p softmax_p(q_j.k_p / sqrt(d)) v_p."""
    Hq, d = len(q), len(q[0])
    L, Hkv = len(K), len(K[0])
    g = Hq // Hkv
    out = []
    for j in range(Hq):
        kv = j // g
        z = [sum(q[j][i] * K[p][kv][i] for i in range(d)) / math.sqrt(d) for p in range(L)]
        m = max(z)
        e = [math.exp(x - m) for x in z]
        tot = sum(e)
        out.append([sum(e[p] * V[p][kv][i] for p in range(L)) / tot for i in range(d)])
    return np.array(out)


def test_softmax_attention_matches_brute_force():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 8))
    K = rng.standard_normal((5, 2, 8)) * 3
    V = rng.standard_normal((5, 2, 8))
    out, lse = softmax_attention(q, K, V)
    assert np.allclose(out, _brute(q.tolist(), K.tolist(), V.tolist()), rtol=0, atol=1e-13)
    z = np.einsum("pd,d->p", K[:, 0], q[0]) / np.sqrt(8)
    assert abs(lse[0] - math.log(sum(math.exp(x) for x in z))) < 1e-12


def test_softmax_attention_matches_torch_sdpa_fp64():
    rng = np.random.default_rng(1)
    Hq, Hkv, L, d = 8, 2, 300, 128
    q = rng.standard_normal((Hq, d))
    K = rng.standard_normal((L, Hkv, d)) * 2
    V = rng.standard_normal((L, Hkv, d))
    out, _ = softmax_attention(q, K, V)
    g = Hq // Hkv
    tq = torch.from_numpy(q)[:, None, :]                             # [Hq, 1, d]
    tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, 0)  # [Hq, L, d]
    tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, 0, :].numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)


def test_single_token_and_identical_keys():
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 16))
    V = rng.standard_normal((1, 1, 16))
    K = rng.standard_normal((1, 1, 16))
    out, _ = softmax_attention(q, K, V)
    assert np.allclose(out, np.repeat(V[0], 4, axis=0), atol=1e-15)
    K = np.repeat(rng.standard_normal((1, 1, 16)), 9, axis=0)
    V = rng.standard_normal((9, 1, 16))
    out, _ = softmax_attention(q, K, V)
    assert np.allclose(out, np.repeat(V.mean(axis=0), 4, axis=0), atol=1e-14)


def test_empty_context():
    out, lse = softmax_attention(np.ones((2, 4)), np.zeros((0, 1, 4)), np.zeros((0, 1, 4)))
    assert np.all(out == 0) and np.all(np.isneginf(lse))


@pytest.mark.parametrize("seed", range(5))
def test_merge_of_random_partition_equals_single_pass(seed):
    rng = np.random.default_rng(seed)
    Hq, Hkv, L, d = 4, 1, 97, 32
    q = rng.standard_normal((Hq, d))
    K = rng.standard_normal((L, Hkv, d)) * 4
    V = rng.standard_normal((L, Hkv, d))
    want, want_lse = softmax_attention(q, K, V)
    labels = rng.integers(0, 4, L)
    parts = [np.nonzero(labels == r)[0] for r in range(4)] + [np.array([], dtype=np.int64)]
    got, got_lse = merge([region_stats(q, K, V, p) for p in parts])
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    assert np.allclose(got_lse, want_lse, rtol=0, atol=1e-12)


def test_rotation_leaves_unquantized_attention_unchanged():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((8, 128))
    K = rng.standard_normal((50, 2, 128)) * 5
    V = rng.standard_normal((50, 2, 128))
    a, _ = softmax_attention(q, K, V)
    b, _ = softmax_attention(rotate_f64(q, 64), rotate_f64(K, 64), V)
    assert np.allclose(a, b, atol=1e-12)


@pytest.fixture(scope="module")
def tiny():
    wl = build_workload(get_config("tiny_1x1024"))
    k, v = seq_kv(wl, 0)
    q = seq_query(wl)
    return wl, bf16_bits(q[0]), bf16_bits(k), bf16_bits(v)


def test_regional_merge_equals_single_pass_on_tiny_workload(tiny):
    wl, q, k, v = tiny
    c = wl.cfg
    cache = quantize_sequence(k, v, c.had_block, c.sink, c.recent)
    a, la = attend(q, cache)
    b, lb = attend_regions(q, cache)
    assert np.allclose(a, b, rtol=0, atol=1e-12)
    assert np.allclose(la, lb, rtol=0, atol=1e-12)


def test_int8_region_is_more_accurate_than_int4(tiny):
    wl, q, k, v = tiny
    c = wl.cfg
    cache = quantize_sequence(k, v, c.had_block, c.sink, c.recent)
    K, V = dequantized_kv(cache)
    from oracle.cache import rotated_keys_f32
    from oracle.quant import dequantize
    yk = rotated_keys_f32(k, c.had_block).astype(np.float64)
    K4 = dequantize(cache.k4, cache.k4_scale, cache.k4_zero)
    e8 = np.abs(K[cache.pos8] - yk[cache.pos8]).mean()
    e4 = np.abs(K4[cache.pos8] - yk[cache.pos8]).mean()
    assert e8 < e4 / 8


def test_quantized_attention_error_vs_unquantized_is_reported(tiny):
    wl, q, k, v = tiny
    c = wl.cfg
    a, _ = attend(q, quantize_sequence(k, v, c.had_block, c.sink, c.recent))
    u, _ = unquantized_attention(q, k, v)
    err = np.abs(a - u).max()
    print(f"tiny workload: max-abs error of INT4/INT8 attention vs unquantized bf16 = {err:.4f}")
    assert err < 2.0
    # the rotated-basis scores equal the unrotated ones: rotation alone changes nothing
    qr = rotated_query(q, c.had_block)
    assert qr.shape == (8, 128)


# ---- causal multi-row attention over the quantized cache (prefill) ----------

def _small_cache(L, H=2, h=16, s=2, w=5, seed=3):
    rng = np.random.default_rng(seed)
    k = torch.from_numpy(rng.standard_normal((L, H, 128)) * 2).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((L, H, 128))).to(torch.bfloat16)
    return quantize_sequence(bf16_bits(k), bf16_bits(v), h, s, w)


def _rows(T, Hq, seed=4):
    rng = np.random.default_rng(seed)
    return bf16_bits(torch.from_numpy(rng.standard_normal((T, Hq, 128))).to(torch.bfloat16))


def test_prefill_last_row_is_decode_attention():
    cache = _small_cache(37)
    q = _rows(6, 4)
    out, lse = prefill_attend(q, cache)
    d_out, d_lse = attend(q[-1], cache)
    assert np.array_equal(out[-1], d_out) and np.array_equal(lse[-1], d_lse)


def test_prefill_rows_match_brute_force():
    """Pure-Python causal softmax per row over the dequantized cache."""
    cache = _small_cache(11, H=1, h=4, s=1, w=3)
    q = _rows(4, 2)
    out, _ = prefill_attend(q, cache)
    K, V = dequantized_kv(cache)
    for t in range(4):
        p = cache.L - 4 + t
        qr = rotated_query(q[t], cache.h)
        ref = _brute(qr.tolist(), K[:p + 1].tolist(), V[:p + 1].tolist())
        assert np.allclose(out[t], ref, rtol=0, atol=1e-12)


def test_prefill_matches_torch_causal_sdpa_fp64():
    """Library routine: fp64 scaled_dot_product_attention with the causal mask of
    rows at positions L - T .. L - 1 over keys 0 .. L - 1."""
    L, T, Hq, Hkv = 70, 20, 8, 2
    cache = _small_cache(L, H=Hkv, h=128, s=4, w=16)
    q = _rows(T, Hq)
    out, _ = prefill_attend(q, cache)
    K, V = dequantized_kv(cache)
    qr = np.stack([rotated_query(q[t], cache.h) for t in range(T)])      # [T, Hq, d]
    g = Hq // Hkv
    tq = torch.from_numpy(qr).permute(1, 0, 2)                              # [Hq, T, d]
    tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(g, 0)       # [Hq, L, d]
    tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(g, 0)
    mask = torch.arange(L)[None, :] <= (L - T + torch.arange(T))[:, None]   # [T, L]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask)
    assert np.allclose(out, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def test_prefill_of_a_whole_sequence_starts_with_the_first_value():
    """T = L: row 0 sees only position 0, so its output is the dequantized v_0."""
    cache = _small_cache(9, H=2, h=8, s=1, w=2)
    q = _rows(9, 4)
    out, lse = prefill_attend(q, cache)
    _, V = dequantized_kv(cache)
    assert np.array_equal(out[0], np.repeat(V[0], 2, axis=0))
    with pytest.raises(ValueError):
        prefill_attend(_rows(10, 4), cache)


@pytest.mark.parametrize("h,seed", [(128, 11), (16, 12), (1, 13)])
def test_attend_with_int8_everywhere_is_within_the_round_trip_bound_of_unquantized(h, seed):
    """End-to-end pin of `attend` (rotation of the query, which cache holds each
    position, 1/sqrt(d), the softmax) against plain attention over the raw bf16
    keys and values, with a bound built from the INT8 round trip alone.

    With every position in the INT8 window (s + w >= L) each dequantized key
    element differs from the exactly rotated key by at most scale/2 (plus the
    fp32 rotation's own error), each value element by scale/2.  If the scores
    move by delta_i, the softmax weights move by at most exp(spread) - 1 in l1
    (spread = max delta - min delta), so each output element moves by at most
    max |v^ - v| + (exp(spread) - 1) * (half the range of that value dim).  The
    deltas are computed here from the oracle's dequantized keys and a query
    rotated by scipy's Hadamard matrix, and checked against the round-trip
    bound before use.  On outlier-free N(0, 1) inputs the bound stays below 0.2
    (the error itself is ~3e-3), while a composition mistake moves the output by
    more: an unrotated query by 0.35-0.4 on these seeds."""
    from scipy.linalg import hadamard

    L, Hkv, g, d = 300, 2, 4, 128
    rng = np.random.default_rng(seed)
    bf = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    k = bf(rng.standard_normal((L, Hkv, d)))
    v = bf(rng.standard_normal((L, Hkv, d)))
    q = bf(rng.standard_normal((Hkv * g, d)))
    kb, vb, qb = bf16_bits(k), bf16_bits(v), bf16_bits(q)
    oc = quantize_sequence(kb, vb, h, 4, 4096)
    assert len(oc.pos8) == L
    out, _ = attend(qb, oc)
    ref, _ = unquantized_attention(qb, kb, vb)

    Hm = np.kron(np.eye(d // h), hadamard(h)) / np.sqrt(h)
    kf = k.to(torch.float64).numpy()
    vf = v.to(torch.float64).numpy()
    qf = q.to(torch.float64).numpy()
    y = kf @ Hm.T                        # exactly rotated keys [L, Hkv, d]
    qt = qf @ Hm.T
    K, V = dequantized_kv(oc)
    # the INT8 round trip: |K^ - y| <= scale/2 + fp32 rotation error, |V^ - v| <= scale/2
    sk = f16_bits_to_f64(oc.k8_scale)[..., None]
    sv = f16_bits_to_f64(oc.v8_scale)[..., None]
    ek = np.abs(K - y)
    ev = np.abs(V - vf)
    assert np.all(ek <= sk / 2 + 1e-5 * np.maximum(1, np.linalg.norm(kf, axis=-1, keepdims=True)))
    assert np.all(ev <= sv / 2 * (1 + 1e-9))
    worst, worst_bound = 0.0, 0.0
    for j in range(Hkv * g):
        kv = j // g
        delta = (K[:, kv] @ qt[j] - kf[:, kv] @ qf[j]) / np.sqrt(d)
        assert np.all(np.abs(delta) <= np.abs(qt[j]) @ ek[:, kv].T / np.sqrt(d) + 1e-9)
        spread = delta.max() - delta.min()
        half = (vf[:, kv].max(axis=0) - vf[:, kv].min(axis=0)) / 2
        bound = ev[:, kv].max(axis=0) + np.expm1(spread) * half
        err = np.abs(out[j] - ref[j])
        assert np.all(err <= bound * (1 + 1e-9) + 1e-12), (j, float(err.max()), float(bound.max()))
        worst = max(worst, float(err.max()))
        worst_bound = max(worst_bound, float(bound.max()))
    assert worst_bound < 0.2, worst_bound


@pytest.mark.parametrize("h", [4, 16, 128])
def test_attend_equals_brute_force_composition(h):
    """`attend` = brute-force softmax (pure-Python loops) of the query rotated by
    scipy's Sylvester Hadamard matrix against the dequantized cache, INT4 and
    INT8 regions both present (s = 2, w = 5, L = 23)."""
    from scipy.linalg import hadamard
    L, Hkv, g, d = 23, 2, 2, 128
    rng = np.random.default_rng(40 + h)
    bf = lambda x: torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16)
    kb = bf16_bits(bf(rng.standard_normal((L, Hkv, d))))
    vb = bf16_bits(bf(rng.standard_normal((L, Hkv, d))))
    q = bf(rng.standard_normal((Hkv * g, d)))
    oc = quantize_sequence(kb, vb, h, 2, 5)
    out, _ = attend(bf16_bits(q), oc)
    Hm = np.kron(np.eye(d // h), hadamard(h)) / np.sqrt(h)
    qt = q.to(torch.float64).numpy() @ Hm.T
    K, V = dequantized_kv(oc)
    ref = _brute(qt.tolist(), K.tolist(), V.tolist())
    assert np.abs(out - ref).max() < 1e-12


def test_unquantized_attention_matches_torch_bf16_sdpa():
    """Plain attention over the raw bf16 tensors: torch converts the bf16 tensors
    itself (not the oracle's bit conversion) and runs fp64 SDPA with the grouped
    heads repeated; a rotated or quantized path would move the result by far more."""
    rng = np.random.default_rng(11)
    Hq, Hkv, L, d = 8, 2, 257, 128
    q = torch.from_numpy(rng.standard_normal((Hq, d)).astype(np.float32)).to(torch.bfloat16)
    k = torch.from_numpy((rng.standard_normal((L, Hkv, d)) * 2).astype(np.float32)).to(torch.bfloat16)
    v = torch.from_numpy(rng.standard_normal((L, Hkv, d)).astype(np.float32)).to(torch.bfloat16)
    out, lse = unquantized_attention(bf16_bits(q), bf16_bits(k), bf16_bits(v))
    g = Hq // Hkv
    tq = q.to(torch.float64)[:, None, :]
    tk = k.to(torch.float64).permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
    tv = v.to(torch.float64).permute(1, 0, 2).repeat_interleave(g, 0).contiguous()
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[:, 0, :].numpy()
    assert np.allclose(out, ref, rtol=0, atol=1e-12)
    z = torch.einsum("hld,hd->hl", tk, tq[:, 0, :]) / math.sqrt(d)
    assert np.allclose(lse, torch.logsumexp(z, dim=1).numpy(), rtol=0, atol=1e-12)
    # the rotated query against unrotated keys is a different function
    out_rot, _ = unquantized_attention(bf16_bits(torch.from_numpy(rotated_query(bf16_bits(q), 128))
                                                 .to(torch.bfloat16)), bf16_bits(k), bf16_bits(v))
    assert np.abs(out_rot - ref).max() > 1e-2
