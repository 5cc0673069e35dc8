"""Shared helpers of the GPU parity tests: build a workload on the device, read
back what the library wrote, and compare it with the oracle."""

from __future__ import annotations

import numpy as np
import torch

from oracle.attention import attend, unquantized_attention
from oracle.cache import quantize_sequence, rotated_keys_f32
from oracle.numerics import bf16_to_f32
from oracle.quant import grouped_tie_flags, tie_flags
from oracle.regions import ring_entry
from workloads import WorkloadConfig, bf16_bits, build_workload

ATOL = 2e-3


def small_config(lengths, *, Hq=8, Hkv=2, P=16, h=64, s=4, w=32, seed=77, name="small", bits=4, key_bits=()):
    return WorkloadConfig(name=name, batch=len(lengths), num_q_heads=Hq, num_kv_heads=Hkv,
                          head_dim=128, lengths="explicit", length_args=tuple(int(x) for x in lengths),
                          page_size=P, had_block=h, sink=s, recent=w, seed=seed, code_bits=bits,
                          key_bits=tuple(key_bits))


def check_workload_invariants(wl):
    """Host-side checks that every index the kernels will use is in bounds."""
    P = wl.page_size
    for b, L in enumerate(wl.lengths):
        n = (int(L) + P - 1) // P
        row = wl.block_table[wl.slots[b]]
        assert n <= wl.block_table.shape[1]
        assert np.all((row[:n] >= 0) & (row[:n] < max(wl.num_pages, 1)))
    assert np.all((wl.slots >= 0) & (wl.slots < wl.num_slots))


def make_device_workload(cfg, keep=(), gen_device="cpu", prefill=True, poison=False, kv_fn=None):
    """Build and fill a workload's cache.  poison=True first fills both pools with
    0xFF bytes (fp16 NaN) so that any read of never-written cache bytes shows.
    kv_fn(b) -> (k, v) replaces the drawn keys and values of row b."""
    from decode_attention_int4_block_amd.harness import DeviceWorkload
    wl = build_workload(cfg)
    check_workload_invariants(wl)
    dw = DeviceWorkload(wl, device="cuda", gen_device=gen_device, keep_host=keep, kv_fn=kv_fn)
    if poison:
        dw.cache.int4_pool.fill_(0xFF)
        dw.cache.int8_pool.fill_(0xFF)
    if prefill:
        dw.prefill()
        dw.append_step()
        torch.cuda.synchronize()
    return dw


def _f16_eq(a, b):
    """fp16 bit patterns equal, with +0 and -0 the same."""
    a = np.asarray(a, np.uint16)
    b = np.asarray(b, np.uint16)
    za = (a & 0x7FFF) == 0
    zb = (b & 0x7FFF) == 0
    return (a == b) | (za & zb)


def compare_cache(dw, b, positions=None):
    """Compare the GPU cache of row b with the oracle's quantization of the same
    bf16 inputs.

    Returns a dict of counts (it raises nothing; `assert_cache_exact` judges it):
    codes and params compared, mismatches, and the mismatches forgiven as
    rounding ties.  A code mismatch is forgiven only where the element's own
    quotient, or its vector's fp32 scale or min, lies within 1e-6 relative of a
    rounding midpoint (oracle.quant.tie_flags); a scale / offset mismatch only
    on the vector flag.  `flagged` counts the elements the gate would forgive,
    mismatched or not, so a test of crafted ties can show it reached them.
    """
    from decode_attention_int4_block_amd.layout import (decode_sub2, decode_sub3, decode_sub4, decode_sub8,
                                                        decode_subg, sub4_index, sub8_index)
    wl = dw.wl
    cfg = wl.cfg
    L = int(wl.lengths[b])
    k, v = dw.host_kv[b]
    kb, vb = bf16_bits(k), bf16_bits(v)
    key_bits = tuple(cfg.key_bits) or None
    oc = quantize_sequence(kb, vb, cfg.had_block, cfg.sink, cfg.recent, main_bits=cfg.code_bits, key_bits=key_bits)
    qmain = (1 << cfg.code_bits) - 1
    decode_main = {2: decode_sub2, 3: decode_sub3}.get(cfg.code_bits, decode_sub4)
    if key_bits:
        def decode_main(blocks, tok):
            return decode_subg(blocks, tok, key_bits, cfg.code_bits)
    H = cfg.num_kv_heads
    P = wl.page_size
    slot = int(wl.slots[b])
    pos = np.arange(L) if positions is None else np.asarray(positions, np.int64)
    stats = dict(codes=0, int4_mismatch=0, int4_ties=0, int8_mismatch=0, int8_ties=0,
                 params=0, params_mismatch=0, params_ties=0, flagged=0)
    yk = rotated_keys_f32(kb, cfg.had_block)
    yv = bf16_to_f32(vb)

    def judge(tag, got, y, codes, qmax):
        el, vec = grouped_tie_flags(y, key_bits) if (tag == "k" and qmax != 255 and key_bits) else tie_flags(y, qmax)
        tie = el | vec[..., None]
        mism = got[tag] != codes
        stats["codes"] += int(mism.size)
        stats["flagged"] += int(tie.sum())
        return mism, tie, vec

    for hk in range(H):
        pages = wl.block_table[slot, pos // P]
        idx = sub4_index(pages, hk, pos % P, H, P)
        got = decode_main(dw.int4_subblocks(idx), (pos % P) % 16)
        for kind, y, codes, sc, ze in (("k", yk, oc.k4, oc.k4_scale, oc.k4_zero),
                                       ("v", yv, oc.v4, oc.v4_scale, oc.v4_zero)):
            mism, tie, vec = judge(kind, got, y[pos, hk], codes[pos, hk], qmain)
            stats["int4_ties"] += int((mism & tie).sum())
            stats["int4_mismatch"] += int((mism & ~tie).sum())
            pm = ~(_f16_eq(got[kind + "_scale"], sc[pos, hk]) & _f16_eq(got[kind + "_zero"], ze[pos, hk]))
            stats["params"] += int(pm.size)
            stats["params_ties"] += int((pm & vec).sum())
            stats["params_mismatch"] += int((pm & ~vec).sum())
        if len(oc.pos8):
            ent = np.array([ring_entry(int(p), cfg.sink, cfg.recent) for p in oc.pos8])
            nr8 = (cfg.sink + cfg.recent + 15) // 16
            idx8 = sub8_index(np.full(len(ent), slot), hk, ent, H, nr8)
            got8 = decode_sub8(dw.int8_subblocks(idx8), ent % 16)
            for kind, y, codes, sc, ze in (("k", yk, oc.k8, oc.k8_scale, oc.k8_zero),
                                           ("v", yv, oc.v8, oc.v8_scale, oc.v8_zero)):
                mism, tie, vec = judge(kind, got8, y[oc.pos8, hk], codes[:, hk], 255)
                stats["int8_ties"] += int((mism & tie).sum())
                stats["int8_mismatch"] += int((mism & ~tie).sum())
                pm = ~(_f16_eq(got8[kind + "_scale"], sc[:, hk]) & _f16_eq(got8[kind + "_zero"], ze[:, hk]))
                stats["params"] += int(pm.size)
                stats["params_ties"] += int((pm & vec).sum())
                stats["params_mismatch"] += int((pm & ~vec).sum())
    return stats


def add_stats(tot, st):
    for k, v in st.items():
        tot[k] = tot.get(k, 0) + v
    return tot


# Mismatches the tie gate may forgive.  Both sides take every rounding decision
# in the same fp32 / fp16 arithmetic in the same order, so the expected count is
# 0; the gate covers an evaluation-order difference at a tie and nothing more.
# At most 1 forgiven code per 1e5 compared, 1 forgiven (scale, offset) pair per
# 1e4 (the vector flag's own rate is ~0.5%, see the oracle's pins).
TIE_CODE_RATE = 1e-5
TIE_PARAM_RATE = 1e-4


def assert_cache_exact(st):
    """Codes, scales and offsets bit-exact; forgiven ties counted and bounded."""
    assert st["int4_mismatch"] == 0 and st["int8_mismatch"] == 0 and st["params_mismatch"] == 0, st
    forgiven = st["int4_ties"] + st["int8_ties"]
    assert forgiven <= TIE_CODE_RATE * max(st["codes"], 1), st
    assert st["params_ties"] <= TIE_PARAM_RATE * max(st["params"], 1), st


def compare_attention(dw, rows, report_unquantized=False):
    """Max-abs error of GPU decode output vs the oracle's fp64 attention for rows."""
    wl = dw.wl
    cfg = wl.cfg
    out = dw.out.cpu().numpy()
    lse = dw.lse.cpu().numpy()
    qb = bf16_bits(dw.q)
    worst, worst_lse, worst_unq = 0.0, 0.0, 0.0
    for b in rows:
        L = int(wl.lengths[b])
        if L == 0:
            assert np.all(out[b] == 0) and np.all(np.isneginf(lse[b]))
            continue
        k, v = dw.host_kv[b]
        kb, vb = bf16_bits(k), bf16_bits(v)
        ref, ref_lse = attend(qb[b], quantize_sequence(kb, vb, cfg.had_block, cfg.sink, cfg.recent,
                                                       main_bits=cfg.code_bits, key_bits=tuple(cfg.key_bits) or None))
        assert np.isfinite(out[b]).all() and np.isfinite(lse[b]).all(), f"non-finite output in row {b}"
        worst = max(worst, float(np.abs(out[b] - ref).max()))
        worst_lse = max(worst_lse, float(np.abs(lse[b] - ref_lse).max()))
        if report_unquantized:
            u, _ = unquantized_attention(qb[b], kb, vb)
            worst_unq = max(worst_unq, float(np.abs(out[b] - u).max()))
    return worst, worst_lse, worst_unq


def attention_error_scaled(dw, rows):
    """Worst |GPU - oracle| / max(1, v_max / 256) over the rows (outputs and lse),
    for crafted rows whose values reach 6e4: fp32 sums of values that large carry
    absolute errors above 2e-3, so the bound is relative to their magnitude."""
    from oracle.cache import dequantized_kv
    cfg = dw.cfg
    out = dw.out.cpu().numpy()
    lse = dw.lse.cpu().numpy()
    qb = bf16_bits(dw.q)
    worst = 0.0
    for b in rows:
        k, v = dw.host_kv[b]
        oc = quantize_sequence(bf16_bits(k), bf16_bits(v), cfg.had_block, cfg.sink, cfg.recent,
                               main_bits=cfg.code_bits, key_bits=tuple(cfg.key_bits) or None)
        ref, ref_lse = attend(qb[b], oc)
        assert np.isfinite(out[b]).all() and np.isfinite(lse[b]).all(), f"non-finite output in row {b}"
        _, V = dequantized_kv(oc)
        scale = max(1.0, float(np.abs(V).max()) / 256.0)
        worst = max(worst, float(np.abs(out[b] - ref).max()) / scale, float(np.abs(lse[b] - ref_lse).max()))
    return worst
