"""Shared helpers of the GPU parity tests: build a workload on the device, read
back what the library wrote, and compare it with the oracle."""

from __future__ import annotations

import numpy as np
import torch

from oracle.attention import attend, unquantized_attention
from oracle.cache import quantize_sequence, rotated_keys_f32
from oracle.numerics import bf16_to_f32
from oracle.quant import tie_near
from oracle.regions import ring_entry
from workloads import WorkloadConfig, bf16_bits, build_workload

ATOL = 2e-3


def small_config(lengths, *, Hq=8, Hkv=2, P=16, h=64, s=4, w=32, seed=77, name="small", bits=4):
    return WorkloadConfig(name=name, batch=len(lengths), num_q_heads=Hq, num_kv_heads=Hkv,
                          head_dim=128, lengths="explicit", length_args=tuple(int(x) for x in lengths),
                          page_size=P, had_block=h, sink=s, recent=w, seed=seed, code_bits=bits)


def check_workload_invariants(wl):
    """Host-side checks that every index the kernels will use is in bounds."""
    P = wl.page_size
    for b, L in enumerate(wl.lengths):
        n = (int(L) + P - 1) // P
        row = wl.block_table[wl.slots[b]]
        assert n <= wl.block_table.shape[1]
        assert np.all((row[:n] >= 0) & (row[:n] < max(wl.num_pages, 1)))
    assert np.all((wl.slots >= 0) & (wl.slots < wl.num_slots))


def make_device_workload(cfg, keep=(), gen_device="cpu", prefill=True, poison=False):
    """Build and fill a workload's cache.  poison=True first fills both pools with
    0xFF bytes (fp16 NaN) so that any read of never-written cache bytes shows."""
    from decode_attention_int4_block_amd.harness import DeviceWorkload
    wl = build_workload(cfg)
    check_workload_invariants(wl)
    dw = DeviceWorkload(wl, device="cuda", gen_device=gen_device, keep_host=keep)
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
    bf16 inputs.  Returns dict of mismatch / tie counts; raises on a mismatch
    that is not near a rounding tie."""
    from decode_attention_int4_block_amd.layout import (decode_sub2, decode_sub3, decode_sub4, decode_sub8,
                                                        sub4_index, sub8_index)
    wl = dw.wl
    cfg = wl.cfg
    L = int(wl.lengths[b])
    k, v = dw.host_kv[b]
    kb, vb = bf16_bits(k), bf16_bits(v)
    oc = quantize_sequence(kb, vb, cfg.had_block, cfg.sink, cfg.recent, main_bits=cfg.code_bits)
    qmain = (1 << cfg.code_bits) - 1
    decode_main = {2: decode_sub2, 3: decode_sub3}.get(cfg.code_bits, decode_sub4)
    H = cfg.num_kv_heads
    P = wl.page_size
    slot = int(wl.slots[b])
    pos = np.arange(L) if positions is None else np.asarray(positions, np.int64)
    stats = dict(int4_mismatch=0, int4_ties=0, int8_mismatch=0, int8_ties=0, params_mismatch=0)
    yk = rotated_keys_f32(kb, cfg.had_block)
    yv = bf16_to_f32(vb)
    for hk in range(H):
        pages = wl.block_table[slot, pos // P]
        idx = sub4_index(pages, hk, pos % P, H, P)
        got = decode_main(dw.int4_subblocks(idx), (pos % P) % 16)
        for kind, y, codes, sc, ze in (("k", yk, oc.k4, oc.k4_scale, oc.k4_zero),
                                       ("v", yv, oc.v4, oc.v4_scale, oc.v4_zero)):
            ties = tie_near(y[pos, hk], qmain)
            mism = got[kind] != codes[pos, hk]
            stats["int4_ties"] += int((mism & ties).sum())
            stats["int4_mismatch"] += int((mism & ~ties).sum())
            pm = ~(_f16_eq(got[kind + "_scale"], sc[pos, hk]) & _f16_eq(got[kind + "_zero"], ze[pos, hk]))
            pm &= ~ties.any(axis=1)
            stats["params_mismatch"] += int(pm.sum())
        if len(oc.pos8):
            ent = np.array([ring_entry(int(p), cfg.sink, cfg.recent) for p in oc.pos8])
            nr8 = (cfg.sink + cfg.recent + 15) // 16
            idx8 = sub8_index(np.full(len(ent), slot), hk, ent, H, nr8)
            got8 = decode_sub8(dw.int8_subblocks(idx8), ent % 16)
            for kind, y, codes, sc, ze in (("k", yk, oc.k8, oc.k8_scale, oc.k8_zero),
                                           ("v", yv, oc.v8, oc.v8_scale, oc.v8_zero)):
                ties = tie_near(y[oc.pos8, hk], 255)
                mism = got8[kind] != codes[:, hk]
                stats["int8_ties"] += int((mism & ties).sum())
                stats["int8_mismatch"] += int((mism & ~ties).sum())
                pm = ~(_f16_eq(got8[kind + "_scale"], sc[:, hk]) & _f16_eq(got8[kind + "_zero"], ze[:, hk]))
                pm &= ~ties.any(axis=1)
                stats["params_mismatch"] += int(pm.sum())
    return stats


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
                                                       main_bits=cfg.code_bits))
        assert np.isfinite(out[b]).all() and np.isfinite(lse[b]).all(), f"non-finite output in row {b}"
        worst = max(worst, float(np.abs(out[b] - ref).max()))
        worst_lse = max(worst_lse, float(np.abs(lse[b] - ref_lse).max()))
        if report_unquantized:
            u, _ = unquantized_attention(qb[b], kb, vb)
            worst_unq = max(worst_unq, float(np.abs(out[b] - u).max()))
    return worst, worst_lse, worst_unq
