"""Benchmark: one decode step of INT4/INT8 KV-cache quantize-append + decode attention.

A step is the whole hot path over one batch: quantize-append of one new token
per row followed by decode attention over the quantized cache.  By default it
is one fused launch (kv_append_decode_attn); --path two-launch times
kv_quant_append followed by kv_decode_attn instead (same bytes written, same
outputs).  The workload is the Qwen3-8B-shaped async-rollout
batch (256 slots, 32 query / 8 KV heads, Pareto(1.5) lengths from 512 clipped
at 32K, 16-token pages, h = 128, s = 4, w = 128), with inputs resident in HBM.

The steps cycle through `--layers` independent copies of the cache, as the
layers of a model would, so the working set (~0.43 GB per copy) exceeds the
256 MB Infinity Cache and each step streams its cache from HBM.

Prints one JSON line (see the fields at the end of main()).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "decode-attn effective KV GB/s + tokens·heads/s; % of MI355X HBM peak"
HBM_PEAK_GBPS = 8000.0
BYTES_INT4 = 136     # K+V codes + fp16 scale/zero of one (token, KV head), INT4
BYTES_INT8 = 264     # same, INT8
BYTES_INT2 = 72      # same, 2-bit main cache
BYTES_INT3 = 104     # same, 3-bit main cache


def region_sizes(L, s, w):
    L = np.asarray(L, np.int64)
    n8 = np.minimum(L, s + w)
    n4 = np.maximum(L - w - s, 0)
    return n4, n8


def decode_bytes(wl):
    """Algorithmic bytes one decode-attention launch must move."""
    c = wl.cfg
    n4, n8 = region_sizes(wl.lengths, c.sink, c.recent)
    main = {2: BYTES_INT2, 3: BYTES_INT3}.get(c.code_bits, BYTES_INT4)
    if c.key_bits:
        # keys with a width per RoPE-block group: 32 dims per group at its width
        # plus fp16 scale / offset, values at code_bits
        main = 4 * sum(c.key_bits) + 4 + 16 * c.code_bits + 4
    kv = int((c.num_kv_heads * (main * n4 + BYTES_INT8 * n8)).sum())
    P = wl.page_size
    lo4, hi4 = c.sink, wl.lengths - c.recent
    pages = np.where(hi4 > lo4, (hi4 + P - 1) // P - lo4 // P, 0)
    bt = int(4 * pages.sum())
    q = c.batch * c.num_q_heads * c.head_dim * 2
    out = c.batch * c.num_q_heads * (c.head_dim + 1) * 4
    meta = c.batch * 8
    return dict(kv=kv, total=kv + bt + q + out + meta, bf16_equiv=int((wl.lengths * c.num_kv_heads * 512).sum()))


def append_bytes(wl):
    c = wl.cfg
    n = int((wl.lengths >= 1).sum())
    ins = n * c.num_kv_heads * c.head_dim * 2 * 2
    # every appended token is written to INT4; the step token is always in the recent window
    outs = n * c.num_kv_heads * (BYTES_INT4 + (BYTES_INT8 if c.sink + c.recent > 0 else 0))
    return ins + outs


def host_facts():
    """The host the CPU baseline ran on."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    mem_gb = None
    try:
        for line in open("/proc/meminfo"):
            if line.startswith("MemTotal"):
                mem_gb = round(int(line.split()[1]) / 2 ** 20, 1)
                break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": model,
            "mem_gib": mem_gb}


def _oracle_worker(name, rows, q_bits, barrier, results):
    """One CPU-baseline process: draw its rows' inputs, wait for the others, then
    run the oracle's decode step (quantization of the row + fp64 attention) on
    each row with single-threaded BLAS; report its timed span."""
    import torch
    from threadpoolctl import threadpool_limits

    from oracle.attention import attend
    from oracle.cache import quantize_sequence
    from workloads import bf16_bits, build_workload, get_config, seq_kv

    torch.set_num_threads(1)
    cfg = get_config(name)
    wl = build_workload(cfg)
    inputs = []
    for b in rows:
        k, v = seq_kv(wl, b, device="cpu")
        inputs.append((b, bf16_bits(k), bf16_bits(v)))
    barrier.wait()
    kvbytes, tok_heads = 0, 0
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for b, kb, vb in inputs:
            attend(q_bits[b], quantize_sequence(kb, vb, cfg.had_block, cfg.sink, cfg.recent))
            L = int(wl.lengths[b])
            n4, n8 = region_sizes([L], cfg.sink, cfg.recent)
            kvbytes += int(cfg.num_kv_heads * (BYTES_INT4 * n4[0] + BYTES_INT8 * n8[0]))
            tok_heads += L * cfg.num_q_heads
        dt = time.perf_counter() - t0
    results.put((dt, kvbytes, tok_heads, len(inputs)))


def cpu_baseline(wl, dw, passes=None, max_procs=16):
    """The oracle as it stands on the host's cores: one process per core (at most
    max_procs), each running the oracle's decode step on its share of the rows
    with single-threaded BLAS.  The rows of the workload are dealt out in a
    seeded order, `passes` times over, so that the sample holds about 10-30 s of
    CPU work; the rate is the processed KV bytes over the slowest process's span.
    """
    import multiprocessing as mp

    c = wl.cfg
    nproc = max(1, min(max_procs, len(os.sched_getaffinity(0))))
    if passes is None:
        # one pass over the rows is 8-60 s of CPU on these hosts at the Qwen3
        # batch's lengths; small batches get more passes
        est = 0.032 * float(wl.lengths.mean()) / 1403.0 * c.batch
        passes = int(max(1, min(8, round(10.0 / max(est, 1e-3)))))
    order = np.concatenate([np.random.default_rng(12345 + i).permutation(c.batch) for i in range(passes)])
    shares = [order[i::nproc].tolist() for i in range(nproc)]
    from workloads import bf16_bits
    qb = bf16_bits(dw.q)
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(nproc)
    results = ctx.Queue()
    procs = [ctx.Process(target=_oracle_worker, args=(c.name, sh, qb, barrier, results)) for sh in shares]
    for p in procs:
        p.start()
    out = [results.get(timeout=600) for _ in procs]
    for p in procs:
        p.join(timeout=60)
    span = max(o[0] for o in out)
    cpu_s = sum(o[0] for o in out)
    kvbytes = sum(o[1] for o in out)
    tok_heads = sum(o[2] for o in out)
    nrows = sum(o[3] for o in out)
    return dict(value=round(kvbytes / span / 1e9, 4), unit="GB/s", cores=nproc, kind="oracle",
                tokens_heads_per_s=round(tok_heads / span, 1), host=host_facts(),
                sample=f"{nrows} row decode steps ({passes} pass(es) over the {c.batch} rows in seeded order), "
                       f"each the oracle's quantization of the row + fp64 attention, dealt to {nproc} processes "
                       f"of one thread each: {cpu_s:.1f} s of CPU in {span:.1f} s")


KERNEL_SOURCES = ("decode.hip", "common.h", "quant.h", "lanes.h", "tiles.h")
MFMA_F16_PEAK_TFLOPS = 2500.0   # MI355X dense fp16 MFMA


def decode_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, "decode_attention_int4_block_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def traffic_from_profile(entry, workload):
    """HBM bytes per launch of an entry point from the committed FETCH_SIZE /
    WRITE_SIZE counter runs, or None when they were taken on other kernel sources."""
    p = os.path.join(ROOT, "profiles", f"{entry}_{workload}_traffic.json")
    if not os.path.exists(p):
        return None
    d = json.load(open(p))
    if d.get("source_sha256") != decode_source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def device_copy_rate(torch, calibration=False, nbytes=1 << 30, reps=5):
    """Bytes read + written per second by the runtime's device-to-device copy of
    1 GiB: a measured ceiling for streaming kernels on this device, as context.
    With calibration=True, one 256 MiB copy runs first (its counters calibrate
    the HBM traffic figures)."""
    if calibration:
        a = torch.ones(256 << 20, dtype=torch.uint8, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    a = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    sec = e0.elapsed_time(e1) / 1e3 / reps
    del a, b
    return round(2 * nbytes / sec / 1e9, 1)


# Protection-budget and rotation variants the KV4-RL page compares against
# ("Main Findings": KV8, KV4 without a side cache, the 16/128 sink/recent split of a
# 144-position budget and its all-sink / all-recent ablations) and the SAW-INT4
# page's naive INT4 (no rotation, h = 1).  Same lengths, seeds and kernels.
def budget_variants(cfg, max_len):
    return [
        ("workload (s=%d, w=%d, h=%d)" % (cfg.sink, cfg.recent, cfg.had_block), {}),
        ("KV4 only (s=0, w=0)", dict(sink=0, recent=0)),
        ("naive INT4 (h=1)", dict(had_block=1)),
        ("budget 16/128", dict(sink=16, recent=128)),
        ("budget 144/0 (all sink)", dict(sink=144, recent=0)),
        ("budget 0/144 (all recent)", dict(sink=0, recent=144)),
        ("KV8 everywhere (s+w >= L)", dict(sink=cfg.sink, recent=max(max_len - cfg.sink, cfg.recent))),
        ("K3V3: 3-bit main cache (s=%d, w=%d)" % (cfg.sink, cfg.recent), dict(code_bits=3)),
        ("K2V2: 2-bit main cache (s=%d, w=%d)" % (cfg.sink, cfg.recent), dict(code_bits=2)),
        ("K(4,3,3,2)V3: key widths per RoPE-block group, h=8 (the bytes of K3V3)",
         dict(code_bits=3, key_bits=(4, 3, 3, 2), had_block=8)),
    ]


def measure_variants(torch, cfg, steps, warmup, only=None):
    """Decode and append time of each budget variant, caches rotated like the main
    measurement (one copy when a copy alone is far beyond the 256 MB Infinity Cache)."""
    from decode_attention_int4_block_amd import QuantKVCache
    from decode_attention_int4_block_amd.harness import DeviceWorkload
    from workloads import build_workload

    base = build_workload(cfg)
    res = []
    for tag, kw in budget_variants(cfg, int(base.lengths.max())):
        if only is not None and not tag.startswith(only):
            continue
        vcfg = cfg.scaled(**kw)
        wl = build_workload(vcfg)
        dw = DeviceWorkload(wl, device="cuda", gen_device="cuda")
        dw.prefill()
        db = decode_bytes(wl)
        copies = [dw.cache]
        if db["total"] < (2 << 30):
            for _ in range(3):
                c2 = QuantKVCache(vcfg.num_kv_heads, wl.page_size, max(wl.num_pages, 1), wl.num_slots,
                                  vcfg.had_block, vcfg.sink, vcfg.recent, code_bits=vcfg.code_bits,
                                  key_bits=vcfg.key_bits or None)
                c2.int4_pool.copy_(dw.cache.int4_pool)
                c2.int8_pool.copy_(dw.cache.int8_pool)
                copies.append(c2)
        def two_launch(i):
            dw.cache = copies[i % len(copies)]
            dw.append_step()
            dw.decode_step()
        prewarm(torch, two_launch, sync=False)
        torch.cuda._sleep(SPIN_CYCLES)
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
        for i in range(warmup + steps):
            dw.cache = copies[i % len(copies)]
            ev = evs[i - warmup] if i >= warmup else None
            if ev:
                ev[0].record()
            dw.append_step()
            if ev:
                ev[1].record()
            dw.decode_step()
            if ev:
                ev[2].record()
        # the fused launch does not serve grouped key widths
        fev = [] if vcfg.key_bits else [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for i in range(len(fev)):
            dw.cache = copies[i % len(copies)]
            fev[i][0].record()
            dw.fused_step()
            fev[i][1].record()
        torch.cuda.synchronize()
        dec = np.array([e[1].elapsed_time(e[2]) for e in evs]) * 1e3
        app = np.array([e[0].elapsed_time(e[1]) for e in evs]) * 1e3
        fus = np.array([e[0].elapsed_time(e[1]) for e in fev]) * 1e3 if fev else None
        us = float(np.median(dec))
        res.append(dict(variant=tag, sink=vcfg.sink, recent=vcfg.recent, had_block=vcfg.had_block,
                        code_bits=vcfg.code_bits, key_bits=list(vcfg.key_bits) or None,
                        decode_algorithmic_bytes=db["total"], decode_us=round(us, 2),
                        append_us=round(float(np.median(app)), 2),
                        fused_us=round(float(np.median(fus)), 2) if fus is not None else None,
                        GBps=round(db["total"] / us / 1e3, 1), hbm_frac=round(db["total"] / us / 1e3 / HBM_PEAK_GBPS, 4)))
        print(f"[bench] variant {tag}: decode {us:.1f} us, {db['total'] / 1e6:.1f} MB", file=sys.stderr, flush=True)
        del dw, copies
        torch.cuda.empty_cache()
    return res


# The pages' own figures for this path, with their hardware: context only (other
# machines, other precisions, relative measures), never a target.
PAGES_CONTEXT = [
    {"figure": "1.34x faster than fp16 FlashAttention2 at 128K context", "hardware": "one NVIDIA H800",
     "what": "packed K3V3 cache (3-bit keys and values), Qwen2.5-3B-Instruct",
     "page": "RoPE-Aware Bit Allocation for KV-Cache Quantization (Block-GTQ), Abstract",
     "here": "long_128k: same heads and context, K4V4 and K3V3 decode timed in `workloads`"},
    {"figure": "4.52x growth of the mean decode-step latency under asynchronous rollout", "hardware": "NVIDIA H200",
     "what": "BF16 KV, Qwen3-4B-Base, iteration-300 trace (KV concentration)",
     "page": "KV4-RL, Main Findings",
     "here": "qwen3_8b_async_256 is the heavy async step this measures"},
]

OTHER_WORKLOADS = ("tiny_1x1024", "qwen3_4b_b64", "long_128k", "refill_512")


def unquantized_error(torch, dw, rows):
    """Max |GPU out - softmax(q k^T / sqrt(d)) v| over sampled rows, the reference
    in fp64 on the host from the same bf16 q, k, v (no rotation, no
    quantization): the quantization's own error, reported, not bounded."""
    from workloads import seq_kv
    cfg = dw.cfg
    g = cfg.num_q_heads // cfg.num_kv_heads
    out = dw.out.cpu().to(torch.float64)
    worst = 0.0
    for b in rows:
        if int(dw.wl.lengths[b]) == 0:
            continue
        k, v = seq_kv(dw.wl, b, device="cuda")
        k = k.cpu().to(torch.float64)                      # [L, Hkv, d]
        v = v.cpu().to(torch.float64)
        q = dw.q[b].cpu().to(torch.float64)                # [Hq, d]
        for j in range(cfg.num_q_heads):
            z = k[:, j // g, :] @ q[j] / float(cfg.head_dim) ** 0.5
            p = torch.softmax(z, dim=0)
            ref = p @ v[:, j // g, :]
            worst = max(worst, float((out[b, j] - ref).abs().max()))
    return worst


def _copies_for(nbytes):
    """Cache copies cycled between steps so that the working set exceeds the
    256 MB Infinity Cache (at most 16; one when a copy alone exceeds 1 GB)."""
    if nbytes > (1 << 30):
        return 1
    return int(min(16, max(4, -(-(640 << 20) // max(nbytes, 1)))))


# GPU time of back-to-back launches run before each timed measurement.  Measured
# on MI355X (shader clock from s_memtime against the 100 MHz real-time counter):
# after an idle spell the clock sits near 2.16 GHz, the first milliseconds of
# sustained launches run up to 30% slower than the settled rate, and the clock
# settles near 2.38 GHz after 20-30 ms.  A few warm-up steps therefore time the
# ramp, not the rate of a sustained decode loop.
PREWARM_MS = 60.0


# A queued spin kernel of this many shader cycles (~2 ms) ahead of per-launch
# timings: the timed launches queue behind it, so that the events time the
# kernels and not the host's launch rate (a 5-us append is launched slower than
# it runs).
SPIN_CYCLES = 5_000_000


def prewarm(torch, fn, ms=PREWARM_MS, sync=True):
    """Runs fn(i) back to back for about `ms` of GPU time (count from one timed
    launch), waits for it unless sync is False; returns the number of launches."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    fn(0)
    e1.record()
    torch.cuda.synchronize()
    n = int(min(20000, max(1, np.ceil(ms / max(e0.elapsed_time(e1), 1e-3)))))
    for i in range(1, n + 1):
        fn(i)
    if sync:
        torch.cuda.synchronize()
    return n + 1


def time_launches(torch, stream, fn, layers, n, warmup=2):
    """Median and p10 / p90 of n launches of fn(cache) timed one by one with HIP
    events on the launch stream, cycling the cache copies, after the pre-warm."""
    prewarm(torch, lambda i: fn(layers[i % len(layers)]), sync=False)
    for i in range(warmup):
        fn(layers[i % len(layers)])
    torch.cuda._sleep(SPIN_CYCLES)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (e0, e1) in enumerate(evs):
        e0.record(stream)
        fn(layers[i % len(layers)])
        e1.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    return float(np.median(us)), float(np.percentile(us, 10)), float(np.percentile(us, 90))


def measure_workload(torch, name, steps):
    """Decode, fused and append timings of one more workload, with its bytes,
    roofline fractions, rates and the error against unquantized attention."""
    from decode_attention_int4_block_amd import QuantKVCache, kv_decode_read_ceiling
    from decode_attention_int4_block_amd.harness import DeviceWorkload
    from workloads import build_workload, get_config

    cfg = get_config(name)
    wl = build_workload(cfg)
    t0 = time.time()
    dw = DeviceWorkload(wl, device="cuda", gen_device="cuda")
    dw.prefill()
    dw.append_step()
    db = decode_bytes(wl)
    ab = append_bytes(wl)
    layers = [dw.cache]
    for _ in range(_copies_for(db["total"]) - 1):
        c2 = QuantKVCache(cfg.num_kv_heads, wl.page_size, max(wl.num_pages, 1), wl.num_slots,
                          cfg.had_block, cfg.sink, cfg.recent, code_bits=cfg.code_bits)
        c2.int4_pool.copy_(dw.cache.int4_pool)
        c2.int8_pool.copy_(dw.cache.int8_pool)
        layers.append(c2)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def on(cache, f):
        dw.cache = cache
        f()

    dec = time_launches(torch, stream, lambda c: on(c, dw.decode_step), layers, steps)
    fus = time_launches(torch, stream, lambda c: on(c, dw.fused_step), layers, steps)
    app = time_launches(torch, stream, lambda c: on(c, dw.append_step), layers, steps)
    ceil = None
    if cfg.group <= 8:
        ceil = time_launches(torch, stream, lambda c: kv_decode_read_ceiling(
            c, dw.q, dw.slots, dw.block_table, dw.ctx_len, workspace=dw.workspace), layers, steps)
    dw.cache = layers[0]
    dw.fused_step()
    torch.cuda.synchronize()
    rows = sorted(set([0, cfg.batch - 1] + [int(x) for x in np.random.default_rng(7).choice(cfg.batch, 2)]))
    rows = rows[:3]
    err = unquantized_error(torch, dw, rows)
    tok_heads = float((wl.lengths * cfg.num_q_heads).sum())
    rec = {
        "workload": name, "batch": cfg.batch, "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
        "page_size": wl.page_size, "had_block": cfg.had_block, "sink": cfg.sink, "recent": cfg.recent,
        "total_tokens": int(wl.lengths.sum()), "cache_copies": len(layers),
        "decode_algorithmic_bytes": db["total"], "decode_kv_bytes": db["kv"], "append_algorithmic_bytes": ab,
        "decode_us": round(dec[0], 2), "decode_us_p10_p90": [round(dec[1], 2), round(dec[2], 2)],
        "fused_us": round(fus[0], 2), "fused_us_p10_p90": [round(fus[1], 2), round(fus[2], 2)],
        "append_us": round(app[0], 2),
        "decode_GBps": round(db["total"] / dec[0] / 1e3, 1),
        "decode_frac": round(db["total"] / dec[0] / 1e3 / HBM_PEAK_GBPS, 4),
        "fused_GBps": round((db["total"] + ab) / fus[0] / 1e3, 1),
        "fused_frac": round((db["total"] + ab) / fus[0] / 1e3 / HBM_PEAK_GBPS, 4),
        "tokens_heads_per_s_decode": round(tok_heads / (dec[0] * 1e-6), 1),
        "read_ceiling_us": round(ceil[0], 2) if ceil else None,
        "read_ceiling_GBps": round(db["total"] / ceil[0] / 1e3, 1) if ceil else None,
        "bf16_equiv_GBps_decode": round(db["bf16_equiv"] / dec[0] / 1e3, 1),
        "max_abs_vs_unquantized_bf16": round(err, 4), "unquantized_rows": rows,
        "setup_s": round(time.time() - t0, 1),
    }
    print(f"[bench] {name}: decode {dec[0]:.1f} us ({rec['decode_frac'] * 100:.1f}%), fused {fus[0]:.1f} us, "
          f"append {app[0]:.1f} us, ceiling {rec['read_ceiling_us']} us", file=sys.stderr, flush=True)
    del dw, layers
    torch.cuda.empty_cache()
    return rec


PREFILL_WORKLOAD = "prefill_qwen3_8b_8x1024"


def prefill_cpu_baseline(wl, q, T, budget_s=6.0):
    """The oracle's causal multi-row attention on a sample: the last rows of the first
    sequence's chunk, one at a time until ~budget_s, single-threaded BLAS."""
    from threadpoolctl import threadpool_limits

    from oracle.attention import rotated_query, softmax_attention
    from oracle.cache import dequantized_kv, quantize_sequence
    from workloads import bf16_bits, seq_kv

    c = wl.cfg
    L0, T0 = int(wl.lengths[0]), int(T[0])
    qb = bf16_bits(q[:T0])
    with threadpool_limits(limits=1):
        k, v = seq_kv(wl, 0, device="cpu")
        t_q = time.perf_counter()
        cache = quantize_sequence(bf16_bits(k), bf16_bits(v), c.had_block, c.sink, c.recent)
        K, V = dequantized_kv(cache)
        t_quant = time.perf_counter() - t_q
        done, flops, t_att = 0, 0, 0.0
        for t in range(T0 - 1, -1, -1):
            p = L0 - T0 + t
            t0 = time.perf_counter()
            softmax_attention(rotated_query(qb[t], c.had_block), K[:p + 1], V[:p + 1])
            t_att += time.perf_counter() - t0
            done += 1
            flops += (p + 1) * c.num_q_heads * 4 * c.head_dim
            if t_att >= budget_s:
                break
    return dict(value=round(flops / t_att / 1e12, 6), unit="TFLOP/s", cores=1, kind="oracle",
                sample=f"the last {done} of {T0} chunk rows of sequence 0 (L = {L0}), fp64 attention over "
                       f"the oracle's dequantized cache, {t_att:.1f} s, 1 thread (quantizing the sequence "
                       f"took another {t_quant:.1f} s)")


def prefill_sub4bit(torch, steps, warmup):
    """The same re-prefill over the 3- and 2-bit main caches."""
    out = []
    for bits in (3, 2):
        px = measure_prefill(torch, steps=steps, warmup=warmup, code_bits=bits)
        out.append({k: px[k] for k in ("code_bits", "us_mean", "us_p10_p90", "algorithmic_flops", "kv_bytes_unique")}
                   | {"achieved_TFLOPs": px["roofline"]["achieved"], "frac_of_fp16_mfma_peak": px["roofline"]["frac"]})
    return out


def measure_prefill(torch, steps, warmup, cpu=False, code_bits=4):
    """kv_prefill_attn on the re-prefill workload: the last `chunk` positions of each
    sequence attended again as causal query rows over the quantized cache (main
    cache of code_bits 4, 3 or 2)."""
    from decode_attention_int4_block_amd import kv_prefill_attn
    from decode_attention_int4_block_amd.harness import DeviceWorkload
    from workloads import build_workload, chunk_queries, get_config

    cfg = get_config(PREFILL_WORKLOAD)
    if code_bits != 4:
        cfg = cfg.scaled(code_bits=code_bits)
    wl = build_workload(cfg)
    dw = DeviceWorkload(wl, device="cuda", gen_device="cuda")
    dw.prefill(include_step_token=True)
    L = wl.lengths.astype(np.int64)
    T = np.minimum(cfg.extra["chunk"], L)
    q = chunk_queries(wl, T, device="cuda")
    q_start = torch.from_numpy(np.concatenate([[0], np.cumsum(T)]).astype(np.int32)).cuda()
    out = torch.empty((int(T.sum()), cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device="cuda")
    lse = torch.empty((int(T.sum()), cfg.num_q_heads), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def launch():
        kv_prefill_attn(dw.cache, q, q_start, dw.slots, dw.block_table, dw.ctx_len, int(T.max()), out=out, lse=lse)

    prewarm(torch, lambda i: launch())
    for _ in range(warmup):
        launch()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e0, e1 in evs:
        e0.record(stream)
        launch()
        e1.record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    # algorithmic work: 2 * 128 flop for q.k and 2 * 128 for p.v per (row, query head, attended key)
    attended = sum(int((L[b] - T[b] + np.arange(1, T[b] + 1)).sum()) for b in range(cfg.batch))
    flops = attended * cfg.num_q_heads * 4 * cfg.head_dim
    # unique cache bytes the chunks' causal prefixes cover (every position up to L)
    n4, n8 = region_sizes(L, cfg.sink, cfg.recent)
    b_main = {4: BYTES_INT4, 3: BYTES_INT3, 2: BYTES_INT2}[code_bits]
    kv_unique = int((cfg.num_kv_heads * (b_main * n4 + BYTES_INT8 * n8)).sum())
    mean_us = float(us.mean())
    achieved = flops / (mean_us * 1e-6) / 1e12
    rec = {
        "workload": cfg.name, "code_bits": code_bits, "sequences": cfg.batch, "chunk_rows": [int(x) for x in T],
        "lengths": [int(x) for x in L], "num_q_heads": cfg.num_q_heads, "num_kv_heads": cfg.num_kv_heads,
        "had_block": cfg.had_block, "sink": cfg.sink, "recent": cfg.recent, "page_size": wl.page_size,
        "launches": steps, "us_mean": round(mean_us, 2),
        "us_p10_p90": [round(float(np.percentile(us, 10)), 2), round(float(np.percentile(us, 90)), 2)],
        "algorithmic_flops": flops, "attended_row_key_pairs_per_q_head": attended,
        "kv_bytes_unique": kv_unique,
        "roofline": {"bound": "mfma", "kernel": "prefill_kernel (kv_prefill_attn)",
                     "achieved": round(achieved, 2), "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4), "traffic": None,
                     "note": "fp16 MFMA peak; each product runs as f16 hi + lo, so the MFMAs issue twice the algorithmic flops"},
    }
    if cpu:
        rec["cpu_baseline"] = prefill_cpu_baseline(wl, q.cpu(), T)
    print(f"[bench] prefill {cfg.name} ({code_bits}-bit): {mean_us:.1f} us, {achieved:.1f} TFLOP/s", file=sys.stderr,
          flush=True)
    del dw, q, out, lse
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen3_8b_async_256")
    ap.add_argument("--layers", type=int, default=4)
    ap.add_argument("--path", choices=["fused", "two-launch"], default="fused",
                    help="the timed step: one kv_append_decode_attn launch, or kv_quant_append + kv_decode_attn")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--variants", action="store_true",
                    help="also time the protection-budget / rotation variants (s, w, h) on the same lengths")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the per-launch records of the other four workloads")
    ap.add_argument("--no-sub4bit", action="store_true",
                    help="skip the decode measurements with the 3- and 2-bit main caches (K3V3, K2V2)")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the kv_prefill_attn measurement on the re-prefill workload")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the kv_prefill_attn measurement (for counter runs of the prefill kernel)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="before warm-up, run one untimed 256 MiB device-to-device copy whose "
                         "FETCH_SIZE / WRITE_SIZE counters scale the decode kernel's")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); "
              "the path is data-parallel over decode rows and is not run across GPUs here.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from decode_attention_int4_block_amd.harness import DeviceWorkload
    from workloads import build_workload, get_config

    if args.prefill_only:
        pf = measure_prefill(torch, steps=args.steps, warmup=args.warmup, cpu=False)
        if not args.no_sub4bit:
            pf["sub4bit"] = prefill_sub4bit(torch, steps=args.steps, warmup=args.warmup)
        print(json.dumps({"prefill": pf}), flush=True)
        return

    cfg = get_config(args.workload)
    wl = build_workload(cfg)
    print(f"[bench] workload {cfg.name}: B={cfg.batch} tokens={int(wl.lengths.sum())} "
          f"max_len={wl.max_len}", file=sys.stderr, flush=True)
    t0 = time.time()
    dw = DeviceWorkload(wl, device="cuda", gen_device="cuda")
    dw.prefill()
    # independent copies of the cache for the rotating "layers"
    layers = [dw.cache]
    from decode_attention_int4_block_amd import QuantKVCache
    for _ in range(args.layers - 1):
        c2 = QuantKVCache(cfg.num_kv_heads, wl.page_size, max(wl.num_pages, 1), wl.num_slots,
                          cfg.had_block, cfg.sink, cfg.recent, code_bits=cfg.code_bits)
        c2.int4_pool.copy_(dw.cache.int4_pool)
        c2.int8_pool.copy_(dw.cache.int8_pool)
        layers.append(c2)
    torch.cuda.synchronize()
    print(f"[bench] prefill + {args.layers} cache copies in {time.time() - t0:.1f} s", file=sys.stderr, flush=True)

    fused = args.path == "fused"

    def step(i, path=None):
        dw.cache = layers[i % len(layers)]
        if (path or args.path) == "fused":
            dw.fused_step()
        else:
            dw.append_step()
            dw.decode_step()

    copy_gbps = device_copy_rate(torch, calibration=args.calibration_copy)
    prewarm_launches = prewarm(torch, lambda i: step(i))
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: K steps back to back, HIP events (on the stream the kernels
    # run on) only at its two ends so that no marker sits between launches
    stream = torch.cuda.current_stream()
    ev_start, ev_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    ev_start.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / args.steps
    step_gpu_ms = ev_start.elapsed_time(ev_end) / args.steps

    # untimed breakdown passes: each launch of the two-launch path between
    # events, and the fused launch between events, queued behind a spin kernel
    torch.cuda._sleep(SPIN_CYCLES)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        dw.cache = layers[i % len(layers)]
        evs[i][0].record(stream)
        dw.append_step()
        evs[i][1].record(stream)
        dw.decode_step()
        evs[i][2].record(stream)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    for i in range(args.steps):
        dw.cache = layers[i % len(layers)]
        fev[i][0].record(stream)
        dw.fused_step()
        fev[i][1].record(stream)
    torch.cuda.synchronize()
    from decode_attention_int4_block_amd import kv_decode_read_ceiling
    ceil_us = time_launches(torch, stream, lambda c: kv_decode_read_ceiling(
        c, dw.q, dw.slots, dw.block_table, dw.ctx_len, workspace=dw.workspace), layers, args.steps)
    app_ms = np.array([e[0].elapsed_time(e[1]) for e in evs])
    dec_ms = np.array([e[1].elapsed_time(e[2]) for e in evs])
    fus_ms = np.array([e[0].elapsed_time(e[1]) for e in fev])

    db = decode_bytes(wl)
    ab = append_bytes(wl)
    tok_heads = float((wl.lengths * cfg.num_q_heads).sum())
    step_s = ms_per_step / 1e3
    value = db["kv"] / step_s / 1e9
    dec_avg_s = float(dec_ms.mean()) / 1e3
    if fused:
        # the fused launch moves the decode bytes and the append bytes; its
        # duration is the timed region's event span per step
        kernel = "kv_append_decode_attn (decode_split_kernel<fused> + decode_combine_kernel)"
        alg_bytes = db["total"] + ab
        achieved = alg_bytes / (step_gpu_ms / 1e3) / 1e9
        traffic = traffic_from_profile("kv_append_decode_attn", cfg.name)
    else:
        kernel = "kv_decode_attn (decode_split_kernel + decode_combine_kernel)"
        alg_bytes = db["total"]
        achieved = alg_bytes / dec_avg_s / 1e9
        traffic = traffic_from_profile("kv_decode_attn", cfg.name)

    rec = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "prewarm": {"gpu_ms": PREWARM_MS, "launches": prewarm_launches,
                    "why": "untimed back-to-back steps before the warm-up, so that the timed steps run at the "
                           "shader clock of a sustained decode loop (it settles 20-30 ms into sustained load)"},
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16-split-f32",
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "batch": cfg.batch, "num_q_heads": cfg.num_q_heads,
            "num_kv_heads": cfg.num_kv_heads, "head_dim": cfg.head_dim, "page_size": wl.page_size,
            "had_block": cfg.had_block, "sink": cfg.sink, "recent": cfg.recent,
            "lengths": f"{cfg.lengths}{tuple(cfg.length_args)}", "total_tokens": int(wl.lengths.sum()),
            "rotating_cache_copies": args.layers,
        },
        "path": args.path,
        "tokens_heads_per_s": round(tok_heads / step_s, 1),
        "hbm_frac": round(value / HBM_PEAK_GBPS, 4),
        "step_gpu_us": round(step_gpu_ms * 1e3, 2),
        "fused_us": round(float(fus_ms.mean()) * 1e3, 2),
        "fused_us_p10_p90": [round(float(np.percentile(fus_ms, 10)) * 1e3, 2),
                             round(float(np.percentile(fus_ms, 90)) * 1e3, 2)],
        "decode_us": round(float(dec_ms.mean()) * 1e3, 2),
        "decode_us_p10_p90": [round(float(np.percentile(dec_ms, 10)) * 1e3, 2),
                              round(float(np.percentile(dec_ms, 90)) * 1e3, 2)],
        "append_us": round(float(app_ms.mean()) * 1e3, 2),
        "decode_kv_bytes": db["kv"],
        "decode_algorithmic_bytes": db["total"],
        "append_algorithmic_bytes": ab,
        "bf16_equiv_GBps_decode": round(db["bf16_equiv"] / dec_avg_s / 1e9, 1),
        "device_copy_GBps_context": copy_gbps,
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "algorithmic_bytes_per_launch": alg_bytes,
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "ceiling": {
                "what": "kv_decode_read_ceiling: this launch's reads (same split, gathers, DMA ring, waits) "
                        "without the arithmetic, per-launch HIP events, median",
                "us": round(ceil_us[0], 2),
                "GBps": round(db["total"] / ceil_us[0] / 1e3, 1),
                "frac_of_peak": round(db["total"] / ceil_us[0] / 1e3 / HBM_PEAK_GBPS, 4),
            },
        },
        "pages_context": PAGES_CONTEXT,
    }
    dw.cache = layers[0]
    dw.fused_step()
    torch.cuda.synchronize()
    rows = sorted(set([0, cfg.batch - 1] + [int(x) for x in np.random.default_rng(7).choice(cfg.batch, 2)]))
    rec["max_abs_vs_unquantized_bf16"] = round(unquantized_error(torch, dw, rows), 4)
    rec["unquantized_rows"] = rows
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(wl, dw)
    if not args.no_workloads:
        rec["workloads"] = [measure_workload(torch, name, steps=max(5, min(args.steps, 20)))
                            for name in OTHER_WORKLOADS if name != cfg.name]
    if not args.no_sub4bit:
        # the 3- and 2-bit main caches (same lengths, seeds and INT8 protection): decode time and bytes
        for tag, key in (("K3V3", "k3v3"), ("K2V2", "k2v2"), ("K(4,3,3,2)V3", "grouped_keys_k4332_v3")):
            kx = measure_variants(torch, cfg, steps=max(5, min(args.steps, 20)), warmup=3, only=tag)
            rec[key] = kx[0] if kx else None
    if not args.no_prefill:
        rec["prefill"] = measure_prefill(torch, steps=max(5, min(args.steps, 20)), warmup=2,
                                         cpu=not args.no_cpu_baseline)
        rec["prefill"]["sub4bit"] = prefill_sub4bit(torch, steps=max(5, min(args.steps, 20)), warmup=2)
    if args.variants:
        del layers
        dw.cache = None
        torch.cuda.empty_cache()
        rec["variants"] = measure_variants(torch, cfg, steps=20, warmup=3)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
