"""GPU parity on crafted rows: the quantizer's edge cases through the C ABI.

Every position of these rows is one of the kinds in `workloads.edge`: constant
vectors (positive, negative, +0, -0), a near-constant vector whose fp16 scale
underflows to 0, one whose fp16 scale is subnormal, vectors already on the
quantization grid, vectors half-way between grid levels (exact rounding ties),
large values near the fp16 range, and N(0, 1).  The first five take the
zero-range guard (fp16 scale 0: every code 0).  Both append paths are run:
`kv_quant_append` + `kv_decode_attn`, and the fused `kv_append_decode_attn`.

Acceptance:
* codes, fp16 scales and offsets bit-exact against the oracle, INT4 (or 3- / 2-
  bit) and INT8, with the tie gate's bound; both paths write the same pool bytes;
  the tie rows are flagged by the gate (so the exact ties were reached) and still
  match exactly, since both sides round them in the same fp32 arithmetic;
* attention finite and within 2e-3 of the oracle's fp64 attention, scaled by
  max(1, v_max / 256) for rows holding the large values (v_max up to 6e4: fp32
  sums of values that large carry absolute errors above 2e-3).
"""

import numpy as np
import pytest
import torch

from gpu_common import (ATOL, add_stats, assert_cache_exact, attention_error_scaled, compare_cache,
                        make_device_workload, small_config)
from oracle.cache import quantize_sequence
from workloads import bf16_bits
from workloads.edge import edge_kv

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _report(name, **kw):
    print(f"[edges] {name}: " + ", ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


# sinks only, inside the window, and rows with an INT4 region
LENGTHS = [1, 2, 5, 33, 37, 70, 200, 301]


@pytest.mark.parametrize("bits", [4, 3, 2])
@pytest.mark.parametrize("h", [1, 128])
def test_crafted_rows_append_and_attend(h, bits):
    cfg = small_config(LENGTHS, h=h, s=4, w=32, seed=2100 + 10 * h + bits, bits=bits)
    rows = list(range(cfg.batch))
    qmax = (1 << bits) - 1

    def kv_fn(b):
        return edge_kv(int(cfg.length_args[b]), cfg.num_kv_heads, h, qmax, seed=7000 + 31 * b + bits, offset=b)

    print(f"[edges] case h={h} bits={bits} lengths={LENGTHS}", flush=True)
    sep = make_device_workload(cfg, keep=rows, poison=True, prefill=False, kv_fn=kv_fn)
    fus = make_device_workload(cfg, keep=rows, poison=True, prefill=False, kv_fn=kv_fn)
    sep.prefill()
    fus.prefill()
    sep.append_step()
    sep.decode_step()
    fus.fused_step()
    torch.cuda.synchronize()

    assert torch.equal(sep.cache.int4_pool, fus.cache.int4_pool), "main pools differ between the two paths"
    assert torch.equal(sep.cache.int8_pool, fus.cache.int8_pool), "INT8 pools differ between the two paths"
    tot = {}
    for b in rows:
        add_stats(tot, compare_cache(sep, b))
    _report(f"h={h} bits={bits} cache", **tot)
    assert_cache_exact(tot)
    # no mismatch at all, ties included: the exact ties are decided the same way
    assert tot["int4_ties"] == 0 and tot["int8_ties"] == 0 and tot["params_ties"] == 0, tot
    if h == 1:
        assert tot["flagged"] > 0, "the crafted tie rows were not reached"
    guarded = 0
    for b in rows:
        k, v = sep.host_kv[b]
        oc = quantize_sequence(bf16_bits(k), bf16_bits(v), h, cfg.sink, cfg.recent, main_bits=bits)
        guarded += int(((oc.k4_scale & 0x7FFF) == 0).sum() + ((oc.v4_scale & 0x7FFF) == 0).sum())
    assert guarded > 0, "no vector took the zero-range guard"
    for name, dw in (("two-launch", sep), ("fused", fus)):
        err = attention_error_scaled(dw, rows)
        _report(f"h={h} bits={bits} {name} attention", scaled_max_abs=f"{err:.2e}", guarded_vectors=guarded)
        assert err <= ATOL
