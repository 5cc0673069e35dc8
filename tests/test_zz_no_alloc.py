"""The no-allocation entry point kv_decode_attn_noalloc against kv_decode_attn.

Both run the same kernels with the same worker count, so their outputs must be
bit-identical; the no-allocation call keeps its workspace in the library's
static device scratch.  Two calls in a row, the second with a smaller batch
(the scratch keeps the first call's contents), then one call too large for the
scratch, which must be rejected on the host.
"""

import numpy as np
import pytest
import torch

from gpu_common import ATOL, compare_attention, make_device_workload, small_config
from workloads import get_config

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(dw):
    from decode_attention_int4_block_amd import kv_decode_attn, kv_decode_attn_noalloc
    out_ws, lse_ws = kv_decode_attn(dw.cache, dw.q, dw.slots, dw.block_table, dw.ctx_len, workspace=dw.workspace)
    out_na = torch.full_like(out_ws, float("nan"))
    lse_na = torch.full_like(lse_ws, float("nan"))
    kv_decode_attn_noalloc(dw.cache, dw.q, dw.slots, dw.block_table, dw.ctx_len, out_na, lse_na)
    torch.cuda.synchronize()
    return out_ws, lse_ws, out_na, lse_na


def test_noalloc_equals_workspace_entry_point_on_two_calls():
    # call 1: the 256-row Qwen3-8B batch as the benchmark runs it
    print("[noalloc] call 1: qwen3_8b_async_256", flush=True)
    big = make_device_workload(get_config("qwen3_8b_async_256"), keep=[], gen_device="cuda")
    o1, l1, n1, m1 = _both(big)
    assert torch.equal(o1, n1) and torch.equal(l1, m1), "call 1: outputs differ from kv_decode_attn"
    del big
    # call 2: a smaller batch with ragged and empty rows; oracle parity on every row
    print("[noalloc] call 2: 7 ragged rows", flush=True)
    cfg = small_config([0, 1, 5, 37, 300, 1025, 0], h=64, s=4, w=32, seed=4242)
    rows = list(range(cfg.batch))
    small = make_device_workload(cfg, keep=[b for b in rows if cfg.length_args[b] > 0])
    o2, l2, n2, m2 = _both(small)
    assert torch.equal(o2, n2) and torch.equal(l2, m2), "call 2: outputs differ from kv_decode_attn"
    small.out.copy_(n2)
    small.lse.copy_(m2)
    err, err_lse, _ = compare_attention(small, rows)
    print(f"[noalloc] call 2 vs oracle: max_abs={err:.2e} lse={err_lse:.2e}", flush=True)
    assert err <= ATOL and err_lse <= ATOL


def test_noalloc_rejects_requests_beyond_the_scratch():
    from decode_attention_int4_block_amd import QuantKVCache, KvqError, kv_decode_attn_noalloc
    B, Hkv, g = 4096, 8, 16                   # needs far more than the 32 MiB scratch
    cache = QuantKVCache(Hkv, 16, 1, B, 128, 4, 128)
    assert cache.workspace_bytes(B, Hkv * g) > (32 << 20)
    q = torch.zeros((B, Hkv * g, 128), dtype=torch.bfloat16, device="cuda")
    i32 = torch.zeros(B, dtype=torch.int32, device="cuda")
    bt = torch.zeros((B, 1), dtype=torch.int32, device="cuda")
    out = torch.zeros((B, Hkv * g, 128), dtype=torch.float32, device="cuda")
    lse = torch.zeros((B, Hkv * g), dtype=torch.float32, device="cuda")
    with pytest.raises(KvqError, match="workspace"):
        kv_decode_attn_noalloc(cache, q, i32, bt, i32, out, lse)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0      # nothing was enqueued
