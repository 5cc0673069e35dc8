"""GPU parity of the 3- and 2-bit main caches (code_bits = 3, 2) under the same
INT8 sink / recent protection (KV4-RL, "Future Directions": caches below 4 bits).

kv_quant_append must write the codes, scales and zeros bit-exact against the
oracle's quantization with qmax = 7 / 3 (and the INT8 copies as for the 4-bit
cache); kv_decode_attn must match the oracle's fp64 attention over its own
sub-4-bit + INT8 cache within 2e-3.
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
    print(f"[sub4bit] {name}: " + ", ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def _check(cfg, name, poison=False):
    rows = list(range(cfg.batch))
    keep = [b for b in rows if cfg.length_args[b] > 0]
    dw = make_device_workload(cfg, keep=keep, poison=poison)
    tot = {}
    for b in keep:
        for k, v in compare_cache(dw, b).items():
            tot[k] = tot.get(k, 0) + v
    assert_cache_exact(tot)
    dw.decode_step()
    torch.cuda.synchronize()
    err, err_lse, _ = compare_attention(dw, rows)
    _report(name, max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}", **tot)
    assert err <= ATOL and err_lse <= ATOL


EDGE = [1, 3, 4, 5, 16, 17, 31, 32, 33, 36, 37, 40, 41, 64, 100, 129, 200, 515]


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("h", [1, 16, 128])
def test_sub4bit_edge_lengths(h, bits):
    _check(small_config(EDGE, h=h, s=4, w=32, seed=3100 + h + 10 * bits, bits=bits), f"{bits}-bit edge lengths h={h}")


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("s,w", [(0, 0), (0, 16), (16, 0), (16, 128), (4, 4000)])
def test_sub4bit_protection_budgets(s, w, bits):
    _check(small_config([1, 3, 17, 40, 129, 300, 1000], h=128, s=s, w=w, seed=3200 + s + w + bits, bits=bits),
           f"{bits}-bit budget s={s} w={w}")


@pytest.mark.parametrize("bits", [2, 3])
@pytest.mark.parametrize("g,Hkv", [(1, 4), (3, 2), (4, 2), (7, 1), (8, 2), (16, 1)])
def test_sub4bit_query_groups(g, Hkv, bits):
    _check(small_config([1, 20, 77, 160, 700], Hq=g * Hkv, Hkv=Hkv, h=128, s=4, w=64, seed=3300 + g + 40 * bits,
                        bits=bits), f"{bits}-bit g={g}")


@pytest.mark.parametrize("bits", [2, 3])
def test_sub4bit_page_sizes_empty_rows_and_poisoned_pools(bits):
    for P in (16, 64, 1024):
        _check(small_config([0, 1, 70, 1500, 0, 2049], P=P, h=64, s=4, w=128, seed=3400 + P + bits, bits=bits),
               f"{bits}-bit P={P}", poison=True)


@pytest.mark.parametrize("bits", [2, 3])
def test_sub4bit_full_size_sampled_rows(bits):
    """The 256-row Qwen3-8B batch with a 3- or 2-bit main cache, sampled rows."""
    from workloads import build_workload
    cfg = get_config("qwen3_8b_async_256").scaled(code_bits=bits)
    wl = build_workload(cfg)
    L = wl.lengths
    rng = np.random.default_rng(13)
    rows = sorted({int(np.argmin(L)), int(np.argmax(L))} |
                  set(int(x) for x in rng.choice(cfg.batch, size=3, replace=False)))
    dw = make_device_workload(cfg, keep=rows, gen_device="cuda")
    tot = {}
    for b in rows:
        Lb = int(L[b])
        positions = np.unique(np.concatenate([np.arange(min(Lb, 40)), np.arange(max(0, Lb - 200), Lb),
                                              rng.integers(0, Lb, size=min(Lb, 300))]))
        for k, v in compare_cache(dw, b, positions).items():
            tot[k] = tot.get(k, 0) + v
    assert_cache_exact(tot)
    dw.decode_step()
    torch.cuda.synchronize()
    err, err_lse, unq = compare_attention(dw, rows, report_unquantized=True)
    _report(f"qwen3_8b_async_256 K{bits}V{bits}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}", vs_unquantized_bf16=f"{unq:.3f}")
    assert err <= ATOL and err_lse <= ATOL
