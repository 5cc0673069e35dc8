"""GPU parity: the HIP library (through the C ABI) against the CPU oracle.

Quantization: codes, fp16 scales and zeros bit-exact (mismatches allowed only
within 1e-6 of a rounding tie; counted and printed).  Attention: max-abs error
within 2e-3 of the oracle's fp64 attention over its own quantization of the
same bf16 inputs; the error against unquantized bf16 attention is printed.
"""

import numpy as np
import pytest
import torch

from gpu_common import (ATOL, assert_cache_exact, compare_attention, compare_cache, make_device_workload,
                        small_config)
from workloads import get_config

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _report(name, **kw):
    print(f"[parity] {name}: " + ", ".join(f"{k}={v}" for k, v in kw.items()), flush=True)


def test_tiny_single_step_cache_and_attention():
    """The tiny non-paged workload (1 x 1024, 8/2 heads, h=128, s=4, w=64)."""
    cfg = get_config("tiny_1x1024")
    dw = make_device_workload(cfg, keep=[0])
    st = compare_cache(dw, 0)
    _report("tiny cache", **st)
    assert_cache_exact(st)
    dw.decode_step()
    torch.cuda.synchronize()
    err, err_lse, unq = compare_attention(dw, [0], report_unquantized=True)
    _report("tiny attention", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}", vs_unquantized_bf16=f"{unq:.3f}")
    assert err <= ATOL and err_lse <= ATOL


EDGE_LENGTHS = [1, 3, 4, 5, 16, 17, 31, 32, 33, 36, 37, 40, 41, 64, 100, 129, 200, 515]


@pytest.mark.parametrize("h", [1, 2, 16, 64, 128])
def test_small_paged_cache_and_attention(h):
    """Ragged lengths around every boundary (s, s+w, page and step edges)."""
    cfg = small_config(EDGE_LENGTHS, h=h, s=4, w=32, seed=100 + h)
    rows = list(range(cfg.batch))
    dw = make_device_workload(cfg, keep=rows)
    tot = {}
    for b in rows:
        st = compare_cache(dw, b)
        for k2, v2 in st.items():
            tot[k2] = tot.get(k2, 0) + v2
    _report(f"small h={h} cache", **tot)
    assert_cache_exact(tot)
    dw.decode_step()
    torch.cuda.synchronize()
    err, err_lse, _ = compare_attention(dw, rows)
    _report(f"small h={h} attention", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


# non-power-of-two groups pad to the next MFMA column count and leave columns unused
@pytest.mark.parametrize("g,Hkv", [(1, 4), (2, 2), (3, 2), (4, 2), (5, 1), (7, 2), (8, 2), (12, 1), (16, 1)])
def test_query_groups(g, Hkv):
    cfg = small_config([1, 40, 300, 777], Hq=g * Hkv, Hkv=Hkv, h=128, s=4, w=64, seed=200 + g)
    rows = list(range(cfg.batch))
    dw = make_device_workload(cfg, keep=rows)
    dw.decode_step()
    torch.cuda.synchronize()
    err, err_lse, _ = compare_attention(dw, rows)
    _report(f"group g={g}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


@pytest.mark.parametrize("s,w", [(0, 0), (0, 16), (16, 0), (16, 128), (4, 4000)])
def test_protection_budgets(s, w):
    """INT4 only (s=w=0), recent only, sinks only, the pages' 16/128 default,
    and INT8 everywhere (s + w >= L)."""
    cfg = small_config([2, 50, 333, 1200], h=128, s=s, w=w, seed=300 + s + w)
    rows = list(range(cfg.batch))
    dw = make_device_workload(cfg, keep=rows)
    tot = {}
    for b in rows:
        for k2, v2 in compare_cache(dw, b).items():
            tot[k2] = tot.get(k2, 0) + v2
    assert_cache_exact(tot)
    dw.decode_step()
    torch.cuda.synchronize()
    err, err_lse, _ = compare_attention(dw, rows)
    _report(f"budget s={s} w={w}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}", **tot)
    assert err <= ATOL and err_lse <= ATOL


def test_page_sizes_and_empty_rows():
    for P in (16, 32, 64, 1024):
        cfg = small_config([0, 1, 70, 1500, 0, 2049], P=P, h=64, s=4, w=128, seed=400 + P)
        rows = list(range(cfg.batch))
        dw = make_device_workload(cfg, keep=[b for b in rows if cfg.length_args[b] > 0])
        dw.decode_step()
        torch.cuda.synchronize()
        err, err_lse, _ = compare_attention(dw, rows)
        _report(f"page P={P}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
        assert err <= ATOL and err_lse <= ATOL


@pytest.mark.parametrize("g,Hkv", [(1, 4), (4, 2), (8, 2), (16, 1)])
def test_unwritten_cache_bytes_never_reach_the_output(g, Hkv):
    """Pools pre-filled with fp16 NaN patterns: positions past each row's context
    share subblocks with valid ones and must be masked, never multiplied by 0."""
    cfg = small_config([1, 5, 17, 33, 50, 97, 130, 301], Hq=g * Hkv, Hkv=Hkv, h=128, s=4, w=32, seed=700 + g)
    rows = list(range(cfg.batch))
    dw = make_device_workload(cfg, keep=rows, poison=True)
    dw.decode_step()
    torch.cuda.synchronize()
    err, err_lse, _ = compare_attention(dw, rows)
    _report(f"poisoned pools g={g}", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}")
    assert err <= ATOL and err_lse <= ATOL


def test_bulk_append_equals_token_by_token():
    """Ordering independence: one bulk append vs one call per position."""
    from decode_attention_int4_block_amd import kv_quant_append
    cfg = small_config([45, 160], h=64, s=4, w=32, seed=500)
    bulk = make_device_workload(cfg, keep=[0, 1])
    seq = make_device_workload(cfg, keep=[0, 1], prefill=False)
    for b in range(cfg.batch):
        k, v = bulk.host_kv[b]
        L = int(cfg.length_args[b])
        slot = int(seq.wl.slots[b])
        for p in range(L):
            la = torch.zeros(seq.wl.num_slots, dtype=torch.int32)
            la[slot] = p + 1
            kv_quant_append(seq.cache, k[p:p + 1].cuda().contiguous(), v[p:p + 1].cuda().contiguous(),
                            torch.tensor([slot], dtype=torch.int32, device="cuda"),
                            torch.tensor([p], dtype=torch.int32, device="cuda"),
                            seq.block_table, la.cuda())
    torch.cuda.synchronize()
    seq.host_kv = bulk.host_kv
    for b in range(cfg.batch):
        assert_cache_exact(compare_cache(seq, b))
    bulk.decode_step()
    seq.decode_step()
    torch.cuda.synchronize()
    assert torch.equal(bulk.out, seq.out)


def test_repeated_decode_is_deterministic():
    cfg = small_config([3000, 17, 900], h=128, s=4, w=128, seed=600)
    dw = make_device_workload(cfg)
    dw.decode_step()
    a = dw.out.clone()
    for _ in range(3):
        dw.decode_step()
    torch.cuda.synchronize()
    assert torch.equal(a, dw.out)


def _segment_pieces(dw, segs):
    """Pieces of each (row, KV head) segment in the last launch, from the
    workspace's first- and last-worker records (256-byte aligned arrays after
    the 256-byte header)."""
    ws = dw.workspace
    first = ws[256:256 + 4 * segs].view(torch.int32).cpu().numpy()
    off = (256 + 4 * segs + 255) // 256 * 256
    last = ws[off:off + 4 * segs].view(torch.int32).cpu().numpy()
    return last - first + 1


# long rows split over hundreds of workers: the combine's helpers fold them
# per (query head, dim slice); the last case has 1024 pieces in one segment
LONG_CASES = [(8, 2, [70000, 5, 3000]), (16, 2, [70000, 700]), (16, 1, [90000]), (6, 2, [70000, 40]),
              (8, 1, [262144])]


@pytest.mark.parametrize("Hq,Hkv,lengths", LONG_CASES)
def test_long_segments(Hq, Hkv, lengths):
    cfg = small_config(lengths, Hq=Hq, Hkv=Hkv, h=128, s=4, w=128, seed=700 + Hq + len(lengths))
    rows = list(range(cfg.batch))
    dw = make_device_workload(cfg, keep=rows, gen_device="cuda")
    dw.decode_step()
    torch.cuda.synchronize()
    n = _segment_pieces(dw, cfg.batch * Hkv)
    err, err_lse, _ = compare_attention(dw, rows)
    _report(f"long segments g={Hq // Hkv} lengths={lengths}", pieces=n.tolist(), max_abs=f"{err:.2e}",
            lse=f"{err_lse:.2e}")
    assert n.max() > 32
    assert err <= ATOL and err_lse <= ATOL


FULL = ["qwen3_4b_b64", "qwen3_8b_async_256", "long_128k", "refill_512"]


@pytest.mark.parametrize("name", FULL)
def test_full_size_sampled_rows(name):
    """Full-size workloads in the benchmark's launch configuration; the oracle
    checks sampled rows (shortest, longest, and a few seeded picks)."""
    cfg = get_config(name)
    from workloads import build_workload
    wl = build_workload(cfg)
    L = wl.lengths
    rng = np.random.default_rng(9)
    pick = {int(np.argmin(L)), int(np.argmax(L))}
    pick |= set(int(x) for x in rng.choice(cfg.batch, size=min(4, cfg.batch), replace=False))
    rows = sorted(pick)
    dw = make_device_workload(cfg, keep=rows, gen_device="cuda")
    tot = {}
    for b in rows:
        Lb = int(L[b])
        positions = np.unique(np.concatenate([np.arange(min(Lb, 40)), np.arange(max(0, Lb - 200), Lb),
                                              rng.integers(0, Lb, size=min(Lb, 300))]))
        for k2, v2 in compare_cache(dw, b, positions).items():
            tot[k2] = tot.get(k2, 0) + v2
    _report(f"{name} cache (sampled rows {rows})", **tot)
    assert_cache_exact(tot)
    dw.decode_step()
    torch.cuda.synchronize()
    err, err_lse, unq = compare_attention(dw, rows, report_unquantized=True)
    _report(f"{name} attention", max_abs=f"{err:.2e}", lse=f"{err_lse:.2e}", vs_unquantized_bf16=f"{unq:.3f}")
    assert err <= ATOL and err_lse <= ATOL
    assert torch.isfinite(dw.out).all()
