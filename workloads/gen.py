"""Seeded generators for decode workloads (inputs only; no method arithmetic).

Recipe (stated once here; the value distributions are those of the tiny
single-step workload and are reused by every workload):

* keys: N(0,1) draws, four seeded channels per KV head (fixed across tokens and
  sequences) scaled by 20, then NeoX rotate-half RoPE with base 1e6 at the
  token's position; computed in fp64 and rounded to bf16 (round-to-nearest-even);
* values and queries: N(0,1) rounded to bf16;
* lengths: see ``draw_lengths``; block tables: a seeded permutation of a page
  pool that holds exactly the pages the sequences need;
* each sequence's keys/values come from a generator keyed by (seed, sequence),
  so any one sequence can be regenerated on its own.

Tensors can be drawn on the CPU or on a GPU; the two devices use different
random streams, so a consumer that compares two implementations must hand both
the same drawn tensors (the GPU-drawn ones are copied to the host for the CPU
side).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .configs import WorkloadConfig


def draw_lengths(cfg: WorkloadConfig, rng: np.random.Generator) -> np.ndarray:
    """Context lengths L_b (each counts the token appended this step)."""
    B = cfg.batch
    a = cfg.length_args
    if cfg.lengths == "fixed":
        L = np.full(B, a[0], dtype=np.int64)
    elif cfg.lengths == "explicit":
        L = np.asarray(a, dtype=np.int64)
        assert len(L) == B
    elif cfg.lengths == "lognormal":
        median, sigma, lo, hi = a
        z = rng.standard_normal(B)
        L = np.rint(median * np.exp(sigma * z)).astype(np.int64)
        L = np.clip(L, lo, hi)
    elif cfg.lengths == "pareto":
        # Pareto type I with scale xm and shape alpha by inverse CDF, then clipped.
        xm, alpha, hi = a
        u = 1.0 - rng.random(B)               # (0, 1]
        L = np.floor(xm * u ** (-1.0 / alpha)).astype(np.int64)
        L = np.clip(L, xm, hi)
    elif cfg.lengths == "uniform":
        lo, hi = a
        L = rng.integers(lo, hi + 1, size=B).astype(np.int64)
    elif cfg.lengths == "refill":
        lo, hi, fresh_frac, fresh_max = a
        L = rng.integers(lo, hi + 1, size=B).astype(np.int64)
        n_fresh = int(round(fresh_frac * B))
        fresh = rng.choice(B, size=n_fresh, replace=False)
        L[fresh] = rng.integers(1, fresh_max + 1, size=n_fresh)
    else:
        raise ValueError(f"unknown length recipe {cfg.lengths!r}")
    return L


@dataclass
class Workload:
    cfg: WorkloadConfig
    lengths: np.ndarray        # [B] int64, includes the token appended this step
    slots: np.ndarray          # [B] int32 slot of each decode row
    num_slots: int
    page_size: int
    num_pages: int
    block_table: np.ndarray    # [num_slots][bt_stride] int32, indexed by slot
    outlier_idx: np.ndarray    # [H_kv][n_outlier] int64 channel indices

    @property
    def bt_stride(self) -> int:
        return int(self.block_table.shape[1])

    @property
    def max_len(self) -> int:
        return int(self.lengths.max()) if len(self.lengths) else 0


def build_workload(cfg: WorkloadConfig) -> Workload:
    rng = np.random.default_rng(cfg.seed)
    L = draw_lengths(cfg, rng)
    B = cfg.batch
    num_slots = B
    slots = rng.permutation(num_slots).astype(np.int32)[:B]
    if cfg.paged:
        P = cfg.page_size
    else:
        # One page per sequence holding the whole context.
        P = int(max(cfg.page_size, int(L.max()), 16))
        P = 1 << (P - 1).bit_length()          # page sizes are powers of two
    npages = (L + P - 1) // P
    num_pages = int(npages.sum())
    bt_stride = max(1, int(npages.max()))
    if cfg.paged:
        pool = rng.permutation(num_pages).astype(np.int32)
    else:
        pool = np.arange(num_pages, dtype=np.int32)
    block_table = np.zeros((num_slots, bt_stride), dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(npages[b])
        block_table[slots[b], :n] = pool[off:off + n]
        off += n
    outlier_idx = np.stack([
        rng.choice(cfg.head_dim, size=cfg.outlier_channels, replace=False)
        for _ in range(cfg.num_kv_heads)
    ]).astype(np.int64)
    return Workload(cfg=cfg, lengths=L, slots=slots, num_slots=num_slots,
                    page_size=P, num_pages=num_pages, block_table=block_table,
                    outlier_idx=outlier_idx)


def _generator(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFF_FFFF_FFFF_FFFF)
    return g


def _rope_neox(x: torch.Tensor, pos0: int, base: float) -> torch.Tensor:
    """Rotate-half RoPE over the last dim of x [L, H, d] (fp64), positions pos0.."""
    L, _, d = x.shape
    half = d // 2
    i = torch.arange(half, dtype=torch.float64, device=x.device)
    theta = base ** (-2.0 * i / d)
    p = torch.arange(pos0, pos0 + L, dtype=torch.float64, device=x.device)
    ang = p[:, None] * theta[None, :]
    c = torch.cos(ang)[:, None, :]
    s = torch.sin(ang)[:, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * c - x2 * s, x2 * c + x1 * s], dim=-1)


def seq_kv(wl: Workload, b: int, device="cpu", pos_range=None):
    """Keys and values (bf16) of sequence b for positions [p0, p1).

    Returns (k, v), each [p1 - p0, H_kv, head_dim] torch.bfloat16 on `device`.
    The draw always covers positions [0, L_b) so that any sub-range equals the
    matching slice of the full sequence.
    """
    cfg = wl.cfg
    Lb = int(wl.lengths[b])
    p0, p1 = (0, Lb) if pos_range is None else pos_range
    g = _generator(device, cfg.seed * 1_000_003 + 7919 * b + 1)
    H, d = cfg.num_kv_heads, cfg.head_dim
    kpre = torch.randn((Lb, H, d), generator=g, device=device, dtype=torch.float32)
    vals = torch.randn((Lb, H, d), generator=g, device=device, dtype=torch.float32)
    kpre = kpre[p0:p1].to(torch.float64)
    scale = torch.ones((H, d), dtype=torch.float64, device=device)
    oi = torch.as_tensor(wl.outlier_idx, device=device)
    scale.scatter_(1, oi, cfg.outlier_scale)
    kpre = kpre * scale[None]
    k = _rope_neox(kpre, p0, cfg.rope_base).to(torch.bfloat16)
    v = vals[p0:p1].to(torch.bfloat16)
    return k, v


def seq_query(wl: Workload, device="cpu") -> torch.Tensor:
    """Decode queries [B, H_q, head_dim] bf16, N(0,1)."""
    cfg = wl.cfg
    g = _generator(device, cfg.seed * 1_000_003 + 17)
    q = torch.randn((cfg.batch, cfg.num_q_heads, cfg.head_dim), generator=g,
                    device=device, dtype=torch.float32)
    return q.to(torch.bfloat16)


def chunk_queries(wl: Workload, rows, device="cpu") -> torch.Tensor:
    """Query rows of a prefill chunk per sequence, [sum(rows), H_q, head_dim] bf16, N(0,1)."""
    cfg = wl.cfg
    g = _generator(device, cfg.seed * 1_000_003 + 29)
    n = int(np.sum(rows))
    q = torch.randn((n, cfg.num_q_heads, cfg.head_dim), generator=g, device=device, dtype=torch.float32)
    return q.to(torch.bfloat16)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy uint16 view of a bf16 tensor's bit patterns."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
