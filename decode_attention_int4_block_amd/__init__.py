"""INT4 KV-cache quantize-append and regional INT4/INT8 decode attention for MI355X.

A thin Python binding over the C ABI in include/kvq.h (libkvq.so, hand-written
gfx950 HIP kernels).  PyTorch only provides device memory and streams; every
step of the computation runs in the library's kernels, and importing the
binding fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes

import torch

from . import _lib
from ._lib import KvqCache, KvqError

__all__ = ["QuantKVCache", "kv_quant_append", "kv_decode_attn", "kv_decode_attn_noalloc", "kv_decode_read_ceiling",
           "kv_append_decode_attn",
           "kv_prefill_attn", "KvqError"]


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev_i32(t, name):
    if t.dtype != torch.int32 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous int32 CUDA tensor")
    return t


def _dev_bf16(t, name):
    if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous bf16 CUDA tensor")
    return t


class QuantKVCache:
    """Device memory of one INT4 paged cache plus its INT8 side cache."""

    def __init__(self, num_kv_heads: int, page_size: int, num_pages: int, num_slots: int,
                 had_block: int, sink: int, recent: int, device="cuda", head_dim: int = 128, code_bits: int = 4,
                 key_bits=None):
        """key_bits: four key widths, one per RoPE-block group (values keep code_bits), or None."""
        self.lib = _lib.load()
        kb = (ctypes.c_int32 * 4)(*(tuple(key_bits) if key_bits else (0, 0, 0, 0)))
        self.desc = KvqCache(num_kv_heads, head_dim, page_size, num_pages, num_slots,
                             had_block, sink, recent, None, None, code_bits, kb)
        self.code_bits = code_bits
        self.key_bits = tuple(key_bits) if key_bits else None
        n4 = self.lib.kvq_int4_pool_bytes(ctypes.byref(self.desc))
        n8 = self.lib.kvq_int8_pool_bytes(ctypes.byref(self.desc))
        if n4 == 0 and num_pages > 0:
            raise KvqError(f"bad cache descriptor: {self.lib.kvq_last_error().decode()}")
        self.int4_pool = torch.empty(max(n4, 256), dtype=torch.uint8, device=device)
        self.int8_pool = torch.empty(max(n8, 256), dtype=torch.uint8, device=device)
        self.desc.int4_pool = self.int4_pool.data_ptr()
        self.desc.int8_pool = self.int8_pool.data_ptr()
        self.num_kv_heads, self.page_size, self.num_pages = num_kv_heads, page_size, num_pages
        self.num_slots, self.had_block, self.sink, self.recent = num_slots, had_block, sink, recent
        self.nr8 = (sink + recent + 15) // 16

    def workspace_bytes(self, B: int, num_q_heads: int) -> int:
        return int(self.lib.kv_decode_attn_workspace_bytes(ctypes.byref(self.desc), B, num_q_heads))

    def new_workspace(self, B: int, num_q_heads: int) -> torch.Tensor:
        n = self.workspace_bytes(B, num_q_heads)
        if n == 0:
            raise KvqError(f"workspace size query failed: {self.lib.kvq_last_error().decode()}")
        return torch.empty(n, dtype=torch.uint8, device=self.int4_pool.device)


def kv_quant_append(cache: QuantKVCache, k, v, slot, pos, block_table, len_after, stream=None):
    """Quantize and append k, v [T, H_kv, 128] bf16 at (slot[T], pos[T])."""
    _dev_bf16(k, "k")
    _dev_bf16(v, "v")
    T = k.shape[0]
    if k.shape != (T, cache.num_kv_heads, 128) or v.shape != k.shape:
        raise ValueError(f"k/v must be [T, {cache.num_kv_heads}, 128], got {tuple(k.shape)}, {tuple(v.shape)}")
    _dev_i32(slot, "slot")
    _dev_i32(pos, "pos")
    _dev_i32(block_table, "block_table")
    _dev_i32(len_after, "len_after")
    if slot.numel() != T or pos.numel() != T:
        raise ValueError("slot and pos need one entry per token")
    st = cache.lib.kv_quant_append(ctypes.byref(cache.desc), _ptr(k), _ptr(v), _ptr(slot), _ptr(pos), T,
                                   _ptr(block_table), block_table.shape[1], _ptr(len_after),
                                   _stream(stream))
    _lib.check(st, "kv_quant_append")


def _decode_args(cache, q, slot, block_table, ctx_len, out, lse, workspace):
    _dev_bf16(q, "q")
    B, Hq, d = q.shape
    _dev_i32(slot, "slot")
    _dev_i32(block_table, "block_table")
    _dev_i32(ctx_len, "ctx_len")
    if slot.numel() != B or ctx_len.numel() != B:
        raise ValueError("slot and ctx_len need one entry per row")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = cache.new_workspace(B, Hq)
    return out, lse, workspace


def kv_decode_attn(cache: QuantKVCache, q, slot, block_table, ctx_len, out=None, lse=None,
                   workspace=None, stream=None):
    """Decode attention of q [B, H_q, 128] bf16; returns (out fp32 [B, H_q, 128], lse [B, H_q])."""
    out, lse, workspace = _decode_args(cache, q, slot, block_table, ctx_len, out, lse, workspace)
    B, Hq = q.shape[0], q.shape[1]
    st = cache.lib.kv_decode_attn(ctypes.byref(cache.desc), _ptr(q), Hq, _ptr(slot), _ptr(block_table),
                                  block_table.shape[1], _ptr(ctx_len), B, _ptr(out), _ptr(lse),
                                  _ptr(workspace), workspace.numel(), _stream(stream))
    _lib.check(st, "kv_decode_attn")
    return out, lse


def kv_decode_read_ceiling(cache: QuantKVCache, q, slot, block_table, ctx_len, workspace=None, stream=None):
    """The memory traffic of kv_decode_attn without its arithmetic (a measured
    bandwidth ceiling for the same access pattern); computes nothing."""
    _dev_bf16(q, "q")
    B, Hq = q.shape[0], q.shape[1]
    _dev_i32(slot, "slot")
    _dev_i32(block_table, "block_table")
    _dev_i32(ctx_len, "ctx_len")
    if workspace is None:
        workspace = cache.new_workspace(B, Hq)
    st = cache.lib.kv_decode_read_ceiling(ctypes.byref(cache.desc), _ptr(q), Hq, _ptr(slot), _ptr(block_table),
                                          block_table.shape[1], _ptr(ctx_len), B, _ptr(workspace),
                                          workspace.numel(), _stream(stream))
    _lib.check(st, "kv_decode_read_ceiling")


def kv_decode_attn_noalloc(cache: QuantKVCache, q, slot, block_table, ctx_len, out, lse, stream=None):
    """kv_decode_attn with the library's static device scratch instead of a
    workspace: the C call allocates nothing (out and lse are the caller's)."""
    _dev_bf16(q, "q")
    B, Hq = q.shape[0], q.shape[1]
    _dev_i32(slot, "slot")
    _dev_i32(block_table, "block_table")
    _dev_i32(ctx_len, "ctx_len")
    if slot.numel() != B or ctx_len.numel() != B:
        raise ValueError("slot and ctx_len need one entry per row")
    st = cache.lib.kv_decode_attn_noalloc(ctypes.byref(cache.desc), _ptr(q), Hq, _ptr(slot), _ptr(block_table),
                                          block_table.shape[1], _ptr(ctx_len), B, _ptr(out), _ptr(lse),
                                          _stream(stream))
    _lib.check(st, "kv_decode_attn_noalloc")
    return out, lse


def kv_append_decode_attn(cache: QuantKVCache, k, v, q, slot, block_table, ctx_len, out=None, lse=None,
                          workspace=None, stream=None):
    """Append k, v [B, H_kv, 128] bf16 at position ctx_len - 1 of each row, then attend q.

    The same cache bytes and outputs as kv_quant_append followed by
    kv_decode_attn, in one launch; returns (out, lse).
    """
    out, lse, workspace = _decode_args(cache, q, slot, block_table, ctx_len, out, lse, workspace)
    B, Hq = q.shape[0], q.shape[1]
    _dev_bf16(k, "k")
    _dev_bf16(v, "v")
    if k.shape != (B, cache.num_kv_heads, 128) or v.shape != k.shape:
        raise ValueError(f"k/v must be [{B}, {cache.num_kv_heads}, 128], got {tuple(k.shape)}, {tuple(v.shape)}")
    st = cache.lib.kv_append_decode_attn(ctypes.byref(cache.desc), _ptr(k), _ptr(v), _ptr(q), Hq, _ptr(slot),
                                         _ptr(block_table), block_table.shape[1], _ptr(ctx_len), B, _ptr(out),
                                         _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream))
    _lib.check(st, "kv_append_decode_attn")
    return out, lse


def kv_prefill_attn(cache: QuantKVCache, q, q_start, slot, block_table, ctx_len, max_rows: int, out=None, lse=None,
                    stream=None):
    """Causal attention of chunks of query rows over the quantized cache.

    q [N, H_q, 128] bf16; rows of sequence b are q_start[b] .. q_start[b + 1] - 1
    (q_start int32 [B + 1] on the device) at positions ctx_len[b] - T_b .. ctx_len[b] - 1.
    max_rows bounds every T_b.  Returns (out fp32 [N, H_q, 128], lse [N, H_q]).
    """
    _dev_bf16(q, "q")
    N, Hq, d = q.shape
    _dev_i32(q_start, "q_start")
    _dev_i32(slot, "slot")
    _dev_i32(block_table, "block_table")
    _dev_i32(ctx_len, "ctx_len")
    B = slot.numel()
    if ctx_len.numel() != B or q_start.numel() != B + 1:
        raise ValueError("slot and ctx_len need one entry per sequence, q_start B + 1")
    if out is None:
        out = torch.empty((N, Hq, d), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((N, Hq), dtype=torch.float32, device=q.device)
    st = cache.lib.kv_prefill_attn(ctypes.byref(cache.desc), _ptr(q), Hq, _ptr(q_start), int(max_rows), _ptr(slot),
                                   _ptr(block_table), block_table.shape[1], _ptr(ctx_len), B, _ptr(out), _ptr(lse),
                                   _stream(stream))
    _lib.check(st, "kv_prefill_attn")
    return out, lse
