"""Drive the library on a synthetic workload: allocate the cache, prefill it
through kv_quant_append, and run decode steps.  Used by the tests, the smoke
check and the benchmark; it only calls the library (no reference maths here).
"""

from __future__ import annotations

import numpy as np
import torch

from workloads import Workload, seq_kv, seq_query

from . import QuantKVCache, kv_append_decode_attn, kv_decode_attn, kv_quant_append


class DeviceWorkload:
    """A workload's cache on the GPU, filled up to L_b - 1 (or L_b) positions.

    The token at position L_b - 1 of each row is the one the timed decode step
    appends; its bf16 k/v are kept in `step_k`, `step_v` ([B, H_kv, 128]).
    """

    def __init__(self, wl: Workload, device="cuda", gen_device=None, keep_host=(), kv_fn=None):
        """kv_fn(b) -> (k, v), each [L_b, H_kv, 128] bf16, replaces the workload's
        drawn keys and values of row b (crafted inputs)."""
        cfg = wl.cfg
        self.kv_fn = kv_fn
        self.wl = wl
        self.cfg = cfg
        self.device = torch.device(device)
        self.gen_device = torch.device(gen_device) if gen_device is not None else self.device
        B = cfg.batch
        self.B = B
        self.cache = QuantKVCache(cfg.num_kv_heads, wl.page_size, max(wl.num_pages, 1), wl.num_slots,
                                  cfg.had_block, cfg.sink, cfg.recent, device=self.device, code_bits=cfg.code_bits,
                                  key_bits=cfg.key_bits or None)
        self.block_table = torch.from_numpy(wl.block_table).to(self.device)
        self.slots = torch.from_numpy(wl.slots.astype(np.int32)).to(self.device)
        self.lengths = wl.lengths.astype(np.int64)
        self.ctx_len = torch.from_numpy(self.lengths.astype(np.int32)).to(self.device)
        self.q = seq_query(wl, device=self.gen_device).to(self.device)
        self.step_k = torch.zeros((B, cfg.num_kv_heads, cfg.head_dim), dtype=torch.bfloat16, device=self.device)
        self.step_v = torch.zeros_like(self.step_k)
        self.step_pos = torch.from_numpy(np.maximum(self.lengths - 1, 0).astype(np.int32)).to(self.device)
        # len_after indexed by slot
        la = np.zeros(wl.num_slots, dtype=np.int32)
        la[wl.slots] = self.lengths
        self.len_after_step = torch.from_numpy(la).to(self.device)
        self.host_kv = {}          # b -> (k bf16 cpu, v bf16 cpu) of the full sequence
        self.keep_host = set(int(b) for b in keep_host)
        self._step_rows = None
        self.workspace = self.cache.new_workspace(B, cfg.num_q_heads)
        self.out = torch.empty((B, cfg.num_q_heads, cfg.head_dim), dtype=torch.float32, device=self.device)
        self.lse = torch.empty((B, cfg.num_q_heads), dtype=torch.float32, device=self.device)

    def prefill(self, include_step_token=False, max_tokens_per_call=1 << 18):
        """Append positions [0, L_b - 1) of every row (and L_b - 1 too if asked)."""
        wl = self.wl
        ks, vs, slots, poss = [], [], [], []
        la_prefill = np.zeros(wl.num_slots, dtype=np.int32)
        pending = 0

        def flush():
            nonlocal ks, vs, slots, poss, pending
            if not ks:
                return
            k = torch.cat(ks).to(self.device)
            v = torch.cat(vs).to(self.device)
            s = torch.from_numpy(np.concatenate(slots).astype(np.int32)).to(self.device)
            p = torch.from_numpy(np.concatenate(poss).astype(np.int32)).to(self.device)
            la = torch.from_numpy(la_prefill).to(self.device)
            kv_quant_append(self.cache, k.contiguous(), v.contiguous(), s, p, self.block_table, la)
            ks, vs, slots, poss, pending = [], [], [], [], 0

        for b in range(self.B):
            L = int(self.lengths[b])
            if L == 0:
                continue
            k, v = self.kv_fn(b) if self.kv_fn is not None else seq_kv(wl, b, device=self.gen_device)
            if b in self.keep_host:
                self.host_kv[b] = (k.cpu(), v.cpu())
            self.step_k[b] = k[L - 1].to(self.device)
            self.step_v[b] = v[L - 1].to(self.device)
            n = L if include_step_token else L - 1
            slot = int(wl.slots[b])
            la_prefill[slot] = n
            if n == 0:
                continue
            ks.append(k[:n])
            vs.append(v[:n])
            slots.append(np.full(n, slot, dtype=np.int32))
            poss.append(np.arange(n, dtype=np.int32))
            pending += n
            if pending >= max_tokens_per_call:
                flush()
        flush()
        torch.cuda.synchronize(self.device)

    def append_step(self, stream=None):
        """Append the step token of every row with L_b >= 1 (position L_b - 1)."""
        if self._step_rows is None:
            rows = np.nonzero(self.lengths >= 1)[0]
            if len(rows) == self.B:
                self._step_rows = (self.step_k, self.step_v, self.slots, self.step_pos)
            else:
                r = torch.from_numpy(rows).to(self.device)
                self._step_rows = (self.step_k[r].contiguous(), self.step_v[r].contiguous(),
                                   self.slots[r].contiguous(), self.step_pos[r].contiguous())
        k, v, s, p = self._step_rows
        kv_quant_append(self.cache, k, v, s, p, self.block_table, self.len_after_step, stream=stream)

    def decode_step(self, stream=None):
        return kv_decode_attn(self.cache, self.q, self.slots, self.block_table, self.ctx_len,
                              out=self.out, lse=self.lse, workspace=self.workspace, stream=stream)

    def fused_step(self, stream=None):
        """append_step and decode_step in one launch (kv_append_decode_attn)."""
        return kv_append_decode_attn(self.cache, self.step_k, self.step_v, self.q, self.slots, self.block_table,
                                     self.ctx_len, out=self.out, lse=self.lse, workspace=self.workspace,
                                     stream=stream)

    # --- inspection helpers (host copies of what the GPU wrote) ----------------
    def int4_subblocks(self, idx: np.ndarray) -> np.ndarray:
        """Main-cache subblocks (INT4, or 3- / 2-bit when the cache holds such codes)."""
        from .layout import SUB2_BYTES, SUB3_BYTES, SUB4_BYTES, subg_bytes
        nb = {2: SUB2_BYTES, 3: SUB3_BYTES}.get(self.cache.code_bits, SUB4_BYTES)
        if self.cache.key_bits:
            nb = subg_bytes(self.cache.key_bits, self.cache.code_bits)
        pool = self.cache.int4_pool[: (self.cache.int4_pool.numel() // nb) * nb]
        t = torch.from_numpy(np.asarray(idx, np.int64)).to(self.device)
        return pool.view(-1, nb).index_select(0, t).cpu().numpy()

    def int8_subblocks(self, idx: np.ndarray) -> np.ndarray:
        from .layout import SUB8_BYTES
        pool = self.cache.int8_pool[: (self.cache.int8_pool.numel() // SUB8_BYTES) * SUB8_BYTES]
        t = torch.from_numpy(np.asarray(idx, np.int64)).to(self.device)
        return pool.view(-1, SUB8_BYTES).index_select(0, t).cpu().numpy()
