"""The five decode workloads and one prefill workload, each named by what it is and its sizes.

Lengths ``L_b`` always count the token appended in the timed decode step.
Shapes follow the Qwen3-4B / Qwen3-8B / Qwen2.5-3B attention layouts the
KV4-RL page (Main Findings) and the Block-GTQ page (Abstract) evaluate on;
page size 16 is the vLLM block size the KV-streams page mentions.
"""

from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class WorkloadConfig:
    name: str
    batch: int              # decode rows (= occupied slots)
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    lengths: str            # length recipe key, see workloads.gen.draw_lengths
    length_args: tuple
    page_size: int
    had_block: int          # Hadamard block size h
    sink: int               # s
    recent: int             # w
    paged: bool = True      # False: one page per sequence, identity block table
    append_each_step: bool = True
    seed: int = 1000
    outlier_channels: int = 4
    outlier_scale: float = 20.0
    rope_base: float = 1.0e6
    code_bits: int = 4      # width of the main cache's codes (4, or 3 or 2 for the sub-4-bit caches)
    key_bits: tuple = ()    # key width per RoPE-block group (four of 2-4; values keep code_bits), or ()
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def scaled(self, **kw) -> "WorkloadConfig":
        """Same recipe with some fields replaced (used for small parity cases)."""
        return replace(self, **kw)


CONFIGS: dict[str, WorkloadConfig] = {
    # Tiny single decode step, non-paged; the case the oracle finishes in seconds.
    "tiny_1x1024": WorkloadConfig(
        name="tiny_1x1024", batch=1, num_q_heads=8, num_kv_heads=2, head_dim=128,
        lengths="fixed", length_args=(1024,), page_size=1024, had_block=128,
        sink=4, recent=64, paged=False, append_each_step=False, seed=1000),
    # Qwen3-4B-shaped decode batch, lognormal lengths (median 2K, sigma 1).
    "qwen3_4b_b64": WorkloadConfig(
        name="qwen3_4b_b64", batch=64, num_q_heads=32, num_kv_heads=8, head_dim=128,
        lengths="lognormal", length_args=(2048, 1.0, 256, 16384), page_size=16,
        had_block=64, sink=4, recent=128, seed=1001),
    # Qwen3-8B-shaped async-rollout heavy step: 256 slots, Pareto(1.5) lengths.
    "qwen3_8b_async_256": WorkloadConfig(
        name="qwen3_8b_async_256", batch=256, num_q_heads=32, num_kv_heads=8, head_dim=128,
        lengths="pareto", length_args=(512, 1.5, 32768), page_size=16,
        had_block=128, sink=4, recent=128, seed=1002),
    # Long-context split-K stress: one 128K sequence, Qwen2.5-3B heads (GQA 8).
    "long_128k": WorkloadConfig(
        name="long_128k", batch=1, num_q_heads=16, num_kv_heads=2, head_dim=128,
        lengths="fixed", length_args=(131072,), page_size=64, had_block=128,
        sink=4, recent=256, seed=1003),
    # Continuous-refill mixed step: 512 slots, uniform lengths, 20% fresh (< 64).
    "refill_512": WorkloadConfig(
        name="refill_512", batch=512, num_q_heads=32, num_kv_heads=8, head_dim=128,
        lengths="refill", length_args=(1, 32768, 0.2, 63), page_size=16,
        had_block=64, sink=4, recent=128, seed=1004),
    # Re-prefill of in-flight rollouts after a policy update (KV4-RL, "Future
    # Directions"): Qwen3-8B heads, 8 sequences of uniform length in [4K, 12K];
    # the last extra["chunk"] positions of each are attended again as one chunk
    # of causal query rows over the quantized cache.
    "prefill_qwen3_8b_8x1024": WorkloadConfig(
        name="prefill_qwen3_8b_8x1024", batch=8, num_q_heads=32, num_kv_heads=8, head_dim=128,
        lengths="uniform", length_args=(4096, 12288), page_size=16,
        had_block=128, sink=4, recent=128, seed=1005, extra={"chunk": 1024}),
}

# Order used when a config is referred to by position.
CONFIG_ORDER = ["tiny_1x1024", "qwen3_4b_b64", "qwen3_8b_async_256", "long_128k", "refill_512"]


def get_config(name_or_index) -> WorkloadConfig:
    if isinstance(name_or_index, int):
        return CONFIGS[CONFIG_ORDER[name_or_index]]
    return CONFIGS[name_or_index]
