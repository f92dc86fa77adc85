"""The five workloads the path is checked and measured on.

Shapes follow the attention shapes of the models the pages discuss: a
Llama-3-8B-shaped layer (32 q-heads / 8 KV heads, head dim 128), a
Qwen3-32B-like layer (64 / 8, 128; 256 KiB of KV per token over 64 layers,
the H20 measurement in [EPD] "KV-Cache 传输"), and a LLaMA-3-70B KV shape
(80 layers, 8 KV heads, 128; 320 KiB per token, 1.34 GB for a 4K prompt in
[DISAGG] "传输的代价").  Block sizes 16 and 32 are the prefill and decode
instances of [DISAGG] "实现"; head shards of 2 and 1 heads are TP 4 and
TP 8 of 8 KV heads ([DISAGG] "布局转换").
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import inputs


@dataclass(frozen=True)
class Workload:
    config_id: int
    name: str
    layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    dtype: str                      # "bf16" or "f32"
    input_scale: float
    pool_blocks: int
    decode_batch: int = 0
    decode_context: tuple = ()      # fixed contexts (empty -> drawn, see below)
    decode_context_range: tuple = ()  # (lo, hi) inclusive uniform draw
    prompt_len: int = 0
    chunk_sizes: tuple = ()
    seed: int = 0
    # relayout (config 4 and the tiny check)
    src_shards: int = 1
    dst_block_size: int = 0
    dst_shards: int = 1
    dst_pool_blocks: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def decode_contexts(self) -> np.ndarray:
        if self.decode_context:
            return np.array(self.decode_context, dtype=np.int32)
        if self.decode_context_range:
            lo, hi = self.decode_context_range
            g = inputs.stream(self.seed, self.config_id, 0, inputs.T_CTX)
            return g.integers(lo, hi + 1, size=self.decode_batch, dtype=np.int64).astype(np.int32)
        return np.zeros(0, dtype=np.int32)


TINY = Workload(
    config_id=1, name="tiny-fp32", layers=1, num_q_heads=4, num_kv_heads=2, head_dim=64,
    block_size=16, dtype="f32", input_scale=1.0, pool_blocks=64,
    decode_batch=4, decode_context=(37, 64, 100, 128), prompt_len=256, chunk_sizes=(64,),
    src_shards=1, dst_block_size=32, dst_shards=2, dst_pool_blocks=32,
)

LLAMA3_8B = Workload(
    config_id=2, name="llama3-8b-attn", layers=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
    block_size=16, dtype="bf16", input_scale=0.5, pool_blocks=8192,
    decode_batch=64, decode_context=(512,) * 64, prompt_len=1024, chunk_sizes=(512,),
    src_shards=4, dst_block_size=32, dst_shards=8, dst_pool_blocks=4096,
)

QWEN3_32B = Workload(
    config_id=3, name="qwen3-32b-attn", layers=64, num_q_heads=64, num_kv_heads=8, head_dim=128,
    block_size=16, dtype="bf16", input_scale=0.5, pool_blocks=16384,
    decode_batch=16, decode_context_range=(2048, 8192), prompt_len=16384, chunk_sizes=(2048, 512),
)

RELAYOUT_70B = Workload(
    config_id=4, name="relayout-llama3-70b", layers=80, num_q_heads=64, num_kv_heads=8, head_dim=128,
    block_size=16, dtype="bf16", input_scale=0.5, pool_blocks=256, prompt_len=4096,
    src_shards=4, dst_block_size=32, dst_shards=8, dst_pool_blocks=128,
)

PDMUX_8B = Workload(
    config_id=5, name="pdmux-llama3-8b", layers=32, num_q_heads=32, num_kv_heads=8, head_dim=128,
    block_size=16, dtype="bf16", input_scale=0.5, pool_blocks=32768,
    decode_batch=128, decode_context=(2048,) * 128, prompt_len=32768, chunk_sizes=(2048, 512),
    extra={"prompt_variant": 16384, "total_cus": 256, "cu_granularity": 8, "min_decode_cus": 32,
           "group_num": 8, "decode_bs_divisor": 36, "token_budget": 65536,
           # stall-free token budgets: the pages' strict (512) and loose (2048) settings
           "stall_free_budgets": (2048, 512)},
)

ALL = {w.config_id: w for w in (TINY, LLAMA3_8B, QWEN3_32B, RELAYOUT_70B, PDMUX_8B)}
