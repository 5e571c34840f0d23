"""Shapes and seeds of the synthetic workloads (no method arithmetic)."""
from __future__ import annotations

from dataclasses import dataclass, field, replace
import math

BLOCK_SIZE = 16


def blocks_needed(seq_lens, block_size: int = BLOCK_SIZE) -> int:
    """Total number of whole blocks that hold ``seq_lens`` tokens."""
    return sum(-(-int(n) // block_size) for n in seq_lens)


def pool_with_spare(need: int, spare: float = 0.10) -> int:
    """Pool size with a fraction of spare blocks on top of what is needed."""
    return need + int(math.ceil(spare * need))


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    seq_lens: tuple
    hq: int
    hkv: int
    head_dim: int
    q_dtype: str            # "f32" | "bf16"
    kv_dtype: str           # "f32" | "bf16" | "e4m3"
    pool_blocks: int
    partition_blocks: int = 0      # 0 = let the library choose
    data_seed: int = 1000
    perm_seed: int = 2000
    outlier_seed: int = 3000
    outlier_prob: float = 0.0
    outlier_mult: float = 8.0
    scale_group: int = 64          # tokens per FP8 scale (e4m3 only)
    block_size: int = BLOCK_SIZE

    @property
    def batch(self) -> int:
        return len(self.seq_lens)

    @property
    def num_tokens(self) -> int:
        return int(sum(self.seq_lens))

    @property
    def max_blocks_per_seq(self) -> int:
        return max(-(-int(n) // self.block_size) for n in self.seq_lens) if self.seq_lens else 0

    def with_(self, **kw) -> "DecodeConfig":
        return replace(self, **kw)


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    prompt_len: int
    chunk: int
    shard_len: int
    hq: int
    hkv: int
    head_dim: int
    dtype: str              # "bf16" (q, and the K/V source values)
    pool_blocks: int
    data_seed: int = 1000
    perm_seed: int = 2000
    kv_dtype: str = "bf16"  # "bf16" | "e4m3" (pool format)
    outlier_seed: int = 3000
    outlier_prob: float = 0.0
    outlier_mult: float = 8.0
    scale_group: int = 64          # tokens per FP8 scale (e4m3 only)
    block_size: int = BLOCK_SIZE

    @property
    def num_chunks(self) -> int:
        return -(-self.prompt_len // self.chunk)

    @property
    def num_shards(self) -> int:
        return -(-self.prompt_len // self.shard_len)

    def with_(self, **kw) -> "PrefillConfig":
        return replace(self, **kw)


def decode_config(name, seq_lens, hq, hkv, head_dim, q_dtype="bf16", kv_dtype=None,
                  pool_blocks=None, seed_index=0, **kw) -> DecodeConfig:
    """A decode workload; the pool defaults to what is needed plus 10 % spare."""
    kv_dtype = kv_dtype or q_dtype
    if pool_blocks is None:
        pool_blocks = pool_with_spare(blocks_needed(seq_lens))
    return DecodeConfig(name=name, seq_lens=tuple(int(n) for n in seq_lens), hq=hq, hkv=hkv,
                        head_dim=head_dim, q_dtype=q_dtype, kv_dtype=kv_dtype,
                        pool_blocks=pool_blocks, data_seed=1000 + seed_index,
                        perm_seed=2000 + seed_index, outlier_seed=3000 + seed_index, **kw)


def prefill_config(name, prompt_len, chunk, shard_len, hq, hkv, head_dim, dtype="bf16",
                   pool_blocks=None, seed_index=0, **kw) -> PrefillConfig:
    if pool_blocks is None:
        pool_blocks = pool_with_spare(blocks_needed([prompt_len]))
    return PrefillConfig(name=name, prompt_len=prompt_len, chunk=chunk, shard_len=shard_len,
                         hq=hq, hkv=hkv, head_dim=head_dim, dtype=dtype, pool_blocks=pool_blocks,
                         data_seed=1000 + seed_index, perm_seed=2000 + seed_index,
                         outlier_seed=3000 + seed_index, **kw)


CONFIGS = {
    "C1": decode_config("C1 tiny decode", (37, 100), 4, 2, 64, q_dtype="f32",
                        pool_blocks=32, seed_index=1),
    "C2": decode_config("C2 Llama-3-8B-like decode B32x8192", (8192,) * 32, 32, 8, 128,
                        seed_index=2),
    "C3": decode_config("C3 70B-like decode B4x131072", (131072,) * 4, 64, 8, 128,
                        partition_blocks=256, seed_index=3),
    "C4": prefill_config("C4 chunked causal prefill 32768", 32768, 4096, 8192, 32, 8, 128,
                         seed_index=4),
    "C4_128K": prefill_config("C4 chunked causal prefill 131072", 131072, 4096, 32768, 32, 8,
                              128, seed_index=6),
    # the 32K chunked prefill over an E4M3 pool (the FP8 KV format of the 1M
    # decode: one scale per 64 tokens per kv head, 1 % of values x8)
    "C4_FP8": prefill_config("C4 chunked causal prefill 32768, E4M3 KV", 32768, 4096, 8192, 32,
                             8, 128, seed_index=7, kv_dtype="e4m3", outlier_prob=0.01,
                             outlier_mult=8.0),
    "C5": decode_config("C5 1M-context FP8-KV decode", (1048576,), 64, 8, 128, q_dtype="bf16",
                        kv_dtype="e4m3", partition_blocks=256, seed_index=5,
                        outlier_prob=0.01, outlier_mult=8.0),
}
