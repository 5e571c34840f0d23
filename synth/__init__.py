"""Seeded synthetic inputs for the paged-KV attention workloads.

This module is shared by the CPU oracle side (tests) and the HIP path (tests,
bench, smoke).  It holds shapes, seeds and random draws only: no attention,
paging, quantisation or merge arithmetic lives here, so neither side can
borrow the other's method code through it.

Workloads (all synthetic, values ~N(0,1)):

* ``C1``  tiny decode: 2 sequences of 37 and 100 tokens, 4 q / 2 kv heads,
  head_dim 64, fp32, 32-block pool.
* ``C2``  Llama-3-8B-like layer decode: 32 x 8192 tokens, 32 q / 8 kv heads,
  head_dim 128, bf16, pool = need + 10 %.
* ``C3``  70B-like long-context decode: 4 x 131072 tokens, 64 q / 8 kv heads,
  bf16, 256-block split-KV partitions.
* ``C4``  chunked causal prefill: one 32768-token prompt in 4096-token query
  chunks, 32 q / 8 kv heads, bf16, KV split in 4 sequential 8192-token shards.
* ``C4_128K`` the same prefill at a 131072-token prompt.
* ``C5``  1M-token decode, 64 q / 8 kv heads, bf16 queries, K/V stored as
  E4M3 with one fp32 scale per 64 tokens per kv head; 1 % of K/V elements are
  multiplied by 8 (outliers).
"""
from .configs import (DecodeConfig, PrefillConfig, CONFIGS, decode_config,
                      prefill_config, blocks_needed, pool_with_spare)
from .gen import (generator, free_order, decode_inputs, prefill_inputs,
                  token_positions)

__all__ = [
    "DecodeConfig", "PrefillConfig", "CONFIGS", "decode_config",
    "prefill_config", "blocks_needed", "pool_with_spare", "generator",
    "free_order", "decode_inputs", "prefill_inputs", "token_positions",
]
