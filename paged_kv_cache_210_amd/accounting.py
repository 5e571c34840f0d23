"""Algorithmic work of the paged-attention path (bytes that must move, flops
that must be done), used to place measured times on the MI355X roofline.

Implementation-only traffic (split-KV partials, shard partials, re-reads) is
never counted here: it is what the roofline fraction is meant to expose.
"""
from __future__ import annotations

ELEM_BYTES = {"f32": 4, "bf16": 2, "e4m3": 1}
BLOCK = 16
SCALE_GROUP = 64

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor spec
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, vendor spec
PCIE_PEAK_GBS = 64.0            # PCIe 5.0 x16 host link, per direction (32 GT/s x 16 lanes)


def block_bytes(hkv, head_dim, kv_dtype):
    """K + V bytes of one physical block (all kv heads), plus its two fp32
    scales per kv head for E4M3 pools: what pkv_copy_blocks moves per block."""
    b = 2 * hkv * 16 * head_dim * ELEM_BYTES[kv_dtype]
    return b + (2 * hkv * 4 if kv_dtype == "e4m3" else 0)


def kv_cache_bytes(layers, kv_heads, head_dim, tokens=1, elem_bytes=2):
    """K and V for ``tokens`` tokens over ``layers`` layers."""
    return 2 * layers * kv_heads * head_dim * elem_bytes * tokens


def ring_step_bytes(batch, heads, local_seq_len, head_dim, elem_bytes=2):
    """K and V of one sequence shard, as sent in one rotation step."""
    return 2 * batch * heads * local_seq_len * head_dim * elem_bytes


def decode_kernel_bytes(seq_lens, hq, hkv, head_dim, q_dtype, kv_dtype):
    """Bytes the split-KV decode kernel must read: every live K/V element once,
    the queries, one table entry per block, the lengths, and (E4M3) one fp32
    scale per 64 tokens per kv head for K and for V."""
    e = ELEM_BYTES[kv_dtype]
    toks = sum(int(n) for n in seq_lens)
    kv = 2 * toks * hkv * head_dim * e
    q = len(seq_lens) * hq * head_dim * ELEM_BYTES[q_dtype]
    table = 4 * sum(-(-int(n) // BLOCK) for n in seq_lens)
    lens = 4 * len(seq_lens)
    scales = 0
    if kv_dtype == "e4m3":
        scales = 2 * 4 * hkv * sum(-(-int(n) // SCALE_GROUP) for n in seq_lens)
    return kv + q + table + lens + scales


def append_bytes(tokens, hkv, head_dim, kv_dtype, src_dtype=None):
    """kv_append of `tokens` tokens: read each token's K and V rows, write them
    into the pool, read its sequence index and position (table reads, one int32
    per token at most, are left out)."""
    src = src_dtype or ("bf16" if kv_dtype == "e4m3" else kv_dtype)
    return tokens * hkv * head_dim * 2 * (ELEM_BYTES[src] + ELEM_BYTES[kv_dtype]) + 8 * tokens


def decode_step_bytes(seq_lens, hq, hkv, head_dim, q_dtype, kv_dtype, src_dtype=None):
    """One decode step: append one token per sequence (read its K/V, write it
    into the pool) plus the attention read, plus writing O."""
    B = len(seq_lens)
    append = append_bytes(B, hkv, head_dim, kv_dtype, src_dtype)
    out = B * hq * head_dim * ELEM_BYTES[q_dtype]
    return append + decode_kernel_bytes(seq_lens, hq, hkv, head_dim, q_dtype, kv_dtype) + out


def visible_pairs(q_pos0, q_len, kv_begin, kv_end, causal=True):
    """Number of (query row, key) pairs a prefill call must score."""
    total = 0
    if not causal:
        return q_len * max(0, kv_end - kv_begin)
    for r in range(q_len):
        hi = min(kv_end, q_pos0 + r + 1)
        total += max(0, hi - kv_begin)
    return total


def prefill_flops(q_pos0, q_len, kv_begin, kv_end, hq, head_dim, causal=True):
    """QK^T and PV: 2 * 2 * d flops per visible (row, key) pair per q head."""
    return 4 * head_dim * hq * visible_pairs(q_pos0, q_len, kv_begin, kv_end, causal)


def causal_prompt_flops(prompt_len, hq, head_dim):
    return 4 * head_dim * hq * (prompt_len * (prompt_len + 1) // 2)
