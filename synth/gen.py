"""Seeded random draws for the workloads.

Recipe (both sides see identical bytes):

* values: one ``torch.Generator`` seeded with ``data_seed`` on the device the
  data is made on; draws in the order q, k, v with ``torch.randn`` in float32,
  then rounded to bf16 (round-to-nearest-even) where the dtype is bf16;
* outliers (FP8 workload): a second generator seeded with ``outlier_seed``
  draws ``torch.rand`` for k then v; elements below ``outlier_prob`` are
  multiplied by ``outlier_mult``, before the bf16 rounding;
* physical block order: ``torch.randperm(pool_blocks)`` from a CPU generator
  seeded with ``perm_seed``; blocks are handed out in that order.

Large workloads are drawn on the GPU (``device="cuda"``) and copied to the
host for the oracle, so both see the same bytes; small ones are drawn on CPU.
"""
from __future__ import annotations

import torch

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def free_order(pool_blocks: int, seed: int) -> torch.Tensor:
    """Seeded permutation of the physical block ids (int32, CPU)."""
    return torch.randperm(int(pool_blocks), generator=generator(seed)).to(torch.int32)


def token_positions(seq_lens):
    """(seq_idx, pos) int32 arrays listing every token, sequence-major."""
    seq_idx = torch.cat([torch.full((int(n),), b, dtype=torch.int32)
                         for b, n in enumerate(seq_lens)]) if len(seq_lens) else torch.zeros(0, dtype=torch.int32)
    pos = torch.cat([torch.arange(int(n), dtype=torch.int32) for n in seq_lens]) \
        if len(seq_lens) else torch.zeros(0, dtype=torch.int32)
    return seq_idx, pos


def _randn(shape, g, device):
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def _outliers(cfg, k, v, device):
    go = generator(cfg.outlier_seed, device)
    mk = torch.rand(k.shape, generator=go, device=device) < cfg.outlier_prob
    k = torch.where(mk, k * cfg.outlier_mult, k)
    del mk
    mv = torch.rand(v.shape, generator=go, device=device) < cfg.outlier_prob
    v = torch.where(mv, v * cfg.outlier_mult, v)
    return k, v


def decode_inputs(cfg, device="cpu"):
    """q [B,Hq,d], k/v [T,Hkv,d] for every token of every sequence, seq_idx/pos [T].

    The source K/V dtype is bf16 for the E4M3 workload (quantised on append)."""
    g = generator(cfg.data_seed, device)
    T = cfg.num_tokens
    q = _randn((cfg.batch, cfg.hq, cfg.head_dim), g, device)
    k = _randn((T, cfg.hkv, cfg.head_dim), g, device)
    v = _randn((T, cfg.hkv, cfg.head_dim), g, device)
    if cfg.outlier_prob > 0:
        k, v = _outliers(cfg, k, v, device)
    src_dt = _DT["bf16"] if cfg.kv_dtype == "e4m3" else _DT[cfg.kv_dtype]
    seq_idx, pos = token_positions(cfg.seq_lens)
    return {
        "q": q.to(_DT[cfg.q_dtype]),
        "k": k.to(src_dt),
        "v": v.to(src_dt),
        "seq_idx": seq_idx,
        "pos": pos,
        "free_order": free_order(cfg.pool_blocks, cfg.perm_seed),
    }


def prefill_inputs(cfg, device="cpu"):
    """q [S,Hq,d], k/v [S,Hkv,d] for the whole prompt of one sequence."""
    g = generator(cfg.data_seed, device)
    S = cfg.prompt_len
    q = _randn((S, cfg.hq, cfg.head_dim), g, device).to(_DT[cfg.dtype])
    k = _randn((S, cfg.hkv, cfg.head_dim), g, device)
    v = _randn((S, cfg.hkv, cfg.head_dim), g, device)
    if cfg.outlier_prob > 0:
        k, v = _outliers(cfg, k, v, device)
    return {"q": q, "k": k.to(_DT[cfg.dtype]), "v": v.to(_DT[cfg.dtype]),
            "free_order": free_order(cfg.pool_blocks, cfg.perm_seed)}
