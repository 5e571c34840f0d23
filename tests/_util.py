"""Shared test helpers: build the oracle's cache and the library's cache from
the same seeded inputs, and compare outputs against the oracle."""
import math
import os
import re

import numpy as np
import torch

from oracle import pkv_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# tolerances (fixed by the attention-output contract for bf16 and E4M3 KV;
# fp32 bounds derived from fp32 accumulation over <= 1e3 keys)
TOL = {"f32": (1e-5, 1e-4), "bf16": (2e-3, 1e-2), "e4m3": (3e-2, 1e-2)}


def header_symbols():
    src = open(os.path.join(ROOT, "include", "pkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkv_[a-z0-9_]+)\s*\(", src)))


def bits(t):
    """bf16 tensor -> uint16 numpy bits (CPU)."""
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def kv_elements(t, fmt):
    """Source K/V tensor -> what the oracle's append takes for this cache format."""
    if fmt == "e4m3":
        return t.detach().cpu().float().numpy()
    if fmt == "bf16":
        return bits(t)
    return t.detach().cpu().numpy()


def frag_pages_logical(k_phys, v_phys, es):
    """Pool pages in the fragment order include/pkv.h documents (bf16: es 2,
    E4M3: es 1; arrays of elements [nb, hkv, 16*d] in any shape) -> logical
    K [nb, hkv, 16, d] and V [nb, hkv, d, 16] (the oracle's layout)."""
    k_phys, v_phys = np.asarray(k_phys), np.asarray(v_phys)
    nb, hkv = k_phys.shape[:2]
    D = k_phys[0, 0].size // 16
    t = np.arange(16)[:, None]
    d = np.arange(D)[None, :]
    c, g, n = d >> 5, (d >> 3) & 3, d >> 4
    cpp, npp = 2 // es, 4 // es
    koff = (c // cpp) * 1024 + ((g << 4) + t) * 16 + (c % cpp) * 8 * es + (d & 7) * es
    voff = (n // npp) * 1024 + (((t >> 2) << 4) + (d & 15)) * 16 + (n % npp) * 4 * es + (t & 3) * es
    assert np.all(koff % es == 0) and np.all(voff % es == 0)
    koff, voff = koff // es, voff // es                     # element offsets, [t, d]
    assert len(np.unique(koff)) == 16 * D and len(np.unique(voff)) == 16 * D
    kf = k_phys.reshape(nb, hkv, 16 * D)
    vf = v_phys.reshape(nb, hkv, 16 * D)
    return kf[:, :, koff], vf[:, :, voff].transpose(0, 1, 3, 2)


def q_elements(t):
    return (bits(t), "bf16") if t.dtype == torch.bfloat16 else (t.detach().cpu().numpy(), "f32")


def oracle_cache(cfg, inp, tables, heads=None, seqs=None):
    """Oracle pool filled sequence by sequence (bulk form of its append)."""
    fmt = cfg.kv_dtype
    cache = O.new_cache(cfg.pool_blocks, cfg.hkv, cfg.head_dim, fmt)
    k = kv_elements(inp["k"], fmt)
    v = kv_elements(inp["v"], fmt)
    start = 0
    for b, n in enumerate(cfg.seq_lens):
        if (seqs is None or b in seqs) and n > 0:
            if fmt == "e4m3":
                O.fp8_group_scales(k[start:start + n], 0, tables[b], cache.k_scale)
                O.fp8_group_scales(v[start:start + n], 0, tables[b], cache.v_scale)
            O.append_sequence(cache, k[start:start + n], v[start:start + n], tables[b], 0,
                              heads=heads)
        start += n
    return cache


def poison_for(fmt):
    return 0x7F if fmt == "e4m3" else float("nan")


def gpu_cache(lib, cfg, inp_dev, tables_dev, poison=True):
    """Library pool filled by pkv_fp8_group_scales + pkv_kv_append."""
    cache = lib.PagedCache.empty(cfg.pool_blocks, cfg.hkv, cfg.head_dim, cfg.kv_dtype,
                                 fill=poison_for(cfg.kv_dtype) if poison else None)
    if cfg.kv_dtype == "e4m3":
        start = 0
        for b, n in enumerate(cfg.seq_lens):
            if n > 0:
                lib.fp8_group_scales(cache, inp_dev["k"][start:start + n],
                                     inp_dev["v"][start:start + n], 0, tables_dev[b])
            start += n
    lib.kv_append(cache, inp_dev["k"], inp_dev["v"], inp_dev["seq_idx"], inp_dev["pos"],
                  tables_dev)
    return cache


def half_ulp(ref, out_fmt):
    """Half a unit in the last place of the output format at |ref| (the
    rounding every correct output of that format may carry)."""
    mant = {"bf16": 7, "f32": 23}[out_fmt]
    a = np.abs(ref)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, 2.0 ** (e - mant - 1), 0.0)


def compare_rows(got, ref, fmt, what="", out_fmt=None):
    """Max abs error and per-row inf-norm relative error against the oracle.

    The absolute bound applies on top of the output format's own rounding:
    |got - ref| <= atol + half_ulp(ref).  (A bf16 output of a value near 2 is
    already up to 3.9e-3 away from the exact value.)"""
    g = got.detach().double().cpu().numpy() if isinstance(got, torch.Tensor) else np.asarray(got)
    ref = np.asarray(ref, dtype=np.float64)
    atol, rrel = TOL[fmt]
    out_fmt = out_fmt or ("f32" if fmt == "f32" else "bf16")
    err = np.maximum(np.abs(g - ref) - half_ulp(ref, out_fmt), 0.0)
    max_abs = float(err.max()) if err.size else 0.0
    denom = np.abs(ref).max(axis=-1)
    rows = err.max(axis=-1)
    live = denom > 0
    row_rel = float((rows[live] / denom[live]).max()) if live.any() else 0.0
    assert np.all(np.isfinite(g)), f"{what}: non-finite output"
    assert np.all(rows[~live] == 0), f"{what}: rows with no keys must be exactly 0"
    assert max_abs <= atol, f"{what}: max abs err {max_abs:.3e} > {atol}"
    assert row_rel <= rrel, f"{what}: row-relative err {row_rel:.3e} > {rrel}"
    return max_abs, row_rel
