#!/usr/bin/env python3
"""Throughput of the paged-attention hot path on one MI355X.

A decode step is one pass of the whole decode path over one batch: append the
newest token of every sequence into the paged pool (pkv_kv_append), then
split-KV attention of that token against every cached key plus the exact
log-sum-exp merge (pkv_paged_attn_decode).  Inputs are resident in HBM before
the timed region starts.

The headline line is the Llama-3-8B-like layer (32 sequences x 8192 tokens,
32 q / 8 kv heads, d 128, bf16).  The 128K decode, the 1M-token E4M3 decode and
the chunked causal prefill are reported under "secondary".  The fp64 CPU oracle
is timed on a bounded sample of the headline workload as "cpu_baseline".

    python bench.py [--gpus 1] [--steps 20] [--warmup 3]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode tok/s + HBM GB/s (% peak); prefill TFLOPS (% MFMA peak) @128K"


def _log(msg):
    print(msg, file=sys.stderr, flush=True)


def _decode_setup(cfg, partition_blocks):
    import torch
    from paged_kv_cache_210_amd import lib
    import synth

    dev = "cuda"
    inp = synth.decode_inputs(cfg, device=dev)
    tables, _ = lib.build_tables(cfg.seq_lens, cfg.pool_blocks, inp["free_order"])
    td = tables.to(dev)
    cache = lib.PagedCache.empty(cfg.pool_blocks, cfg.hkv, cfg.head_dim, cfg.kv_dtype, device=dev)
    lens_l = list(cfg.seq_lens)
    ends = torch.tensor(lens_l, device=dev).cumsum(0) - 1          # newest token of each seq
    keep = torch.ones(cfg.num_tokens, dtype=torch.bool, device=dev)
    keep[ends] = False
    seq_idx, pos = inp["seq_idx"].to(dev), inp["pos"].to(dev)
    if cfg.kv_dtype == "e4m3":
        start = 0
        for b, n in enumerate(lens_l):
            lib.fp8_group_scales(cache, inp["k"][start:start + n], inp["v"][start:start + n], 0,
                                 td[b])
            start += n
    lib.kv_append(cache, inp["k"][keep].contiguous(), inp["v"][keep].contiguous(), seq_idx[keep].contiguous(),
                  pos[keep].contiguous(), td)
    step_in = {
        "k": inp["k"][ends].contiguous(), "v": inp["v"][ends].contiguous(),
        "seq": torch.arange(cfg.batch, dtype=torch.int32, device=dev),
        "pos": torch.tensor([n - 1 for n in lens_l], dtype=torch.int32, device=dev),
    }
    # a second pool with the same contents: timed steps alternate between the
    # two, so a step's pages were last read two steps earlier, with the whole
    # other pool (1 GiB or more) read in between, and none of them is still in
    # L2 or the last-level cache
    twin = lib.PagedCache(cache.k.clone(), cache.v.clone(), cache.kv_dtype,
                          None if cache.k_scale is None else cache.k_scale.clone(),
                          None if cache.v_scale is None else cache.v_scale.clone())
    q = inp["q"]
    lens = torch.tensor(lens_l, dtype=torch.int32, device=dev)
    P = lib.decode_partitions(cache, q.dtype, cfg.batch, cfg.hq, td.shape[1], partition_blocks)
    part = (torch.empty(P, cfg.batch, cfg.hq, cfg.head_dim, dtype=torch.float32, device=dev),
            torch.empty(P, cfg.batch, cfg.hq, dtype=torch.float32, device=dev),
            torch.empty(P, cfg.batch, cfg.hq, dtype=torch.float32, device=dev))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=dev)
    del inp, keep
    torch.cuda.synchronize()
    # the folded step needs bf16 q, a bf16 or E4M3 pool and at most 16 query
    # heads per kv head
    folded = (cfg.q_dtype == "bf16" and cfg.kv_dtype in ("bf16", "e4m3") and
              cfg.hq // cfg.hkv <= 16)
    return dict(cache=cache, caches=(cache, twin), td=td, q=q, lens=lens, part=part, out=out,
                lse=lse, step_in=step_in, tables=tables, partitions=P, folded=folded)


def bench_decode(cfg, steps, warmup, partition_blocks=0):
    """Returns (ms per step, ms per split-KV decode kernel, ms per merge, state).

    A step appends the newest token of every sequence and attends with it:
    pkv_paged_attn_decode_step_partial (the append folded into the decode
    launch) + pkv_attn_lse_merge, the launches of pkv_paged_attn_decode_step
    (shapes it refuses would take pkv_kv_append + pkv_paged_attn_decode_partial
    + pkv_attn_lse_merge).  In the timed steps two events bracket the decode
    launch, so the dominant kernel is timed on its own; the merge launch is
    timed in a pass of its own afterwards, and so is the step with no events
    at all (reported beside, not as the value: each event recorded between
    launches costs a few microseconds).  Steps alternate between two pools
    holding the same KV, so no step reads pages still cached from the one
    before."""
    import torch
    from paged_kv_cache_210_amd import lib

    st = _decode_setup(cfg, partition_blocks)
    s = st["step_in"]
    po, pm, pl = st["part"]
    it = [0]

    def step(dec_ev=None, merge_ev=None):
        cache = st["caches"][it[0] % 2]
        it[0] += 1
        if st["folded"]:
            if dec_ev is not None:
                dec_ev[0].record()
            lib.paged_attn_decode_step(cache, s["k"], s["v"], st["q"], st["td"], st["lens"],
                                       partition_blocks=partition_blocks, partial=True,
                                       part=st["part"])
        else:
            lib.kv_append(cache, s["k"], s["v"], s["seq"], s["pos"], st["td"])
            if dec_ev is not None:
                dec_ev[0].record()
            lib.paged_attn_decode_partial(cache, st["q"], st["td"], st["lens"],
                                          partition_blocks=partition_blocks, part=st["part"])
        if dec_ev is not None:
            dec_ev[1].record()
        if merge_ev is not None:
            merge_ev[0].record()
        lib.attn_lse_merge(po, pm, pl, out=st["out"], with_state=False, out_lse=st["lse"])
        if merge_ev is not None:
            merge_ev[1].record()

    def timed(k, dec=False, merge=False):
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(k)]
        mevs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(k)]
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        start.record()
        for i in range(k):
            step(evs[i] if dec else None, mevs[i] if merge else None)
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) / k, evs, mevs

    for _ in range(warmup):
        step()
    # the timed steps: events only around the decode launch (each event
    # recorded between launches adds a few microseconds to a step)
    ms_step, evs, _ = timed(steps, dec=True)
    dec = sorted(e[0].elapsed_time(e[1]) for e in evs)
    st["decode_ms_median"], st["decode_ms_min"] = dec[len(dec) // 2], dec[0]
    ms_dec = sum(dec) / steps
    # after the timed steps: the merge launch on its own, and the step with no
    # events at all
    _, _, mevs = timed(steps, merge=True)
    ms_merge = sum(e[0].elapsed_time(e[1]) for e in mevs) / steps
    st["ms_per_step_no_events"], _, _ = timed(steps)
    return ms_step, ms_dec, ms_merge, st


def decode_record(cfg, steps, warmup, partition_blocks):
    from paged_kv_cache_210_amd import accounting as A

    ms_step, ms_dec, ms_merge, st = bench_decode(cfg, steps, warmup, partition_blocks)
    kbytes = A.decode_kernel_bytes(cfg.seq_lens, cfg.hq, cfg.hkv, cfg.head_dim, cfg.q_dtype,
                                   cfg.kv_dtype)
    step_bytes = A.decode_step_bytes(cfg.seq_lens, cfg.hq, cfg.hkv, cfg.head_dim, cfg.q_dtype,
                                     cfg.kv_dtype)
    if st["folded"]:       # the folded append reads the new K/V and writes it into the pool
        kbytes += A.append_bytes(cfg.batch, cfg.hkv, cfg.head_dim, cfg.kv_dtype) - 8 * cfg.batch
    gbs = kbytes / (ms_dec * 1e-3) / 1e9
    rec = {
        "workload": cfg.name,
        "tok_per_s": cfg.batch / (ms_step * 1e-3),
        "ms_per_step": ms_step,
        "step_hbm_gbs": step_bytes / (ms_step * 1e-3) / 1e9,
        "merge_ms": ms_merge,
        "ms_per_step_no_events": st["ms_per_step_no_events"],
        "partitions": st["partitions"],
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": A.HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / A.HBM_PEAK_GBS, "traffic": measured_traffic(cfg),
                     "kernel": ("decode_mfma_kernel with the append folded in "
                                "(pkv_paged_attn_decode_step_partial)" if st["folded"] else
                                "decode_mfma_kernel (pkv_paged_attn_decode_partial)"),
                     "ms_per_launch": ms_dec, "ms_per_launch_median": st["decode_ms_median"],
                     "ms_per_launch_min": st["decode_ms_min"], "bytes_per_launch": kbytes},
    }
    return rec, st


def measured_traffic(cfg):
    """HBM bytes per launch of the decode kernel from the committed counter
    runs (profiles/decode_hbm_traffic.json), or None when the kernel source has
    changed since they were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "decode_hbm_traffic.json")
    src = os.path.join(ROOT, "paged_kv_cache_210_amd", "csrc", "decode.hip")
    key = {"C2": "C2", "C3": "C3", "C5": "C5"}.get(cfg.name.split()[0])
    try:
        rec = json.load(open(path))
        if hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["kernel_source_sha256"]:
            return None
        return rec["workloads"][key]["traffic_bytes"]
    except (OSError, KeyError, ValueError):
        return None


def _prefill_setup(cfg):
    import torch
    from paged_kv_cache_210_amd import lib
    import synth

    dev = "cuda"
    inp = synth.prefill_inputs(cfg, device=dev)
    tables, _ = lib.build_tables([cfg.prompt_len], cfg.pool_blocks, inp["free_order"])
    td = tables.to(dev)
    cache = lib.PagedCache.empty(cfg.pool_blocks, cfg.hkv, cfg.head_dim, cfg.kv_dtype, device=dev)
    C, S = cfg.chunk, cfg.shard_len
    max_parts = -(-cfg.prompt_len // S)
    part = (torch.empty(max_parts, C, cfg.hq, cfg.head_dim, dtype=torch.float32, device=dev),
            torch.empty(max_parts, C, cfg.hq, dtype=torch.float32, device=dev),
            torch.empty(max_parts, C, cfg.hq, dtype=torch.float32, device=dev))
    out = torch.empty_like(inp["q"])
    lse1 = torch.empty(C, cfg.hq, dtype=torch.float32, device=dev)
    pos = torch.arange(cfg.prompt_len, dtype=torch.int32, device=dev)
    seq = torch.zeros(C, dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    return dict(inp=inp, td=td, cache=cache, part=part, out=out, lse1=lse1, pos=pos, seq=seq)


def prefill_pass(cfg, st, ev=None):
    """One chunked pass over the prompt: per chunk append its K/V (for an E4M3
    pool: first the chunk's 64-token group scales), attend to each visible KV
    shard (partial form), merge the shards by LSE; a chunk that sees a single
    shard is attended in the final form, with nothing to merge."""
    from paged_kv_cache_210_amd import lib

    C, S = cfg.chunk, cfg.shard_len
    inp, td, cache, (po, pm, pl) = st["inp"], st["td"], st["cache"], st["part"]
    for c in range(cfg.num_chunks):
        a, b = c * C, min((c + 1) * C, cfg.prompt_len)
        if ev is not None:
            ev.append(("append", c))
        if cfg.kv_dtype == "e4m3":
            lib.fp8_group_scales(cache, inp["k"][a:b], inp["v"][a:b], a, td[0])
        lib.kv_append(cache, inp["k"][a:b], inp["v"][a:b], st["seq"][:b - a], st["pos"][a:b], td)
        q = inp["q"][a:b]
        nsh = -(-b // S)
        if ev is not None:
            ev.append(("start", c))
        if nsh == 1:          # one shard holds every visible key: nothing to merge
            lib.paged_attn_prefill(cache, q, a, td[0], 0, b, True, out=st["out"][a:b],
                                   out_lse=st["lse1"][:b - a])
        else:
            for j in range(nsh):
                lib.paged_attn_prefill(cache, q, a, td[0], j * S, min((j + 1) * S, b), True,
                                       partial=True,
                                       part=(po[j, :b - a], pm[j, :b - a], pl[j, :b - a]))
            lib.attn_lse_merge(po[:nsh, :b - a], pm[:nsh, :b - a], pl[:nsh, :b - a],
                               out=st["out"][a:b], with_state=False)
        if ev is not None:
            ev.append(("end", c))


def prefill_record(cfg, reps):
    import torch
    from paged_kv_cache_210_amd import accounting as A

    st = _prefill_setup(cfg)
    prefill_pass(cfg, st)                      # warm-up pass
    torch.cuda.synchronize()
    marks = []
    events = {}

    class _Ev(list):
        def append(self, item):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            events[item] = e

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    attn_ms = append_ms = 0.0
    start.record()
    for _ in range(reps):
        events.clear()
        ev = _Ev()
        prefill_pass(cfg, st, ev)
        torch.cuda.synchronize()
        attn_ms += sum(events[("start", c)].elapsed_time(events[("end", c)])
                       for c in range(cfg.num_chunks))
        append_ms += sum(events[("append", c)].elapsed_time(events[("start", c)])
                         for c in range(cfg.num_chunks))
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end) / reps
    attn_ms /= reps
    append_ms /= reps
    abytes = A.append_bytes(cfg.prompt_len, cfg.hkv, cfg.head_dim, cfg.kv_dtype)
    flops = A.causal_prompt_flops(cfg.prompt_len, cfg.hq, cfg.head_dim)
    tflops = flops / (attn_ms * 1e-3) / 1e12
    del st
    torch.cuda.empty_cache()
    return {
        "workload": cfg.name,
        "prompt_tok_per_s": cfg.prompt_len / (total_ms * 1e-3),
        "ms_per_prompt": total_ms,
        "attn_ms_per_prompt": attn_ms,
        "tflops": tflops,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": A.BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / A.BF16_MFMA_PEAK_TFLOPS,
                     "traffic": None,
                     "kernel": "pkv_paged_attn_prefill (all shards) + pkv_attn_lse_merge",
                     "mfma": ("fp16 x fp16 (E4M3 tiles dequantised to fp16, q converted)"
                              if cfg.kv_dtype == "e4m3" else "bf16 (K Q^T), fp16 (P V)"),
                     "flops_per_prompt": flops},
        "kv_dtype": cfg.kv_dtype,
        "kv_append": {"ms_per_prompt": append_ms, "bytes_per_prompt": abytes,
                      "includes": "kv_append" + (" + fp8_group_scales (scales read the chunk once "
                                                 "more, not counted in bytes)"
                                                 if cfg.kv_dtype == "e4m3" else ""),
                      "gbs": abytes / (append_ms * 1e-3) / 1e9,
                      "frac_of_hbm_peak": abytes / (append_ms * 1e-3) / 1e9 / A.HBM_PEAK_GBS},
    }


def block_copy_record(reps=5, blocks=8192, cow_blocks=32):
    """pkv_copy_blocks on the Llama-3-8B-like layer's pool layout (8 kv heads,
    d 128, bf16: 64 KiB per block): offload of `blocks` blocks from HBM to a
    pinned host pool and page-in back (PCIe-bound), the same number copied
    inside HBM, and one copy-on-write launch of `cow_blocks` single blocks (one
    per sequence after a fork).  Times are HIP events on the launching stream."""
    import torch
    from paged_kv_cache_210_amd import accounting as A
    from paged_kv_cache_210_amd import lib

    hkv, d = 8, 128
    nb = 2 * blocks
    dev = lib.PagedCache.empty(nb, hkv, d, "bf16")
    dev.k.normal_()
    dev.v.normal_()
    host = lib.PagedCache.empty(blocks, hkv, d, "bf16", pinned=True)
    perm = torch.randperm(nb, generator=torch.Generator().manual_seed(7)).to(torch.int32)
    src, dst = perm[:blocks].cuda(), perm[blocks:].cuda()
    slots = torch.arange(blocks, dtype=torch.int32, device="cuda")
    per_block = A.block_bytes(hkv, d, "bf16")

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    out_ms = timed(lambda: lib.copy_blocks(dev, host, src, slots))
    in_ms = timed(lambda: lib.copy_blocks(host, dev, slots, dst))
    hbm_ms = timed(lambda: lib.copy_blocks(dev, dev, src, dst))
    cow_ms = timed(lambda: lib.copy_blocks(dev, dev, src[:cow_blocks], dst[:cow_blocks]))
    moved = blocks * per_block
    rec = {
        "workload": f"pkv_copy_blocks, {blocks} blocks of 8 kv heads x d 128 bf16 "
                    f"({moved / 2**20:.0f} MiB), random block ids",
        "offload_gbs": moved / (out_ms * 1e-3) / 1e9,
        "page_in_gbs": moved / (in_ms * 1e-3) / 1e9,
        "pcie_peak_gbs": A.PCIE_PEAK_GBS,
        "offload_frac_of_pcie": moved / (out_ms * 1e-3) / 1e9 / A.PCIE_PEAK_GBS,
        "page_in_frac_of_pcie": moved / (in_ms * 1e-3) / 1e9 / A.PCIE_PEAK_GBS,
        "hbm_copy_gbs_read_plus_write": 2 * moved / (hbm_ms * 1e-3) / 1e9,
        "hbm_frac": 2 * moved / (hbm_ms * 1e-3) / 1e9 / A.HBM_PEAK_GBS,
        "cow_launch_us": cow_ms * 1e3,
        "cow_blocks": cow_blocks,
    }
    del dev, host
    torch.cuda.empty_cache()
    return rec


def hbm_copy_record(reps=20, nbytes=1 << 30):
    """A plain device-to-device copy of a known size: the attainable-bandwidth
    context for the decode roofline, and the reference kernel for scaling the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    return {"workload": f"device copy of {nbytes} bytes", "bytes_read": nbytes,
            "bytes_written": nbytes, "ms": ms, "gbs": 2 * nbytes / (ms * 1e-3) / 1e9}


def cpu_baseline_decode(cfg, budget_s):
    """The fp64 oracle, as it stands, on a bounded sample of the same decode
    step: append the newest token of each sampled sequence, then attention over
    all its keys.  Sequences are added until the budget is used; when the whole
    batch takes less, the steps are repeated over the batch (re-appending a
    token writes the same slot with the same values) until it is used."""
    import numpy as np
    import torch
    from oracle import pkv_oracle as O
    import synth

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas_threads = 1
    inp = synth.decode_inputs(cfg, device="cuda")
    order = inp["free_order"].numpy()
    tables, _ = O.build_tables(cfg.seq_lens, cfg.pool_blocks, order)

    def bits(t):
        return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    cache = O.new_cache(cfg.pool_blocks, cfg.hkv, cfg.head_dim, cfg.kv_dtype)
    q = bits(inp["q"])
    done, spent = 0, 0.0
    start = 0
    newest = []

    def timed_step(b, n, kn, vn):
        t0 = time.perf_counter()
        O.append(cache, kn, vn, np.array([b], np.int32), np.array([n - 1], np.int32), tables)
        O.decode(cache, q[b:b + 1], "bf16", tables[b:b + 1], [n])
        return time.perf_counter() - t0

    for b, n in enumerate(cfg.seq_lens):
        k = bits(inp["k"][start:start + n])
        v = bits(inp["v"][start:start + n])
        O.append_sequence(cache, k[:n - 1], v[:n - 1], tables[b], 0)        # untimed pre-fill
        newest.append((k[n - 1:n], v[n - 1:n]))
        spent += timed_step(b, n, *newest[b])
        done += 1
        start += n
        if spent >= budget_s:
            break
    passes = 1
    while spent < budget_s and done == passes * cfg.batch:
        for b, n in enumerate(cfg.seq_lens):
            spent += timed_step(b, n, *newest[b])
            done += 1
            if spent >= budget_s:
                break
        passes += 1
    seqs = min(done, cfg.batch)
    return {"value": done / spent, "unit": "tok/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{done} decode steps over {seqs} of {cfg.batch} sequences of {cfg.name} "
                      f"(append newest token + decode over {cfg.seq_lens[0]} keys, all "
                      f"{cfg.hq} heads), {spent:.1f} s of CPU time",
            "host_cpus": len(os.sched_getaffinity(0))}


def cpu_baseline_prefill(cfg, budget_s, device="cuda"):
    """The fp64 oracle, as it stands, on a bounded sample of the same causal
    prefill: query rows taken from the end of the prompt (the longest ones),
    each against all of its visible keys, all heads.  The rate is attention
    flops (4*d per visible key per head) per second, the same unit as the GPU
    figure; the prompt's KV is put into the oracle pool untimed."""
    import numpy as np
    import torch
    from oracle import pkv_oracle as O
    import synth

    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        blas_threads = 1
    inp = synth.prefill_inputs(cfg, device=device)
    tables, _ = O.build_tables([cfg.prompt_len], cfg.pool_blocks, inp["free_order"].numpy())

    def bits(t):
        return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    cache = O.new_cache(cfg.pool_blocks, cfg.hkv, cfg.head_dim, "bf16")
    O.append_sequence(cache, bits(inp["k"]), bits(inp["v"]), tables[0], 0)   # untimed
    q = bits(inp["q"])
    rows, pairs, spent = 0, 0, 0.0
    for r in range(cfg.prompt_len - 1, -1, -1):
        t0 = time.perf_counter()
        O.prefill(cache, q[r:r + 1], "bf16", r, tables[0], 0, r + 1, True)
        spent += time.perf_counter() - t0
        rows += 1
        pairs += r + 1
        if spent >= budget_s:
            break
    flops = 4 * cfg.head_dim * cfg.hq * pairs
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(blas_threads),
            "kind": "oracle",
            "sample": f"{rows} query rows (the last ones) of {cfg.name}, each against all its "
                      f"visible keys, all {cfg.hq} heads, {spent:.1f} s of CPU time",
            "host_cpus": len(os.sched_getaffinity(0))}


# Blocks per decode partition: the 131072-token workload is defined with
# 256-block partitions; the others use the library's choice (0), which for the
# 1M-token workload is 128 partitions of 512 blocks (1024 workgroups).
PARTITION_BLOCKS = {"C2": 0, "C3": 256, "C5": 0}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-secondary", action="store_true", help="headline workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", choices=["C2", "C3", "C5", "C4", "C4_128K", "C4_FP8", "hbm_copy",
                                       "block_copy"],
                    help="run one workload and print its record (for profiling)")
    ap.add_argument("--prefill-reps", type=int, default=2)
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path "
              "(see the sharding notes); run with --gpus 1", file=sys.stderr)
        return 2

    import torch
    import synth
    from paged_kv_cache_210_amd import lib

    lib.load()
    torch.cuda.init()
    if args.only == "hbm_copy":
        print(json.dumps(hbm_copy_record(args.steps)), flush=True)
        return 0
    if args.only == "block_copy":
        print(json.dumps(block_copy_record()), flush=True)
        return 0
    if args.only:
        c = synth.CONFIGS[args.only]
        _log(f"[bench] only {c.name}")
        if args.only.startswith("C4"):
            rec = prefill_record(c, args.prefill_reps)
        else:
            rec, _ = decode_record(c, args.steps, args.warmup,
                                   PARTITION_BLOCKS[args.only])
        print(json.dumps(rec), flush=True)
        return 0
    cfg = synth.CONFIGS["C2"]
    _log(f"[bench] headline {cfg.name}: warmup {args.warmup}, steps {args.steps}")
    head, st = decode_record(cfg, args.steps, args.warmup, 0)
    del st
    torch.cuda.empty_cache()
    _log(f"[bench] {head['tok_per_s']:.0f} tok/s, decode {head['roofline']['achieved']:.0f} GB/s")

    secondary = []
    if not args.no_secondary:
        for name in ("C3", "C5"):
            pb = PARTITION_BLOCKS[name]
            c = synth.CONFIGS[name]
            _log(f"[bench] secondary {c.name}")
            rec, st = decode_record(c, args.steps, args.warmup, pb)
            del st
            torch.cuda.empty_cache()
            rec["partition_blocks"] = pb
            secondary.append(rec)
            _log(f"[bench]   {rec['tok_per_s']:.0f} tok/s, {rec['roofline']['achieved']:.0f} GB/s")

        for name in ("C4", "C4_128K", "C4_FP8"):
            c = synth.CONFIGS[name]
            _log(f"[bench] secondary {c.name}")
            rec = prefill_record(c, args.prefill_reps)
            if name == "C4" and not args.no_cpu_baseline:
                rec["cpu_baseline"] = cpu_baseline_prefill(c, args.cpu_seconds / 2)
                rec["cpu_baseline"]["gpu_speedup"] = rec["tflops"] / rec["cpu_baseline"]["value"]
            secondary.append(rec)
            _log(f"[bench]   {rec['tflops']:.0f} TFLOP/s, {rec['ms_per_prompt']:.2f} ms/prompt; "
                 f"kv_append {rec['kv_append']['gbs']:.0f} GB/s")

    if not args.no_secondary:
        bc = block_copy_record()
        secondary.append(bc)
        _log(f"[bench] block copies: offload {bc['offload_gbs']:.1f} GB/s, page-in "
             f"{bc['page_in_gbs']:.1f} GB/s, in HBM {bc['hbm_copy_gbs_read_plus_write']:.0f} GB/s")

    copy = hbm_copy_record()
    _log(f"[bench] plain device copy: {copy['gbs']:.0f} GB/s")

    cpu = None
    if not args.no_cpu_baseline:
        _log("[bench] cpu baseline (fp64 oracle)")
        cpu = cpu_baseline_decode(cfg, args.cpu_seconds)
        cpu["gpu_speedup"] = head["tok_per_s"] / cpu["value"]

    line = {
        "metric": METRIC,
        "value": head["tok_per_s"],
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) q/k/v, shuffled physical blocks",
        "config": {"workload": cfg.name, "batch": cfg.batch, "seq_len": cfg.seq_lens[0],
                   "q_heads": cfg.hq, "kv_heads": cfg.hkv, "head_dim": cfg.head_dim,
                   "block_size": 16, "kv_dtype": cfg.kv_dtype, "pool_blocks": cfg.pool_blocks,
                   "step": "append 1 token/seq folded into split-KV decode (pkv_paged_attn_decode_step) + LSE merge"},
        "ms_per_step_no_events": head["ms_per_step_no_events"],
        "merge_ms": head["merge_ms"],
        "decode_hbm_gbs": head["roofline"]["achieved"],
        "hbm_copy_gbs": copy["gbs"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
