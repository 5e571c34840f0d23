#!/usr/bin/env python3
"""Throughput of the paged-attention hot path on one MI355X.

A decode step is one pass of the whole decode path over one batch: append the
newest token of every sequence into the paged pool (pkv_kv_append), then
split-KV attention of that token against every cached key plus the exact
log-sum-exp merge (pkv_paged_attn_decode).  Inputs are resident in HBM before
the timed region starts.

The headline is the 128K decode (4 sequences x 131072 tokens, 64 q / 8 kv
heads, d 128, bf16, 256-block partitions); the 131072-token chunked causal
prefill is carried beside it ("prefill_128k"), and the 8K and 1M-token (E4M3)
decodes, the 32K prefills (bf16 and E4M3), block copies and the page-in
overlap are reported under "secondary".  Every decode and prefill record
carries the fp64 CPU oracle timed on a bounded sample of the same workload
("cpu_baseline") and the GPU's error against it.

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
    before.  Each timed pass is queued behind a GPU spin, so it measures the
    GPU running the steps back to back, not the host issuing them."""
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
        # the GPU spins (about 8 ms, more for long runs) while the host queues
        # the k steps, so a pause of the host between two launches (the
        # Python binding takes longer to issue a C2 step than some of the
        # steps take) cannot leave the GPU idle inside the timed region
        torch.cuda._sleep(20_000_000 + 500_000 * k)
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


def decode_record(cfg, steps, warmup, partition_blocks, keep_rows=None):
    """Timed decode steps of one workload; returns (record, GPU output of the
    rows in keep_rows as float64 [len(keep_rows), Hq, d] on the host)."""
    import torch
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
        "partition_blocks": partition_blocks,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": A.HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / A.HBM_PEAK_GBS, "traffic": measured_traffic(cfg),
                     "kernel": ("decode_mfma_kernel with the append folded in "
                                "(pkv_paged_attn_decode_step_partial)" if st["folded"] else
                                "decode_mfma_kernel (pkv_paged_attn_decode_partial)"),
                     "ms_per_launch": ms_dec, "ms_per_launch_median": st["decode_ms_median"],
                     "ms_per_launch_min": st["decode_ms_min"], "bytes_per_launch": kbytes,
                     "clock_ghz_observed": observed_clock(_key(cfg))},
    }
    rows = None
    if keep_rows is not None:
        rows = st["out"][list(keep_rows)].double().cpu().numpy()
    del st
    torch.cuda.empty_cache()
    return rec, rows


def _key(cfg):
    """The workload's name in synth.CONFIGS (C2, C3, C4_128K, ...)."""
    import synth

    return next((k for k, c in synth.CONFIGS.items() if c == cfg), cfg.name)


def _gated(path, key):
    """A committed counter figure, or None when a kernel source it was taken
    with has changed since (each record stores the sha256 of its sources)."""
    import hashlib

    try:
        rec = json.load(open(os.path.join(ROOT, path)))
        w = rec["workloads"][key]
        shas = dict(rec.get("kernel_source_sha256", {}))
        shas.update(w.get("kernel_source_sha256", {}))
        for src, sha in shas.items():
            if hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest() != sha:
                return None
        return w
    except (OSError, KeyError, ValueError, TypeError, AttributeError):
        return None


def measured_traffic(cfg):
    """HBM bytes per launch of the decode kernel from the committed counter
    runs (profiles/decode_hbm_traffic.json), or None when the kernel source has
    changed since they were taken."""
    w = _gated("profiles/decode_hbm_traffic.json", _key(cfg))
    return None if w is None else w["traffic_bytes"]


def prefill_traffic(cfg):
    """HBM bytes per prompt of the prefill kernel launches from the committed
    FETCH_SIZE / WRITE_SIZE runs (profiles/prefill_hbm_traffic.json), or None
    when the kernel source has changed since."""
    w = _gated("profiles/prefill_hbm_traffic.json", _key(cfg))
    return None if w is None else w["traffic_bytes_per_prompt"]


def observed_clock(key):
    """Average shader clock over the dominant kernel's launches (GPU-active
    cycles per XCD from GRBM_GUI_ACTIVE over the traced kernel time) from the
    committed counter run (profiles/observed_clock.json), or None when the
    kernel source has changed since."""
    w = _gated("profiles/observed_clock.json", key)
    return None if w is None else w["clock_ghz"]


def chunk_plan(cfg):
    """The chunked pass over a prompt: for each 4096-token (cfg.chunk) query
    chunk c, rows [a, b), the KV shard ranges it attends to, in order.  Shards
    are the contiguous cfg.shard_len-token ranges of the keys written so far
    (the chunk's own included); a chunk that sees one shard only is attended
    in the final form, the others as one partial per shard merged by LSE."""
    C, S = cfg.chunk, cfg.shard_len
    plan = []
    for c in range(cfg.num_chunks):
        a, b = c * C, min((c + 1) * C, cfg.prompt_len)
        shards = [(j * S, min((j + 1) * S, b)) for j in range(-(-b // S))]
        plan.append((c, a, b, shards))
    return plan


def prefill_setup(cfg, poison=False):
    """Device state of one prompt: inputs drawn on the GPU, the table from the
    library allocator, an empty pool (NaN / 0x7F codes when poison), shard
    partial buffers and the output."""
    import torch
    from paged_kv_cache_210_amd import lib
    import synth

    dev = "cuda"
    inp = synth.prefill_inputs(cfg, device=dev)
    tables, _ = lib.build_tables([cfg.prompt_len], cfg.pool_blocks, inp["free_order"])
    td = tables.to(dev)
    fill = None
    if poison:
        fill = 0x7F if cfg.kv_dtype == "e4m3" else float("nan")
    cache = lib.PagedCache.empty(cfg.pool_blocks, cfg.hkv, cfg.head_dim, cfg.kv_dtype, device=dev,
                                 fill=fill)
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
    return dict(inp=inp, tables=tables, td=td, cache=cache, part=part, out=out, lse1=lse1,
                pos=pos, seq=seq)


def append_chunk(cfg, st, a, b):
    """The append of prompt rows [a, b): for an E4M3 pool the group scales and
    the append in one pass (pkv_kv_append_fp8_groups), else pkv_kv_append."""
    from paged_kv_cache_210_amd import lib

    inp, td, cache = st["inp"], st["td"], st["cache"]
    if cfg.kv_dtype == "e4m3":
        lib.kv_append_fp8_groups(cache, inp["k"][a:b], inp["v"][a:b], a, td[0])
    else:
        lib.kv_append(cache, inp["k"][a:b], inp["v"][a:b], st["seq"][:b - a], st["pos"][a:b], td)


def prefill_pass(cfg, st, ev=None):
    """One chunked pass over the prompt (chunk_plan): per chunk append its K/V
    (append_chunk), then attend to its shards and merge them by LSE into
    st["out"]."""
    from paged_kv_cache_210_amd import lib

    inp, td, cache, (po, pm, pl) = st["inp"], st["td"], st["cache"], st["part"]
    for c, a, b, shards in chunk_plan(cfg):
        append_chunk(cfg, st, a, b)
        q = inp["q"][a:b]
        if ev is not None:
            ev.append(("start", c))
        if len(shards) == 1:          # one shard holds every visible key: nothing to merge
            lo, hi = shards[0]
            lib.paged_attn_prefill(cache, q, a, td[0], lo, hi, True, out=st["out"][a:b],
                                   out_lse=st["lse1"][:b - a])
        else:
            for j, (lo, hi) in enumerate(shards):
                lib.paged_attn_prefill(cache, q, a, td[0], lo, hi, True, partial=True,
                                       part=(po[j, :b - a], pm[j, :b - a], pl[j, :b - a]))
            n = len(shards)
            lib.attn_lse_merge(po[:n, :b - a], pm[:n, :b - a], pl[:n, :b - a],
                               out=st["out"][a:b], with_state=False)
        if ev is not None:
            ev.append(("end", c))


def prefill_record(cfg, reps, keep_rows=None):
    """Timed chunked passes over one prompt; returns (record, GPU output rows
    keep_rows as float64 on the host)."""
    import torch
    from paged_kv_cache_210_amd import accounting as A

    st = prefill_setup(cfg)
    prefill_pass(cfg, st)                      # warm-up pass
    torch.cuda.synchronize()
    events = {}

    class _Ev(list):
        def append(self, item):
            e = torch.cuda.Event(enable_timing=True)
            e.record()
            events[item] = e

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    attn_ms = 0.0
    start.record()
    for _ in range(reps):
        events.clear()
        ev = _Ev()
        prefill_pass(cfg, st, ev)
        torch.cuda.synchronize()
        attn_ms += sum(events[("start", c)].elapsed_time(events[("end", c)])
                       for c in range(cfg.num_chunks))
    end.record()
    torch.cuda.synchronize()
    total_ms = start.elapsed_time(end) / reps
    attn_ms /= reps
    # the appends of a prompt on their own, back to back (each writes the same
    # values into the same slots again), two events around the batch; the GPU
    # first spins for ~10 ms so that every append is queued before the first
    # runs (the host takes longer to issue a call than a chunk's append takes
    # on the GPU)
    plan = chunk_plan(cfg)
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(20_000_000)
    a0.record()
    for _ in range(reps):
        for _, a, b, _ in plan:
            append_chunk(cfg, st, a, b)
    a1.record()
    torch.cuda.synchronize()
    append_ms = a0.elapsed_time(a1) / reps
    abytes = A.append_bytes(cfg.prompt_len, cfg.hkv, cfg.head_dim, cfg.kv_dtype)
    flops = A.causal_prompt_flops(cfg.prompt_len, cfg.hq, cfg.head_dim)
    tflops = flops / (attn_ms * 1e-3) / 1e12
    rows = None
    if keep_rows is not None:
        rows = st["out"][torch.tensor(list(keep_rows), device="cuda")].double().cpu().numpy()
    del st
    torch.cuda.empty_cache()
    rec = {
        "workload": cfg.name,
        "prompt_tok_per_s": cfg.prompt_len / (total_ms * 1e-3),
        "ms_per_prompt": total_ms,
        "attn_ms_per_prompt": attn_ms,
        "tflops": tflops,
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": A.BF16_MFMA_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": tflops / A.BF16_MFMA_PEAK_TFLOPS,
                     "traffic": prefill_traffic(cfg),
                     "traffic_unit": "HBM bytes per prompt, prefill_kernel launches",
                     "kernel": "pkv_paged_attn_prefill (all shards) + pkv_attn_lse_merge",
                     "mfma": ("fp16 x fp16 (E4M3 tiles dequantised to fp16, q converted)"
                              if cfg.kv_dtype == "e4m3" else "bf16 (K Q^T), fp16 (P V)"),
                     "flops_per_prompt": flops,
                     "clock_ghz_observed": observed_clock(_key(cfg))},
        "kv_dtype": cfg.kv_dtype,
        "kv_append": {"ms_per_prompt": append_ms, "bytes_per_prompt": abytes,
                      "chunks": cfg.num_chunks,
                      "includes": ("pkv_kv_append_fp8_groups (group scales and append in one "
                                   "pass)" if cfg.kv_dtype == "e4m3" else "pkv_kv_append") +
                                  ", the prompt's chunk appends back to back",
                      "gbs": abytes / (append_ms * 1e-3) / 1e9,
                      "frac_of_hbm_peak": abytes / (append_ms * 1e-3) / 1e9 / A.HBM_PEAK_GBS},
    }
    return rec, rows


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


def page_in_overlap_record(steps=20, warmup=3, blocks=2048, reps=3):
    """The prefetch of KV offload beside decode: C2 decode steps (the folded
    step + merge, as timed for the C2 record) on the current stream while
    pkv_copy_blocks pages `blocks` blocks (C2's format, 64 KiB each) in from a
    pinned host pool on a second stream.  Reported: the decode steps alone,
    the page-in alone, both together (from one start event to the later of
    the two ends), the overlap fraction (t_decode + t_page_in - t_both) /
    min(t_decode, t_page_in), and the decode kernel's GB/s while the page-in
    runs.  Medians over `reps` repetitions of each."""
    import statistics
    import torch
    import synth
    from paged_kv_cache_210_amd import accounting as A
    from paged_kv_cache_210_amd import lib

    cfg = synth.CONFIGS["C2"]
    st = _decode_setup(cfg, 0)
    s_in = st["step_in"]
    po, pm, pl = st["part"]
    it = [0]

    def step(ev=None):
        cache = st["caches"][it[0] % 2]
        it[0] += 1
        if ev is not None:
            ev[0].record()
        lib.paged_attn_decode_step(cache, s_in["k"], s_in["v"], st["q"], st["td"], st["lens"],
                                   partial=True, part=st["part"])
        if ev is not None:
            ev[1].record()
        lib.attn_lse_merge(po, pm, pl, out=st["out"], with_state=False, out_lse=st["lse"])

    hkv, d = cfg.hkv, cfg.head_dim
    host = lib.PagedCache.empty(blocks, hkv, d, "bf16", pinned=True)
    host.k.copy_(torch.randn(host.k.shape).to(torch.bfloat16))
    host.v.copy_(torch.randn(host.v.shape).to(torch.bfloat16))
    dst = lib.PagedCache.empty(blocks, hkv, d, "bf16")
    perm = torch.randperm(blocks, generator=torch.Generator().manual_seed(8)).to(torch.int32)
    src_ids = perm.cuda()
    dst_ids = torch.arange(blocks, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    main = torch.cuda.current_stream()
    E = lambda: torch.cuda.Event(enable_timing=True)    # noqa: E731

    def run(decode, page_in):
        torch.cuda.synchronize()
        t0, end_m, end_s = E(), E(), E()
        evs = [[E(), E()] for _ in range(steps)] if decode else []
        t0.record(main)
        side.wait_event(t0)
        if page_in:
            lib.copy_blocks(host, dst, src_ids, dst_ids, stream=side)
        end_s.record(side)
        if decode:
            for i in range(steps):
                step(evs[i])
        end_m.record(main)
        torch.cuda.synchronize()
        both = max(t0.elapsed_time(end_m), t0.elapsed_time(end_s))
        dec = sum(e[0].elapsed_time(e[1]) for e in evs)
        return both, dec

    for _ in range(warmup):
        step()
    run(True, True)
    t_dec, t_pg, t_both, k_alone, k_both = [], [], [], [], []
    for _ in range(reps):
        b, k = run(True, False)
        t_dec.append(b)
        k_alone.append(k)
        t_pg.append(run(False, True)[0])
        b, k = run(True, True)
        t_both.append(b)
        k_both.append(k)
    med = statistics.median
    td, tp, tb = med(t_dec), med(t_pg), med(t_both)
    kbytes = A.decode_kernel_bytes(cfg.seq_lens, cfg.hq, cfg.hkv, cfg.head_dim, cfg.q_dtype,
                                   cfg.kv_dtype)
    kbytes += A.append_bytes(cfg.batch, cfg.hkv, cfg.head_dim, cfg.kv_dtype) - 8 * cfg.batch
    moved = blocks * A.block_bytes(hkv, d, "bf16")
    rec = {
        "workload": f"{cfg.name}: {steps} decode steps on one stream while {blocks} blocks "
                    f"({moved / 2**20:.0f} MiB) page in from pinned host memory on another",
        "decode_alone_ms": td, "page_in_alone_ms": tp, "both_ms": tb,
        "overlap_frac": (td + tp - tb) / min(td, tp),
        "page_in_gbs_alone": moved / (tp * 1e-3) / 1e9,
        "decode_gbs_alone": kbytes * steps / (med(k_alone) * 1e-3) / 1e9,
        "decode_gbs_during_page_in": kbytes * steps / (med(k_both) * 1e-3) / 1e9,
        "decode_tok_per_s_during_page_in": cfg.batch * steps / (tb * 1e-3),
        "reps": reps,
    }
    del st, host, dst
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


# ---------------------------------------------------------------- oracle baselines
def _threads():
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        return 1


def oracle_error(got, ref):
    """Error of bf16 GPU outputs against the oracle on the same rows:
    max |got - ref|, the same beyond the output's own rounding (half a bf16 ulp
    of ref), and the per-row inf-norm relative error (max over rows of
    max_i |got_i - ref_i| / max_i |ref_i|), rows being the last axis."""
    import numpy as np

    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = np.abs(got - ref)
    a = np.abs(ref)
    half_ulp = np.where(a > 0, 2.0 ** (np.floor(np.log2(np.where(a > 0, a, 1.0))) - 8), 0.0)
    den = a.max(axis=-1)
    live = den > 0
    rel = (diff.max(axis=-1)[live] / den[live]).max() if live.any() else 0.0
    return {"max_abs": float(diff.max()),
            "max_abs_beyond_bf16_rounding": float(np.maximum(diff - half_ulp, 0).max()),
            "row_rel": float(rel), "rows": int(np.prod(got.shape[:-1]))}


def _kv_host(t, fmt):
    """Source K/V rows (device tensor) -> what the oracle's append takes."""
    import numpy as np
    import torch

    if fmt == "e4m3":
        return t.float().cpu().numpy()
    return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def cpu_baseline_decode(cfg, budget_s, gpu_rows=None, seqs=None, kv_heads=None,
                        piece=1 << 16):
    """The fp64 oracle, as it stands, on a bounded sample of the same decode
    step: for each sampled sequence, append its newest token, then attention
    of its query over all its keys, for the query heads of the sampled kv
    heads (all by default).  Sequences are taken in turn, and the turns
    repeated (re-appending a token writes the same slot with the same values)
    until the CPU budget is used.  With kv_heads sampled, a step does that
    fraction of a token's work, so the rate is scaled by it (tokens/s =
    steps * len(kv_heads) / Hkv / time).  The sampled outputs are compared
    with the GPU's (gpu_rows [len(seqs), Hq, d], in the order of seqs)."""
    import numpy as np
    import torch
    from oracle import pkv_oracle as O
    import synth

    seqs = list(range(cfg.batch)) if seqs is None else list(seqs)
    heads = list(range(cfg.hkv)) if kv_heads is None else list(kv_heads)
    G = cfg.hq // cfg.hkv
    qheads = [g * G + i for g in heads for i in range(G)]
    inp = synth.decode_inputs(cfg, device="cuda")
    tables, _ = O.build_tables(cfg.seq_lens, cfg.pool_blocks, inp["free_order"].numpy())
    cache = O.new_cache(cfg.pool_blocks, cfg.hkv, cfg.head_dim, cfg.kv_dtype)
    q = inp["q"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    starts = np.concatenate([[0], np.cumsum(cfg.seq_lens)[:-1]])
    newest = {}
    setup0 = time.perf_counter()
    for b in seqs:                                     # untimed: the pool before the step
        n, a = cfg.seq_lens[b], int(starts[b])
        for p0 in range(0, n, piece):
            p1 = min(n, p0 + piece)
            k = _kv_host(inp["k"][a + p0:a + p1], cfg.kv_dtype)
            v = _kv_host(inp["v"][a + p0:a + p1], cfg.kv_dtype)
            if cfg.kv_dtype == "e4m3":                 # scales from every token, newest included
                O.fp8_group_scales(k, p0, tables[b], cache.k_scale)
                O.fp8_group_scales(v, p0, tables[b], cache.v_scale)
            m = min(p1, n - 1) - p0
            if m > 0:
                O.append_sequence(cache, k[:m], v[:m], tables[b], p0, heads=heads)
            if p1 == n:
                newest[b] = (k[n - 1 - p0:n - p0], v[n - 1 - p0:n - p0])
    setup_s = time.perf_counter() - setup0
    del inp
    done, spent, outs = 0, 0.0, {}
    while spent < budget_s:
        for b in seqs:
            n = cfg.seq_lens[b]
            t0 = time.perf_counter()
            O.append(cache, newest[b][0], newest[b][1], np.array([b], np.int32),
                     np.array([n - 1], np.int32), tables)
            r = O.decode(cache, q[b:b + 1], cfg.q_dtype, tables[b:b + 1], [n],
                         kv_heads=None if kv_heads is None else heads)
            spent += time.perf_counter() - t0
            outs[b] = r["o"][0][qheads]
            done += 1
            if spent >= budget_s:
                break
    frac = len(heads) / cfg.hkv
    what = (f"all {cfg.hq} heads" if frac == 1 else
            f"the {len(qheads)} query heads of kv head(s) {heads}, i.e. {frac:g} of a token's "
            f"work per step, rate scaled by that fraction")
    rec = {"value": done * frac / spent, "unit": "tok/s", "cores": int(_threads()),
           "kind": "oracle",
           "sample": f"{done} decode steps (append the newest token, attend over all "
                     f"{cfg.seq_lens[seqs[0]]} keys, {what}) taking turns over "
                     f"{len(seqs)} of {cfg.batch} sequences of {cfg.name}, {spent:.1f} s of "
                     f"CPU time (+{setup_s:.1f} s untimed to fill the oracle pool)",
           "host_cpus": len(os.sched_getaffinity(0))}
    if gpu_rows is not None:
        got = [gpu_rows[i][qheads] for i, b in enumerate(seqs) if b in outs]
        want = [outs[b] for b in seqs if b in outs]
        rec["gpu_error_vs_oracle"] = oracle_error(np.stack(got), np.stack(want))
        rec["gpu_error_vs_oracle"]["sequences"] = [b for b in seqs if b in outs]
        rec["gpu_error_vs_oracle"]["q_heads"] = "all" if frac == 1 else qheads
    return rec


def cpu_baseline_prefill(cfg, budget_s, gpu_rows=None, edge_rows=()):
    """The fp64 oracle, as it stands, on a bounded sample of the same causal
    prefill: query rows taken from the end of the prompt (the longest ones),
    each against all of its visible keys, all heads, timed until the CPU
    budget is used; the rate is attention flops (4*d per visible key per head)
    per second, the GPU figure's unit.  The prompt's KV is put into the oracle
    pool untimed (E4M3: scales per chunk, as the GPU pass makes them).  The
    timed rows and the untimed edge_rows are compared with the GPU's output
    (gpu_rows: the rows of prefill_rows(cfg, edge_rows), in order)."""
    import numpy as np
    import torch
    from oracle import pkv_oracle as O
    import synth

    inp = synth.prefill_inputs(cfg, device="cuda")
    tables, _ = O.build_tables([cfg.prompt_len], cfg.pool_blocks, inp["free_order"].numpy())
    cache = O.new_cache(cfg.pool_blocks, cfg.hkv, cfg.head_dim, cfg.kv_dtype)
    setup0 = time.perf_counter()
    for c, a, b, _ in chunk_plan(cfg):
        k = _kv_host(inp["k"][a:b], cfg.kv_dtype)
        v = _kv_host(inp["v"][a:b], cfg.kv_dtype)
        if cfg.kv_dtype == "e4m3":
            O.fp8_group_scales(k, a, tables[0], cache.k_scale)
            O.fp8_group_scales(v, a, tables[0], cache.v_scale)
        O.append_sequence(cache, k, v, tables[0], a)
    q = inp["q"].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    setup_s = time.perf_counter() - setup0
    del inp
    got_rows, outs, pairs, spent = [], {}, 0, 0.0
    for r in range(cfg.prompt_len - 1, -1, -1):
        t0 = time.perf_counter()
        res = O.prefill(cache, q[r:r + 1], "bf16", r, tables[0], 0, r + 1, True)
        spent += time.perf_counter() - t0
        outs[r] = res["o"][0]
        pairs += r + 1
        if spent >= budget_s:
            break
    timed_rows = sorted(outs)
    for r in edge_rows:                              # untimed rows for the error only
        if r not in outs:
            outs[r] = O.prefill(cache, q[r:r + 1], "bf16", r, tables[0], 0, r + 1, True)["o"][0]
    flops = 4 * cfg.head_dim * cfg.hq * pairs
    rec = {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(_threads()),
           "kind": "oracle",
           "sample": f"{len(timed_rows)} query rows (the last ones) of {cfg.name}, each against "
                     f"all its visible keys, all {cfg.hq} heads, {spent:.1f} s of CPU time "
                     f"(+{setup_s:.1f} s untimed to fill the oracle pool)",
           "host_cpus": len(os.sched_getaffinity(0)), "timed_rows": len(timed_rows)}
    if gpu_rows is not None:
        rows = prefill_rows(cfg, edge_rows)
        sel = [i for i, r in enumerate(rows) if r in outs]
        rec["gpu_error_vs_oracle"] = oracle_error(gpu_rows[sel],
                                                  np.stack([outs[rows[i]] for i in sel]))
        rec["gpu_error_vs_oracle"]["query_rows"] = [rows[i] for i in sel]
    return rec


def prefill_rows(cfg, edge_rows, n_tail=64):
    """Rows whose GPU output is kept for the oracle comparison: the edge rows
    and the last n_tail rows of the prompt (more than the oracle's budget
    reaches: the comparison takes those it computed)."""
    tail = list(range(cfg.prompt_len - n_tail, cfg.prompt_len))
    return sorted(set(list(edge_rows) + tail))


def edge_rows_of(cfg):
    """First rows, the ends of the first chunk and of every shard."""
    rows = {0, 1, 63, 64, cfg.chunk - 1, cfg.chunk}
    for j in range(1, cfg.num_shards):
        rows |= {j * cfg.shard_len - 1, j * cfg.shard_len}
    return sorted(r for r in rows if r < cfg.prompt_len)


# Blocks per decode partition: the 131072-token workload is defined with
# 256-block partitions; the others use the library's choice (0), which for the
# 1M-token workload is 128 partitions of 512 blocks (1024 workgroups).
PARTITION_BLOCKS = {"C2": 0, "C3": 256, "C5": 0}
# Sequences (and, for the 1M-token workload, kv heads: filling the oracle's
# E4M3 pool for all 8 would take minutes) whose output the oracle recomputes.
ORACLE_SEQS = {"C2": None, "C3": [0, 1, 2, 3], "C5": [0]}
ORACLE_KV_HEADS = {"C2": None, "C3": None, "C5": [3]}
# CPU seconds of each oracle baseline, as fractions of --cpu-seconds.
CPU_SHARE = {"C2": 0.5, "C3": 0.6, "C5": 0.8, "C4": 0.4, "C4_128K": 0.6, "C4_FP8": 0.4}


def decode_with_baseline(name, args):
    import synth

    c = synth.CONFIGS[name]
    seqs = ORACLE_SEQS[name]
    keep = list(range(c.batch)) if seqs is None else seqs
    _log(f"[bench] decode {c.name}")
    rec, rows = decode_record(c, args.steps, args.warmup, PARTITION_BLOCKS[name], keep_rows=keep)
    _log(f"[bench]   {rec['tok_per_s']:.0f} tok/s, decode {rec['roofline']['achieved']:.0f} GB/s")
    if not args.no_cpu_baseline:
        _log(f"[bench]   oracle baseline {name}")
        rec["cpu_baseline"] = cpu_baseline_decode(c, args.cpu_seconds * CPU_SHARE[name], rows,
                                                  seqs=keep, kv_heads=ORACLE_KV_HEADS[name])
        rec["cpu_baseline"]["gpu_speedup"] = rec["tok_per_s"] / rec["cpu_baseline"]["value"]
        _log(f"[bench]   oracle {rec['cpu_baseline']['value']:.3g} tok/s; GPU error "
             f"{rec['cpu_baseline'].get('gpu_error_vs_oracle')}")
    return rec


def prefill_with_baseline(name, args):
    import synth

    c = synth.CONFIGS[name]
    edges = edge_rows_of(c)
    keep = prefill_rows(c, edges)
    _log(f"[bench] prefill {c.name}")
    rec, rows = prefill_record(c, args.prefill_reps, keep_rows=keep)
    _log(f"[bench]   {rec['tflops']:.0f} TFLOP/s, {rec['ms_per_prompt']:.2f} ms/prompt; "
         f"kv_append {rec['kv_append']['gbs']:.0f} GB/s")
    if not args.no_cpu_baseline:
        _log(f"[bench]   oracle baseline {name}")
        rec["cpu_baseline"] = cpu_baseline_prefill(c, args.cpu_seconds * CPU_SHARE[name], rows,
                                                   edge_rows=edges)
        rec["cpu_baseline"]["gpu_speedup"] = rec["tflops"] / rec["cpu_baseline"]["value"]
        _log(f"[bench]   oracle {rec['cpu_baseline']['value']:.3g} TFLOP/s; GPU error "
             f"{rec['cpu_baseline'].get('gpu_error_vs_oracle')}")
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-secondary", action="store_true", help="headline workloads only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="CPU budget unit of the oracle baselines (each takes a share)")
    ap.add_argument("--only", choices=["C2", "C3", "C5", "C4", "C4_128K", "C4_FP8", "hbm_copy",
                                       "block_copy", "page_in_overlap"],
                    help="run one workload and print its record (for profiling; no oracle)")
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
    if args.only == "page_in_overlap":
        print(json.dumps(page_in_overlap_record(args.steps, args.warmup)), flush=True)
        return 0
    if args.only:
        c = synth.CONFIGS[args.only]
        _log(f"[bench] only {c.name}")
        if args.only.startswith("C4"):
            rec, _ = prefill_record(c, args.prefill_reps)
        else:
            rec, _ = decode_record(c, args.steps, args.warmup, PARTITION_BLOCKS[args.only])
        print(json.dumps(rec), flush=True)
        return 0

    # headline: the 128K decode, with the 128K chunked prefill beside it
    head = decode_with_baseline("C3", args)
    pre128 = prefill_with_baseline("C4_128K", args)
    secondary = []
    if not args.no_secondary:
        for name in ("C2", "C5"):
            secondary.append(decode_with_baseline(name, args))
        for name in ("C4", "C4_FP8"):
            secondary.append(prefill_with_baseline(name, args))
        bc = block_copy_record()
        secondary.append(bc)
        _log(f"[bench] block copies: offload {bc['offload_gbs']:.1f} GB/s, page-in "
             f"{bc['page_in_gbs']:.1f} GB/s, in HBM {bc['hbm_copy_gbs_read_plus_write']:.0f} GB/s")
        ov = page_in_overlap_record(args.steps, args.warmup)
        secondary.append(ov)
        _log(f"[bench] page-in beside decode: overlap {ov['overlap_frac']:.2f}, decode "
             f"{ov['decode_gbs_during_page_in']:.0f} GB/s during the page-in "
             f"({ov['decode_gbs_alone']:.0f} alone), page-in {ov['page_in_gbs_alone']:.1f} GB/s")
    copy = hbm_copy_record()
    _log(f"[bench] plain device copy: {copy['gbs']:.0f} GB/s")

    cfg = synth.CONFIGS["C3"]
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
                   "partition_blocks": PARTITION_BLOCKS["C3"],
                   "step": "append 1 token/seq folded into split-KV decode "
                           "(pkv_paged_attn_decode_step) + LSE merge"},
        "ms_per_step_no_events": head["ms_per_step_no_events"],
        "merge_ms": head["merge_ms"],
        "decode_hbm_gbs": head["roofline"]["achieved"],
        "hbm_copy_gbs": copy["gbs"],
        "roofline": head["roofline"],
        "cpu_baseline": head.get("cpu_baseline"),
        "prefill_128k": pre128,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
