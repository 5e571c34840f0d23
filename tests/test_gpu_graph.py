"""A decode step (kv_append of one token per sequence + split-KV decode + LSE
merge, or the same with the append folded into the decode launch) captured in
a HIP graph and replayed: every replay, with unrelated eager work between
replays, must give bit for bit what the eager step gives."""
import pytest
import torch

import synth
from tests._util import gpu_cache

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def lib():
    from paged_kv_cache_210_amd import lib as L
    L.load()
    return L


@pytest.mark.parametrize("kv_dtype,pb,folded", [("bf16", 0, False), ("bf16", 4, False),
                                                ("e4m3", 2, False), ("bf16", 0, True),
                                                ("bf16", 4, True)])
def test_decode_step_graph_replays_match_eager(lib, kv_dtype, pb, folded):
    """folded: the step is pkv_paged_attn_decode_step_partial (append inside
    the decode launch) + merge instead of append + decode + merge."""
    cfg = synth.decode_config("graph", (300, 1000, 17, 64), 16, 4, 128, q_dtype="bf16",
                              kv_dtype=kv_dtype, seed_index=31)
    host = synth.decode_inputs(cfg, device="cpu")
    inp = {k: host[k].to(DEV) for k in ("q", "k", "v", "seq_idx", "pos")}
    tables, _ = lib.build_tables(cfg.seq_lens, cfg.pool_blocks, host["free_order"])
    td = tables.to(DEV)
    cache = gpu_cache(lib, cfg, inp, td, poison=True)
    lens = torch.tensor(cfg.seq_lens, dtype=torch.int32, device=DEV)
    # the step re-appends each sequence's last token (same values, same slot)
    last = torch.cumsum(lens, 0) - 1
    k1, v1 = inp["k"][last].contiguous(), inp["v"][last].contiguous()
    seq = torch.arange(cfg.batch, dtype=torch.int32, device=DEV)
    pos = (lens - 1).to(torch.int32)
    B, hq, D = inp["q"].shape
    P = lib.decode_partitions(cache, torch.bfloat16, B, hq, td.shape[1], pb)

    def buffers():
        part = (torch.empty(P, B, hq, D, device=DEV), torch.empty(P, B, hq, device=DEV),
                torch.empty(P, B, hq, device=DEV))
        return part, torch.empty(B, hq, D, dtype=torch.bfloat16, device=DEV), \
            torch.empty(B, hq, device=DEV)

    def step(part, out, lse):
        if folded:
            lib.paged_attn_decode_step(cache, k1, v1, inp["q"], td, lens, partition_blocks=pb,
                                       partial=True, part=part)
        else:
            lib.kv_append(cache, k1, v1, seq, pos, td)
            lib.paged_attn_decode_partial(cache, inp["q"], td, lens, partition_blocks=pb,
                                          part=part)
        lib.attn_lse_merge(*part, out=out, with_state=False, out_lse=lse)

    pe, oe, le = buffers()
    step(pe, oe, le)
    torch.cuda.synchronize()
    pool_k = cache.k.clone()

    pg, og, lg = buffers()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step(pg, og, lg)
    torch.cuda.current_stream().wait_stream(side)
    with torch.cuda.graph(graph):
        step(pg, og, lg)

    other_q = torch.randn(B, hq, D, device=DEV).to(torch.bfloat16)
    for r in range(3):
        og.zero_()
        lg.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(og.view(torch.int16), oe.view(torch.int16)), f"replay {r}: out"
        assert torch.equal(lg, le), f"replay {r}: lse"
        assert torch.equal(cache.k.view(torch.uint8), pool_k.view(torch.uint8)), f"replay {r}: pool"
        # unrelated eager work on the same stream between replays
        po2, o2, l2 = buffers()
        lib.paged_attn_decode_partial(cache, other_q, td, lens, partition_blocks=pb, part=po2)
        lib.attn_lse_merge(*po2, out=o2, with_state=False, out_lse=l2)
        torch.cuda.synchronize()
