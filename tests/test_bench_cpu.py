"""Host-side checks of bench.py: the one-GPU refusal, and that the chunked
prefill pass it times scores every causal (row, key) pair of the prompt
exactly once, so the flops it divides by are the work its calls do."""
import pytest

import bench
import synth
from paged_kv_cache_210_amd import accounting as A


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


@pytest.mark.parametrize("name", ["C4", "C4_128K", "C4_FP8"])
def test_chunked_pass_covers_the_causal_prompt_once(name):
    """bench.chunk_plan, the plan bench.prefill_pass runs: chunks tile the
    prompt in order, each chunk's shards tile [0, chunk end) in order, a
    single shard is the final form, and the flops of the calls add up to the
    causal prompt's."""
    cfg = synth.CONFIGS[name]
    plan = bench.chunk_plan(cfg)
    assert [a for _, a, _, _ in plan] == list(range(0, cfg.prompt_len, cfg.chunk))
    assert plan[-1][2] == cfg.prompt_len
    done = 0
    for c, a, b, shards in plan:
        assert shards[0][0] == 0 and shards[-1][1] == b
        assert all(shards[j][1] == shards[j + 1][0] for j in range(len(shards) - 1))
        assert all(hi - lo <= cfg.shard_len for lo, hi in shards)
        done += sum(A.prefill_flops(a, b - a, lo, hi, cfg.hq, cfg.head_dim) for lo, hi in shards)
    assert done == A.causal_prompt_flops(cfg.prompt_len, cfg.hq, cfg.head_dim)
    assert done == 4 * cfg.head_dim * cfg.hq * cfg.prompt_len * (cfg.prompt_len + 1) // 2
    # the 32K prompt: 8 chunks, the first two in the final form, 20 shard calls
    if name == "C4":
        assert [len(sh) for *_, sh in plan] == [1, 1, 2, 2, 3, 3, 4, 4]


def test_oracle_error_fields():
    """bench.oracle_error: raw max abs, the part beyond bf16 output rounding,
    and the per-row relative error."""
    import numpy as np
    ref = np.array([[1.0, 0.5], [0.0, 0.0], [2.0, -4.0]])
    got = ref + np.array([[2.0 ** -9, 0], [0, 0], [0, 2.0 ** -5]])
    e = bench.oracle_error(got, ref)
    assert e["max_abs"] == 2.0 ** -5
    # 2^-9 at 1.0 is within half a bf16 ulp (2^-8); 2^-5 at 4.0 is one ulp,
    # half of which (2^-6) lies beyond the output rounding
    assert e["max_abs_beyond_bf16_rounding"] == 2.0 ** -6
    assert e["row_rel"] == max(2.0 ** -9 / 1.0, 2.0 ** -5 / 4.0)
    assert e["rows"] == 3


def test_edge_rows_and_kept_rows():
    cfg = synth.CONFIGS["C4"]
    edges = bench.edge_rows_of(cfg)
    assert edges == [0, 1, 63, 64, 4095, 4096, 8191, 8192, 16383, 16384, 24575, 24576]
    kept = bench.prefill_rows(cfg, edges)
    assert kept[:len(edges)] == edges and kept[-1] == cfg.prompt_len - 1
    assert len(kept) == len(edges) + 64
