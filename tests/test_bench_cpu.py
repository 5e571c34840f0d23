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


@pytest.mark.parametrize("name", ["C4", "C4_128K"])
def test_chunked_pass_covers_the_causal_prompt_once(name):
    cfg = synth.CONFIGS[name]
    C, S, n = cfg.chunk, cfg.shard_len, cfg.prompt_len
    done = 0
    for a in range(0, n, C):
        b = min(a + C, n)
        nsh = -(-b // S)
        # one shard: the final form over [0, b); several: a partial per shard
        ranges = [(0, b)] if nsh == 1 else [(j * S, min((j + 1) * S, b)) for j in range(nsh)]
        done += sum(A.prefill_flops(a, b - a, lo, hi, cfg.hq, cfg.head_dim)
                    for lo, hi in ranges)
    assert done == A.causal_prompt_flops(n, cfg.hq, cfg.head_dim)
    assert done == 4 * cfg.head_dim * cfg.hq * n * (n + 1) // 2
