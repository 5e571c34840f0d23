"""Pins for the CPU oracle: it is checked against things other than itself.

* brute force: torch's scaled_dot_product_attention in float64 on CPU, run on
  contiguous (never paged) K/V with an explicit boolean mask;
* closed forms of softmax attention (one key, constant V, zero query, scale
  invariance, a dominant score, equal queries in a GQA group);
* invariants: permutation of physical blocks, chunked merge == full softmax,
  merge associativity, prefill row p == decode at length p+1;
* the E4M3 codec against torch.float8_e4m3fn and hand-derived codes.
"""
import math

import numpy as np
import pytest
import torch

from oracle import pkv_oracle as O
import synth

RNG = np.random.default_rng(7)


def _bits(t):
    """bf16 torch tensor -> uint16 numpy bits."""
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _paged(seq_lens, hkv, d, fmt, pool_blocks, perm_seed, k, v, fill=None):
    """Tables from a seeded permutation and a pool filled by oracle.append."""
    order = synth.free_order(pool_blocks, perm_seed).numpy()
    tables, waste = O.build_tables(seq_lens, pool_blocks, order)
    cache = O.new_cache(pool_blocks, hkv, d, fmt, fill=fill)
    seq_idx, pos = synth.token_positions(seq_lens)
    O.append(cache, k, v, seq_idx.numpy(), pos.numpy(), tables)
    return cache, tables, waste


def _sdpa(q, K, V, mask, scale):
    """Library brute force: q [R,d], K/V [n,d] float64, mask bool [R,n]."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(K)[None, None]
    vt = torch.from_numpy(V)[None, None]
    mt = torch.from_numpy(mask)[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)
    return o[0, 0].numpy()


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_decode_matches_sdpa_on_contiguous_kv(fmt):
    cfg = synth.CONFIGS["C1"] if fmt == "f32" else synth.decode_config(
        "tiny bf16", (5, 16, 17, 50), 8, 2, 128, q_dtype="bf16", seed_index=11)
    inp = synth.decode_inputs(cfg)
    conv = (lambda t: t.numpy()) if fmt == "f32" else _bits
    cache, tables, _ = _paged(cfg.seq_lens, cfg.hkv, cfg.head_dim, fmt, cfg.pool_blocks,
                              cfg.perm_seed, conv(inp["k"]), conv(inp["v"]))
    out = O.decode(cache, conv(inp["q"]), fmt, tables, cfg.seq_lens)
    kf = inp["k"].double().numpy()
    vf = inp["v"].double().numpy()
    qf = inp["q"].double().numpy()
    G = cfg.hq // cfg.hkv
    start = 0
    for b, n in enumerate(cfg.seq_lens):
        for h in range(cfg.hq):
            K = kf[start:start + n, h // G]
            V = vf[start:start + n, h // G]
            ref = _sdpa(qf[b, h][None], K, V, np.ones((1, n), bool), 1 / math.sqrt(cfg.head_dim))
            np.testing.assert_allclose(out["o"][b, h], ref[0], rtol=1e-12, atol=1e-13)
        start += n


@pytest.mark.parametrize("q_pos0,kv_begin,kv_end,causal", [
    (0, 0, 40, True), (24, 0, 64, True), (33, 10, 57, True), (20, 0, 50, False),
    (5, 30, 70, True),   # rows before kv_begin see nothing: empty rows
])
def test_prefill_matches_sdpa_with_mask(q_pos0, kv_begin, kv_end, causal):
    hq, hkv, d, T = 4, 2, 64, 24
    n_total = max(kv_end, q_pos0 + T)
    g = torch.Generator().manual_seed(99)
    q = torch.randn(T, hq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(n_total, hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(n_total, hkv, d, generator=g).to(torch.bfloat16)
    pool = O.BLOCK and (n_total // 16 + 4)
    cache, tables, _ = _paged([n_total], hkv, d, "bf16", pool, 5, _bits(k), _bits(v))
    out = O.prefill(cache, _bits(q), "bf16", q_pos0, tables[0], kv_begin, kv_end, causal)
    qf, kf, vf = q.double().numpy(), k.double().numpy(), v.double().numpy()
    t = np.arange(kv_end)
    for h in range(hq):
        for r in range(T):
            vis = (t >= kv_begin) & (t < kv_end)
            if causal:
                vis &= t <= q_pos0 + r
            if not vis.any():
                assert np.all(out["o"][r, h] == 0) and out["m"][r, h] == -np.inf
                assert out["l"][r, h] == 0 and out["lse"][r, h] == -np.inf
                continue
            K, V = kf[:kv_end, h // 2][vis], vf[:kv_end, h // 2][vis]
            ref = _sdpa(qf[r, h][None], K, V, np.ones((1, len(K)), bool), 1 / 8.0)
            np.testing.assert_allclose(out["o"][r, h], ref[0], rtol=1e-12, atol=1e-13)
            # lse against scipy's logsumexp of the raw scores
            from scipy.special import logsumexp
            assert abs(out["lse"][r, h] - logsumexp(K @ qf[r, h] / 8.0)) < 1e-12


# ---------------------------------------------------------------- closed forms
def _one_seq_cache(K, V, fmt="f32", pool=8, seed=3):
    n, d = K.shape
    k = K[:, None, :].astype(np.float32)
    v = V[:, None, :].astype(np.float32)
    cache, tables, _ = _paged([n], 1, d, fmt, pool, seed, k, v)
    return cache, tables


def test_single_key_returns_its_value():
    K = RNG.standard_normal((1, 64)).astype(np.float32)
    V = RNG.standard_normal((1, 64)).astype(np.float32)
    cache, tables = _one_seq_cache(K, V)
    q = RNG.standard_normal((1, 1, 64)).astype(np.float32)
    out = O.decode(cache, q, "f32", tables, [1])
    np.testing.assert_array_equal(out["o"][0, 0], V[0].astype(np.float64))
    assert out["l"][0, 0] == 1.0


def test_zero_query_gives_mean_of_values():
    K = RNG.standard_normal((37, 64)).astype(np.float32)
    V = RNG.standard_normal((37, 64)).astype(np.float32)
    cache, tables = _one_seq_cache(K, V)
    out = O.decode(cache, np.zeros((1, 1, 64), np.float32), "f32", tables, [37])
    np.testing.assert_allclose(out["o"][0, 0], V.astype(np.float64).mean(0), rtol=1e-13, atol=1e-14)
    assert out["l"][0, 0] == 37.0 and out["m"][0, 0] == 0.0


def test_constant_values_give_that_constant():
    K = RNG.standard_normal((50, 64)).astype(np.float32)
    V = np.tile(RNG.standard_normal((1, 64)).astype(np.float32), (50, 1))
    cache, tables = _one_seq_cache(K, V)
    q = RNG.standard_normal((1, 1, 64)).astype(np.float32)
    out = O.decode(cache, q, "f32", tables, [50])
    np.testing.assert_allclose(out["o"][0, 0], V[0].astype(np.float64), rtol=1e-13, atol=1e-14)


def test_scale_invariance():
    K = RNG.standard_normal((40, 64)).astype(np.float32)
    V = RNG.standard_normal((40, 64)).astype(np.float32)
    q = RNG.standard_normal((1, 1, 64)).astype(np.float32)
    c1, t1 = _one_seq_cache(K, V)
    c2, t2 = _one_seq_cache(K * np.float32(4.0), V)         # exact in fp32
    a = O.decode(c1, q, "f32", t1, [40], scale=0.3)
    b = O.decode(c2, q, "f32", t2, [40], scale=0.075)
    np.testing.assert_allclose(a["o"], b["o"], rtol=1e-13, atol=1e-14)


def test_dominant_score_selects_its_value():
    K = (RNG.standard_normal((30, 64)) * 0.01).astype(np.float32)
    q = np.zeros((1, 1, 64), np.float32)
    q[0, 0, 3] = 1.0
    K[17, 3] = 400.0                           # score 50 after 1/8 scaling
    V = RNG.standard_normal((30, 64)).astype(np.float32)
    cache, tables = _one_seq_cache(K, V)
    out = O.decode(cache, q, "f32", tables, [30])
    np.testing.assert_allclose(out["o"][0, 0], V[17], rtol=1e-15, atol=1e-18)


def test_equal_queries_in_a_gqa_group_give_equal_outputs():
    cfg = synth.decode_config("gqa", (33, 70), 8, 2, 64, q_dtype="f32", seed_index=12)
    inp = synth.decode_inputs(cfg)
    q = inp["q"].numpy().copy()
    q[:, 1] = q[:, 0]
    q[:, 6] = q[:, 5]
    cache, tables, _ = _paged(cfg.seq_lens, 2, 64, "f32", cfg.pool_blocks, cfg.perm_seed,
                              inp["k"].numpy(), inp["v"].numpy())
    out = O.decode(cache, q, "f32", tables, cfg.seq_lens)
    np.testing.assert_array_equal(out["o"][:, 1], out["o"][:, 0])
    np.testing.assert_array_equal(out["o"][:, 6], out["o"][:, 5])
    assert not np.array_equal(out["o"][:, 0], out["o"][:, 5])   # different kv heads


# ---------------------------------------------------------------- invariants
def test_block_permutation_invariance_bitwise():
    cfg = synth.CONFIGS["C1"]
    inp = synth.decode_inputs(cfg)
    k, v, q = inp["k"].numpy(), inp["v"].numpy(), inp["q"].numpy()
    c1, t1, _ = _paged(cfg.seq_lens, 2, 64, "f32", 32, 2001, k, v)
    c2, t2, _ = _paged(cfg.seq_lens, 2, 64, "f32", 32, 777, k, v)
    assert not np.array_equal(t1, t2)
    a = O.decode(c1, q, "f32", t1, cfg.seq_lens)
    b = O.decode(c2, q, "f32", t2, cfg.seq_lens)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


def test_stray_reads_never_happen_poisoned_pool():
    cfg = synth.CONFIGS["C1"]
    inp = synth.decode_inputs(cfg)
    k, v, q = inp["k"].numpy(), inp["v"].numpy(), inp["q"].numpy()
    c1, t1, _ = _paged(cfg.seq_lens, 2, 64, "f32", 32, 2001, k, v)
    c2, t2, _ = _paged(cfg.seq_lens, 2, 64, "f32", 32, 2001, k, v, fill=np.nan)
    a = O.decode(c1, q, "f32", t1, cfg.seq_lens)
    b = O.decode(c2, q, "f32", t2, cfg.seq_lens)
    assert np.all(np.isfinite(b["o"]))
    np.testing.assert_array_equal(a["o"], b["o"])


@pytest.mark.parametrize("cuts", [[0, 48, 200], [0, 0, 1, 2, 100, 200], [0, 17, 17, 150, 199, 200],
                                  [0, 200]])
def test_chunked_merge_equals_full_softmax(cuts):
    hq, hkv, d, T, n = 4, 2, 64, 8, 200
    g = torch.Generator().manual_seed(5)
    q = torch.randn(T, hq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(n, hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(n, hkv, d, generator=g).to(torch.bfloat16)
    cache, tables, _ = _paged([n], hkv, d, "bf16", 20, 9, _bits(k), _bits(v))
    full = O.prefill(cache, _bits(q), "bf16", n - T, tables[0], 0, n, True)
    parts = []
    for a, b in zip(cuts[:-1], cuts[1:]):
        p = O.prefill(cache, _bits(q), "bf16", n - T, tables[0], a, b, True)
        parts.append((p["o_un"], p["m"], p["l"]))
    Om, M, L = O.lse_merge(parts)
    np.testing.assert_allclose(Om, full["o"], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(O.lse_of(M, L), full["lse"], rtol=1e-13, atol=1e-13)


def test_merge_is_associative_and_all_empty_is_empty():
    shape = (3, 5)
    def part(seed, empty=False):
        r = np.random.default_rng(seed)
        if empty:
            return np.zeros(shape + (8,)), np.full(shape, -np.inf), np.zeros(shape)
        return r.standard_normal(shape + (8,)), r.standard_normal(shape) * 3, r.random(shape) + 0.5
    A, B, C = part(1), part(2), part(3)
    def as_part(merged):
        o, m, l = merged
        return o * l[..., None], m, l
    left = O.lse_merge([as_part(O.lse_merge([A, B])), C])
    right = O.lse_merge([A, as_part(O.lse_merge([B, C]))])
    flat = O.lse_merge([A, B, C])
    for x, y in ((left, flat), (right, flat)):
        np.testing.assert_allclose(x[0], y[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(x[2] * np.exp(x[1] - y[1]), y[2], rtol=1e-13)
    E = part(0, empty=True)
    stale = (np.full(shape + (8,), np.nan), np.full(shape, -np.inf), np.zeros(shape))
    o3, m3, l3 = O.lse_merge([A, stale, B])
    o4, m4, l4 = O.lse_merge([A, B])
    np.testing.assert_array_equal(o3, o4)
    o, m, l = O.lse_merge([E, E])
    assert np.all(o == 0) and np.all(m == -np.inf) and np.all(l == 0)
    o2, m2, l2 = O.lse_merge([E, A, E])
    np.testing.assert_allclose(o2, A[0] / A[2][..., None], rtol=1e-14)


def test_prefill_row_equals_decode_at_that_length():
    hq, hkv, d, n = 4, 2, 64, 90
    g = torch.Generator().manual_seed(21)
    q = torch.randn(n, hq, d, generator=g).to(torch.bfloat16)
    k = torch.randn(n, hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(n, hkv, d, generator=g).to(torch.bfloat16)
    cache, tables, _ = _paged([n], hkv, d, "bf16", 12, 4, _bits(k), _bits(v))
    pre = O.prefill(cache, _bits(q), "bf16", 0, tables[0], 0, n, True)
    for p in (0, 15, 16, 47, 89):
        dec = O.decode(cache, _bits(q[p:p + 1]), "bf16", tables[:1], [p + 1])
        np.testing.assert_allclose(pre["o"][p], dec["o"][0], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------- allocator
def test_allocator_waste_bound_brute_force():
    for n in range(0, 700):
        alloc = O.Allocator(64)
        alloc.reserve(0, n)
        w = alloc.waste_slots(0)
        assert w == 16 * (-(-n // 16)) - n and 0 <= w <= 15
        if n >= 210:                  # ratio form of the 6.25 % bound
            assert w <= (-(-n // 16)) and w / (16 * (-(-n // 16))) <= 1 / 16
    # the ratio form fails below 210 (e.g. 209 tokens waste 15 of 224 slots)
    alloc = O.Allocator(64)
    alloc.reserve(0, 209)
    assert alloc.waste_slots(0) / 224 > 1 / 16


def test_allocator_grows_on_demand_and_never_double_owns():
    order = synth.free_order(40, 123).numpy()
    alloc = O.Allocator(40, order)
    lens = [0, 0, 0]
    r = np.random.default_rng(3)
    handed = []
    for step in range(300):
        s = int(r.integers(0, 3))
        before = len(alloc.tables.get(s, []))
        lens[s] += int(r.integers(0, 6))
        try:
            row = alloc.reserve(s, lens[s])
        except O.OutOfBlocks:
            alloc.release(s)
            lens[s] = 0
            continue
        handed.extend(row[before:])
        owned = [b for t in alloc.tables.values() for b in t]
        assert len(owned) == len(set(owned))
        assert len(owned) + alloc.free_count() == 40
        assert len(row) == -(-lens[s] // 16)
    # the first blocks handed out follow the free order
    assert handed[:5] == list(order[:5])


def test_allocator_exhaustion_and_reuse():
    alloc = O.Allocator(3, [2, 0, 1])
    assert alloc.reserve(0, 33) == [2, 0, 1]
    with pytest.raises(O.OutOfBlocks):
        alloc.reserve(1, 1)
    alloc2 = O.Allocator(3, [2, 0, 1])
    alloc2.reserve(0, 16)
    with pytest.raises(O.OutOfBlocks):          # needs 3 more, 2 free: nothing changes
        alloc2.reserve(0, 64)
    assert alloc2.free_count() == 2 and alloc2.waste_slots(0) == 0
    alloc.release(0)
    assert alloc.reserve(1, 16) == [2]


def test_build_tables_pads_with_minus_one():
    tables, waste = O.build_tables([37, 100], 32, synth.free_order(32, 2001).numpy())
    assert tables.shape == (2, 7)
    assert list(tables[0, 3:]) == [-1] * 4 and (tables[1] >= 0).all()
    assert waste == [11, 12]
    assert len(set(tables[tables >= 0].tolist())) == 10


# ---------------------------------------------------------------- E4M3 codec
def test_e4m3_decode_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    mine = O.e4m3_decode(np.arange(256, dtype=np.uint8))
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(mine), nan)
    np.testing.assert_array_equal(mine[~nan], ref[~nan])
    assert mine[0x7E] == 448.0 and mine[0x01] == 2.0 ** -9 and mine[0x08] == 2.0 ** -6


def test_e4m3_encode_roundtrip_and_ties():
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    vals = O.e4m3_decode(np.array(finite, np.uint8)).astype(np.float32)
    np.testing.assert_array_equal(O.e4m3_encode(vals), np.array(finite, np.uint8))
    cases = [(1.0625, 0x38), (1.1875, 0x3A), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02),
             (-1.0625, 0xB8), (449.0, 0x7E), (1e6, 0x7E), (-1e30, 0xFE), (464.0, 0x7E),
             (0.0, 0x00), (-0.0, 0x80), (-2.0 ** -11, 0x80)]
    for x, c in cases:
        assert O.e4m3_encode(np.float32(x)) == c, (x, hex(c))
    assert O.e4m3_encode(np.float32(np.nan)) == 0x7F


def test_e4m3_encode_matches_torch_in_range():
    x = (np.random.default_rng(0).standard_normal(200000) * 60).astype(np.float32)
    x = np.concatenate([x, (np.random.default_rng(1).standard_normal(20000) * 0.01).astype(np.float32)])
    x = np.clip(x, -448, 448)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_encode(x), ref)


def test_group_scales_map_group_max_to_448():
    cfg = synth.decode_config("fp8", (150, 64), 2, 2, 64, q_dtype="bf16", kv_dtype="e4m3",
                              seed_index=13, outlier_prob=0.01)
    inp = synth.decode_inputs(cfg)
    kf = inp["k"].float().numpy()
    order = synth.free_order(cfg.pool_blocks, cfg.perm_seed).numpy()
    tables, _ = O.build_tables(cfg.seq_lens, cfg.pool_blocks, order)
    cache = O.new_cache(cfg.pool_blocks, 2, 64, "e4m3")
    start = 0
    for b, n in enumerate(cfg.seq_lens):
        O.fp8_group_scales(kf[start:start + n], 0, tables[b], cache.k_scale)
        start += n
    # every block of a 64-token group carries the same scale
    row = tables[0]
    for g0 in range(0, 150, 64):
        blocks = row[g0 // 16: min(g0 + 64, 150) // 16 + (1 if min(g0 + 64, 150) % 16 else 0)]
        vals = {float(cache.k_scale[b, 1]) for b in blocks}
        assert len(vals) == 1
        amax = np.abs(kf[g0:min(g0 + 64, 150), 1]).max()
        s = vals.pop()
        assert s == np.float32(amax / np.float32(448))
        code = O.e4m3_encode(np.float32(np.float32(amax) * np.float32(1 / np.float32(s))))
        assert code == 0x7E
    assert np.all(O.group_scale(np.float32(0.0)) == 1.0)
    assert np.all(O.group_scale(np.float32(1e-43)) == 1.0)


def test_fp8_append_dequant_error_within_half_ulp():
    d = 64
    x = (np.random.default_rng(2).standard_normal((64, 1, d)) * 3).astype(np.float32)
    cache = O.new_cache(8, 1, d, "e4m3")
    tables, _ = O.build_tables([64], 8, np.arange(8))
    O.fp8_group_scales(x, 0, tables[0], cache.k_scale)
    O.fp8_group_scales(x, 0, tables[0], cache.v_scale)
    O.append(cache, x, x, np.zeros(64, np.int32), np.arange(64, dtype=np.int32), tables)
    K, V = O.gather_kv(cache, tables[0], 64, 0)
    s = float(cache.k_scale[tables[0][0], 0])
    y = x[:, 0].astype(np.float64) / s
    err = np.abs(K / s - x[:, 0].astype(np.float64) / s)
    # half an E4M3 ulp: 2^(e-4) for normals (|y| >= 2^-6), 2^-10 for subnormals (+ f32 rounding)
    bound = np.where(np.abs(y) >= 2 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 1e-30))) - 4),
                     2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)
    np.testing.assert_array_equal(K, V)


def test_fp8_attention_is_attention_over_dequantised_values():
    d, n = 64, 80
    r = np.random.default_rng(4)
    x = (r.standard_normal((n, 1, d))).astype(np.float32)
    y = (r.standard_normal((n, 1, d))).astype(np.float32)
    cache = O.new_cache(8, 1, d, "e4m3")
    tables, _ = O.build_tables([n], 8, np.arange(8)[::-1].copy())
    O.fp8_group_scales(x, 0, tables[0], cache.k_scale)
    O.fp8_group_scales(y, 0, tables[0], cache.v_scale)
    O.append(cache, x, y, np.zeros(n, np.int32), np.arange(n, dtype=np.int32), tables)
    # dequantised values rebuilt independently from the stored codes and scales
    Kd = np.zeros((n, d)); Vd = np.zeros((n, d))
    for t in range(n):
        blk = tables[0][t // 16]
        Kd[t] = torch.from_numpy(cache.k[blk, 0, t % 16].copy()).view(torch.float8_e4m3fn).double().numpy() \
            * float(cache.k_scale[blk, 0])
        Vd[t] = torch.from_numpy(cache.v[blk, 0, :, t % 16].copy()).view(torch.float8_e4m3fn).double().numpy() \
            * float(cache.v_scale[blk, 0])
    q = r.standard_normal((1, 1, d)).astype(np.float32)
    out = O.decode(cache, q, "f32", tables, [n])
    ref = _sdpa(q[0].astype(np.float64), Kd, Vd, np.ones((1, n), bool), 1 / 8.0)
    np.testing.assert_allclose(out["o"][0], ref, rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- append
def test_append_places_tokens_by_table():
    tables = np.array([[3, 1, -1], [0, 2, 4]], np.int32)
    cache = O.new_cache(5, 2, 8, "f32", fill=-7.0)
    k = np.arange(3 * 2 * 8, dtype=np.float32).reshape(3, 2, 8)
    v = -k
    O.append(cache, k, v, np.array([0, 1, 1], np.int32), np.array([17, 0, 40], np.int32), tables)
    np.testing.assert_array_equal(cache.k[1, :, 1, :], k[0])
    np.testing.assert_array_equal(cache.v[1, :, :, 1], v[0])
    np.testing.assert_array_equal(cache.k[0, :, 0, :], k[1])
    np.testing.assert_array_equal(cache.k[4, :, 8, :], k[2])
    np.testing.assert_array_equal(cache.v[4, :, :, 8], v[2])
    assert (cache.k == -7).sum() == cache.k.size - 3 * 16


@pytest.mark.parametrize("fmt", ["bf16", "e4m3"])
def test_bulk_append_equals_token_append(fmt):
    hkv, d, n = 2, 64, 150
    g = torch.Generator().manual_seed(8)
    k = torch.randn(n, hkv, d, generator=g).to(torch.bfloat16)
    v = torch.randn(n, hkv, d, generator=g).to(torch.bfloat16)
    order = synth.free_order(14, 31).numpy()
    tables, _ = O.build_tables([n], 14, order)
    a = O.new_cache(14, hkv, d, fmt)
    b = O.new_cache(14, hkv, d, fmt)
    if fmt == "e4m3":
        kk, vv = k.float().numpy(), v.float().numpy()
        for c in (a, b):
            O.fp8_group_scales(kk, 0, tables[0], c.k_scale)
            O.fp8_group_scales(vv, 0, tables[0], c.v_scale)
    else:
        kk, vv = _bits(k), _bits(v)
    O.append(a, kk, vv, np.zeros(n, np.int32), np.arange(n, dtype=np.int32), tables)
    O.append_sequence(b, kk[:37], vv[:37], tables[0], 0, chunk=16)
    O.append_sequence(b, kk[37:], vv[37:], tables[0], 37, chunk=50)
    np.testing.assert_array_equal(a.k, b.k)
    np.testing.assert_array_equal(a.v, b.v)
    c = O.new_cache(14, hkv, d, fmt)
    if fmt == "e4m3":
        c.k_scale[:], c.v_scale[:] = a.k_scale, a.v_scale
    O.append_sequence(c, kk, vv, tables[0], 0, heads=[1])
    np.testing.assert_array_equal(c.k[:, 1], a.k[:, 1])
    assert not c.k[:, 0].any()


# ---------------------------------------------------------------- prefix sharing
def _chain_hashes(tokens):
    """Caller-side prefix hashes: hash j covers tokens [0, 16(j+1))."""
    out, h = [], 1469598103934665603
    for j in range(len(tokens) // 16):
        for t in tokens[16 * j:16 * j + 16]:
            h = ((h ^ int(t)) * 1099511628211) % (1 << 64)
        out.append(h)
    return out


def _check_sharing_state(alloc, nb):
    held = {}
    for s, t in alloc.tables.items():
        for b in t:
            held[b] = held.get(b, 0) + 1
    for b in range(nb):
        assert alloc.refcount(b) == held.get(b, 0)
    assert not set(held) & set(alloc.free)
    assert len(held) + alloc.free_count() == nb
    assert len(set(alloc.free)) == len(alloc.free)
    for h, b in alloc.by_hash.items():
        assert alloc.hash_of[b] == h and b in held


def test_sharing_allocator_keeps_every_sequence_its_own_tokens():
    """Brute force against the plain definition: every sequence owns its list
    of token values.  Tokens are written through the table into an oracle pool
    (K = the token value), shared blocks are copied with copy_blocks when
    reserve_cow names a pair, sequences fork and take over published prefixes,
    and after every step each sequence reads back exactly its own tokens."""
    nb = 48
    alloc = O.Allocator(nb, synth.free_order(nb, 99).numpy())
    cache = O.new_cache(nb, 1, 4, "f32", fill=np.nan)
    truth = {}
    r = np.random.default_rng(5)
    next_val = [1.0]

    def write(seq, n_new):
        toks = []
        for _ in range(n_new):
            toks.append(next_val[0])
            next_val[0] += 1.0
        return toks

    for step in range(1500):
        op = r.random()
        seqs = sorted(truth)
        if op < 0.45 or not seqs:                       # grow a sequence
            s = int(r.integers(0, 8))
            old = truth.get(s, [])
            toks = write(s, int(r.integers(1, 24)))
            try:
                table, pair = alloc.reserve_cow(s, len(old) + len(toks))
            except O.OutOfBlocks:
                continue
            if pair is not None:
                O.copy_blocks(cache, cache, [pair[0]], [pair[1]])
            tab = np.array([table], dtype=np.int32)
            vals = np.array(toks, dtype=np.float32)[:, None, None] * np.ones((1, 1, 4), np.float32)
            O.append(cache, vals, vals, np.zeros(len(toks), np.int32),
                     np.arange(len(old), len(old) + len(toks)), tab)
            truth[s] = old + toks
        elif op < 0.6:                                  # fork
            s = seqs[int(r.integers(0, len(seqs)))]
            d = int(r.integers(0, 8))
            if d in truth:
                continue
            alloc.fork(s, d)
            truth[d] = list(truth[s])
        elif op < 0.72:                                 # publish full blocks
            s = seqs[int(r.integers(0, len(seqs)))]
            hs = _chain_hashes(truth[s])
            alloc.publish_prefix(s, hs)
        elif op < 0.82:                                 # a new sequence reuses a prefix
            s = seqs[int(r.integers(0, len(seqs)))]
            d = int(r.integers(0, 8))
            if d in truth:
                continue
            extra = write(d, 5)
            want = _chain_hashes(truth[s]) + _chain_hashes(truth[s] + extra)[len(truth[s]) // 16:]
            m = alloc.match_prefix(d, want)
            published = [h for h in want if h in alloc.by_hash]
            assert m <= len(want)
            truth[d] = truth[s][:16 * m]
            assert m == 0 or alloc.tables[d] == [alloc.by_hash[h] for h in want[:m]]
            assert set(want[:m]) <= set(published)
        else:                                           # release
            s = seqs[int(r.integers(0, len(seqs)))]
            alloc.release(s)
            del truth[s]
        _check_sharing_state(alloc, nb)
        for s, toks in truth.items():
            assert alloc.lens[s] == len(toks)
            if toks:
                K, _ = O.gather_kv(cache, alloc.tables[s], len(toks), 0)
                assert np.array_equal(K[:, 0], np.array(toks)), (step, s)


def test_plain_reserve_refuses_to_write_into_a_shared_block():
    alloc = O.Allocator(8)
    alloc.reserve(0, 20)                         # blocks 0, 1 (block 1 partly filled)
    alloc.fork(0, 1)
    assert alloc.refcount(1) == 2
    with pytest.raises(O.SharedBlock):
        alloc.reserve(0, 21)
    assert alloc.lens[0] == 20 and alloc.free_count() == 6
    table, pair = alloc.reserve_cow(1, 40)       # fresh block first, then growth
    assert pair == (1, 2) and table == [0, 2, 3]
    assert alloc.refcount(1) == 1 and alloc.refcount(0) == 2
    assert alloc.reserve(0, 32) == [0, 1]        # sole holder now: writes in place
    alloc2 = O.Allocator(4)
    alloc2.reserve(0, 32)                        # full last block: growth never copies
    alloc2.fork(0, 1)
    assert alloc2.reserve_cow(1, 33) == ([0, 1, 2], None)
    alloc3 = O.Allocator(2)
    alloc3.reserve(0, 20)
    alloc3.fork(0, 1)
    with pytest.raises(O.OutOfBlocks):           # no block left for the copy
        alloc3.reserve_cow(1, 21)
    assert alloc3.tables[1] == [0, 1] and alloc3.refcount(1) == 2


def test_published_prefix_leaves_index_when_freed():
    alloc = O.Allocator(8)
    toks = list(range(40))
    alloc.reserve(0, 40)
    hs = _chain_hashes(toks)
    with pytest.raises(ValueError):              # the third block is not full
        alloc.publish_prefix(0, hs + [123])
    alloc.publish_prefix(0, hs)
    assert alloc.match_prefix(5, hs) == 2 and alloc.lens[5] == 32
    assert alloc.tables[5] == alloc.tables[0][:2]
    assert alloc.match_prefix(6, [hs[0], 999, hs[1]]) == 1
    alloc.release(0)
    alloc.release(5)
    assert alloc.by_hash and alloc.refcount(alloc.tables[6][0]) == 1
    alloc.release(6)
    assert not alloc.by_hash and alloc.free_count() == 8
    assert alloc.match_prefix(7, hs) == 0


# ---------------------------------------------------------------- KV offload
def _read_back(alloc, dev, host, seq, n):
    """Token values of sequence `seq` ([n]) read through its page table: from
    the device pool for resident blocks, from its host slot otherwise."""
    out = []
    for j in range(-(-n // 16)):
        b, slot, _ = alloc.block_state(seq, j)
        pool, blk = (host, slot) if b == O.OFFLOADED else (dev, b)
        cnt = min(16, n - 16 * j)
        out.extend(pool.k[blk, 0, :cnt, 0].tolist())
    return out


def test_offload_page_table_keeps_every_sequence_its_own_tokens():
    """Brute force against the plain definition with a host tier [P3 section
    4.2]: every sequence owns its list of token values; blocks move between the
    device pool and host slots (O.copy_blocks over the returned pairs), grow,
    fork, publish / match prefixes and release in random order, and after
    every step each sequence reads back exactly its own tokens through its page
    table; device blocks and host slots are each held once or free."""
    nb, nh = 40, 24
    alloc = O.Allocator(nb, synth.free_order(nb, 41).numpy())
    alloc.set_host_slots(nh)
    dev = O.new_cache(nb, 1, 4, "f32", fill=np.nan)
    host = O.new_cache(nh, 1, 4, "f32", fill=np.nan)
    truth = {}
    r = np.random.default_rng(11)
    nxt = [1.0]
    moved = {"out": 0, "in": 0}
    for step in range(2000):
        op = r.random()
        seqs = sorted(truth)
        if op < 0.3 or not seqs:                           # grow
            s = int(r.integers(0, 6))
            old = truth.get(s, [])
            toks = [nxt[0] + i for i in range(int(r.integers(1, 24)))]
            try:
                table, pair = alloc.reserve_cow(s, len(old) + len(toks))
            except (O.OutOfBlocks, O.Offloaded):
                continue
            nxt[0] += len(toks)
            if pair is not None:
                O.copy_blocks(dev, dev, [pair[0]], [pair[1]])
            vals = np.array(toks, np.float32)[:, None, None] * np.ones((1, 1, 4), np.float32)
            O.append(dev, vals, vals, np.zeros(len(toks), np.int32),
                     np.arange(len(old), len(old) + len(toks)), np.array([table], np.int32))
            truth[s] = old + toks
        elif op < 0.5:                                     # offload a range
            s = seqs[int(r.integers(0, len(seqs)))]
            first, count = int(r.integers(0, 6)), int(r.integers(0, 6))
            try:
                pairs = alloc.offload(s, first, count)
            except (O.OutOfBlocks, O.SharedBlock):
                continue
            O.copy_blocks(dev, host, [p[0] for p in pairs], [p[1] for p in pairs])
            moved["out"] += len(pairs)
        elif op < 0.7:                                     # page a range back in
            s = seqs[int(r.integers(0, len(seqs)))]
            first, count = int(r.integers(0, 6)), int(r.integers(0, 6))
            try:
                pairs = alloc.page_in(s, first, count)
            except O.OutOfBlocks:
                continue
            O.copy_blocks(host, dev, [p[0] for p in pairs], [p[1] for p in pairs])
            moved["in"] += len(pairs)
        elif op < 0.78:                                    # fork
            s = seqs[int(r.integers(0, len(seqs)))]
            d = int(r.integers(0, 6))
            if d in truth:
                continue
            try:
                alloc.fork(s, d)
            except O.Offloaded:
                assert O.OFFLOADED in alloc.tables[s]
                continue
            truth[d] = list(truth[s])
        elif op < 0.86:                                    # publish, then a new one matches
            s = seqs[int(r.integers(0, len(seqs)))]
            alloc.publish_prefix(s, _chain_hashes(truth[s]))
            d = int(r.integers(0, 6))
            if d not in truth:
                m = alloc.match_prefix(d, _chain_hashes(truth[s]))
                truth[d] = truth[s][:16 * m]
        else:                                              # release
            s = seqs[int(r.integers(0, len(seqs)))]
            alloc.release(s)
            del truth[s]
        # invariants: device blocks held or free, host slots used or free, once each
        held, slots = {}, []
        for s, t in alloc.tables.items():
            for j, b in enumerate(t):
                if b == O.OFFLOADED:
                    slots.append(alloc.slot_of[s][j])
                else:
                    assert alloc.slot_of[s][j] == -1
                    held[b] = held.get(b, 0) + 1
        assert all(alloc.refcount(b) == held.get(b, 0) for b in range(nb))
        assert sorted(list(held) + alloc.free) == list(range(nb))
        assert sorted(slots + alloc.host_free) == list(range(nh))
        assert all(h not in alloc.hash_of or True for h in slots)
        assert all(b in held for b in alloc.hash_of)
        for s, toks in truth.items():
            assert _read_back(alloc, dev, host, s, len(toks)) == toks, (step, s)
    assert moved["out"] > 50 and moved["in"] > 20


def test_offload_refusals_and_coldest_order():
    alloc = O.Allocator(8)
    alloc.set_host_slots(3)
    alloc.reserve(0, 40)                        # blocks 0, 1, 2 (the last partly filled)
    assert alloc.offload(0, 2, 1) == [(2, 0)]
    assert alloc.table(0) == [0, 1, O.OFFLOADED] and alloc.block_state(0, 2) == (O.OFFLOADED, 0, -1)
    for n in (41, 48):                          # the growth would write into host memory
        with pytest.raises(O.Offloaded):
            alloc.reserve(0, n)
    assert alloc.lens[0] == 40 and alloc.reserve(0, 40) == [0, 1, O.OFFLOADED]
    with pytest.raises(O.Offloaded):            # host slots are not shared
        alloc.fork(0, 1)
    assert alloc.page_in(0, 0, 8) == [(0, 3)]   # the free list's front: block 3
    alloc.fork(0, 1)
    with pytest.raises(O.SharedBlock):          # shared blocks stay on the device
        alloc.offload(0, 0, 1)
    alloc.release(1)
    assert alloc.reserve(2, 64) == [4, 5, 6, 7]
    with pytest.raises(O.OutOfBlocks):          # 4 blocks, 3 free host slots: nothing moves
        alloc.offload(2, 0, 4)
    assert O.OFFLOADED not in alloc.table(2) and alloc.host_free_count() == 3
    alloc.touch(0, 0, 3, 7)
    alloc.touch(2, 1, 2, 3)
    alloc.touch(2, 0, 1, 9)
    # candidates: full, resident blocks held by one table (seq 0's partly
    # filled third block is not one); never read (-1) first, then by step
    assert alloc.coldest(10) == [(2, 3), (2, 1), (2, 2), (0, 0), (0, 1), (2, 0)]
    assert alloc.coldest(2) == [(2, 3), (2, 1)]
    assert alloc.block_state(2, 0) == (4, -1, 9)
