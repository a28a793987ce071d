"""Pins for the oracle's paged attention (no GPU).

The oracle is checked against things other than itself:

* a library routine: torch's scaled_dot_product_attention in float64 over
  the *logical* per-token K/V drawn by the generator (K/V repeated per
  group for grouped-query heads), so the allocator replay, the pool scatter
  and the table walk are all exercised end to end;
* closed forms: a single key returns its value exactly; a zero query or a
  zero scale returns the mean of the values; a dominant key returns its
  value;
* the invariant the pages state (storage is scattered, the math is not):
  any two free orders give bit-identical outputs;
* the log-sum-exp identity: partitioned attention merged equals unsplit;
* brute force: a loop-only restatement on tiny inputs;
* sensitivity: mistakes planted in a copy of the oracle fail these pins.
"""
import math

import numpy as np
import pytest
import torch

import oracle.attention as oa
from oracle.cache import replay
from synthetic import make_workload
from synthetic.workloads import custom


def sdpa_reference(w, rows=None):
    """torch SDPA (float64, CPU) over the generator's logical K/V of each sequence."""
    G = w.group
    out = np.zeros((w.batch, w.num_q_heads, w.head_dim))
    q = oa.widen(w.q)
    for b in (range(w.batch) if rows is None else rows):
        L = int(w.seq_lens[b])
        if L == 0:
            continue
        k, v = w.sequence_kv(b)
        K = torch.from_numpy(oa.widen(k)).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, L, D]
        V = torch.from_numpy(oa.widen(v)).permute(1, 0, 2).repeat_interleave(G, dim=0)
        Q = torch.from_numpy(q[b]).unsqueeze(1)  # [Hq, 1, D]
        o = torch.nn.functional.scaled_dot_product_attention(Q, K.contiguous(), V.contiguous(), scale=w.scale)
        out[b] = o.squeeze(1).numpy()
    return out


def oracle_out(w, **kw):
    pool, _, tables, _, _ = replay(w)
    return oa.paged_decode(w.q, pool.k, pool.v, tables, w.seq_lens, w.scale, **kw), pool, tables


CASES = [
    dict(seed=0, dtype="f32", num_q_heads=8, num_kv_heads=8, head_dim=64, block_size=16, lens=[14, 60, 1, 33]),
    dict(seed=1, dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, lens=[1, 17, 200, 513]),
    dict(seed=2, dtype="bf16", num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=8, lens=[3, 40, 129]),
    dict(seed=3, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=32, lens=[31, 32, 33, 95]),
    dict(seed=4, dtype="f32", num_q_heads=6, num_kv_heads=3, head_dim=64, block_size=8, lens=[0, 5, 77]),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c['dtype']}-G{c['num_q_heads']//c['num_kv_heads']}-bs{c['block_size']}")
def test_matches_torch_sdpa_over_logical_kv(case):
    w = custom(**case)
    got, _, _ = oracle_out(w)
    ref = sdpa_reference(w)
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_tiny_workload_matches_sdpa():
    w = make_workload("tiny")
    got, pool, tables = oracle_out(w)
    np.testing.assert_allclose(got, sdpa_reference(w), rtol=0, atol=1e-12)
    # unwritten slots stay NaN in the pool, and the result never touches them
    assert np.isnan(pool.k).any()


def test_shrunken_trace_workloads_match_sdpa():
    for w in (make_workload("llama_70b", batch=4, len_lo=20, len_hi=90),
              make_workload("prefix_share", prompts=2, samples=3, prompt_len=37, tail_max=20)):
        got, _, _ = oracle_out(w)
        np.testing.assert_allclose(got, sdpa_reference(w), rtol=0, atol=1e-12)


def test_single_key_returns_its_value_exactly():
    w = custom(seed=7, dtype="bf16", num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16, lens=[1, 1])
    got, _, _ = oracle_out(w)
    for b in range(2):
        _, v = w.sequence_kv(b)
        vv = oa.widen(v)[0]  # [Hkv, D]
        assert np.array_equal(got[b], np.repeat(vv, 4, axis=0))


def test_zero_query_or_zero_scale_gives_mean_of_values():
    w = custom(seed=8, dtype="f32", num_q_heads=4, num_kv_heads=2, head_dim=64, block_size=8, lens=[13, 50])
    pool, _, tables, _, _ = replay(w)
    zero_q = np.zeros_like(w.q)
    for q, scale in ((zero_q, w.scale), (w.q, 0.0)):
        got = oa.paged_decode(q, pool.k, pool.v, tables, w.seq_lens, scale)
        for b in range(2):
            _, v = w.sequence_kv(b)
            mean = oa.widen(v).mean(axis=0)  # [Hkv, D]
            np.testing.assert_allclose(got[b], np.repeat(mean, 2, axis=0), rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value():
    w = custom(seed=9, dtype="f32", num_q_heads=2, num_kv_heads=1, head_dim=64, block_size=16, lens=[40])
    pool, _, tables, _, _ = replay(w)
    q = np.zeros((1, 2, 64), np.float32)
    q[0, :, 0] = 1.0
    # make position 23 carry a huge first key component
    phys, off = tables[0][23 // 16], 23 % 16
    pool.k[phys, 0, off, 0] = 1e4
    got = oa.paged_decode(q, pool.k, pool.v, tables, w.seq_lens, 1.0)
    np.testing.assert_allclose(got[0, 0], oa.widen(pool.v[phys, 0, off]), atol=1e-12)


def test_block_placement_does_not_change_the_result():
    base = dict(dtype="bf16", num_q_heads=32, num_kv_heads=8, head_dim=128, block_size=16, lens=[77, 300, 5])
    w1 = custom(seed=11, **base)
    w2 = custom(seed=11, **base)
    w2.free_order = np.arange(w2.num_blocks, dtype=np.int32)  # identity placement
    w3 = custom(seed=11, **base)
    w3.free_order = w3.free_order[::-1].copy()
    outs = []
    tables = []
    for w in (w1, w2, w3):
        o, _, t = oracle_out(w)
        outs.append(o)
        tables.append(t)
    assert not np.array_equal(tables[0], tables[1])
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("bs", [8, 16, 32])
def test_loop_oracle_agrees_on_tiny_inputs(bs):
    w = custom(seed=20 + bs, dtype="bf16", num_q_heads=4, num_kv_heads=2, head_dim=8, block_size=bs,
               lens=[1, bs - 1, bs + 3 if bs + 3 <= 40 else 40])
    pool, _, tables, _, _ = replay(w)
    a = oa.paged_decode(w.q, pool.k, pool.v, tables, w.seq_lens, w.scale)
    b = oa.paged_decode_loops(w.q, pool.k, pool.v, tables, w.seq_lens, w.scale)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


@pytest.mark.parametrize("P", [16, 32, 512])
def test_split_merge_equals_unsplit(P):
    w = custom(seed=30, dtype="bf16", num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
               lens=[1, 15, 16, 17, 700, 1500])
    pool, _, tables, _, _ = replay(w)
    whole = oa.paged_decode(w.q, pool.k, pool.v, tables, w.seq_lens, w.scale)
    split = oa.paged_decode_split(w.q, pool.k, pool.v, tables, w.seq_lens, w.scale, P)
    np.testing.assert_allclose(split, whole, rtol=1e-12, atol=1e-13)


def test_merge_of_one_partition_is_that_partition():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 32))
    K = rng.standard_normal((50, 2, 32))
    V = rng.standard_normal((50, 2, 32))
    parts = oa.partition_stats(q, K, V, 0.3, 64)
    assert len(parts) == 1
    np.testing.assert_allclose(oa.merge_partitions(parts), parts[0][2], rtol=0, atol=1e-15)
    np.testing.assert_allclose(parts[0][2], oa.dense_attention(q, K, V, 0.3), rtol=0, atol=1e-14)


def test_grouped_heads_equal_repeated_kv_heads():
    w = custom(seed=40, dtype="bf16", num_q_heads=16, num_kv_heads=4, head_dim=64, block_size=16, lens=[33, 90])
    pool, _, tables, _, _ = replay(w)
    gqa = oa.paged_decode(w.q, pool.k, pool.v, tables, w.seq_lens, w.scale)
    mha = oa.paged_decode(w.q, np.repeat(pool.k, 4, axis=1), np.repeat(pool.v, 4, axis=1), tables,
                          w.seq_lens, w.scale)
    assert np.array_equal(gqa, mha)


def test_empty_sequence_gives_zero_row():
    w = custom(seed=41, dtype="f32", num_q_heads=4, num_kv_heads=4, head_dim=64, block_size=16, lens=[0, 9])
    got, _, _ = oracle_out(w)
    assert np.array_equal(got[0], np.zeros_like(got[0]))
    assert np.abs(got[1]).sum() > 0


# ---------------------------------------------------------------- sensitivity
def _mutants():
    def wrong_group(q, K, V, scale):
        Hq, D = q.shape
        Hkv = K.shape[1]
        out = np.zeros((Hq, D))
        for h in range(Hq):
            g = h % Hkv  # interleaved instead of consecutive grouping
            s = scale * (K[:, g, :] @ q[h])
            p = np.exp(s - s.max())
            out[h] = (p @ V[:, g, :]) / p.sum()
        return out

    def no_scale(q, K, V, scale):
        return ORIG_DENSE(q, K, V, 1.0)

    def drop_last_token(q, K, V, scale):
        return ORIG_DENSE(q, K[:-1] if len(K) > 1 else K, V[:-1] if len(V) > 1 else V, scale)

    def keys_as_values(q, K, V, scale):
        return ORIG_DENSE(q, K, K, scale)

    return {"wrong_group": wrong_group, "no_scale": no_scale, "drop_last_token": drop_last_token,
            "keys_as_values": keys_as_values}


ORIG_DENSE = oa.dense_attention


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_planted_mistakes_fail_the_library_pin(name, monkeypatch):
    """A mistake planted in the oracle (on the CPU) must break the SDPA pin."""
    w = custom(**CASES[1])
    ref = sdpa_reference(w)
    monkeypatch.setattr(oa, "dense_attention", _mutants()[name])
    got, _, _ = oracle_out(w)
    assert np.abs(got - ref).max() > 1e-3


def test_planted_table_walk_mistake_fails_the_library_pin(monkeypatch):
    w = custom(**CASES[1])
    ref = sdpa_reference(w)

    def off_by_one_block(k_cache, v_cache, table, seq_len):
        bs = k_cache.shape[2]
        pos = np.arange(seq_len)
        phys = np.asarray(table)[np.minimum(pos // bs + (pos % bs == bs - 1), len(table) - 1)]
        return oa.widen(k_cache[phys, :, pos % bs, :]), oa.widen(v_cache[phys, :, pos % bs, :])

    monkeypatch.setattr(oa, "gather_sequence", off_by_one_block)
    got, _, _ = oracle_out(w)
    assert not np.allclose(got, ref, atol=1e-3, equal_nan=False)
