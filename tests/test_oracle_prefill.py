"""Pins for the oracle's causal multi-token query (oracle.attention.paged_prefill), no GPU.

* a library routine: a full prefill (every token new, M = L) equals torch's
  scaled_dot_product_attention with is_causal=True in float64 over the
  generator's logical K/V;
* chunking does not change a token's row: the last M rows of a full prefill
  equal a chunk of M new tokens with the same queries (so chunks, too, are
  pinned to the library routine);
* one new token is the decode: M = 1 equals the (separately pinned) decode;
* sensitivity: an off-by-one causal limit planted in a copy fails the pins.
"""
import numpy as np
import pytest
import torch

import oracle.attention as oa
from oracle.cache import replay
from synthetic import multi_query
from synthetic.workloads import custom


def setup(dtype, hq, hkv, d, bs, lens, seed=3):
    w = custom(seed=seed, dtype=dtype, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, block_size=bs, lens=lens)
    pool, _, tables, _, _ = replay(w)
    return w, pool, tables


def sdpa_causal(w, b, q_rows):
    """torch SDPA, is_causal, float64, over the logical K/V of request b (all L tokens as queries)."""
    k, v = w.sequence_kv(b)
    G = w.group
    K = torch.from_numpy(oa.widen(k)).permute(1, 0, 2).repeat_interleave(G, dim=0)  # [Hq, L, D]
    V = torch.from_numpy(oa.widen(v)).permute(1, 0, 2).repeat_interleave(G, dim=0)
    Q = torch.from_numpy(oa.widen(q_rows)).permute(1, 0, 2)  # [Hq, L, D]
    o = torch.nn.functional.scaled_dot_product_attention(Q, K, V, is_causal=True, scale=w.scale)
    return o.permute(1, 0, 2).numpy()


CASES = [
    ("f32", 8, 8, 64, 16, [14, 60, 1, 33]),
    ("bf16", 32, 8, 128, 16, [40, 77, 5]),
    ("bf16", 16, 2, 64, 8, [30, 9]),
]


@pytest.mark.parametrize("case", CASES)
def test_full_prefill_matches_sdpa_causal(case):
    w, pool, tables = setup(*case)
    q, qs = multi_query(w, w.seq_lens, seed=1)
    got = oa.paged_prefill(q, pool.k, pool.v, tables, w.seq_lens, qs, w.scale)
    for b in range(w.batch):
        ref = sdpa_causal(w, b, q[qs[b]:qs[b + 1]])
        assert np.abs(got[qs[b]:qs[b + 1]] - ref).max() < 1e-12


@pytest.mark.parametrize("case", CASES)
def test_chunks_equal_the_tail_of_a_full_prefill(case):
    w, pool, tables = setup(*case)
    qf, qsf = multi_query(w, w.seq_lens, seed=1)
    full = oa.paged_prefill(qf, pool.k, pool.v, tables, w.seq_lens, qsf, w.scale)
    for frac in (1, 2, 3):
        m = np.maximum(1, w.seq_lens // (frac + 1)).astype(np.int64)
        m = np.minimum(m, w.seq_lens)
        qs = np.zeros(w.batch + 1, dtype=np.int32)
        qs[1:] = np.cumsum(m)
        q = np.concatenate([qf[qsf[b + 1] - m[b]:qsf[b + 1]] for b in range(w.batch)])
        got = oa.paged_prefill(q, pool.k, pool.v, tables, w.seq_lens, qs, w.scale)
        for b in range(w.batch):
            assert np.array_equal(got[qs[b]:qs[b + 1]], full[qsf[b + 1] - m[b]:qsf[b + 1]])


def test_one_new_token_is_the_decode():
    w, pool, tables = setup("bf16", 32, 8, 128, 16, [40, 77, 5, 1])
    q, qs = multi_query(w, np.ones(w.batch, dtype=np.int64), seed=2)
    got = oa.paged_prefill(q, pool.k, pool.v, tables, w.seq_lens, qs, w.scale)
    ref = oa.paged_decode(q, pool.k, pool.v, tables, w.seq_lens, w.scale)
    assert np.array_equal(got, ref)


def test_empty_chunk_leaves_no_rows():
    w, pool, tables = setup("f32", 8, 8, 64, 16, [14, 60])
    q, qs = multi_query(w, np.array([0, 3]), seed=2)
    got = oa.paged_prefill(q, pool.k, pool.v, tables, w.seq_lens, qs, w.scale)
    assert got.shape == (3, 8, 64) and qs.tolist() == [0, 0, 3]


def test_planted_causal_off_by_one_fails_the_pins(monkeypatch):
    w, pool, tables = setup(*CASES[1])
    q, qs = multi_query(w, w.seq_lens, seed=1)
    ref = np.concatenate([sdpa_causal(w, b, q[qs[b]:qs[b + 1]]) for b in range(w.batch)])
    orig = oa.dense_attention
    # a limit one short: each token misses its own key (the first one sees one key anyway)
    monkeypatch.setattr(oa, "dense_attention", lambda qq, K, V, s: orig(qq, K[:-1] if len(K) > 1 else K,
                                                                        V[:-1] if len(V) > 1 else V, s))
    got = oa.paged_prefill(q, pool.k, pool.v, tables, w.seq_lens, qs, w.scale)
    assert np.abs(got - ref).max() > 1e-3
