"""Paged single-query decode attention in float64 (test infrastructure).

What it computes, from the pages:

* "PagedAttention MCQ" page, code sketch: for every logical position ``pos``
  in ``[0, seq_len)`` the keys and values are fetched through the request's
  block table (block ``table[pos // block_size]``, offset
  ``pos % block_size``), stacked in position order, and handed to standard
  scaled dot-product attention.
* "Paged Attention" (mbrenndoerfer.com), chapter introduction: the gain
  comes from memory management alone; the attention algorithm itself is
  unchanged.  So the result is exactly softmax(scale * q K^T) V over the
  sequence's tokens in order, whatever blocks hold them.

Readings where the pages are silent:

* grouped-query attention: query head ``h`` reads KV head
  ``h // (num_q_heads // num_kv_heads)``;
* ``seq_len`` counts the decode token itself (it is written to the cache
  first), so a length-1 sequence attends to its own key only;
* a sequence of length 0 yields a zero output row;
* only positions below ``seq_len`` are read, so a slot past the end may hold
  anything (NaN included) without effect;
* ``scale`` is an argument (the workloads use 1/sqrt(head_dim)).

Precision: every input is widened exactly to float64 (bfloat16 bit patterns
by a 16-bit shift) and all arithmetic is float64 with a two-pass softmax.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np


def widen(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of float32 data or of bfloat16 bit patterns (uint16)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if x.dtype in (np.float32, np.float64):
        return x.astype(np.float64)
    raise TypeError(f"unsupported input type {x.dtype}")


def gather_sequence(k_cache, v_cache, table, seq_len: int) -> Tuple[np.ndarray, np.ndarray]:
    """Walk one request's block table: K and V of positions [0, seq_len), [L, Hkv, D] float64."""
    bs = k_cache.shape[2]
    pos = np.arange(seq_len)
    phys = np.asarray(table)[pos // bs]
    off = pos % bs
    # advanced indices on axes 0 and 2 with a slice between them put the
    # position axis first: the result is [L, Hkv, D]
    return widen(k_cache[phys, :, off, :]), widen(v_cache[phys, :, off, :])


def dense_attention(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for one sequence.  q [Hq, D]; K, V [L, Hkv, D] -> [Hq, D]."""
    Hq, D = q.shape
    L, Hkv, _ = K.shape
    out = np.zeros((Hq, D))
    if L == 0:
        return out
    G = Hq // Hkv
    for h in range(Hq):
        g = h // G
        s = scale * (K[:, g, :] @ q[h])
        m = s.max()
        p = np.exp(s - m)
        out[h] = (p @ V[:, g, :]) / p.sum()
    return out


def paged_decode(q, k_cache, v_cache, block_tables, seq_lens, scale: float, rows=None) -> np.ndarray:
    """Decode output for every sequence b (or just ``rows``): [B, Hq, D] float64.

    q [B, Hq, D]; k_cache, v_cache [NB, Hkv, bs, D]; block_tables [B, W];
    seq_lens [B].  Rows not listed in ``rows`` stay zero.
    """
    qd = widen(q)
    B, Hq, D = qd.shape
    out = np.zeros((B, Hq, D))
    for b in (range(B) if rows is None else rows):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        K, V = gather_sequence(k_cache, v_cache, block_tables[b], L)
        out[b] = dense_attention(qd[b], K, V, scale)
    return out


def paged_prefill(q, k_cache, v_cache, block_tables, seq_lens, query_start, scale: float,
                  rows=None) -> np.ndarray:
    """Causal multi-token query (prefill, chunked prefill, verification): [T, Hq, D] float64.

    The cache grows by the tokens a step adds ("Paged attention in LLMs",
    "The cache being stored"), so a request with ``seq_lens[b]`` = L cached
    tokens whose last M are new has query rows ``query_start[b] ..
    query_start[b+1] - 1``; query token i sits at position L - M + i and, as
    in any autoregressive model, sees the keys at positions up to its own.
    Each row is therefore exactly the decode of that token over the first
    L - M + i + 1 positions.  Only the requests in ``rows`` are computed when
    given; the others' rows stay zero.
    """
    qd = widen(q)
    T, Hq, D = qd.shape
    out = np.zeros((T, Hq, D))
    B = len(seq_lens)
    for b in (range(B) if rows is None else rows):
        t0, t1 = int(query_start[b]), int(query_start[b + 1])
        L, M = int(seq_lens[b]), t1 - t0
        if M == 0:
            continue
        K, V = gather_sequence(k_cache, v_cache, block_tables[b], L)
        for i in range(M):
            p = L - M + i
            out[t0 + i] = dense_attention(qd[t0 + i], K[: p + 1], V[: p + 1], scale)
    return out


def paged_decode_loops(q, k_cache, v_cache, block_tables, seq_lens, scale: float) -> np.ndarray:
    """The same result with plain Python loops and no array arithmetic (tiny inputs only)."""
    import math

    B = len(q)
    Hq, D = len(q[0]), len(q[0][0])
    Hkv, bs = len(k_cache[0]), len(k_cache[0][0])
    G = Hq // Hkv
    qd = widen(np.asarray(q)).tolist()
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        keys, values = [], []
        for pos in range(L):
            phys = int(block_tables[b][pos // bs])
            off = pos % bs
            keys.append(widen(k_cache[phys, :, off, :]).tolist())
            values.append(widen(v_cache[phys, :, off, :]).tolist())
        for h in range(Hq):
            g = h // G
            scores = []
            for pos in range(L):
                acc = 0.0
                for d in range(D):
                    acc += qd[b][h][d] * keys[pos][g][d]
                scores.append(scale * acc)
            m = max(scores)
            weights = [math.exp(s - m) for s in scores]
            total = sum(weights)
            for d in range(D):
                acc = 0.0
                for pos in range(L):
                    acc += weights[pos] * values[pos][g][d]
                out[b][h][d] = acc / total
    return np.array(out, dtype=np.float64).reshape(B, Hq, D)


def partition_stats(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float,
                    partition_size: int) -> List[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
    """Split one sequence into partitions [j*P, min((j+1)*P, L)) and summarise each.

    For partition j and every query head: m_j = max of its scaled scores,
    l_j = sum of exp(score - m_j), o_j = (sum of exp(score - m_j) v) / l_j,
    i.e. o_j is the attention output over that partition alone.
    Returns [(m_j [Hq], l_j [Hq], o_j [Hq, D])].
    """
    Hq, D = q.shape
    L, Hkv, _ = K.shape
    G = Hq // Hkv
    parts = []
    for start in range(0, L, partition_size):
        stop = min(start + partition_size, L)
        m = np.empty(Hq)
        l = np.empty(Hq)
        o = np.empty((Hq, D))
        for h in range(Hq):
            g = h // G
            s = scale * (K[start:stop, g, :] @ q[h])
            m[h] = s.max()
            p = np.exp(s - m[h])
            l[h] = p.sum()
            o[h] = (p @ V[start:stop, g, :]) / l[h]
        parts.append((m, l, o))
    return parts


def merge_partitions(parts) -> np.ndarray:
    """Log-sum-exp merge: M = max_j m_j, w_j = l_j exp(m_j - M), out = sum w_j o_j / sum w_j."""
    m = np.stack([p[0] for p in parts])  # [P, Hq]
    l = np.stack([p[1] for p in parts])
    o = np.stack([p[2] for p in parts])  # [P, Hq, D]
    M = m.max(axis=0)
    w = l * np.exp(m - M)
    return (w[:, :, None] * o).sum(axis=0) / w.sum(axis=0)[:, None]


def paged_decode_split(q, k_cache, v_cache, block_tables, seq_lens, scale: float,
                       partition_size: int) -> np.ndarray:
    """Decode through per-partition summaries and the log-sum-exp merge."""
    qd = widen(q)
    B, Hq, D = qd.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        L = int(seq_lens[b])
        if L <= 0:
            continue
        K, V = gather_sequence(k_cache, v_cache, block_tables[b], L)
        out[b] = merge_partitions(partition_stats(qd[b], K, V, scale, partition_size))
    return out
