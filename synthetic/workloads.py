"""Seeded synthetic workloads for single-query decode over a block-paged KV cache.

Every random draw comes from its own numpy PCG64 stream keyed by
``SeedSequence([seed, config_id, stream, item])``, so a value never depends
on the order in which other values were drawn, and the oracle and the HIP
path see bit-identical inputs.

A workload is a list of allocator operations (``Op``) plus the key/value
vectors of every token those operations append.  The operations say *what*
happens to each sequence (it starts, grows, forks, finishes); which physical
block or slot a token lands in is decided by whichever allocator replays the
list, never here.  The list ends with one decode-step token per measured
sequence, the token the decode query belongs to.

Values are float32 draws from N(0, 1); for bfloat16 workloads they are
rounded to nearest-even and carried as uint16 bit patterns.

Workload shapes (the sizes of the five decode layers the path is measured on):

* ``tiny``: 4 sequences of lengths 14, 60, 1, 33; block size 16; 8 query and
  8 KV heads; head dim 64; float32; a 64-block pool in a shuffled free order.
* ``llama3_8b``: 64 sequences, lengths uniform in [512, 4096]; 32 query / 8 KV
  heads (GQA 4); head dim 128; block size 16; bfloat16; pool = total demand
  + 10 % in a shuffled free order.
* ``llama_70b``: 256 sequences, lengths uniform in [1024, 8192]; 64 query /
  8 KV heads (GQA 8); head dim 128; block size 16; bfloat16; the pool is
  fragmented by an interleaved arrival/finish trace of 512 requests.
* ``prefix_share``: 32 prompts x 8 parallel samples; the 2040-token prompt is
  stored once and forked, every sample then grows its own tail of 0..512
  tokens (the first tail token of a forked sample copies the partially
  filled last prompt block); 32 query / 8 KV heads; head dim 128; bfloat16.
* ``long_ctx_bs{8,16,32}``: 8 sequences, lengths uniform in [32768, 131072];
  32 query / 8 KV heads; head dim 128; bfloat16; split into 512-token
  partitions; the same lengths and values for each block size.

The Llama-3-8B, 70B and long-context shapes also come in float32
(``dtype="f32"``, names ending ``_f32``): the same lengths, placement and
draws, left unrounded, for parity at the float32 tolerance at full size.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np

# stream ids of SeedSequence([seed, config_id, stream, item])
S_LENS = 0
S_FREE_ORDER = 1
S_TRACE = 2
S_Q = 3
S_KV = 4
S_TAILS = 5
S_FINISH_ORDER = 6
S_MEMTRACE = 7

PROMPT_OWNER_BASE = 1 << 20  # KV owner id of prompt p in prefix sharing


def _rng(seed: int, config_id: int, stream: int, item: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, config_id, stream, item])))


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return uint16 bits.

    Inputs here are finite normal draws, so the NaN/Inf corner of the
    rounding rule never arises; it is handled anyway (NaN stays a quiet NaN).
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    if nan.any():
        r[nan] = np.uint16(0x7FC0)
    return r


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass
class Op:
    """One allocator operation of a workload trace.

    kind: 'add' (start sequence ``seq``), 'append' (``n`` more tokens),
    'fork' (``seq`` starts as a copy of ``parent``'s table), 'free'.
    write: the appended tokens' K/V are written into the cache (False for
    requests whose contents the measured step never reads).
    decode: this append is the decode-step token of a measured sequence.
    """

    kind: str
    seq: int
    n: int = 0
    parent: int = -1
    write: bool = True
    decode: bool = False


@dataclass
class Workload:
    name: str
    config_id: int
    seed: int
    dtype: str  # 'f32' or 'bf16'
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    scale: float
    partition_size: int  # 0: single pass; else tokens per split partition
    seq_ids: List[int]  # measured batch: row b of q / block_tables is seq_ids[b]
    seq_lens: np.ndarray  # int32 [B], final length including the decode token
    free_order: np.ndarray  # int32 [num_blocks], initial free-block order
    ops: List[Op]
    q: np.ndarray  # [B, Hq, D]; uint16 bf16 bits or float32
    # runs(seq, start, end) -> [(kv owner id, first position in the owner's stream, count)]
    _runs: Callable[[int, int, int], List[Tuple[int, int, int]]] = field(repr=False, default=None)
    _owner_len: Dict[int, int] = field(repr=False, default_factory=dict)
    _kv_cache: Dict[int, Tuple[np.ndarray, np.ndarray]] = field(repr=False, default_factory=dict)
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.seq_ids)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def np_dtype(self):
        return np.uint16 if self.dtype == "bf16" else np.float32

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if len(self.seq_lens) else 0

    def kv_read_bytes(self) -> int:
        """Bytes of K and V the decode step must read: sum(L) * 2 * Hkv * D * sizeof."""
        return int(self.seq_lens.astype(np.int64).sum()) * 2 * self.num_kv_heads * self.head_dim * self.elem_bytes

    def _owner_kv(self, owner: int) -> Tuple[np.ndarray, np.ndarray]:
        hit = self._kv_cache.get(owner)
        if hit is not None:
            return hit
        n = self._owner_len[owner]
        g = _rng(self.seed, self.config_id, S_KV, owner)
        shape = (n, self.num_kv_heads, self.head_dim)
        k = g.standard_normal(shape, dtype=np.float32)
        v = g.standard_normal(shape, dtype=np.float32)
        if self.dtype == "bf16":
            k, v = bf16_bits_from_f32(k), bf16_bits_from_f32(v)
        self._kv_cache[owner] = (k, v)
        return k, v

    def token_kv(self, seq: int, start: int, n: int) -> Tuple[np.ndarray, np.ndarray]:
        """K and V of tokens [start, start+n) of ``seq``: two [n, Hkv, D] arrays."""
        if n == 0:
            shape = (0, self.num_kv_heads, self.head_dim)
            return np.empty(shape, self.np_dtype), np.empty(shape, self.np_dtype)
        pieces_k, pieces_v = [], []
        for owner, opos, run in self._runs(seq, start, start + n):
            k, v = self._owner_kv(owner)
            pieces_k.append(k[opos:opos + run])
            pieces_v.append(v[opos:opos + run])
        if len(pieces_k) == 1:
            return pieces_k[0], pieces_v[0]
        return np.concatenate(pieces_k), np.concatenate(pieces_v)

    def sequence_kv(self, b: int) -> Tuple[np.ndarray, np.ndarray]:
        """Logical K/V of measured sequence b over positions [0, L_b)."""
        return self.token_kv(self.seq_ids[b], 0, int(self.seq_lens[b]))

    def drop_kv(self) -> None:
        """Forget generated K/V arrays (they are regenerated on demand)."""
        self._kv_cache.clear()


def _draw_q(seed, cfg, B, Hq, D, dtype):
    q = _rng(seed, cfg, S_Q).standard_normal((B, Hq, D), dtype=np.float32)
    return bf16_bits_from_f32(q) if dtype == "bf16" else q


def _simple_batch(name, cfg, seed, dtype, Hq, Hkv, D, bs, lens, num_blocks, partition_size=0):
    """Each sequence prefills L-1 tokens, then every sequence appends its decode token."""
    lens = np.asarray(lens, dtype=np.int32)
    B = len(lens)
    ops: List[Op] = []
    for b in range(B):
        ops.append(Op("add", b))
        if lens[b] > 1:
            ops.append(Op("append", b, n=int(lens[b]) - 1))
    for b in range(B):
        if lens[b] >= 1:  # an empty sequence has no decode token; its output row is zero
            ops.append(Op("append", b, n=1, decode=True))
    free_order = _rng(seed, cfg, S_FREE_ORDER, bs).permutation(num_blocks).astype(np.int32)
    w = Workload(
        name=name, config_id=cfg, seed=seed, dtype=dtype, num_q_heads=Hq, num_kv_heads=Hkv,
        head_dim=D, block_size=bs, num_blocks=num_blocks, scale=1.0 / math.sqrt(D),
        partition_size=partition_size, seq_ids=list(range(B)), seq_lens=lens,
        free_order=free_order, ops=ops, q=_draw_q(seed, cfg, B, Hq, D, dtype),
    )
    w._runs = lambda seq, a, e: [(seq, a, e - a)]
    w._owner_len = {b: int(lens[b]) for b in range(B)}
    return w


def _pool_for(lens, bs, slack=1.1):
    need = sum(-(-int(L) // bs) for L in lens)
    return max(1, int(math.ceil(slack * need)))


def tiny(seed: int = 0, **_):
    """4 sequences {14, 60, 1, 33}, bs 16, 8/8 heads, D 64, fp32, 64-block pool."""
    return _simple_batch("tiny", 0, seed, "f32", 8, 8, 64, 16, [14, 60, 1, 33], 64)


def _named(base: str, dtype: str) -> str:
    return base if dtype == "bf16" else f"{base}_{dtype}"


def llama3_8b(seed: int = 0, batch: int = 64, len_lo: int = 512, len_hi: int = 4096, dtype: str = "bf16", **_):
    lens = _rng(seed, 1, S_LENS).integers(len_lo, len_hi + 1, size=batch)
    return _simple_batch(_named("llama3_8b", dtype), 1, seed, dtype, 32, 8, 128, 16, lens, _pool_for(lens, 16))


def long_ctx(seed: int = 0, block_size: int = 16, batch: int = 8, len_lo: int = 32768,
             len_hi: int = 131072, partition_size: int = 512, dtype: str = "bf16", **_):
    lens = _rng(seed, 4, S_LENS).integers(len_lo, len_hi + 1, size=batch)
    w = _simple_batch(_named(f"long_ctx_bs{block_size}", dtype), 4, seed, dtype, 32, 8, 128, block_size, lens,
                      _pool_for(lens, block_size), partition_size=partition_size)
    return w


def llama_70b(seed: int = 0, batch: int = 256, len_lo: int = 1024, len_hi: int = 8192, dtype: str = "bf16", **_):
    """Interleaved arrival/finish trace that fragments the pool.

    2*batch requests draw target lengths; requests [0, batch) survive and are
    measured, requests [batch, 2*batch) finish.  Phase 1: a seeded random
    pick among unfinished requests appends up to one block of tokens, until
    survivors hold floor(L/2) tokens and finishers hold L.  Phase 2: the
    finishers are freed in a seeded order.  Phase 3: survivors grow to L-1
    by the same interleaving; then each appends its decode token.  Finishers'
    tokens are never written to the cache.
    """
    cfg, bs = 2, 16
    R = 2 * batch
    targets = _rng(seed, cfg, S_LENS).integers(len_lo, len_hi + 1, size=R).astype(np.int64)
    g = _rng(seed, cfg, S_TRACE)
    ops: List[Op] = [Op("add", r) for r in range(R)]
    length = np.zeros(R, dtype=np.int64)

    def grow(goal):
        live = [r for r in range(R) if length[r] < goal[r]]
        while live:
            i = int(g.integers(len(live)))
            r = live[i]
            n = int(min(bs, goal[r] - length[r]))
            ops.append(Op("append", r, n=n, write=r < batch))
            length[r] += n
            if length[r] >= goal[r]:
                live[i] = live[-1]
                live.pop()

    goal1 = np.where(np.arange(R) < batch, targets // 2, targets)
    grow(goal1)
    # pool sizing: blocks held at the end of phase 1 and of phase 3 (no sharing here)
    peak1 = int(sum(-(-int(x) // bs) for x in length))
    finish = _rng(seed, cfg, S_FINISH_ORDER).permutation(np.arange(batch, R))
    for r in finish:
        ops.append(Op("free", int(r)))
        length[r] = 0
    goal3 = np.where(np.arange(R) < batch, targets - 1, 0)
    grow(goal3)
    for r in range(batch):
        ops.append(Op("append", r, n=1, decode=True))
        length[r] += 1
    peak3 = int(sum(-(-int(x) // bs) for x in length[:batch]))
    num_blocks = int(math.ceil(1.1 * max(peak1, peak3)))
    lens = targets[:batch].astype(np.int32)
    w = Workload(
        name=_named("llama_70b", dtype), config_id=cfg, seed=seed, dtype=dtype, num_q_heads=64, num_kv_heads=8,
        head_dim=128, block_size=bs, num_blocks=num_blocks, scale=1.0 / math.sqrt(128),
        partition_size=0, seq_ids=list(range(batch)), seq_lens=lens,
        free_order=_rng(seed, cfg, S_FREE_ORDER).permutation(num_blocks).astype(np.int32),
        ops=ops, q=_draw_q(seed, cfg, batch, 64, 128, dtype),
    )
    w._runs = lambda seq, a, e: [(seq, a, e - a)]
    w._owner_len = {r: int(targets[r]) for r in range(batch)}
    w.meta["requests"] = R
    return w


def prefix_share(seed: int = 0, prompts: int = 32, samples: int = 8, prompt_len: int = 2040,
                 tail_max: int = 512, block_size: int = 16, dtype: str = "bf16", num_q_heads: int = 32,
                 num_kv_heads: int = 8, head_dim: int = 128, **_):
    """Parallel sampling: each prompt is stored once and forked to every sample.

    Sample s of prompt p is sequence ``samples*p + s``.  Sample 0 prefills the
    prompt and is forked ``samples-1`` times; sample tails t ~ U{0..tail_max}
    count generated tokens before the measured step.  At step k = 1, 2, ...
    every sample with k <= t+1 appends one token, in sequence-id order; the
    token of step t+1 is that sample's decode token.  L = prompt_len + t + 1.
    The shape keywords exist for small parity cases; the defaults are the
    measured workload.
    """
    cfg, bs = 3, block_size
    B = prompts * samples
    tails = _rng(seed, cfg, S_TAILS).integers(0, tail_max + 1, size=B).astype(np.int64)
    ops: List[Op] = []
    for p in range(prompts):
        root = samples * p
        ops.append(Op("add", root))
        ops.append(Op("append", root, n=prompt_len))
        for s in range(1, samples):
            ops.append(Op("fork", root + s, parent=root))
    for step in range(1, int(tails.max()) + 2):
        for seq in range(B):
            if step <= tails[seq] + 1:
                ops.append(Op("append", seq, n=1, decode=(step == tails[seq] + 1)))
    lens = (prompt_len + tails + 1).astype(np.int32)
    base = prompt_len - prompt_len % bs
    bound = prompts * (-(-prompt_len // bs)) + sum(-(-(int(L) - base) // bs) for L in lens)
    num_blocks = int(math.ceil(1.1 * bound))
    w = Workload(
        name="prefix_share", config_id=cfg, seed=seed, dtype=dtype, num_q_heads=num_q_heads,
        num_kv_heads=num_kv_heads, head_dim=head_dim, block_size=bs, num_blocks=num_blocks,
        scale=1.0 / math.sqrt(head_dim),
        partition_size=0, seq_ids=list(range(B)), seq_lens=lens,
        free_order=_rng(seed, cfg, S_FREE_ORDER).permutation(num_blocks).astype(np.int32),
        ops=ops, q=_draw_q(seed, cfg, B, num_q_heads, head_dim, dtype),
    )

    def runs(seq, a, e):
        out = []
        if a < prompt_len:  # prompt tokens come from the prompt's own stream
            m = min(e, prompt_len)
            out.append((PROMPT_OWNER_BASE + seq // samples, a, m - a))
            a = m
        if a < e:
            out.append((seq, a - prompt_len, e - a))
        return out

    w._runs = runs
    w._owner_len = {PROMPT_OWNER_BASE + p: prompt_len for p in range(prompts)}
    w._owner_len.update({seq: int(tails[seq]) + 1 for seq in range(B)})
    w.meta.update(prompts=prompts, samples=samples, prompt_len=prompt_len)
    return w


WORKLOADS = {
    "tiny": tiny,
    "llama3_8b": llama3_8b,
    "llama_70b": llama_70b,
    "prefix_share": prefix_share,
    "long_ctx_bs8": lambda seed=0, **kw: long_ctx(seed, block_size=8, **kw),
    "long_ctx_bs16": lambda seed=0, **kw: long_ctx(seed, block_size=16, **kw),
    "long_ctx_bs32": lambda seed=0, **kw: long_ctx(seed, block_size=32, **kw),
    # the same shapes in float32
    "llama3_8b_f32": lambda seed=0, **kw: llama3_8b(seed, dtype="f32", **kw),
    "llama_70b_f32": lambda seed=0, **kw: llama_70b(seed, dtype="f32", **kw),
    "long_ctx_bs8_f32": lambda seed=0, **kw: long_ctx(seed, block_size=8, dtype="f32", **kw),
    "long_ctx_bs16_f32": lambda seed=0, **kw: long_ctx(seed, block_size=16, dtype="f32", **kw),
    "long_ctx_bs32_f32": lambda seed=0, **kw: long_ctx(seed, block_size=32, dtype="f32", **kw),
}


def make_workload(name: str, seed: int = 0, **overrides) -> Workload:
    """Build a named workload.  Keyword overrides shrink it for parity tests
    (e.g. ``batch=6, len_lo=1, len_hi=700``)."""
    return WORKLOADS[name](seed=seed, **overrides)


def custom(seed: int, dtype: str, num_q_heads: int, num_kv_heads: int, head_dim: int,
           block_size: int, lens, num_blocks: Optional[int] = None, partition_size: int = 0,
           config_id: int = 99) -> Workload:
    """A plain prefill-then-decode batch of arbitrary shape (for edge cases)."""
    lens = [int(x) for x in lens]
    nb = num_blocks if num_blocks is not None else _pool_for(lens, block_size, slack=1.25) + 2
    return _simple_batch("custom", config_id, seed, dtype, num_q_heads, num_kv_heads, head_dim,
                         block_size, lens, nb, partition_size)


@dataclass
class MemoryTrace:
    """A request trace for the KV-memory accounting: arrival step, prompt and
    reply lengths of each request, in arrival order."""
    arrival: np.ndarray  # int32 [R], non-decreasing
    prompt: np.ndarray  # int32 [R], >= 1
    reply: np.ndarray  # int32 [R], 0 .. max_reply
    max_reply: int


def memory_trace(seed: int = 0, requests: int = 2000, mean_gap: float = 0.5, prompt_lo: int = 16,
                 prompt_hi: int = 512, reply_mean: float = 300.0, max_reply: int = 2048) -> MemoryTrace:
    """Seeded request trace.  The pages give no length distribution; this one
    takes Poisson arrivals (exponential gaps of ``mean_gap`` steps, rounded
    down), prompts uniform in [prompt_lo, prompt_hi] and replies exponential
    with mean ``reply_mean`` rounded down and capped at ``max_reply`` (the
    pages' example reserves 2,048 tokens for a reply)."""
    g = _rng(seed, 100, S_MEMTRACE)
    gaps = g.exponential(mean_gap, size=requests)
    arrival = np.floor(np.cumsum(gaps)).astype(np.int64)
    arrival -= arrival[0] if requests else 0
    prompt = g.integers(prompt_lo, prompt_hi + 1, size=requests)
    reply = np.minimum(np.floor(g.exponential(reply_mean, size=requests)), max_reply)
    return MemoryTrace(arrival.astype(np.int32), prompt.astype(np.int32), reply.astype(np.int32), max_reply)


def multi_query(w: Workload, query_lens, seed: int = 0):
    """Queries for a multi-token step over workload ``w``: request b's last
    ``query_lens[b]`` tokens (positions L_b - M_b .. L_b - 1, whose keys and
    values the workload already holds) get fresh N(0, 1) queries.  Returns
    (q [T, Hq, D] in the workload dtype, query_start int32 [B + 1])."""
    m = np.asarray(query_lens, dtype=np.int64)
    assert m.shape == (w.batch,)
    qs = np.zeros(w.batch + 1, dtype=np.int32)
    qs[1:] = np.cumsum(m)
    g = _rng(seed, w.config_id, S_Q, 1)
    q = g.standard_normal((int(qs[-1]), w.num_q_heads, w.head_dim), dtype=np.float32)
    return (bf16_bits_from_f32(q) if w.dtype == "bf16" else q), qs
