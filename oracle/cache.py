"""KV pool on the CPU (test infrastructure; see the package header).

Layout follows the "PagedAttention MCQ" page's code sketch, which holds the
pool as ``[num_blocks, 2, num_layers, num_kv_heads, block_size, d_head]``.
One layer's keys (index 0 of the K/V axis) and values (index 1) are the two
arrays ``[num_blocks, num_kv_heads, block_size, head_dim]`` kept here.

Values are held as raw bit patterns (uint16 for bfloat16, float32 for
float32) so every comparison with the device pool can be exact.  A fresh
pool is filled with a quiet-NaN pattern: any slot the method never wrote
stays NaN, and a reader that touches one produces NaN.

Writes follow the pages: "Paged attention in LLMs", section "The cache being
stored" (each step adds one token's keys and values), and the MCQ page's
sketch (a position's slot is block ``table[pos // bs]``, offset
``pos % bs``): the token written to slot ``s`` lands at block
``s // block_size``, offset ``s % block_size``.  A copy-on-write copies one
whole physical block (MCQ page, comparison table, "Copy on write blocks").
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np

from .allocator import BlockAllocatorModel

NAN_BF16 = np.uint16(0x7FC0)
NAN_F32_BITS = np.uint32(0x7FC00000)


class KVPool:
    def __init__(self, num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, dtype: str):
        self.num_blocks, self.num_kv_heads = num_blocks, num_kv_heads
        self.block_size, self.head_dim, self.dtype = block_size, head_dim, dtype
        shape = (num_blocks, num_kv_heads, block_size, head_dim)
        if dtype == "bf16":
            self.k = np.full(shape, NAN_BF16, dtype=np.uint16)
            self.v = np.full(shape, NAN_BF16, dtype=np.uint16)
        elif dtype == "f32":
            self.k = np.full(shape, NAN_F32_BITS, dtype=np.uint32).view(np.float32)
            self.v = np.full(shape, NAN_F32_BITS, dtype=np.uint32).view(np.float32)
        else:
            raise ValueError(dtype)

    def write(self, slots: Sequence[int], k: np.ndarray, v: np.ndarray) -> None:
        """Store token i's K/V ([Hkv, D] each) at slot slots[i]; a negative slot is skipped."""
        bs = self.block_size
        slots = np.asarray(slots, dtype=np.int64)
        keep = slots >= 0
        s = slots[keep]
        # one call writes distinct slots (numpy leaves the winner of a repeated
        # index unspecified), so the order of the tokens does not matter
        if len(np.unique(s)) != len(s):
            raise ValueError("repeated slot in one write")
        self.k[s // bs, :, s % bs, :] = np.asarray(k)[keep]
        self.v[s // bs, :, s % bs, :] = np.asarray(v)[keep]

    def copy_block(self, src: int, dst: int) -> None:
        self.k[dst] = self.k[src]
        self.v[dst] = self.v[src]

    def bits(self) -> Tuple[np.ndarray, np.ndarray]:
        """Raw bit views of the K and V arrays (uint16 or uint32)."""
        if self.dtype == "bf16":
            return self.k, self.v
        return self.k.view(np.uint32), self.v.view(np.uint32)


def replay(workload, include_decode: bool = True):
    """Run a workload's operation list in order through the allocator model and the pool.

    Each append allocates (and copies on write) first, then writes the new
    tokens' K/V.  Returns (pool, allocator, block_tables [B, max_blocks] int32,
    decode_slots [B] int64 (-1 where a sequence has no decode token),
    record) where ``record`` lists, per operation, the slots and copy pairs
    the allocator produced.  With include_decode False the decode-step
    tokens are allocated but not written.
    """
    w = workload
    alloc = BlockAllocatorModel(w.num_blocks, w.block_size, w.free_order)
    pool = KVPool(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, w.dtype)
    decode_slot: Dict[int, int] = {}
    record: List[Tuple[List[int], List[Tuple[int, int]]]] = []
    for op in w.ops:
        if op.kind == "add":
            alloc.add_seq(op.seq)
            record.append(([], []))
        elif op.kind == "fork":
            alloc.fork(op.parent, op.seq)
            record.append(([], []))
        elif op.kind == "free":
            alloc.free_seq(op.seq)
            record.append(([], []))
        elif op.kind == "append":
            start = alloc.lens[op.seq]
            slots, copies = alloc.append(op.seq, op.n)
            record.append((slots, copies))
            for src, dst in copies:
                pool.copy_block(src, dst)
            if op.decode:
                decode_slot[op.seq] = slots[-1]
            if op.write and (include_decode or not op.decode):
                k, v = w.token_kv(op.seq, start, op.n)
                pool.write(slots, k, v)
        else:
            raise ValueError(op.kind)
    B = w.batch
    width = max([len(alloc.tables[s]) for s in w.seq_ids] + [1])
    tables = np.zeros((B, width), dtype=np.int32)
    for b, s in enumerate(w.seq_ids):
        t = alloc.tables[s]
        tables[b, :len(t)] = t
    dslots = np.array([decode_slot.get(s, -1) for s in w.seq_ids], dtype=np.int64)
    return pool, alloc, tables, dslots, record
