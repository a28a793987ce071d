"""Block allocator model (test infrastructure; see the package header).

Follows the pages:

* "Paged attention in LLMs", section "The fix": the cache is cut into
  fixed-size blocks that need not be adjacent; a request takes a new block
  only when its current one is full, from wherever a free one is.
* same page, "Keeping track: the block table": each request owns a table
  mapping its logical block index (0, 1, 2, ...) to a physical block, so the
  sequence reads in order even though storage is scattered.
* same page, "Sharing blocks": requests with a common prefix (parallel
  samples, beam search) point their own tables at the same physical blocks.
* "PagedAttention MCQ" page, comparison table row "Beam search / best of N":
  shared blocks are copied on write.
* "PagedAttention MCQ" page, code sketch: position ``pos`` lives in physical
  block ``table[pos // block_size]`` at offset ``pos % block_size``.

Readings where the pages are silent:

* the free pool is a FIFO queue seeded with a given order; freed blocks
  join its tail, walked from logical block 0 upward;
* a slot is the integer ``physical_block * block_size + offset``;
* a fork shares every block of the parent, the partially filled tail
  included; the first append of a holder that finds its last block shared
  (reference count > 1) copies that whole block to a fresh one and records
  the (source, destination) pair; the last holder writes in place;
* an append that cannot be satisfied changes nothing (all or nothing).
"""
from __future__ import annotations

from collections import deque
from typing import Dict, List, Optional, Sequence, Tuple


class OutOfBlocks(Exception):
    pass


class UnknownSequence(Exception):
    pass


class BlockAllocatorModel:
    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("bad pool shape")
        self.num_blocks = num_blocks
        self.block_size = block_size
        order = range(num_blocks) if free_order is None else [int(x) for x in free_order]
        if sorted(order) != list(range(num_blocks)):
            raise ValueError("free_order must be a permutation of the pool")
        self.free: deque = deque(order)
        self.ref: List[int] = [0] * num_blocks
        self.tables: Dict[int, List[int]] = {}
        self.lens: Dict[int, int] = {}

    # -- requests -------------------------------------------------------
    def add_seq(self, seq: int) -> None:
        if seq in self.tables:
            raise ValueError(f"sequence {seq} exists")
        self.tables[seq] = []
        self.lens[seq] = 0

    def _need(self, seq: int, n: int) -> int:
        """Fresh blocks that appending n tokens to seq will take."""
        bs = self.block_size
        length = self.lens[seq]
        table = self.tables[seq]
        need = 0
        if n > 0 and length % bs != 0 and self.ref[table[-1]] > 1:
            need += 1  # the shared partial tail block is copied first
        # positions length .. length+n-1 that start a new block
        first_new = -(-length // bs)  # logical index of the first block not yet held
        last = (length + n - 1) // bs if n > 0 else first_new - 1
        need += max(0, last - first_new + 1)
        return need

    def append(self, seq: int, n: int) -> Tuple[List[int], List[Tuple[int, int]]]:
        """Append n tokens to seq.  Returns (slots of the n tokens, copy pairs)."""
        if seq not in self.tables:
            raise UnknownSequence(seq)
        if n < 0:
            raise ValueError("negative token count")
        if self._need(seq, n) > len(self.free):
            raise OutOfBlocks(seq)
        bs = self.block_size
        table = self.tables[seq]
        slots: List[int] = []
        copies: List[Tuple[int, int]] = []
        for _ in range(n):
            pos = self.lens[seq]
            if pos % bs == 0:
                phys = self.free.popleft()
                self.ref[phys] = 1
                table.append(phys)
            elif self.ref[table[-1]] > 1:
                src = table[-1]
                dst = self.free.popleft()
                self.ref[src] -= 1
                self.ref[dst] = 1
                table[-1] = dst
                copies.append((src, dst))
            slots.append(table[pos // bs] * bs + pos % bs)
            self.lens[seq] = pos + 1
        return slots, copies

    def fork(self, parent: int, child: int) -> None:
        if parent not in self.tables:
            raise UnknownSequence(parent)
        if child in self.tables:
            raise ValueError(f"sequence {child} exists")
        self.tables[child] = list(self.tables[parent])
        self.lens[child] = self.lens[parent]
        for phys in self.tables[child]:
            self.ref[phys] += 1

    def free_seq(self, seq: int) -> None:
        if seq not in self.tables:
            raise UnknownSequence(seq)
        for phys in self.tables.pop(seq):
            self.ref[phys] -= 1
            if self.ref[phys] == 0:
                self.free.append(phys)
        del self.lens[seq]

    def move_to(self, other: "BlockAllocatorModel", seqs: Sequence[int]) -> List[Tuple[int, int]]:
        """Swap the given sequences out to (or back in from) another pool.

        The MCQ page lists easy preemption among what paging gives; it says no
        more.  Reading: each distinct block the sequences hold here is given
        one fresh block there, in order of first appearance, so what they
        share stays shared; the sequences are then freed here in the given
        order.  Returns the (here, there) block pairs whose contents must be
        copied.  All or nothing.
        """
        seqs = list(seqs)
        if len(set(seqs)) != len(seqs) or other.block_size != self.block_size:
            raise ValueError("bad move")
        for s in seqs:
            if s not in self.tables:
                raise UnknownSequence(s)
            if s in other.tables:
                raise ValueError(f"sequence {s} exists there")
        order: List[int] = []
        for s in seqs:
            for b in self.tables[s]:
                if b not in order:
                    order.append(b)
        if len(order) > len(other.free):
            raise OutOfBlocks(seqs)
        there = {b: other.free.popleft() for b in order}
        for b in order:
            other.ref[there[b]] = 0
        for s in seqs:
            other.tables[s] = [there[b] for b in self.tables[s]]
            other.lens[s] = self.lens[s]
            for b in other.tables[s]:
                other.ref[b] += 1
            self.free_seq(s)
        return [(b, there[b]) for b in order]

    # -- accounting (pages' worked example: slots held / used / wasted) ----
    def held_slots(self, seqs: Optional[Sequence[int]] = None) -> int:
        """Slots of the distinct physical blocks the given requests hold."""
        seqs = list(self.tables) if seqs is None else seqs
        blocks = set()
        for s in seqs:
            blocks.update(self.tables[s])
        return len(blocks) * self.block_size

    def used_slots(self, seqs: Optional[Sequence[int]] = None) -> int:
        """Distinct tokens stored: a position shared by several holders counts once."""
        seqs = list(self.tables) if seqs is None else seqs
        used = set()
        bs = self.block_size
        for s in seqs:
            t = self.tables[s]
            for pos in range(self.lens[s]):
                used.add(t[pos // bs] * bs + pos % bs)
        return len(used)

    def wasted_slots(self, seqs: Optional[Sequence[int]] = None) -> int:
        return self.held_slots(seqs) - self.used_slots(seqs)

    def block_fill(self, seq: int) -> List[int]:
        """Tokens stored in each of seq's blocks, in table order."""
        bs = self.block_size
        L = self.lens[seq]
        return [min(bs, L - j * bs) for j in range(len(self.tables[seq]))]


class ContiguousReservationModel:
    """The scheme the pages replace: one run of ``max_len`` slots per request.

    "Paged attention in LLMs", section "Why the memory gets wasted": every
    request reserves the maximum reply length up front in one unbroken run;
    free memory between runs is usable only by a request that fits a gap.
    Slots are a line ``[0, capacity)``; a request takes the lowest-addressed
    free run long enough for it (first fit).
    """

    def __init__(self, capacity: int, max_len: int):
        self.capacity = capacity
        self.max_len = max_len
        self.runs: Dict[int, Tuple[int, int]] = {}  # seq -> (start, length)
        self.lens: Dict[int, int] = {}

    def free_gaps(self) -> List[Tuple[int, int]]:
        taken = sorted(self.runs.values())
        gaps, cur = [], 0
        for start, length in taken:
            if start > cur:
                gaps.append((cur, start - cur))
            cur = max(cur, start + length)
        if cur < self.capacity:
            gaps.append((cur, self.capacity - cur))
        return gaps

    def admit(self, seq: int, reserve: Optional[int] = None) -> bool:
        need = self.max_len if reserve is None else reserve
        for start, length in self.free_gaps():
            if length >= need:
                self.runs[seq] = (start, need)
                self.lens[seq] = 0
                return True
        return False

    def place(self, seq: int, start: int, length: int) -> None:
        """Pin a request's run at a given address (to build a given layout)."""
        self.runs[seq] = (start, length)
        self.lens[seq] = 0

    def grow(self, seq: int, n: int) -> None:
        if self.lens[seq] + n > self.runs[seq][1]:
            raise OutOfBlocks(seq)
        self.lens[seq] += n

    def release(self, seq: int) -> None:
        del self.runs[seq]
        del self.lens[seq]

    def held_slots(self, seq: int) -> int:
        return self.runs[seq][1]

    def used_slots(self, seq: int) -> int:
        return self.lens[seq]

    def wasted_slots(self, seq: int) -> int:
        return self.held_slots(seq) - self.used_slots(seq)
