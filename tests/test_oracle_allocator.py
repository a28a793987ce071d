"""Pins for the oracle's allocator model and CPU pool (no GPU).

Each check ties the model to something other than itself: the numbers of
the pages' worked examples (tests/golden), the invariants the pages state
(the sequence reads in order, shared prefixes are stored once, each request
keeps its own table), and brute force over every short operation sequence
on tiny pools.
"""
import itertools
import json
import os
import random

import numpy as np
import pytest

from oracle.allocator import BlockAllocatorModel, ContiguousReservationModel, OutOfBlocks
from oracle.cache import KVPool

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- the pages' numbers
def test_worked_example_fourteen_tokens():
    g = golden("worked_example.json")
    n, bs = g["reply_tokens"], g["block_size"]
    paged = BlockAllocatorModel(num_blocks=8, block_size=bs)
    paged.add_seq(0)
    paged.append(0, n)
    assert len(paged.tables[0]) == g["paged"]["blocks"]
    assert paged.held_slots() == g["paged"]["held"]
    assert paged.used_slots() == g["paged"]["used"]
    assert paged.wasted_slots() == g["paged"]["wasted"]
    assert paged.block_fill(0) == g["block_fill"]

    flat = ContiguousReservationModel(capacity=g["reservation_slots"], max_len=g["reservation_slots"])
    assert flat.admit(0)
    flat.grow(0, n)
    assert flat.held_slots(0) == g["contiguous"]["held"]
    assert flat.used_slots(0) == g["contiguous"]["used"]
    assert flat.wasted_slots(0) == g["contiguous"]["wasted"]


def test_reservation_waste_inside():
    g = golden("reservation_waste.json")["inside_reservation"]
    flat = ContiguousReservationModel(capacity=g["limit"], max_len=g["limit"])
    assert flat.admit(0)
    flat.grow(0, g["reply_tokens"])
    assert flat.wasted_slots(0) == g["unused"]


def test_gaps_do_not_admit_a_contiguous_run_but_blocks_do():
    g = golden("reservation_waste.json")["between_reservations"]
    gaps = g["free_gaps"]
    # lay out: gap, 1 taken slot, gap, 1 taken slot, gap
    cap = sum(gaps) + len(gaps) - 1
    flat = ContiguousReservationModel(capacity=cap, max_len=g["request_in_one_run"])
    addr = 0
    for i, gap in enumerate(gaps[:-1]):
        addr += gap
        flat.place(100 + i, addr, 1)
        addr += 1
    assert [length for _, length in flat.free_gaps()] == gaps
    assert sum(length for _, length in flat.free_gaps()) == g["free_total"]
    assert flat.admit(0) is g["admitted"]
    # the same free slots cut into blocks of 2: any free block fits any request
    paged = BlockAllocatorModel(num_blocks=g["free_total"] // 2, block_size=2)
    paged.add_seq(0)
    paged.append(0, g["request_in_one_run"])
    assert paged.lens[0] == g["request_in_one_run"]


def test_tail_waste_bounded_by_block_size_minus_one():
    g = golden("tail_waste.json")
    bs = g["block_size"]
    rng = random.Random(5)
    worst = 0
    for _ in range(300):
        L = rng.randint(1, 200)
        a = BlockAllocatorModel(num_blocks=64, block_size=bs)
        a.add_seq(0)
        a.append(0, L)
        w = a.wasted_slots()
        assert 0 <= w <= bs - 1
        assert w == (-L) % bs
        worst = max(worst, w)
    assert worst == g["max_wasted_per_request"]


# ---------------------------------------------------------------- invariants
def check_invariants(a: BlockAllocatorModel):
    bs = a.block_size
    ref = [0] * a.num_blocks
    for seq, t in a.tables.items():
        assert len(t) == -(-a.lens[seq] // bs)
        for phys in t:
            ref[phys] += 1
    assert ref == a.ref
    assert sum(a.ref) == sum(len(t) for t in a.tables.values())
    assert len(a.free) + sum(1 for r in a.ref if r > 0) == a.num_blocks
    assert len(set(a.free)) == len(a.free)
    assert all(a.ref[b] == 0 for b in a.free)


def token_pool(a: BlockAllocatorModel):
    """A pool whose K payload is a token identity: (owner, position) packed in float32."""
    return KVPool(a.num_blocks, 1, a.block_size, 1, "f32")


def read_back(pool: KVPool, a: BlockAllocatorModel, seq):
    bs = a.block_size
    t = a.tables[seq]
    return [float(pool.k[t[p // bs], 0, p % bs, 0]) for p in range(a.lens[seq])]


class Shadow:
    """Per-sequence token identities, tracked without any allocator."""

    def __init__(self):
        self.tokens = {}
        self.next_id = 1.0

    def add(self, seq):
        self.tokens[seq] = []

    def append(self, seq, n):
        ids = []
        for _ in range(n):
            ids.append(self.next_id)
            self.next_id += 1.0
        self.tokens[seq].extend(ids)
        return ids

    def fork(self, parent, child):
        self.tokens[child] = list(self.tokens[parent])

    def free(self, seq):
        del self.tokens[seq]


def run_op(a, pool, shadow, op):
    kind = op[0]
    if kind == "add":
        a.add_seq(op[1])
        shadow.add(op[1])
    elif kind == "append":
        seq, n = op[1], op[2]
        before = (list(a.free), list(a.ref), {s: list(t) for s, t in a.tables.items()}, dict(a.lens))
        try:
            slots, copies = a.append(seq, n)
        except OutOfBlocks:
            after = (list(a.free), list(a.ref), {s: list(t) for s, t in a.tables.items()}, dict(a.lens))
            assert before == after, "an append that fails must change nothing"
            return False
        old_table = before[2][seq]
        new_table = a.tables[seq]
        if copies:
            assert len(copies) == 1
            src, dst = copies[0]
            # copy-on-write replaces exactly the last entry the table had
            assert old_table[:-1] == new_table[:len(old_table) - 1]
            assert old_table[-1] == src and new_table[len(old_table) - 1] == dst
        else:
            assert new_table[:len(old_table)] == old_table
        for src, dst in copies:
            pool.copy_block(src, dst)
        ids = shadow.append(seq, n)
        pool.write(slots, np.array(ids, np.float32).reshape(-1, 1, 1), np.zeros((n, 1, 1), np.float32))
    elif kind == "fork":
        a.fork(op[1], op[2])
        shadow.fork(op[1], op[2])
        assert a.tables[op[1]] == a.tables[op[2]]
    elif kind == "free":
        a.free_seq(op[1])
        shadow.free(op[1])
    return True


def check_contents(a, pool, shadow):
    # "the sequence stays in order" and "each request keeps its own table":
    # walking any live request's table yields exactly the tokens it appended
    for seq in a.tables:
        assert read_back(pool, a, seq) == shadow.tokens[seq]


@pytest.mark.parametrize("seed", range(12))
def test_random_traces_keep_invariants_and_contents(seed):
    rng = random.Random(seed)
    bs = rng.choice([1, 2, 3, 4, 5, 16])
    nb = rng.randint(4, 40)
    order = list(range(nb))
    rng.shuffle(order)
    a = BlockAllocatorModel(nb, bs, order)
    pool = token_pool(a)
    shadow = Shadow()
    next_seq = 0
    for _ in range(300):
        live = list(a.tables)
        r = rng.random()
        if r < 0.15 or not live:
            run_op(a, pool, shadow, ("add", next_seq))
            next_seq += 1
        elif r < 0.7:
            run_op(a, pool, shadow, ("append", rng.choice(live), rng.randint(0, 2 * bs + 1)))
        elif r < 0.85:
            run_op(a, pool, shadow, ("fork", rng.choice(live), next_seq))
            next_seq += 1
        else:
            run_op(a, pool, shadow, ("free", rng.choice(live)))
        check_invariants(a)
        check_contents(a, pool, shadow)


def test_brute_force_short_operation_sequences():
    """Every sequence of up to 5 operations over 3 request ids, pools of 1..4 blocks of 2."""
    alphabet = []
    for s in range(3):
        alphabet += [("append", s, 1), ("append", s, 3), ("free", s)]
    alphabet += [("fork", 0, 1), ("fork", 0, 2), ("fork", 1, 2)]
    checked = 0
    for nb in (1, 2, 3, 4):
        for depth in range(1, 6 if nb <= 2 else 5):
            for seq in itertools.product(alphabet, repeat=depth):
                a = BlockAllocatorModel(nb, 2, list(reversed(range(nb))))
                pool = token_pool(a)
                shadow = Shadow()
                a.add_seq(0)
                shadow.add(0)
                for op in seq:
                    kind = op[0]
                    if kind == "append" and op[1] not in a.tables:
                        continue
                    if kind == "free" and op[1] not in a.tables:
                        continue
                    if kind == "fork" and (op[1] not in a.tables or op[2] in a.tables):
                        continue
                    run_op(a, pool, shadow, op)
                    check_invariants(a)
                    check_contents(a, pool, shadow)
                checked += 1
    assert checked > 10000


def test_copy_on_write_only_for_shared_partial_tail():
    a = BlockAllocatorModel(16, 4)
    a.add_seq(0)
    a.append(0, 6)  # blocks: full, partial (2 of 4)
    for c in (1, 2):
        a.fork(0, c)
    shared_tail = a.tables[0][-1]
    assert a.ref[shared_tail] == 3
    _, copies0 = a.append(0, 1)
    _, copies1 = a.append(1, 1)
    _, copies2 = a.append(2, 1)  # last holder writes in place
    assert len(copies0) == 1 and copies0[0][0] == shared_tail
    assert len(copies1) == 1 and copies1[0][0] == shared_tail
    assert copies2 == []
    assert a.tables[2][-1] == shared_tail
    # the full first block stays shared by all three
    assert a.ref[a.tables[0][0]] == 3
    # a shared FULL tail is never copied: the next token opens a new block
    b = BlockAllocatorModel(16, 4)
    b.add_seq(0)
    b.append(0, 8)
    b.fork(0, 1)
    _, c = b.append(1, 1)
    assert c == [] and b.tables[1][:2] == b.tables[0][:2]


def test_out_of_blocks_changes_nothing_and_counts_the_copy():
    a = BlockAllocatorModel(3, 4)
    a.add_seq(0)
    a.append(0, 6)  # 2 blocks
    a.fork(0, 1)
    # appending 3 tokens to seq 1 needs a copy of the shared tail + 0 new blocks = 1 block
    a.append(1, 2)
    assert len(a.free) == 0
    with pytest.raises(OutOfBlocks):
        a.append(0, 3)  # 6+3 = 9 tokens -> needs a 3rd block, none free
    check_invariants(a)


def test_free_returns_blocks_in_table_order_to_the_tail():
    a = BlockAllocatorModel(6, 2, [5, 4, 3, 2, 1, 0])
    a.add_seq(0)
    a.append(0, 5)  # takes 5, 4, 3
    assert a.tables[0] == [5, 4, 3]
    a.free_seq(0)
    assert list(a.free) == [2, 1, 0, 5, 4, 3]


def test_pool_write_touches_only_the_named_slots():
    for dtype in ("bf16", "f32"):
        pool = KVPool(5, 2, 4, 3, dtype)
        before_k, before_v = (x.copy() for x in pool.bits())
        slots = [7, 0, 19]
        k = np.arange(3 * 2 * 3).reshape(3, 2, 3).astype(np.uint16 if dtype == "bf16" else np.float32)
        pool.write(slots + [-1], np.concatenate([k, k[:1]]), np.concatenate([k, k[:1]]) + 1)
        kb, vb = pool.bits()
        touched = np.zeros(kb.shape, bool)
        for i, s in enumerate(slots):
            touched[s // 4, :, s % 4, :] = True
            assert np.array_equal(pool.k[s // 4, :, s % 4, :], k[i])
            assert np.array_equal(pool.v[s // 4, :, s % 4, :], k[i] + 1)
        assert np.array_equal(kb[~touched], before_k[~touched])
        assert np.array_equal(vb[~touched], before_v[~touched])
        pool.copy_block(1, 3)
        assert np.array_equal(pool.bits()[0][3], pool.bits()[0][1])
