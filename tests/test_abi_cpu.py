"""libpa on the host (no GPU): exports, argument validation, allocator parity.

* every function include/pa.h declares is exported by the built library;
* the kernel entry points reject bad arguments on the host, before any HIP
  call (these calls pass no device memory, so nothing is launched);
* the C++ allocator and the oracle's allocator model agree bit for bit
  (slots, copy pairs, tables, lengths, reference counts, the free queue in
  order) over the workloads' operation lists and over random traces.
"""
import ctypes
import os
import random
import re

import numpy as np
import pytest

import paged_kv_cache_348_amd as pa
from paged_kv_cache_348_amd import _lib
from oracle.allocator import BlockAllocatorModel, OutOfBlocks, UnknownSequence
from synthetic import make_workload

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    inc = os.path.join(ROOT, "include")
    text = "".join(open(os.path.join(inc, f)).read() for f in sorted(os.listdir(inc)) if f.endswith(".h"))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert len(names) >= 15
    h = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(h, n), f"{n} declared in include/ but not exported"
    assert sorted(n for n, _, _ in _lib.SIGNATURES) == names


@pytest.mark.host_lib
def test_status_strings():
    for code in range(7):
        assert pa.status_string(code) not in ("", "?", "unknown status")


def _l():
    return pa.lib()


def fake(addr=0x10000):
    return ctypes.c_void_p(addr)  # never dereferenced: validation fails first


@pytest.mark.parametrize("args,expect", [
    # (T, Hkv, D, bs, NB, dtype)
    ((-1, 8, 128, 16, 10, 1), pa.PA_ERR_INVALID_ARG),
    ((4, 0, 128, 16, 10, 1), pa.PA_ERR_INVALID_ARG),
    ((4, 8, 96, 16, 10, 1), pa.PA_ERR_UNSUPPORTED),
    ((4, 8, 128, 12, 10, 1), pa.PA_ERR_UNSUPPORTED),
    ((4, 8, 128, 16, 10, 7), pa.PA_ERR_UNSUPPORTED),
    ((4, 8, 128, 16, -1, 1), pa.PA_ERR_INVALID_ARG),
])
def test_cache_write_rejects_bad_shapes(args, expect):
    T, hkv, d, bs, nb, dt = args
    st = _l().pa_cache_write(fake(), fake(), fake(), fake(), fake(), T, hkv, d, bs, nb, dt, None)
    assert st == expect


def test_cache_write_null_and_misaligned_pointers():
    st = _l().pa_cache_write(None, fake(), fake(), fake(), fake(), 4, 8, 128, 16, 10, 1, None)
    assert st == pa.PA_ERR_INVALID_ARG
    st = _l().pa_cache_write(fake(0x10008), fake(), fake(), fake(), fake(), 4, 8, 128, 16, 10, 1, None)
    assert st == pa.PA_ERR_INVALID_ARG
    # zero tokens: nothing to do, no pointer needed
    assert _l().pa_cache_write(None, None, None, None, None, 0, 8, 128, 16, 10, 1, None) == pa.PA_OK


def test_copy_blocks_validation():
    assert _l().pa_copy_blocks(fake(), fake(), None, 3, 8, 128, 16, 10, 1, None) == pa.PA_ERR_INVALID_ARG
    assert _l().pa_copy_blocks(fake(), fake(), fake(), -1, 8, 128, 16, 10, 1, None) == pa.PA_ERR_INVALID_ARG
    assert _l().pa_copy_blocks(fake(), fake(), fake(), 3, 8, 100, 16, 10, 1, None) == pa.PA_ERR_UNSUPPORTED
    assert _l().pa_copy_blocks(None, None, None, 0, 8, 128, 16, 10, 1, None) == pa.PA_OK


def decode_call(**kw):
    a = dict(q=fake(), kc=fake(), vc=fake(), bt=fake(), sl=fake(), hkv=8, scale=0.1, out=fake(), stream=None,
             B=4, hq=32, d=128, bs=16, nb=100, mb=8, dt=1, ps=0, ws=None, wsb=0)
    a.update(kw)
    return _l().pa_decode(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["hkv"], a["scale"], a["out"], a["stream"],
                          a["B"], a["hq"], a["d"], a["bs"], a["nb"], a["mb"], a["dt"], a["ps"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,expect", [
    (dict(hq=30), pa.PA_ERR_INVALID_ARG),            # Hq % Hkv
    (dict(hq=8 * 17), pa.PA_ERR_UNSUPPORTED),        # group of 17 heads
    (dict(d=96), pa.PA_ERR_UNSUPPORTED),
    (dict(bs=24), pa.PA_ERR_UNSUPPORTED),
    (dict(dt=5), pa.PA_ERR_UNSUPPORTED),
    (dict(B=-1), pa.PA_ERR_INVALID_ARG),
    (dict(hkv=0), pa.PA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), pa.PA_ERR_INVALID_ARG),
    (dict(ps=48), pa.PA_ERR_UNSUPPORTED),            # not a multiple of 32
    (dict(ps=16 * 65 // 32 * 32 + 32 * 32), pa.PA_ERR_UNSUPPORTED),  # over 64 blocks
    (dict(ps=512, mb=64, ws=None), pa.PA_ERR_INVALID_ARG),           # workspace needed
    (dict(ps=512, mb=64, ws=fake(0x10100), wsb=16), pa.PA_ERR_INVALID_ARG),  # too small
    (dict(q=None), pa.PA_ERR_INVALID_ARG),
    (dict(out=fake(0x10004)), pa.PA_ERR_INVALID_ARG),
    (dict(B=0, q=None, kc=None, vc=None, bt=None, sl=None, out=None), pa.PA_OK),
    (dict(ps=-1, ws=None), pa.PA_ERR_INVALID_ARG),                   # balanced split needs a workspace
    (dict(ps=-1, B=1025), pa.PA_ERR_UNSUPPORTED),                     # too many sequences to balance
    (dict(ps=-2), pa.PA_ERR_INVALID_ARG),
])
def test_decode_rejects_bad_arguments(kw, expect):
    assert decode_call(**kw) == expect


def decode_append_call(**kw):
    a = dict(q=fake(), k=fake(), v=fake(), slots=fake(), kc=fake(), vc=fake(), bt=fake(), sl=fake(), hkv=8,
             scale=0.1, out=fake(), stream=None, B=4, hq=32, d=128, bs=16, nb=100, mb=8, dt=1,
             ws=fake(0x20000), wsb=1 << 30)
    a.update(kw)
    return _l().pa_decode_append(a["q"], a["k"], a["v"], a["slots"], a["kc"], a["vc"], a["bt"], a["sl"], a["hkv"],
                                 a["scale"], a["out"], a["stream"], a["B"], a["hq"], a["d"], a["bs"], a["nb"],
                                 a["mb"], a["dt"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,expect", [
    (dict(k=None), pa.PA_ERR_INVALID_ARG),                 # the new tokens are required
    (dict(v=None), pa.PA_ERR_INVALID_ARG),
    (dict(slots=None), pa.PA_ERR_INVALID_ARG),
    (dict(k=fake(0x10008)), pa.PA_ERR_INVALID_ARG),        # rows must be 16-byte aligned
    (dict(slots=fake(0x10004)), pa.PA_ERR_INVALID_ARG),    # int64 slots
    (dict(ws=None), pa.PA_ERR_INVALID_ARG),                # the balanced split's workspace
    (dict(wsb=16), pa.PA_ERR_INVALID_ARG),
    (dict(B=1025), pa.PA_ERR_UNSUPPORTED),                 # too many sequences to balance
    (dict(hq=30), pa.PA_ERR_INVALID_ARG),
    (dict(d=96), pa.PA_ERR_UNSUPPORTED),
    (dict(bs=24), pa.PA_ERR_UNSUPPORTED),
    (dict(dt=5), pa.PA_ERR_UNSUPPORTED),
    (dict(nb=-1), pa.PA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), pa.PA_ERR_INVALID_ARG),
    (dict(B=0, q=None, k=None, v=None, slots=None, kc=None, vc=None, bt=None, sl=None, out=None, ws=None),
     pa.PA_OK),
])
def test_decode_append_rejects_bad_arguments(kw, expect):
    """The one-launch decode step validates everything on the host, before any launch."""
    assert decode_append_call(**kw) == expect


def test_workspace_size_formula():
    # partitions of 512 over 8 blocks of 16 = 128 tokens: one partition, no workspace
    assert pa.decode_workspace_bytes(4, 32, 8, 128, 16, 8, 512) == 0
    assert pa.decode_workspace_bytes(4, 32, 8, 128, 16, 8, 0) == 0
    cnt = _l().pa_decode_counter_bytes()
    assert cnt >= 2048 * 4 and cnt % 256 == 0  # one counter per wave of a balanced call, whatever the batch
    n = pa.decode_workspace_bytes(64, 32, 8, 128, 16, 256, 512)
    rows = 64 * 32 * 8
    assert n >= cnt + rows * 128 * 4 + rows * 2 * 4 and n % 256 == 0
    # balanced split: counters plus two partial slots of G heads per wave
    nb = pa.decode_workspace_bytes(64, 32, 8, 128, 16, 256, pa.PA_PARTITION_BALANCED)
    assert nb >= cnt + 2 * 2048 * 4 * (128 + 2) * 4 and nb % 256 == 0
    assert pa.decode_workspace_bytes(64, 32, 8, 128, 16, 256, -2) == 0
    assert pa.decode_workspace_bytes(64, 30, 8, 128, 16, 256, 512) == 0  # heads not grouped evenly


# ---------------------------------------------------------------- allocator parity
def state_of_model(m: BlockAllocatorModel):
    return ({s: list(t) for s, t in m.tables.items()}, dict(m.lens), list(m.ref), list(m.free))


def state_of_lib(a: pa.Allocator, seqs, nb):
    tables, lens = {}, {}
    for s in seqs:
        t, n = a.table(s)
        tables[s], lens[s] = t, n
    return tables, lens, [a.refcount(b) for b in range(nb)], a.free_list()


def replay_both(w):
    m = BlockAllocatorModel(w.num_blocks, w.block_size, w.free_order)
    a = pa.Allocator(w.num_blocks, w.block_size, w.free_order)
    live = set()
    for op in w.ops:
        if op.kind == "add":
            m.add_seq(op.seq)
            a.add_seq(op.seq)
            live.add(op.seq)
        elif op.kind == "fork":
            m.fork(op.parent, op.seq)
            a.fork(op.parent, op.seq)
            live.add(op.seq)
        elif op.kind == "free":
            m.free_seq(op.seq)
            a.free(op.seq)
            live.discard(op.seq)
        else:
            s1, c1 = m.append(op.seq, op.n)
            s2, c2 = a.append(op.seq, op.n)
            assert list(s2) == s1 and c2 == c1
    return m, a, live


@pytest.mark.host_lib
@pytest.mark.parametrize("name,kw", [
    ("tiny", {}),
    ("llama3_8b", {}),
    ("llama_70b", dict(batch=24, len_lo=100, len_hi=900)),
    ("prefix_share", dict(prompts=3, samples=8, prompt_len=2040, tail_max=40)),
    ("long_ctx_bs8", dict(batch=3, len_lo=1000, len_hi=5000)),
])
def test_allocator_matches_model_on_workloads(name, kw):
    w = make_workload(name, **kw)
    m, a, live = replay_both(w)
    assert set(live) == set(m.tables)
    assert state_of_lib(a, sorted(live), w.num_blocks) == state_of_model(m)
    tables, lens = a.batch_tables(w.seq_ids, pad=-7)
    for b, s in enumerate(w.seq_ids):
        t = m.tables[s]
        assert list(tables[b, :len(t)]) == t and all(tables[b, len(t):] == -7)
        assert lens[b] == m.lens[s] == w.seq_lens[b]


@pytest.mark.host_lib
@pytest.mark.parametrize("seed", range(6))
def test_allocator_matches_model_on_random_traces(seed):
    rng = random.Random(100 + seed)
    bs = rng.choice([1, 3, 8, 16])
    nb = rng.randint(3, 30)
    order = list(range(nb))
    rng.shuffle(order)
    m = BlockAllocatorModel(nb, bs, order)
    a = pa.Allocator(nb, bs, order)
    nxt = 0
    for _ in range(400):
        live = sorted(m.tables)
        r = rng.random()
        if r < 0.15 or not live:
            m.add_seq(nxt)
            a.add_seq(nxt)
            nxt += 1
        elif r < 0.7:
            s, n = rng.choice(live), rng.randint(0, 3 * bs)
            try:
                exp = m.append(s, n)
            except OutOfBlocks:
                with pytest.raises(pa.PAError) as e:
                    a.append(s, n)
                assert e.value.status == pa.PA_ERR_OOM
            else:
                got = a.append(s, n)
                assert list(got[0]) == exp[0] and got[1] == exp[1]
        elif r < 0.85:
            p = rng.choice(live)
            m.fork(p, nxt)
            a.fork(p, nxt)
            nxt += 1
        else:
            s = rng.choice(live)
            m.free_seq(s)
            a.free(s)
        live = sorted(m.tables)
        assert state_of_lib(a, live, nb) == ({s: m.tables[s] for s in live}, {s: m.lens[s] for s in live},
                                             list(m.ref), list(m.free))


@pytest.mark.host_lib
def test_allocator_error_codes():
    a = pa.Allocator(4, 2)
    with pytest.raises(pa.PAError) as e:
        a.append(5, 1)
    assert e.value.status == pa.PA_ERR_NOT_FOUND
    a.add_seq(1)
    with pytest.raises(pa.PAError) as e:
        a.add_seq(1)
    assert e.value.status == pa.PA_ERR_EXISTS
    with pytest.raises(pa.PAError) as e:
        a.fork(9, 2)
    assert e.value.status == pa.PA_ERR_NOT_FOUND
    with pytest.raises(pa.PAError) as e:
        a.free(9)
    assert e.value.status == pa.PA_ERR_NOT_FOUND
    a.append(1, 8)
    with pytest.raises(pa.PAError) as e:
        a.append(1, 1)
    assert e.value.status == pa.PA_ERR_OOM
    assert a.table(1) == ([0, 1, 2, 3], 8)
    with pytest.raises(ValueError):
        pa.Allocator(3, 2, [0, 0, 1])
    h = pa.lib().pa_alloc_create(-1, 2, None)
    assert not h


def test_stream_read_validation():
    assert _l().pa_bench_stream_read(None, 16, fake(), 0, None) == pa.PA_ERR_INVALID_ARG
    assert _l().pa_bench_stream_read(fake(0x10004), 16, fake(), 0, None) == pa.PA_ERR_INVALID_ARG
    assert _l().pa_bench_stream_read(fake(), 17, fake(), 0, None) == pa.PA_ERR_INVALID_ARG
    assert _l().pa_bench_stream_read(fake(), 16, fake(), -1, None) == pa.PA_ERR_INVALID_ARG
    assert _l().pa_bench_stream_read(fake(), 0, fake(), 0, None) == pa.PA_OK


def test_value_position_permutes_each_block():
    import torch
    for bs in (8, 16, 32):
        for dt in (torch.bfloat16, torch.float32):
            pos = [pa.value_position(o, bs, dt) for o in range(bs)]
            assert sorted(pos) == list(range(bs))
            assert all(pa.value_position(p, bs, dt) == o for o, p in enumerate(pos))  # an involution
            if dt == torch.float32 or bs == 8:
                assert pos == list(range(bs))
            else:
                # within each 16 offsets: 0-3, 8-11, 4-7, 12-15
                assert pos[:16] == [0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15]
                assert all(p // 16 == o // 16 for o, p in enumerate(pos))


# ---------------------------------------------------------------- shared-prefix decode (host side)
def shared_call(**kw):
    a = dict(q=fake(), kc=fake(), vc=fake(), bt=fake(), sl=fake(), hkv=8, scale=0.1, out=fake(), stream=None,
             B=16, hq=32, d=128, bs=16, nb=100, mb=40, dt=1, groups=fake(), pblk=fake(), ng=2, mg=8, mp=30, ps=512,
             ws=fake(0x10000), wsb=1 << 30)
    a.update(kw)
    return _l().pa_decode_shared_prefix(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["hkv"], a["scale"], a["out"],
                                        a["stream"], a["B"], a["hq"], a["d"], a["bs"], a["nb"], a["mb"], a["dt"],
                                        a["groups"], a["pblk"], a["ng"], a["mg"], a["mp"], a["ps"], a["ws"], a["wsb"])


@pytest.mark.parametrize("kw,expect", [
    (dict(mg=17), pa.PA_ERR_UNSUPPORTED),                # 17 requests x 4 heads > 64 columns
    (dict(mg=9, dt=0), pa.PA_ERR_UNSUPPORTED),           # float32, head dim 128: 32 columns at most
    (dict(hq=8 * 17), pa.PA_ERR_UNSUPPORTED),
    (dict(mg=0), pa.PA_ERR_INVALID_ARG),
    (dict(mp=41), pa.PA_ERR_INVALID_ARG),                # prefix longer than the table
    (dict(mp=-1), pa.PA_ERR_INVALID_ARG),
    (dict(ng=-1), pa.PA_ERR_INVALID_ARG),
    (dict(ng=17), pa.PA_ERR_UNSUPPORTED),                # more groups than requests
    (dict(ps=0), pa.PA_ERR_UNSUPPORTED),
    (dict(ps=48), pa.PA_ERR_UNSUPPORTED),
    (dict(ps=-1), pa.PA_ERR_UNSUPPORTED),                # the balanced split is not offered here
    (dict(groups=None), pa.PA_ERR_INVALID_ARG),
    (dict(pblk=None), pa.PA_ERR_INVALID_ARG),
    (dict(ws=None), pa.PA_ERR_INVALID_ARG),
    (dict(wsb=64), pa.PA_ERR_INVALID_ARG),
    (dict(ws=fake(0x10010)), pa.PA_ERR_INVALID_ARG),      # not 256-byte aligned
    (dict(d=96), pa.PA_ERR_UNSUPPORTED),
    (dict(scale=float("inf")), pa.PA_ERR_INVALID_ARG),
    (dict(B=0, q=None, kc=None, vc=None, bt=None, sl=None, out=None, groups=None, pblk=None, ng=0, ws=None),
     pa.PA_OK),
])
def test_shared_prefix_decode_rejects_bad_arguments(kw, expect):
    assert shared_call(**kw) == expect


def test_shared_prefix_max_group():
    import torch
    assert pa.shared_prefix_max_group(32, 8, 128, torch.bfloat16) == 16
    assert pa.shared_prefix_max_group(64, 8, 128, torch.bfloat16) == 8
    assert pa.shared_prefix_max_group(64, 8, 128, torch.float32) == 4
    assert pa.shared_prefix_max_group(8, 8, 64, torch.float32) == 64
    assert pa.shared_prefix_max_group(16, 1, 64, torch.bfloat16) == 4


def test_shared_prefix_workspace_size():
    cnt = _l().pa_decode_counter_bytes()
    # prefix: 30 blocks of 16 = 480 tokens -> 1 partition; own part: 640 tokens -> 2 partitions;
    # the partials sit after pa_decode's (untouched) counter region, then one merge counter
    # per (request, kv-head), at most one per query head
    n = pa.decode_shared_prefix_workspace_bytes(16, 32, 128, 16, 40, 30, 512)
    rows = 16 * 32 * 3
    assert n >= cnt + rows * 128 * 4 + rows * 2 * 4 + 16 * 32 * 4 and n % 256 == 0
    assert pa.decode_shared_prefix_workspace_bytes(16, 32, 128, 16, 40, 41, 512) == 0
    assert pa.decode_shared_prefix_workspace_bytes(16, 32, 128, 16, 40, 30, 0) == 0


def plan(tables, lens, bs=16, mg=8, mins=1):
    p = pa.plan_shared_prefix(np.array(tables, dtype=np.int32), np.array(lens, dtype=np.int32), bs, mg, mins)
    return [tuple(g) for g in p.groups.tolist()], p.prefix_blocks.tolist(), p.max_group, p.max_prefix_blocks


@pytest.mark.host_lib
def test_plan_groups_requests_with_common_leading_blocks():
    # three requests share blocks 5, 6, 7; the fourth shares nothing
    t = [[5, 6, 7, 10], [5, 6, 7, 11], [5, 6, 7, 12], [9, 1, 2, 3]]
    assert plan(t, [64, 60, 50, 64]) == ([(0, 3)], [3, 3, 3, 0], 3, 3)
    # the shared count stops at the blocks wholly inside the shortest member
    assert plan(t, [64, 60, 40, 64]) == ([(0, 3)], [2, 2, 2, 0], 3, 2)
    # a member whose length covers no whole block breaks the group (nothing shared)
    assert plan(t, [64, 60, 15, 64]) == ([(0, 2)], [3, 3, 0, 0], 2, 3)
    # min_shared_blocks
    assert plan(t, [64, 64, 64, 64], mins=4) == ([], [0, 0, 0, 0], 1, 0)
    # max_group_size caps a run of identical tables
    same = [[1, 2, 3]] * 5
    assert plan(same, [48] * 5, mg=2) == ([(0, 2), (2, 2)], [3, 3, 3, 3, 0], 2, 3)
    # empty batch and one request
    assert plan(np.zeros((0, 3)), [], mg=2) == ([], [], 1, 0)
    assert plan([[1, 2]], [32]) == ([], [0], 1, 0)


@pytest.mark.host_lib
def test_plan_stops_when_a_join_would_save_fewer_reads():
    # A and B share 10 blocks; C shares 2 with them: (2 members, 10 blocks) saves 10 reads,
    # (3 members, 2 blocks) would save 4, so C starts its own group with D
    A = list(range(100, 112))
    B = A[:10] + [200, 201]
    C = A[:2] + [300 + i for i in range(10)]
    D = C[:8] + [400, 401, 402, 403]
    g, p, mg, mp = plan([A, B, C, D], [192] * 4)
    assert g == [(0, 2), (2, 2)] and p == [10, 10, 8, 8] and mg == 2 and mp == 10
    # but a third member that keeps most of the shared blocks does join: 3 x 9 >= 2 x 10
    E = A[:9] + [500, 501, 502]
    g, p, _, _ = plan([A, B, E], [192] * 3)
    assert g == [(0, 3)] and p == [9, 9, 9]


@pytest.mark.host_lib
def test_plan_on_the_prefix_sharing_workload():
    w = make_workload("prefix_share", seed=0, prompts=4, samples=8, prompt_len=2040, tail_max=40)
    a = pa.Allocator(w.num_blocks, w.block_size, w.free_order)
    for op in w.ops:
        if op.kind == "add":
            a.add_seq(op.seq)
        elif op.kind == "fork":
            a.fork(op.parent, op.seq)
        elif op.kind == "append":
            a.append(op.seq, op.n)
    tables, lens = a.batch_tables(w.seq_ids)
    g, p, mg, mp = plan(tables, lens, mg=8)
    # every sample of a prompt shares the prompt's 127 full blocks; the partial
    # 128th was copied on write by all but the last sample
    assert g == [(8 * i, 8) for i in range(4)] and p == [127] * 32 and mg == 8 and mp == 127


def test_plan_check_enforces_one_group_per_shared_request():
    ok = pa.SharedPrefixPlan(np.array([[0, 3], [5, 2]], np.int32), np.array([4, 4, 4, 0, 0, 2, 2], np.int32), 3, 4)
    ok.check()
    # a prefix above the bound is allowed (its row is NaN), and so is a request in no group with 0
    pa.SharedPrefixPlan(ok.groups, np.array([4, 9, 4, 0, 0, 2, 2], np.int32), 3, 4).check()
    with pytest.raises(ValueError, match="overlaps"):
        pa.SharedPrefixPlan(np.array([[0, 3], [2, 2]], np.int32), ok.prefix_blocks, 3, 4).check()
    with pytest.raises(ValueError, match="outside"):
        pa.SharedPrefixPlan(np.array([[6, 2]], np.int32), ok.prefix_blocks, 3, 4).check()
    with pytest.raises(ValueError, match="no group"):
        pa.SharedPrefixPlan(ok.groups, np.array([4, 4, 4, 1, 0, 2, 2], np.int32), 3, 4).check()


@pytest.mark.host_lib
def test_plan_rejects_bad_arguments():
    t = np.zeros((2, 3), np.int32)
    ln = np.zeros(2, np.int32)
    g = np.zeros(4, np.int32)
    pb = np.zeros(2, np.int32)
    n1, n2, n3 = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    P = _lib.P_I32

    def call(B=2, W=3, bs=16, mg=4, mins=1, groups=g):
        return _l().pa_plan_shared_prefix(t.ctypes.data_as(P), ln.ctypes.data_as(P), B, W, bs, mg, mins,
                                          groups.ctypes.data_as(P) if groups is not None else None,
                                          pb.ctypes.data_as(P), ctypes.byref(n1), ctypes.byref(n2),
                                          ctypes.byref(n3))
    assert call() == pa.PA_OK
    assert call(B=-1) == pa.PA_ERR_INVALID_ARG
    assert call(bs=0) == pa.PA_ERR_INVALID_ARG
    assert call(mg=0) == pa.PA_ERR_INVALID_ARG
    assert call(mins=0) == pa.PA_ERR_INVALID_ARG
    assert call(groups=None) == pa.PA_ERR_INVALID_ARG


# ---------------------------------------------------------------- multi-token query (host side)
def prefill_call(**kw):
    a = dict(q=fake(), kc=fake(), vc=fake(), bt=fake(), sl=fake(), qs=fake(), hkv=8, scale=0.1, out=fake(),
             stream=None, B=4, T=16, hq=32, d=128, bs=16, nb=100, mb=8, dt=1, mq=4)
    a.update(kw)
    return _l().pa_prefill(a["q"], a["kc"], a["vc"], a["bt"], a["sl"], a["qs"], a["hkv"], a["scale"], a["out"],
                           a["stream"], a["B"], a["T"], a["hq"], a["d"], a["bs"], a["nb"], a["mb"], a["dt"], a["mq"],
                           a.get("ws"), a.get("wsb", 0))


@pytest.mark.parametrize("kw,expect", [
    (dict(hq=30), pa.PA_ERR_INVALID_ARG),
    (dict(hq=8 * 17), pa.PA_ERR_UNSUPPORTED),
    (dict(d=96), pa.PA_ERR_UNSUPPORTED),
    (dict(bs=24), pa.PA_ERR_UNSUPPORTED),
    (dict(dt=7), pa.PA_ERR_UNSUPPORTED),
    (dict(B=-1), pa.PA_ERR_INVALID_ARG),
    (dict(T=-1), pa.PA_ERR_INVALID_ARG),
    (dict(mq=-1), pa.PA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), pa.PA_ERR_INVALID_ARG),
    (dict(qs=None), pa.PA_ERR_INVALID_ARG),
    (dict(out=fake(0x10008)), pa.PA_ERR_INVALID_ARG),
    (dict(qs=fake(0x10002)), pa.PA_ERR_INVALID_ARG),
    (dict(B=0, q=None, kc=None, vc=None, bt=None, sl=None, qs=None, out=None), pa.PA_OK),
    (dict(T=0, q=None, out=None), pa.PA_OK),
    (dict(mq=0), pa.PA_OK),
    (dict(ws=fake(0x10100), wsb=16), pa.PA_ERR_INVALID_ARG),   # balanced path: workspace too small
    (dict(ws=fake(0x10010), wsb=1 << 30), pa.PA_ERR_INVALID_ARG),  # not 256-byte aligned
    # 20 new tokens x 4 heads over tables of 200 blocks: key partitions
    (dict(mq=20, mb=200, ws=fake(0x10100), wsb=16), pa.PA_ERR_INVALID_ARG),       # workspace too small
    (dict(mq=20, mb=200, ws=fake(0x10010), wsb=1 << 30), pa.PA_ERR_INVALID_ARG),  # not 256-byte aligned
])
def test_prefill_rejects_bad_arguments(kw, expect):
    assert prefill_call(**kw) == expect


def test_prefill_workspace_size():
    cnt = _l().pa_decode_counter_bytes()
    # arguments: B, T, Hq, Hkv, D, block size, table width, max new tokens
    # 4 new tokens x 4 heads = 16 columns: the balanced path, with counters and 16-column slots
    n = pa.prefill_workspace_bytes(64, 256, 32, 8, 128, 16, 256, 4)
    assert n >= cnt + 2 * 2048 * 16 * 130 * 4 and n % 256 == 0
    assert pa.prefill_workspace_bytes(8, 128, 8, 8, 64, 16, 256, 16) > 0  # G = 1: 16 tokens
    # 5 new tokens x 4 heads = 20 columns: 512 tile waves over tables of 4096 tokens, so
    # 2 key partitions: per query row 2 partials of D + 2 floats
    n = pa.prefill_workspace_bytes(64, 320, 32, 8, 128, 16, 256, 5)
    rows = 320 * 32
    assert n >= cnt + rows * 2 * 130 * 4 and n % 256 == 0
    assert pa.prefill_workspace_bytes(64, 320, 32, 8, 128, 16, 128, 5) == 0     # one partition: tiles only
    assert pa.prefill_workspace_bytes(64, 2048, 32, 8, 128, 16, 256, 32) == 0   # 1,024 tile waves
    assert pa.prefill_workspace_bytes(64, 32768, 32, 8, 128, 16, 256, 512) == 0  # 16,384 tile waves
    assert pa.prefill_workspace_bytes(1025, 4100, 32, 8, 128, 16, 256, 4) == 0   # many waves already
    assert pa.prefill_workspace_bytes(64, 320, 32, 7, 128, 16, 256, 5) == 0      # Hq not a multiple of Hkv
