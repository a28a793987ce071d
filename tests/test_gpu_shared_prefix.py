"""GPU parity of the shared-prefix decode (pa_decode_shared_prefix) against the oracle.

Requests forked from one prompt share the prompt's blocks; the shared-prefix
decode reads those blocks once per group, but its result is still each
request's own attention over its own tokens, so the reference is the
oracle's paged decode of the same replayed pool (1e-5 float32, 2e-2
bfloat16).  Covered: every block size, head dims 64 and 128, group sizes
1..16 query heads per kv-head and 1..8 requests per group (1..4 column
tiles), prompts shorter than one shared step, prompts on and off step
boundaries, zero-length tails, partial groupings (groups capped below the
sample count, requests left out of any group), and the documented error
rows (a bad shared table entry, a group larger than the launch bound, a
prefix above the stated maximum: NaN rows only where promised).
"""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_348_amd as pa  # noqa: E402
from paged_kv_cache_348_amd.workload import build_device_batch  # noqa: E402
import oracle.attention as oa  # noqa: E402
from oracle.cache import replay  # noqa: E402
from synthetic import make_workload  # noqa: E402

TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(*a):
    print("[gpu-shared]", *a, flush=True)
    sys.stdout.flush()


def out_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def oracle_out(w):
    pool, _, tables, _, _ = replay(w)
    return oa.paged_decode(w.q, pool.k, pool.v, tables, w.seq_lens, w.scale)


def check(got, ref, dtype, what, rows=None):
    rows = list(range(got.shape[0])) if rows is None else list(rows)
    g, r = got[rows], ref[rows]
    assert not np.isnan(g).any(), f"{what}: NaN in output"
    err = np.abs(g - r)
    say(f"{what}: max abs err {err.max() if err.size else 0:.3e}")
    assert err.max() <= TOL[dtype], (what, float(err.max()))


# (label, prefix_share keywords, partition sizes)
CASES = [
    ("bf16-G4-bs16", dict(prompts=3, samples=8, prompt_len=300, tail_max=70), (64, 256, 512, 1024)),
    ("bf16-G4-bs8", dict(prompts=2, samples=8, prompt_len=333, tail_max=50, block_size=8), (64, 512)),
    ("bf16-G4-bs32", dict(prompts=2, samples=6, prompt_len=1000, tail_max=90, block_size=32), (64, 512)),
    ("bf16-G8-bs16", dict(prompts=2, samples=8, prompt_len=515, tail_max=40, num_q_heads=64), (128, 512)),
    ("bf16-G1-bs16", dict(prompts=3, samples=4, prompt_len=260, tail_max=30, num_q_heads=8), (96,)),
    ("bf16-G16-D64", dict(prompts=2, samples=4, prompt_len=200, tail_max=20, num_q_heads=16, num_kv_heads=1,
                          head_dim=64), (64,)),
    ("bf16-short-prompt", dict(prompts=2, samples=8, prompt_len=20, tail_max=30), (64,)),
    ("bf16-step-aligned", dict(prompts=2, samples=8, prompt_len=256, tail_max=0), (64, 512)),
    ("bf16-many-partials", dict(prompts=1, samples=4, prompt_len=2500, tail_max=1200), (32,)),  # > 64 per row
    ("f32-G1-D64", dict(prompts=2, samples=5, prompt_len=150, tail_max=40, dtype="f32", num_q_heads=8,
                        head_dim=64), (32, 128)),
    ("f32-G4-D128", dict(prompts=2, samples=8, prompt_len=180, tail_max=30, dtype="f32"), (64,)),
    ("f32-G8-D128-bs8", dict(prompts=2, samples=8, prompt_len=170, tail_max=25, dtype="f32", num_q_heads=64,
                             block_size=8), (64,)),  # groups of 4: 32 columns at most in float32, head dim 128
    ("f32-G4-D64-bs32", dict(prompts=2, samples=16, prompt_len=170, tail_max=25, dtype="f32", num_q_heads=32,
                             head_dim=64, block_size=32), (64,)),  # 16 x 4 = 64 columns
    # group sizes that do not divide 16 (a group's columns span tiles unevenly)
    ("bf16-G3", dict(prompts=2, samples=8, prompt_len=300, tail_max=70, num_q_heads=24), (64, 512)),
    ("bf16-G5", dict(prompts=3, samples=7, prompt_len=210, tail_max=40, num_q_heads=40), (128,)),
    ("bf16-G6", dict(prompts=2, samples=9, prompt_len=290, tail_max=33, num_q_heads=48), (64,)),
    # a large batch: 1040 requests in 65 groups of 16
    ("bf16-1040-requests", dict(prompts=65, samples=16, prompt_len=40, tail_max=20), (64,)),
]


@pytest.mark.parametrize("label,kw,parts", CASES, ids=[c[0] for c in CASES])
def test_shared_prefix_decode_matches_oracle(label, kw, parts):
    w = make_workload("prefix_share", seed=7, **kw)
    say(label, "B", w.batch, "max L", w.max_seq_len, "bs", w.block_size, "G", w.group)
    ref = oracle_out(w)
    dev = build_device_batch(w)
    dev.cache_append()
    plan = dev.shared_plan()
    say(label, "groups", plan.num_groups, "max group", plan.max_group, "prefix blocks", plan.max_prefix_blocks)
    per_group = pa.shared_prefix_max_group(w.num_q_heads, w.num_kv_heads, w.head_dim, dev.q.dtype)
    assert plan.max_group == min(per_group, kw["samples"])
    assert plan.num_groups == kw["prompts"] * -(-kw["samples"] // plan.max_group)
    for ps in parts:
        out = dev.attend_shared(plan, partition_size=ps)
        torch.cuda.synchronize()
        check(out_f64(out), ref, w.dtype, f"{label} ps={ps}")


def test_partial_groupings_and_workspace_reuse():
    """Groups capped below the sample count, and requests left out of every group."""
    w = make_workload("prefix_share", seed=3, prompts=4, samples=8, prompt_len=400, tail_max=60)
    ref = oracle_out(w)
    dev = build_device_batch(w)
    dev.cache_append()
    for mg in (3, 2, 8):
        plan = dev.shared_plan(max_group_size=mg)
        assert plan.max_group <= mg
        out = dev.attend_shared(plan, partition_size=128)
        torch.cuda.synchronize()
        check(out_f64(out), ref, w.dtype, f"max group {mg}")
    # keep only the groups of prompts 1 and 3; the other requests go alone
    full = dev.shared_plan()
    keep = [i for i in range(full.num_groups) if full.groups[i, 0] // 8 in (1, 3)]
    pblk = np.zeros_like(full.prefix_blocks)
    for i in keep:
        s0, n = full.groups[i]
        pblk[s0:s0 + n] = full.prefix_blocks[s0]
    part = pa.SharedPrefixPlan(full.groups[keep].copy(), pblk, full.max_group, full.max_prefix_blocks).to("cuda")
    out = dev.attend_shared(part, partition_size=256)
    torch.cuda.synchronize()
    check(out_f64(out), ref, w.dtype, "two of four groups")
    # an empty plan is the plain split decode; with no prefix launch a fill
    # kernel clears the merge counters, so a second call on the same
    # workspace (rows of two 256-token partitions) must agree as well
    none = pa.SharedPrefixPlan(np.zeros((0, 2), np.int32), np.zeros(w.batch, np.int32), 1, 0).to("cuda")
    assert int(w.seq_lens.max()) > 256
    for call in range(2):
        out = dev.attend_shared(none, partition_size=256)
        torch.cuda.synchronize()
        check(out_f64(out), ref, w.dtype, f"no groups, call {call}")


def test_shared_prefix_error_rows_without_fault():
    """Bad shared entry, oversized group, prefix above its bound: NaN rows exactly where documented."""
    w = make_workload("prefix_share", seed=5, prompts=3, samples=4, prompt_len=300, tail_max=20)
    ref = oracle_out(w)
    dev = build_device_batch(w)
    dev.cache_append()
    plan = dev.shared_plan()
    assert plan.num_groups == 3 and plan.max_group == 4

    # 1) a shared entry of group 1 (requests 4..7) points outside the pool
    tables = dev.block_tables.clone()
    tables[4:8, 2] = w.num_blocks + 5
    out = pa.decode_shared_prefix(dev.q, dev.k_cache, dev.v_cache, tables, dev.seq_lens, w.num_kv_heads, w.scale,
                                  plan, partition_size=64)
    torch.cuda.synchronize()
    got = out_f64(out)
    assert np.isnan(got[4:8]).all()
    check(got, ref, w.dtype, "bad entry: other rows", rows=[0, 1, 2, 3, 8, 9, 10, 11])

    # 2) the launch is sized for groups of 2: the groups of 4 give NaN rows
    out = pa.decode_shared_prefix(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.seq_lens, w.num_kv_heads,
                                  w.scale, plan, partition_size=64, max_group_size=2)
    torch.cuda.synchronize()
    assert np.isnan(out_f64(out)).all()

    # 3) request 9 claims a prefix above max_prefix_blocks
    pblk = plan.prefix_blocks.copy()
    pblk[9] = plan.max_prefix_blocks + 1
    bad = pa.SharedPrefixPlan(plan.groups.copy(), pblk, plan.max_group, plan.max_prefix_blocks).to("cuda")
    out = pa.decode_shared_prefix(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, dev.seq_lens, w.num_kv_heads,
                                  w.scale, bad, partition_size=64)
    torch.cuda.synchronize()
    got = out_f64(out)
    assert np.isnan(got[9]).all()
    check(got, ref, w.dtype, "prefix above bound: other rows", rows=[r for r in range(w.batch) if r != 9])

    # 4) an empty request outside any group gives a zero row
    lens = dev.seq_lens.clone()
    lens[0] = 0
    pblk = plan.prefix_blocks.copy()
    pblk[0:4] = 0
    groups = plan.groups[1:].copy()
    p4 = pa.SharedPrefixPlan(groups, pblk, plan.max_group, plan.max_prefix_blocks).to("cuda")
    out = pa.decode_shared_prefix(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, lens, w.num_kv_heads, w.scale,
                                  p4, partition_size=64)
    torch.cuda.synchronize()
    got = out_f64(out)
    assert (got[0] == 0).all()
    check(got, ref, w.dtype, "zero-length row: other rows", rows=range(1, w.batch))

    # 5) request 1 is shorter than its group's shared part: its row is NaN, its group's others are not
    lens = dev.seq_lens.clone()
    lens[1] = 100
    out = pa.decode_shared_prefix(dev.q, dev.k_cache, dev.v_cache, dev.block_tables, lens, w.num_kv_heads, w.scale,
                                  plan, partition_size=64)
    torch.cuda.synchronize()
    got = out_f64(out)
    assert np.isnan(got[1]).all()
    check(got, ref, w.dtype, "short member: other rows", rows=[r for r in range(w.batch) if r != 1])
