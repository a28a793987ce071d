"""Decode-step benchmark on one MI355X: paged single-query decode attention.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload llama3_8b]
                    [--partition-size P] [--no-cpu]

One step is one pass of the whole hot path over one batch: the cache append
of every sequence's decode token and the decode attention.  With the
balanced split (the default for the Llama-3-8B and 70B shapes) both run in
one launch (pa_decode_append: the launch stores the new tokens and attends
to them from their input rows); otherwise, or with --step separate, the
step is pa_cache_write followed by pa_decode (with its split-sequence merge
when partitioned).  The
inputs (pool, block tables, queries, decode tokens) are resident in HBM
before the timed region starts.  The default workload is the
Llama-3-8B-shaped decode layer: 64 sequences, 32 query / 8 KV heads, head
dim 128, block size 16, bfloat16, lengths uniform in [512, 4096], blocks
placed by a seeded random permutation of a pool sized to demand + 10 %.

Printed: one JSON line with decode tokens/s (``value``), the KV-read
bandwidth, a roofline entry for the decode kernel (algorithmic KV bytes per
launch / its average duration, timed with HIP events on the launch stream)
and the CPU oracle timed on this host's cores on the same workload
(``cpu_baseline``; it runs before the GPU is touched).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from synthetic import make_workload  # noqa: E402

HBM_PEAK_GBPS = 8000.0
HOST_LINK_GBPS = 64.0  # PCIe 5.0 x16, one direction
PARTITION_BALANCED = -1  # the library's balanced split (PA_PARTITION_BALANCED)
# launch configuration per workload, the faster mode as measured on MI355X
# (the long-context ones use their own 512-token partitions with the
# log-sum-exp merge; with prefix sharing, fixed partitions dispatch the
# samples of one prompt together, so their shared blocks are read while
# still in L2 / MALL)
DEFAULT_PARTITION = {"llama3_8b": PARTITION_BALANCED, "llama_70b": PARTITION_BALANCED, "prefix_share": 1024}
# decode entry point per workload: with prefix sharing, the shared-prefix
# decode reads each prompt's blocks once for all of its samples
DEFAULT_DECODE = {"prefix_share": "shared"}
WORKLOAD_TEXT = {
    "llama3_8b": "Llama-3-8B-shaped decode layer: batch 64, 32 q / 8 kv heads (GQA 4), d_head 128, block 16, "
                 "bf16, seq_lens U[512,4096], seeded random block permutation of a pool = demand + 10%",
    "llama_70b": "70B-shaped decode layer: batch 256, 64 q / 8 kv heads (GQA 8), d_head 128, block 16, bf16, "
                 "seq_lens U[1024,8192], pool fragmented by an interleaved arrival/finish trace",
    "prefix_share": "parallel sampling: 32 prompts x 8 samples, shared 2040-token prompt, tails U[0,512], "
                    "copy-on-write of the partial prompt block, 32 q / 8 kv heads, d_head 128, bf16",
    "long_ctx_bs8": "long-context split decode: batch 8, seq_lens U[32768,131072], 32 q / 8 kv heads, d_head 128, "
                    "bf16, block 8, 512-token partitions + log-sum-exp merge",
    "long_ctx_bs16": "long-context split decode: batch 8, seq_lens U[32768,131072], 32 q / 8 kv heads, d_head 128, "
                     "bf16, block 16, 512-token partitions + log-sum-exp merge",
    "long_ctx_bs32": "long-context split decode: batch 8, seq_lens U[32768,131072], 32 q / 8 kv heads, d_head 128, "
                     "bf16, block 32, 512-token partitions + log-sum-exp merge",
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def measured_traffic(workload: str, mode: str = "split", fused: bool = False):
    """HBM bytes per decode launch from the committed counter summary of this
    workload (rocprofv3 FETCH_SIZE + WRITE_SIZE, scaled by their
    calibrations), or None when there is none or the decode sources changed
    since it was taken."""
    import hashlib

    kernel = "pa_decode_shared_prefix" if mode == "shared" else ("pa_decode_append" if fused else "pa_decode")
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip().split()[0] if v.strip() else ""
    h = hashlib.sha256()
    srcs = ("pa_shared.hip" if mode == "shared" else "pa_decode.hip", "pa_decode_common.h", "pa_device.h")
    for f in srcs:
        h.update(open(os.path.join(ROOT, "paged_kv_cache_348_amd", "csrc", f), "rb").read())
    if fields.get("source_sha256") != h.hexdigest() or "traffic_bytes_per_launch" not in fields:
        return None
    return int(fields["traffic_bytes_per_launch"])


# ---------------------------------------------------------------------------- CPU baseline (the oracle)

_CPU = {}
# Worker processes of the oracle's pool at most: a one-GPU share of the host
# (what the machine gives one GPU's jobs, whatever the affinity mask shows).
CPU_POOL_CAP = 16


def host_cores():
    """(cores in this process's affinity, worker processes used)."""
    affinity = len(os.sched_getaffinity(0))
    return affinity, max(1, min(CPU_POOL_CAP, affinity))


def close_pool(p):
    """End a worker pool by letting its workers exit (close + join): a
    terminate() would signal them, which a profiler attached to this
    process reports as an abort."""
    p.close()
    p.join()


def _cpu_init():
    try:
        from threadpoolctl import threadpool_limits

        threadpool_limits(1)
    except Exception:
        pass


def _cpu_one(b):
    import oracle.attention as oa

    c = _CPU
    L = int(c["lens"][b])
    if L <= 0:
        return b, np.zeros(c["q"].shape[1:])
    K, V = oa.gather_sequence(c["k"], c["v"], c["tables"][b], L)
    return b, oa.dense_attention(oa.widen(c["q"][b]), K, V, c["scale"])


def cpu_baseline(w, min_seconds: float = 10.0, max_passes: int = 10000):
    """Time the oracle over the workload's sequences on this host's cores.

    The pool is built by the oracle's own replay (untimed); the timed part
    is the block-table walk and float64 attention of every sequence, one
    sequence per task in a process pool.  Whole passes over the batch
    repeat until ``min_seconds`` of wall time have gone by.
    """
    import multiprocessing as mp

    from oracle.cache import replay

    t0 = time.perf_counter()
    pool, _, tables, _, _ = replay(w)
    log(f"oracle replay {time.perf_counter() - t0:.1f}s")
    _CPU.update(k=pool.k, v=pool.v, tables=tables, lens=w.seq_lens, q=w.q, scale=w.scale)
    affinity, cores = host_cores()
    ctx = mp.get_context("fork")
    out = np.zeros((w.batch, w.num_q_heads, w.head_dim))
    order = sorted(range(w.batch), key=lambda b: -int(w.seq_lens[b]))  # longest first
    p = ctx.Pool(cores, initializer=_cpu_init)
    try:
        passes = 0
        t0 = time.perf_counter()
        while True:
            for b, o in p.imap_unordered(_cpu_one, order):
                out[b] = o
            passes += 1
            el = time.perf_counter() - t0
            if el >= min_seconds or passes >= max_passes:
                break
    finally:
        close_pool(p)
    tok = passes * w.batch
    res = {
        "value": tok / el,
        "unit": "decode tokens/s",
        "cores": cores,
        "affinity_cores": affinity,
        "kind": "oracle",
        "sample": f"the whole batch ({w.batch} sequences, sum L = {int(w.seq_lens.sum())}) x {passes} passes, "
                  f"{el:.1f} s; float64 numpy, one sequence per task in a {cores}-process pool "
                  f"({affinity} cores in this process's affinity, capped at {CPU_POOL_CAP})",
        "kv_read_gbps": passes * w.kv_read_bytes() / el / 1e9,
    }
    _CPU.clear()
    return res, out


def _cpu_prefill_one(b):
    import oracle.attention as oa

    c = _CPU
    out = oa.paged_prefill(c["q"], c["k"], c["v"], c["tables"], c["lens"], c["qs"], c["scale"], rows=[b])
    return b, out[c["qs"][b]:c["qs"][b + 1]]


def cpu_prefill_baseline(w, q, qs, min_seconds: float = 10.0, max_passes: int = 1000):
    """The oracle's causal multi-token query, one request per task, until
    ``min_seconds`` have gone by (whole requests; longest first)."""
    import multiprocessing as mp

    from oracle.cache import replay

    pool, _, tables, _, _ = replay(w)
    _CPU.update(k=pool.k, v=pool.v, tables=tables, lens=w.seq_lens, q=q, qs=qs, scale=w.scale)
    affinity, cores = host_cores()
    ctx = mp.get_context("fork")
    order = sorted(range(w.batch), key=lambda b: -int(w.seq_lens[b]))
    out = np.zeros((int(qs[-1]), w.num_q_heads, w.head_dim))
    done_tok, done_req = 0, 0
    p = ctx.Pool(cores, initializer=_cpu_init)
    try:
        t0 = time.perf_counter()
        for _ in range(max_passes):
            for b, o in p.imap_unordered(_cpu_prefill_one, order):
                out[qs[b]:qs[b + 1]] = o
                done_tok += int(qs[b + 1] - qs[b])
                done_req += 1
            el = time.perf_counter() - t0
            if el >= min_seconds:
                break
    finally:
        close_pool(p)
    _CPU.clear()
    return {"value": done_tok / el, "unit": "query tokens/s", "cores": cores, "affinity_cores": affinity,
            "kind": "oracle",
            "sample": f"{done_req} requests ({done_tok} query tokens), {el:.1f} s; float64 numpy, one request per "
                      f"task in a {cores}-process pool ({affinity} cores in this process's affinity, capped at "
                      f"{CPU_POOL_CAP})"}, out


def prefill_flops(w, qs) -> float:
    """4 * D flops per (query token, visible key, query head): QK^T and PV."""
    tot = 0
    for b in range(w.batch):
        L, M = int(w.seq_lens[b]), int(qs[b + 1] - qs[b])
        tot += M * (L - M) + M * (M + 1) // 2  # sum over i of (L - M + i + 1)
    return 4.0 * w.head_dim * w.num_q_heads * tot


def prefill_main(args, w):
    """--prefill M: the last M tokens of every request are new and attend causally (pa_prefill)."""
    import torch

    import paged_kv_cache_348_amd as pa
    from paged_kv_cache_348_amd.workload import build_device_batch, to_device
    from synthetic import multi_query

    m = np.minimum(w.seq_lens.astype(np.int64), args.prefill)
    q, qs = multi_query(w, m, seed=args.seed)
    T = int(qs[-1])
    flops = prefill_flops(w, qs)
    kv_bytes = w.kv_read_bytes()
    log(f"multi-token query: {w.batch} requests, {args.prefill} new tokens each (T {T}), {flops / 1e9:.1f} GFLOP")
    cpu, ref = (None, None)
    if not args.no_cpu:
        cpu, ref = cpu_prefill_baseline(w, q, qs, min_seconds=args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']:.1f} query tok/s on {cpu['cores']} cores")
    dev = build_device_batch(w, device="cuda", partition_size=0)
    dev.cache_append()
    w.drop_kv()
    qd = to_device(q, w.dtype, "cuda")
    qsd = torch.from_numpy(qs).to("cuda")
    out = torch.empty_like(qd)
    maxq = int(m.max())
    stream = torch.cuda.current_stream()
    wsb = pa.prefill_workspace_bytes(w.batch, T, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                     dev.max_blocks, maxq)
    ws = pa.new_workspace(wsb) if wsb else None  # the faster paths' workspace, made once
    path = pa.prefill_path(w.batch, w.num_q_heads, w.num_kv_heads, maxq, wsb, bf16=w.dtype == "bf16",
                           head_dim=w.head_dim, block_size=w.block_size)
    log(f"pa_prefill path: {path}")

    def call():
        pa.prefill(qd, dev.k_cache, dev.v_cache, dev.block_tables, dev.seq_lens, qsd, w.num_kv_heads, w.scale, maxq,
                   out=out, workspace=ws)

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    runs = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        runs.append(a.elapsed_time(b) / args.steps)
    ms = float(np.median(runs))
    err = None
    if ref is not None:
        err = float(np.abs(out.float().cpu().numpy().astype(np.float64) - ref).max())
        log(f"full-size parity vs oracle: max abs err {err:.3e}")
    tflops = flops / (ms * 1e-3) / 1e12
    gbps = kv_bytes / (ms * 1e-3) / 1e9
    peak_tf = 2500.0 if w.dtype == "bf16" else 157.3
    frac_m, frac_h = tflops / peak_tf, gbps / HBM_PEAK_GBPS
    mfma_bound = frac_m >= frac_h
    res = {
        "metric": "causal multi-token query tokens/s over the paged cache on 1 MI355X",
        "value": T / (ms * 1e-3),
        "unit": "query tokens/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v rounded to bf16; seeded lengths and block placement)",
        "config": {"workload": WORKLOAD_TEXT[args.workload] + f"; the last {args.prefill} tokens of each request "
                   "are new queries with a causal mask", "name": w.name, "seed": args.seed, "batch": w.batch,
                   "query_tokens": T, "new_tokens_per_request": args.prefill, "sum_seq_len": int(w.seq_lens.sum()),
                   "step": f"pa_prefill ({path})"},
        "roofline": {
            "bound": "mfma" if mfma_bound else "hbm", "kernel": "pa_prefill",
            "achieved": tflops if mfma_bound else gbps, "peak": peak_tf if mfma_bound else HBM_PEAK_GBPS,
            "unit": "TFLOP/s" if mfma_bound else "GB/s", "frac": frac_m if mfma_bound else frac_h,
            "traffic": None, "flop_per_launch": flops, "algorithmic_bytes_per_launch": kv_bytes,
            "other": {"tflops": tflops, "kv_read_gbps": gbps},
        },
        "runs_ms": runs,
        "cpu_baseline": cpu,
        "max_abs_err_vs_oracle": err,
    }
    print(json.dumps(res), flush=True)
    return 0


def append_main(args, w):
    """--append: pa_cache_write of every sequence's prefill tokens (positions
    0 .. L-2, with the slots the allocator gave them and their own values) in
    one call, timed with HIP events on the launch stream.  The writes repeat
    the pool's contents, so it is unchanged.  Algorithmic bytes: each
    token's keys and values read once and written once."""
    import torch

    import paged_kv_cache_348_amd as pa
    from paged_kv_cache_348_amd.workload import build_device_batch, to_device

    if any(op.kind == "fork" for op in w.ops):
        print("--append takes workloads without shared blocks", file=sys.stderr)
        return 2
    dev = build_device_batch(w, device="cuda", partition_size=0)
    bs = w.block_size
    slots, ks, vs = [], [], []
    for b in range(w.batch):
        n = int(dev.host_lens[b]) - 1
        if n <= 0:
            continue
        pos = np.arange(n)
        slots.append(dev.host_tables[b][pos // bs].astype(np.int64) * bs + pos % bs)
        k, v = w.token_kv(w.seq_ids[b], 0, n)
        ks.append(k)
        vs.append(v)
    w.drop_kv()
    T = int(sum(len(x) for x in slots))
    sl = torch.from_numpy(np.concatenate(slots)).cuda()
    kd = to_device(np.concatenate(ks), w.dtype, "cuda")
    vd = to_device(np.concatenate(vs), w.dtype, "cuda")
    del ks, vs
    stream = torch.cuda.current_stream()

    def call():
        pa.cache_write(kd, vd, sl, dev.k_cache, dev.v_cache)

    for _ in range(args.warmup):
        call()
    runs = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        runs.append(a.elapsed_time(b) / args.steps)
    ms = float(np.median(runs))
    per_tok = 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    algo = 2 * T * per_tok  # read + write
    gbps = algo / (ms * 1e-3) / 1e9

    # reference: a plain device copy of the same keys and values (the same
    # bytes read and written, contiguous on both sides), timed the same way
    ck, cv = torch.empty_like(kd), torch.empty_like(vd)

    def copy():
        ck.copy_(kd)
        cv.copy_(vd)

    for _ in range(args.warmup):
        copy()
    copy_runs = []
    for _ in range(3):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(args.steps):
            copy()
        b.record(stream)
        torch.cuda.synchronize()
        copy_runs.append(a.elapsed_time(b) / args.steps)
    ms_copy = float(np.median(copy_runs))
    del ck, cv
    res = {
        "metric": "bulk cache append (pa_cache_write) tokens/s on 1 MI355X",
        "value": T / (ms * 1e-3), "unit": "appended tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic (the workload's own prefill tokens and slots)",
        "config": {"workload": WORKLOAD_TEXT.get(args.workload, w.name), "name": w.name, "tokens": T,
                   "step": "pa_cache_write of every prefill token in one call"},
        "roofline": {"bound": "hbm", "kernel": "pa_cache_write", "achieved": gbps, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": gbps / HBM_PEAK_GBPS, "traffic": None,
                     "algorithmic_bytes_per_launch": algo},
        "runs_ms": runs,
        "copy_same_bytes": {"what": "plain device copy of the same keys and values (read + write)",
                            "ms": ms_copy, "gbps": algo / (ms_copy * 1e-3) / 1e9,
                            "frac_of_8tbs": algo / (ms_copy * 1e-3) / 1e9 / HBM_PEAK_GBPS},
    }
    print(json.dumps(res), flush=True)
    return 0


# ---------------------------------------------------------------------------- GPU


def shared_read_bytes(w, plan) -> int:
    """KV bytes the shared-prefix decode must read: each group's shared part
    once, plus every request's own tokens."""
    a = max(32, w.block_size)
    per_tok = 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    shared = (plan.prefix_blocks.astype(np.int64) * w.block_size) // a * a
    own = int((w.seq_lens.astype(np.int64) - shared).sum())
    once = sum(int(shared[s0]) for s0, _ in plan.groups)
    return (own + once) * per_tok


def gpu_bench(w, steps: int, warmup: int, partition_size: int, decode_mode: str, cold_iters: int = 20,
              fused: bool = False):
    import torch

    from paged_kv_cache_348_amd.workload import build_device_batch

    dev_name = torch.cuda.get_device_name(0)
    log(f"device {dev_name}")
    t0 = time.perf_counter()
    dev = build_device_batch(w, device="cuda", partition_size=partition_size)
    torch.cuda.synchronize()
    log(f"device pool built in {time.perf_counter() - t0:.1f}s, NB {w.num_blocks}, width {dev.max_blocks}")
    w.drop_kv()
    stream = torch.cuda.current_stream()
    plan = None
    if decode_mode == "shared":
        plan = dev.shared_plan()
        log(f"shared-prefix plan: {plan.num_groups} groups, up to {plan.max_group} requests, "
            f"up to {plan.max_prefix_blocks} shared blocks")
        attend = lambda: dev.attend_shared(plan, partition_size=partition_size)  # noqa: E731
    elif fused:
        attend = dev.append_and_attend  # the append runs in the same launch
    else:
        attend = dev.attend

    def step():
        if not fused:
            dev.cache_append()
        attend()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # timed region: `steps` whole steps (cache append + decode)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms_step = ev0.elapsed_time(ev1) / steps
    out = dev.out.float().cpu().numpy().astype(np.float64)

    # decode alone.  Hot: `n` launches back to back between one event pair
    # (per-launch events would add their own gaps).  Cold: one event pair per
    # launch, each after a 1 GiB read that evicts L2 and MALL (a read leaves
    # no dirty lines to write back during the timed launch).
    def time_decode_hot(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(n):
            attend()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    def time_decode_cold(n):
        scratch = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for a, b in evs:
            scratch.amax()
            a.record(stream)
            attend()
            b.record(stream)
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in evs])
        del scratch
        return t

    def time_decode_single(n):
        # hot launches timed like the cold ones, one event pair each: the
        # difference to the back-to-back time is what a per-launch event pair
        # adds (the wait between the first event and the kernel's start)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        torch.cuda.synchronize()
        for a, b in evs:
            a.record(stream)
            attend()
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs])

    hot = np.array([time_decode_hot(max(steps, 20)) for _ in range(3)])
    cold = time_decode_cold(cold_iters)
    single = time_decode_single(cold_iters)

    # calibration: a plain streaming read of the same byte count
    import paged_kv_cache_348_amd as pa

    read_bytes = shared_read_bytes(w, plan) if plan is not None else w.kv_read_bytes()
    per_tok = 2 * w.num_kv_heads * w.head_dim * w.elem_bytes
    algo_bytes = read_bytes + (int((w.seq_lens >= 1).sum()) * per_tok if fused else 0)  # + the stored new tokens
    nbytes = (read_bytes + 4095) // 4096 * 4096
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    for _ in range(3):
        pa.stream_read(buf, sink)
    sr = []
    for _ in range(max(steps, 20)):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        pa.stream_read(buf, sink)
        b.record(stream)
        sr.append((a, b))
    torch.cuda.synchronize()
    sr_ms = float(np.mean([a.elapsed_time(b) for a, b in sr]))
    del buf

    # swap: the blocks of the first sequences out to a pinned host pool and
    # back into the same blocks (the pool is unchanged afterwards)
    nseq = min(8, w.batch)
    blocks = sorted({int(b) for r in range(nseq) for b in dev.host_tables[r][: -(-int(dev.host_lens[r]) // w.block_size)]})
    nsw = len(blocks)
    ks, vs = pa.kv_cache_shapes(nsw, w.num_kv_heads, w.block_size, w.head_dim, dev.k_cache.dtype)
    hk = torch.empty(ks, dtype=dev.k_cache.dtype, pin_memory=True)
    hv = torch.empty(vs, dtype=dev.v_cache.dtype, pin_memory=True)
    ids = torch.tensor(blocks, dtype=torch.int32)
    seq = torch.arange(nsw, dtype=torch.int32)
    out_pairs = torch.stack([ids, seq], 1).contiguous().cuda()
    in_pairs = torch.stack([seq, ids], 1).contiguous().cuda()
    swap = {}
    for name, args in (("out", (dev.k_cache, dev.v_cache, hk, hv, out_pairs)),
                       ("in", (hk, hv, dev.k_cache, dev.v_cache, in_pairs))):
        pa.swap_blocks(*args)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(5):
            pa.swap_blocks(*args)
        b.record(stream)
        torch.cuda.synchronize()
        swap[name] = a.elapsed_time(b) / 5
    swap_bytes = nsw * 2 * w.num_kv_heads * w.block_size * w.head_dim * w.elem_bytes
    del hk, hv

    # cache append alone
    ca0, ca1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ca0.record(stream)
    for _ in range(steps):
        dev.cache_append()
    ca1.record(stream)
    torch.cuda.synchronize()
    ms_append = ca0.elapsed_time(ca1) / steps
    return dict(ms_step=ms_step, wall_s=t_wall, hot_ms=hot, cold_ms=cold, single_ms=single, ms_append=ms_append,
                out=out,
                stream_read_gbps=nbytes / (sr_ms * 1e-3) / 1e9,
                device=dev_name, width=dev.max_blocks, launches=dev.launches,
                read_bytes=read_bytes, algo_bytes=algo_bytes, swap_ms=swap, swap_bytes=swap_bytes, swap_blocks=nsw)


def cold_only_main(args, w, ps, mode, fused):
    """N decode launches of the step, each right after a 1 GiB read that
    evicts L2 and MALL (a read leaves no dirty lines to write back during the
    launch), with no events: under a kernel trace every launch of the decode
    kernel is a cold one, timed without event overhead."""
    import torch

    from paged_kv_cache_348_amd.workload import build_device_batch

    dev = build_device_batch(w, device="cuda", partition_size=ps)
    w.drop_kv()
    if mode == "shared":
        plan = dev.shared_plan()
        attend = lambda: dev.attend_shared(plan, partition_size=ps)  # noqa: E731
    elif fused:
        attend = dev.append_and_attend
    else:
        dev.cache_append()
        attend = dev.attend
    scratch = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.cold_only):
        scratch.amax()
        attend()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(json.dumps({"cold_only": args.cold_only, "workload": w.name, "partition_size": ps, "decode": mode,
                      "fused": fused, "wall_s": el}), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama3_8b", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--partition-size", type=int, default=None)
    ap.add_argument("--decode", choices=("split", "shared"), default=None,
                    help="split: pa_decode; shared: pa_decode_shared_prefix (reads blocks shared by forked "
                         "requests once per group); default: shared for prefix_share, else split")
    ap.add_argument("--step", choices=("fused", "separate"), default=None,
                    help="fused: cache append and decode in one launch (pa_decode_append, balanced split only); "
                         "separate: pa_cache_write then the decode; default: fused with the balanced split")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--block-order", choices=("seeded", "identity"), default="seeded",
                    help="identity: the free pool starts in address order, so each sequence's blocks are "
                         "mostly adjacent (the block-table lookup-overhead comparison)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cold-only", type=int, default=0, metavar="N",
                    help="run only N decode launches of the step, each after a 1 GiB read that evicts L2 and "
                         "MALL, with no events around them (for a kernel trace of cold launches), then print "
                         "one JSON line")
    ap.add_argument("--append", action="store_true",
                    help="measure the bulk cache append instead: pa_cache_write of every sequence's prefill tokens "
                         "(positions 0 .. L-2, their own slots and values) in one call")
    ap.add_argument("--prefill", type=int, default=0,
                    help="measure pa_prefill instead: the last N tokens of each request are new queries "
                         "(causal multi-token query: speculative verification, chunked prefill)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the library has no multi-GPU path; "
              "the decode would shard by sequence or KV head with no exchange", file=sys.stderr)
        return 2
    if int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py is a single-process, single-GPU benchmark", file=sys.stderr)
        return 2

    w = make_workload(args.workload, seed=args.seed)
    if args.block_order == "identity":
        w.free_order = np.arange(w.num_blocks, dtype=np.int32)
    if args.prefill > 0:
        return prefill_main(args, w)
    if args.append:
        return append_main(args, w)
    ps = args.partition_size
    mode = args.decode or DEFAULT_DECODE.get(args.workload, "split")
    if ps is None:
        ps = w.partition_size or DEFAULT_PARTITION.get(args.workload, 0)
    if mode == "shared" and ps <= 0:
        ps = 512
    fused = (args.step or ("fused" if ps == PARTITION_BALANCED and mode == "split" else "separate")) == "fused"
    if fused and (ps != PARTITION_BALANCED or mode != "split"):
        print("--step fused runs on the balanced split (pa_decode_append)", file=sys.stderr)
        return 2
    kv_bytes = w.kv_read_bytes()
    log(f"workload {w.name}: B {w.batch}, sum L {int(w.seq_lens.sum())}, KV bytes {kv_bytes / 1e9:.3f} GB, "
        f"partition {ps}, decode {mode}")
    if args.cold_only:
        return cold_only_main(args, w, ps, mode, fused)

    cpu, ref = (None, None)
    if not args.no_cpu:
        cpu, ref = cpu_baseline(w, min_seconds=args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']:.1f} tok/s on {cpu['cores']} cores")

    g = gpu_bench(w, args.steps, args.warmup, ps, mode, fused=fused)
    ms = g["ms_step"]
    hot, cold = g["hot_ms"], g["cold_ms"]
    t_dec = float(np.median(hot)) * 1e-3
    read_bytes = g["read_bytes"]  # what the decode must read: logical KV bytes, or unique ones when shared
    algo_bytes = g["algo_bytes"]  # + the new tokens' stores when the append runs in the same launch
    # the dominant kernel's launch time: with the one-launch step, the timed
    # region's own average (one launch per step); otherwise the decode alone,
    # back to back between one event pair (median of three runs)
    t_launch = ms * 1e-3 if fused else t_dec
    achieved = algo_bytes / t_launch / 1e9
    t_cold = float(np.median(cold)) * 1e-3
    # per-launch event gap, measured on hot launches in this run
    gap = max(0.0, float(np.median(g["single_ms"])) - float(np.median(hot))) * 1e-3
    err = None
    if ref is not None:
        err = float(np.abs(g["out"] - ref).max())
        log(f"full-size parity vs oracle: max abs err {err:.3e}")
    flop = 4.0 * w.head_dim * w.num_q_heads * float(w.seq_lens.sum())
    res = {
        "metric": "decode attention tokens/s and KV-read HBM GB/s (% of 8 TB/s) on 1 MI355X",
        "value": w.batch / (ms * 1e-3),
        "unit": "decode tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v rounded to bf16; seeded lengths and block placement)",
        "config": {
            "workload": WORKLOAD_TEXT[args.workload],
            "name": w.name,
            "seed": args.seed,
            "batch": w.batch,
            "sum_seq_len": int(w.seq_lens.sum()),
            "num_q_heads": w.num_q_heads,
            "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim,
            "block_size": w.block_size,
            "num_blocks": w.num_blocks,
            "partition_size": ps,
            "step": ("pa_decode_append (the decode tokens' cache append and the decode in one launch)" if fused
                     else "pa_cache_write (decode tokens) + "
                     + ("pa_decode_shared_prefix" if mode == "shared" else "pa_decode")),
            "decode": mode,
            "block_order": args.block_order,
        },
        "kv_read_gbps_step": kv_bytes / (ms * 1e-3) / 1e9,
        "kv_logical_bytes": kv_bytes,
        "kv_unique_read_bytes": read_bytes,
        "kv_read_frac_of_8tbs_step": kv_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "decode_us": {"hot": float(np.median(hot)) * 1e3, "hot_runs": [float(x) * 1e3 for x in hot],
                      "cold_median": float(np.median(cold)) * 1e3, "cold_min": float(cold.min()) * 1e3,
                      "hot_one_event_pair_each": float(np.median(g["single_ms"])) * 1e3,
                      "event_pair_gap": gap * 1e6},
        "cache_append_us": g["ms_append"] * 1e3,
        "swap": {  # pa_swap_blocks to / from a pinned host pool (host link: PCIe 5.0 x16, 64 GB/s each way)
            "blocks": g["swap_blocks"], "bytes": g["swap_bytes"],
            "out_gbps": g["swap_bytes"] / (g["swap_ms"]["out"] * 1e-3) / 1e9,
            "in_gbps": g["swap_bytes"] / (g["swap_ms"]["in"] * 1e-3) / 1e9,
            "host_link_peak_gbps": HOST_LINK_GBPS,
        },
        "stream_read_gbps_same_bytes": g["stream_read_gbps"],
        "kv_tokens_per_s": float(w.seq_lens.sum()) / t_dec,
        "roofline": {
            "bound": "hbm",
            "kernel": "pa_decode_shared_prefix" if mode == "shared" else ("pa_decode_append" if fused else "pa_decode"),
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "timing": ("timed region: one launch per step" if fused else
                       "decode alone, back-to-back launches between one event pair"),
            # L2 and MALL evicted before each launch (a 1 GiB read), one event
            # pair per launch, median of the launches
            "achieved_cold": algo_bytes / t_cold / 1e9,
            "frac_cold": algo_bytes / t_cold / 1e9 / HBM_PEAK_GBPS,
            # the same cold median less the event-pair gap measured on hot
            # launches timed the same way (a kernel trace of cold launches,
            # bench.py --cold-only, times the kernel with no events at all)
            "frac_cold_net": algo_bytes / max(t_cold - gap, 1e-9) / 1e9 / HBM_PEAK_GBPS,
            "traffic": (measured_traffic(args.workload, mode, fused)
                        if ps == DEFAULT_PARTITION.get(args.workload, ps)
                        and mode == DEFAULT_DECODE.get(args.workload, "split") else None),
            "algorithmic_bytes_per_launch": algo_bytes,
            "flop_per_launch": flop,
        },
        "cpu_baseline": cpu,
        "max_abs_err_vs_oracle": err,
        "device": g["device"],
    }
    if cpu is not None:
        cpu.pop("kv_read_gbps", None)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
