"""Device state for a workload's decode step, built through libpa.

Replays a workload's allocator operations through the library's host
allocator and writes the appended tokens into a device pool with the
library's kernels (pa_cache_write, pa_copy_blocks).  Launches are batched:
pending block copies run before pending token writes, and a batch is
flushed whenever the next copy touches a block that pending work touches,
or a write repeats a pending slot, so the final pool equals a token-by-token
replay.  The decode-step tokens (one per measured sequence) are not written
here: they are the cache append of the measured step.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

from . import (PA_PARTITION_BALANCED, Allocator, cache_write, check_slots, copy_blocks, decode, decode_append,
               decode_shared_prefix,
               decode_shared_prefix_workspace_bytes, decode_workspace_bytes, new_kv_cache, new_workspace,
               plan_shared_prefix, shared_prefix_max_group)


def _torch():
    import torch

    return torch


def to_device(arr: np.ndarray, dtype_name: str, device):
    """Host array (uint16 bf16 bits or float32) -> device tensor of the cache dtype."""
    torch = _torch()
    arr = np.ascontiguousarray(arr)
    if dtype_name == "bf16":
        return torch.from_numpy(arr.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(arr.astype(np.float32, copy=False)).to(device)


@dataclass
class DeviceBatch:
    workload: object
    allocator: Allocator
    q: object
    k_cache: object
    v_cache: object
    block_tables: object  # int32 [B, max_blocks]
    seq_lens: object  # int32 [B]
    dec_k: object  # [T, Hkv, D] decode-step tokens (T = sequences with L >= 1)
    dec_v: object
    dec_slots: object  # int64 [T]
    out: object
    workspace: Optional[object]
    partition_size: int
    host_tables: np.ndarray
    host_lens: np.ndarray
    host_dec_slots: np.ndarray
    launches: dict = field(default_factory=dict)
    shared_workspace: Optional[object] = None
    # the decode step's new tokens per sequence for the fused append
    # (pa_decode_append): row b is position L_b - 1, stored at new_slots[b]
    # (-1: a sequence without a decode-step token, its last position already
    # in the cache, or L_b = 0)
    new_k: Optional[object] = None
    new_v: Optional[object] = None
    new_slots: Optional[object] = None
    fused_workspace: Optional[object] = None

    @property
    def max_blocks(self) -> int:
        return int(self.host_tables.shape[1])

    def cache_append(self, stream=None) -> None:
        cache_write(self.dec_k, self.dec_v, self.dec_slots, self.k_cache, self.v_cache, stream=stream)

    def append_and_attend(self, stream=None, out=None):
        """The cache append and the decode in one launch (pa_decode_append)."""
        w = self.workload
        if self.fused_workspace is None:
            self.fused_workspace = new_workspace(
                decode_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                       self.max_blocks, PA_PARTITION_BALANCED), self.q.device)
        return decode_append(self.q, self.new_k, self.new_v, self.new_slots, self.k_cache, self.v_cache,
                             self.block_tables, self.seq_lens, w.num_kv_heads, w.scale,
                             out=self.out if out is None else out, workspace=self.fused_workspace, stream=stream)

    def attend(self, stream=None, partition_size: Optional[int] = None, out=None):
        w = self.workload
        ps = self.partition_size if partition_size is None else partition_size
        ws = self.workspace
        need = decode_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size,
                                      self.max_blocks, ps)
        if need and (ws is None or ws.numel() < need):
            ws = new_workspace(need, self.q.device)
            if partition_size is None:
                self.workspace = ws
        return decode(self.q, self.k_cache, self.v_cache, self.block_tables, self.seq_lens, w.num_kv_heads, w.scale,
                      out=self.out if out is None else out, partition_size=ps, workspace=ws, stream=stream)

    def shared_plan(self, max_group_size: Optional[int] = None, min_shared_blocks: int = 1):
        """Plan (host) and upload the shared-prefix grouping of this batch's tables."""
        w = self.workload
        mg = (shared_prefix_max_group(w.num_q_heads, w.num_kv_heads, w.head_dim, self.q.dtype)
              if max_group_size is None else max_group_size)
        plan = plan_shared_prefix(self.host_tables, self.host_lens, w.block_size, mg, min_shared_blocks)
        return plan.to(self.q.device)

    def attend_shared(self, plan, partition_size: int = 512, stream=None, out=None, workspace=None):
        """Decode attention through the shared-prefix path (pa_decode_shared_prefix)."""
        w = self.workload
        ws = workspace
        if ws is None:
            need = decode_shared_prefix_workspace_bytes(w.batch, w.num_q_heads, w.head_dim, w.block_size,
                                                        self.max_blocks, plan.max_prefix_blocks, partition_size)
            ws = self.shared_workspace
            if need and (ws is None or ws.numel() < need):
                ws = self.shared_workspace = new_workspace(need, self.q.device)
        return decode_shared_prefix(self.q, self.k_cache, self.v_cache, self.block_tables, self.seq_lens,
                                    w.num_kv_heads, w.scale, plan, partition_size=partition_size,
                                    out=self.out if out is None else out, workspace=ws, stream=stream)

    def step(self, stream=None, partition_size: Optional[int] = None):
        """One decode step: append the decode tokens, then attend."""
        self.cache_append(stream)
        return self.attend(stream, partition_size)


class _Batcher:
    def __init__(self, w, k_cache, v_cache, device, max_tokens: int):
        self.w, self.kc, self.vc, self.device = w, k_cache, v_cache, device
        self.max_tokens = max_tokens
        self.copies: List[Tuple[int, int]] = []
        self.slots: List[np.ndarray] = []
        self.ks: List[np.ndarray] = []
        self.vs: List[np.ndarray] = []
        self.slot_set = set()
        self.blocks = set()  # blocks touched by pending copies or writes
        self.ntok = 0
        self.launches = {"cache_write": 0, "copy_blocks": 0}

    def add_copy(self, src: int, dst: int) -> None:
        if src in self.blocks or dst in self.blocks:
            self.flush()
        self.copies.append((src, dst))
        self.blocks.update((src, dst))

    def add_write(self, slots: np.ndarray, k: np.ndarray, v: np.ndarray) -> None:
        if any(int(s) in self.slot_set for s in slots):
            self.flush()
        bs = self.w.block_size
        self.slots.append(slots)
        self.ks.append(k)
        self.vs.append(v)
        self.slot_set.update(int(s) for s in slots)
        self.blocks.update(int(s) // bs for s in slots)
        self.ntok += len(slots)
        if self.ntok >= self.max_tokens:
            self.flush()

    def flush(self) -> None:
        torch = _torch()
        if self.copies:
            pairs = torch.tensor(np.array(self.copies, dtype=np.int32), device=self.device)
            copy_blocks(self.kc, self.vc, pairs)
            self.launches["copy_blocks"] += 1
        if self.slots:
            host = np.concatenate(self.slots).astype(np.int64)
            check_slots(host, self.w.num_blocks * self.w.block_size)  # distinct, inside the pool
            slots = torch.from_numpy(host).to(self.device)
            k = to_device(np.concatenate(self.ks), self.w.dtype, self.device)
            v = to_device(np.concatenate(self.vs), self.w.dtype, self.device)
            cache_write(k, v, slots, self.kc, self.vc)
            self.launches["cache_write"] += 1
        self.copies, self.slots, self.ks, self.vs = [], [], [], []
        self.slot_set, self.blocks, self.ntok = set(), set(), 0


def build_device_batch(w, device="cuda", partition_size: Optional[int] = None, nan_fill: bool = True,
                       table_width: Optional[int] = None, table_pad: Optional[int] = None,
                       flush_tokens: int = 1 << 17) -> DeviceBatch:
    """Replay ``w``'s operations on the device; return the decode step's inputs.

    nan_fill poisons the pool first, so slots the replay never writes hold NaN.
    table_pad fills block-table entries past each sequence's blocks (default:
    a block no measured sequence uses, when one exists, else 0).
    """
    torch = _torch()
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    alloc = Allocator(w.num_blocks, w.block_size, w.free_order)
    kc, vc = new_kv_cache(w.num_blocks, w.num_kv_heads, w.block_size, w.head_dim, dt, device, nan_fill=nan_fill)
    bat = _Batcher(w, kc, vc, device, flush_tokens)
    dec = {}
    length = {}  # tokens per live sequence, tracked here to avoid table queries
    for op in w.ops:
        if op.kind == "add":
            alloc.add_seq(op.seq)
            length[op.seq] = 0
        elif op.kind == "fork":
            alloc.fork(op.parent, op.seq)
            length[op.seq] = length[op.parent]
        elif op.kind == "free":
            alloc.free(op.seq)
            del length[op.seq]
        elif op.kind == "append":
            start = length[op.seq]
            slots, copies = alloc.append(op.seq, op.n)
            length[op.seq] = start + op.n
            for src, dst in copies:
                bat.add_copy(src, dst)
            if op.decode:
                dec[op.seq] = int(slots[-1])
            elif op.write:
                k, v = w.token_kv(op.seq, start, op.n)
                bat.add_write(slots, k, v)
        else:
            raise ValueError(op.kind)
    bat.flush()

    used = set()
    width = table_width
    tabs = [alloc.table(s)[0] for s in w.seq_ids]
    for t in tabs:
        used.update(t)
    if width is None:
        width = max([len(t) for t in tabs] + [1])
    if table_pad is None:
        free = alloc.free_list()
        table_pad = free[0] if free else (0 if not used else min(used))
    tables, lens = alloc.batch_tables(w.seq_ids, width=width, pad=table_pad)

    # decode-step tokens, in batch order (sequences without one are skipped)
    rows = [b for b, s in enumerate(w.seq_ids) if s in dec]
    dslots = np.array([dec[w.seq_ids[b]] for b in rows], dtype=np.int64)
    check_slots(dslots, w.num_blocks * w.block_size)
    dk, dv = [], []
    for b in rows:  # the decode token is the last position, L - 1
        k, v = w.token_kv(w.seq_ids[b], int(lens[b]) - 1, 1)
        dk.append(k)
        dv.append(v)
    shape = (0, w.num_kv_heads, w.head_dim)
    # per-sequence rows for the fused append: position L - 1 of every sequence
    nk = np.zeros((w.batch, w.num_kv_heads, w.head_dim), w.np_dtype)
    nv = np.zeros_like(nk)
    nslots = np.full(w.batch, -1, dtype=np.int64)
    for i, b in enumerate(rows):
        nk[b], nv[b], nslots[b] = dk[i][0], dv[i][0], dslots[i]
    for b, s in enumerate(w.seq_ids):
        if s not in dec and lens[b] >= 1:
            k, v = w.token_kv(s, int(lens[b]) - 1, 1)
            nk[b], nv[b] = k[0], v[0]
    dk = np.concatenate(dk) if dk else np.empty(shape, w.np_dtype)
    dv = np.concatenate(dv) if dv else np.empty(shape, w.np_dtype)

    ps = w.partition_size if partition_size is None else partition_size
    need = (decode_workspace_bytes(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, width, ps)
            if w.batch else 0)
    ws = new_workspace(need, device) if need else None
    q = to_device(w.q, w.dtype, device)
    return DeviceBatch(
        workload=w, allocator=alloc, q=q, k_cache=kc, v_cache=vc,
        block_tables=torch.from_numpy(tables).to(device), seq_lens=torch.from_numpy(lens).to(device),
        dec_k=to_device(dk, w.dtype, device), dec_v=to_device(dv, w.dtype, device),
        dec_slots=torch.from_numpy(dslots).to(device), out=torch.empty_like(q), workspace=ws,
        partition_size=ps, host_tables=tables, host_lens=lens, host_dec_slots=dslots, launches=bat.launches,
        new_k=to_device(nk, w.dtype, device), new_v=to_device(nv, w.dtype, device),
        new_slots=torch.from_numpy(nslots).to(device),
    )
