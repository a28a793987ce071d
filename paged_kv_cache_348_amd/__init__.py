"""Paged KV-cache decode attention for AMD MI355X (gfx950).

A thin Python binding over libpa.so (include/pa.h): argument marshalling
only.  Every step of the decode path (cache append, block copy, decode
attention, log-sum-exp merge) runs in the library's HIP kernels; the block
allocator runs in the library's host C++.  PyTorch supplies device memory
and streams.

Device cache layout (per layer), X = 16 bytes / element size:
    k_cache [num_blocks, num_kv_heads, head_dim // X, block_size, X]
    v_cache [num_blocks, num_kv_heads, head_dim, block_size]
where a bfloat16 value of in-block offset o with block_size 16 or 32 sits
at ``value_position(o)`` (bits 2 and 3 of o swapped).  ``logical_view``
presents both as [num_blocks, num_kv_heads, block_size, head_dim], the
pages' per-layer layout.
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from ._lib import (PA_MEM_CONTIGUOUS, PA_MEM_PAGED, MemStats)
from ._lib import (PA_BF16, PA_PARTITION_BALANCED, PA_ERR_EXISTS, PA_ERR_INVALID_ARG, PA_ERR_LAUNCH, PA_ERR_NOT_FOUND, PA_ERR_OOM,
                   PA_ERR_UNSUPPORTED, PA_F32, PA_OK, P_I32, P_I64, PAError, check, lib, status_string)

__all__ = [
    "PAError", "Allocator", "cache_write", "check_slots", "copy_blocks", "decode", "decode_workspace_bytes", "new_kv_cache",
    "kv_cache_shapes", "logical_view", "value_position", "stream_read", "PA_OK", "PA_ERR_INVALID_ARG", "PA_ERR_UNSUPPORTED", "PA_ERR_OOM",
    "PA_ERR_NOT_FOUND", "PA_ERR_LAUNCH", "PA_ERR_EXISTS", "PA_PARTITION_BALANCED", "status_string", "lib",
    "new_workspace", "SharedPrefixPlan", "plan_shared_prefix", "decode_shared_prefix",
    "decode_shared_prefix_workspace_bytes", "shared_prefix_max_group", "simulate_memory", "PA_MEM_CONTIGUOUS",
    "PA_MEM_PAGED", "swap_blocks", "decode_append", "decode_append_noalloc", "prefill", "prefill_workspace_bytes", "prefill_path",
]


def _torch():
    import torch

    return torch


def _dtype_code(dtype) -> int:
    torch = _torch()
    if dtype == torch.bfloat16:
        return PA_BF16
    if dtype == torch.float32:
        return PA_F32
    raise TypeError(f"unsupported dtype {dtype} (bfloat16 or float32)")


def _elem_bytes(dtype) -> int:
    return 2 if _dtype_code(dtype) == PA_BF16 else 4


def _on_stream(stream):
    """Context for the tensors a call makes itself (``out``, a zero-filled
    workspace): they are allocated, and the workspace filled, on the launch
    stream, so the launch follows the fill in stream order and the caching
    allocator does not hand the memory to another stream while the launch
    may still use it.  With no stream given the launch stream is the current
    one and nothing changes."""
    import contextlib

    return contextlib.nullcontext() if stream is None else _torch().cuda.stream(stream)


def _stream_ptr(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


def _dev(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def kv_cache_shapes(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int,
                    dtype) -> Tuple[Tuple[int, ...], Tuple[int, ...]]:
    x = 16 // _elem_bytes(dtype)
    if head_dim % x:
        raise ValueError("head_dim must be a multiple of 16 bytes of elements")
    return ((num_blocks, num_kv_heads, head_dim // x, block_size, x), (num_blocks, num_kv_heads, head_dim, block_size))


def new_kv_cache(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int, dtype=None,
                 device="cuda", nan_fill: bool = False):
    """Allocate one layer's (k_cache, v_cache).  ``nan_fill`` poisons every slot with NaN."""
    torch = _torch()
    dtype = torch.bfloat16 if dtype is None else dtype
    ks, vs = kv_cache_shapes(num_blocks, num_kv_heads, block_size, head_dim, dtype)
    if nan_fill:
        k = torch.full(ks, float("nan"), dtype=dtype, device=device)
        v = torch.full(vs, float("nan"), dtype=dtype, device=device)
    else:
        k = torch.empty(ks, dtype=dtype, device=device)
        v = torch.empty(vs, dtype=dtype, device=device)
    return k, v


def _pool_dims(k_cache, v_cache):
    if k_cache.dim() != 5 or v_cache.dim() != 4:
        raise ValueError("k_cache must be [NB, Hkv, D/X, bs, X] and v_cache [NB, Hkv, D, bs]")
    nb, hkv, dx, bs, x = k_cache.shape
    d = dx * x
    if tuple(v_cache.shape) != (nb, hkv, d, bs) or k_cache.dtype != v_cache.dtype:
        raise ValueError("k_cache and v_cache disagree")
    if x * _elem_bytes(k_cache.dtype) != 16:
        raise ValueError("innermost key axis must span 16 bytes")
    return nb, hkv, bs, d


def value_position(offset: int, block_size: int, dtype) -> int:
    """Position along v_cache's last axis of the value with in-block offset ``offset``."""
    if _dtype_code(dtype) == PA_BF16 and block_size >= 16:
        return (offset & ~12) | ((offset & 4) << 1) | ((offset & 8) >> 1)
    return offset


def logical_view(k_cache, v_cache):
    """Both caches as [NB, Hkv, bs, D] (new tensors gathered from the device layout)."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    perm = [value_position(o, bs, v_cache.dtype) for o in range(bs)]
    idx = _torch().tensor(perm, device=v_cache.device)
    return (k_cache.permute(0, 1, 3, 2, 4).reshape(nb, hkv, bs, d),
            v_cache.index_select(3, idx).transpose(2, 3).contiguous())


def cache_write(k, v, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """Write token t's K/V ([T, Hkv, D] each) into slot slot_mapping[t] (int64; < 0 skips)."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    T = k.shape[0] if k.dim() == 3 else 0
    if k.shape != v.shape or (T and tuple(k.shape[1:]) != (hkv, d)):
        raise ValueError("k and v must be [T, num_kv_heads, head_dim]")
    if slot_mapping.dtype != _torch().int64 or slot_mapping.numel() != T:
        raise ValueError("slot_mapping must be int64 [T]")
    if k.dtype != k_cache.dtype:
        raise ValueError("k/v and cache dtypes differ")
    if T == 0:
        return
    check(lib().pa_cache_write(_dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping"),
                               _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), T, hkv, d, bs, nb,
                               _dtype_code(k.dtype), _stream_ptr(stream)), "pa_cache_write")


def check_slots(slot_mapping, num_slots: int) -> None:
    """Host check of an append's slots (pa_check_slots): raises PAError
    naming the first repeated or out-of-pool entry.  Negative slots pass."""
    sl = np.ascontiguousarray(np.asarray(slot_mapping, dtype=np.int64).reshape(-1))
    bad = ctypes.c_int32(-1)
    st = lib().pa_check_slots(sl.ctypes.data_as(P_I64), sl.shape[0], int(num_slots), ctypes.byref(bad))
    if st != PA_OK:
        where = f"pa_check_slots (entry {bad.value}: slot {int(sl[bad.value])})" if bad.value >= 0 else "pa_check_slots"
        raise PAError(st, where)


def copy_blocks(k_cache, v_cache, pairs, stream=None) -> None:
    """Copy whole blocks: pairs is int32 [n, 2] of (source, destination)."""
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    if pairs.dtype != _torch().int32 or (pairs.numel() and (pairs.dim() != 2 or pairs.shape[1] != 2)):
        raise ValueError("pairs must be int32 [n, 2]")
    n = pairs.shape[0] if pairs.numel() else 0
    if n == 0:
        return
    check(lib().pa_copy_blocks(_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(pairs, "pairs"), n, hkv, d,
                               bs, nb, _dtype_code(k_cache.dtype), _stream_ptr(stream)), "pa_copy_blocks")


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                           max_blocks_per_seq: int, partition_size: int) -> int:
    return int(lib().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                               max_blocks_per_seq, partition_size))


def new_workspace(nbytes: int, device="cuda"):
    """A decode workspace: zero-filled, as the balanced split's counters require."""
    return _torch().zeros(max(int(nbytes), 1), dtype=_torch().uint8, device=device)


def decode(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads: int, scale: float, out=None,
           partition_size: int = 0, workspace=None, stream=None):
    """Decode attention; returns ``out`` [B, Hq, D] (q's dtype).

    partition_size: 0 single pass, > 0 fixed partitions, PA_PARTITION_BALANCED
    (-1) the balanced split.  ``workspace`` (uint8 device tensor) must come
    from new_workspace() or be otherwise zero-filled before its first use.
    """
    torch = _torch()
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    if hkv != num_kv_heads:
        raise ValueError("num_kv_heads does not match the cache")
    B, hq, dq = q.shape
    if dq != d or q.dtype != k_cache.dtype:
        raise ValueError("q must be [B, Hq, head_dim] in the cache dtype")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks]")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        raise ValueError("seq_lens must be int32 [B]")
    if out is None:
        with _on_stream(stream):
            out = torch.empty_like(q)
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    mb = block_tables.shape[1]
    need = decode_workspace_bytes(B, hq, hkv, d, bs, mb, partition_size) if B else 0
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            with _on_stream(stream):
                workspace = new_workspace(need, q.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    check(lib().pa_decode(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                          _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), hkv, float(scale),
                          _dev(out, "out"), _stream_ptr(stream), B, hq, d, bs, nb, mb, _dtype_code(q.dtype),
                          partition_size, ws_ptr, ws_bytes), "pa_decode")
    return out


def decode_append(q, k, v, slot_mapping, k_cache, v_cache, block_tables, seq_lens, num_kv_heads: int, scale: float,
                  out=None, workspace=None, stream=None):
    """One decode step in one launch (pa_decode_append): stores k[b], v[b]
    ([B, Hkv, D], sequence b's token at position seq_lens[b] - 1) in slot
    slot_mapping[b] (int64 [B]; out of range skips) and returns the decode
    attention over positions 0 .. seq_lens[b] - 1, reading that position from
    k[b], v[b].  Balanced split; ``workspace`` as for decode()."""
    torch = _torch()
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    if hkv != num_kv_heads:
        raise ValueError("num_kv_heads does not match the cache")
    B, hq, dq = q.shape
    if dq != d or q.dtype != k_cache.dtype:
        raise ValueError("q must be [B, Hq, head_dim] in the cache dtype")
    if tuple(k.shape) != (B, hkv, d) or k.shape != v.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [B, num_kv_heads, head_dim] in the cache dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != B:
        raise ValueError("slot_mapping must be int64 [B]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks]")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        raise ValueError("seq_lens must be int32 [B]")
    if out is None:
        with _on_stream(stream):
            out = torch.empty_like(q)
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if B == 0:
        return out
    mb = block_tables.shape[1]
    need = decode_workspace_bytes(B, hq, hkv, d, bs, mb, PA_PARTITION_BALANCED)
    if workspace is None:
        with _on_stream(stream):
            workspace = new_workspace(need, q.device)
    check(lib().pa_decode_append(_dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping"),
                                 _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
                                 _dev(seq_lens, "seq_lens"), hkv, float(scale), _dev(out, "out"), _stream_ptr(stream),
                                 B, hq, d, bs, nb, mb, _dtype_code(q.dtype), _dev(workspace, "workspace"),
                                 workspace.numel() * workspace.element_size()), "pa_decode_append")
    return out


def decode_append_noalloc(q, k, v, slot_mapping, k_cache, v_cache, block_tables, seq_lens, num_kv_heads: int,
                          scale: float, out, stream=None):
    """decode_append without a workspace and without allocating
    (pa_decode_append_noalloc): the library's static per-GPU scratch holds
    the balanced split's counters and partials.  ``out`` must be given.
    Calls that overlap on one GPU race (they share the scratch)."""
    torch = _torch()
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    if hkv != num_kv_heads:
        raise ValueError("num_kv_heads does not match the cache")
    B, hq, dq = q.shape
    if dq != d or q.dtype != k_cache.dtype:
        raise ValueError("q must be [B, Hq, head_dim] in the cache dtype")
    if tuple(k.shape) != (B, hkv, d) or k.shape != v.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [B, num_kv_heads, head_dim] in the cache dtype")
    if slot_mapping.dtype != torch.int64 or slot_mapping.numel() != B:
        raise ValueError("slot_mapping must be int64 [B]")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks]")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        raise ValueError("seq_lens must be int32 [B]")
    if out is None or tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must be given and match q")
    if B == 0:
        return out
    check(lib().pa_decode_append_noalloc(
        _dev(q, "q"), _dev(k, "k"), _dev(v, "v"), _dev(slot_mapping, "slot_mapping"), _dev(k_cache, "k_cache"),
        _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"), hkv, float(scale),
        _dev(out, "out"), _stream_ptr(stream), B, hq, d, bs, nb, block_tables.shape[1], _dtype_code(q.dtype)),
        "pa_decode_append_noalloc")
    return out


class SharedPrefixPlan:
    """Groups of consecutive requests whose block tables start alike (pa_plan_shared_prefix).

    Host arrays: ``groups`` int32 [num_groups, 2] (first request, members),
    ``prefix_blocks`` int32 [B]; ``to(device)`` adds their device copies.
    """

    def __init__(self, groups, prefix_blocks, max_group: int, max_prefix_blocks: int):
        self.groups = groups
        self.prefix_blocks = prefix_blocks
        self.max_group = int(max_group)
        self.max_prefix_blocks = int(max_prefix_blocks)
        self.d_groups = None
        self.d_prefix_blocks = None

    @property
    def num_groups(self) -> int:
        return int(self.groups.shape[0])

    def check(self) -> None:
        """The plan's invariant (what pa_plan_shared_prefix returns): groups
        lie in the batch and do not overlap, and every request whose
        prefix_blocks is in 1 .. max_prefix_blocks lies in a group (else its
        rows would be unspecified).  Raises ValueError."""
        B = int(self.prefix_blocks.shape[0])
        owner = np.full(B, -1, dtype=np.int64)
        for i, (s0, n) in enumerate(np.asarray(self.groups, dtype=np.int64).reshape(-1, 2)):
            if s0 < 0 or n < 1 or s0 + n > B:
                raise ValueError(f"group {i} ({s0}, {n}) is outside the batch of {B}")
            if (owner[s0:s0 + n] >= 0).any():
                raise ValueError(f"group {i} overlaps another group")
            owner[s0:s0 + n] = i
        pb = np.asarray(self.prefix_blocks)
        loose = np.nonzero((pb > 0) & (pb <= self.max_prefix_blocks) & (owner < 0))[0]
        if len(loose):
            raise ValueError(f"request {int(loose[0])} has shared prefix blocks but no group")

    def to(self, device="cuda"):
        self.check()
        torch = _torch()
        g = self.groups if self.num_groups else np.zeros((1, 2), dtype=np.int32)
        self.d_groups = torch.from_numpy(np.ascontiguousarray(g)).to(device)
        self.d_prefix_blocks = torch.from_numpy(np.ascontiguousarray(self.prefix_blocks)).to(device)
        return self


def shared_prefix_max_group(num_q_heads: int, num_kv_heads: int, head_dim: int, dtype) -> int:
    """Largest group pa_decode_shared_prefix takes for this shape: 64 query
    columns per wave (32 for float32 with head dim 128) over the group's heads."""
    cols = 32 if (_dtype_code(dtype) == PA_F32 and head_dim == 128) else 64
    return max(1, cols // (num_q_heads // num_kv_heads))


def plan_shared_prefix(block_tables, seq_lens, block_size: int, max_group_size: int,
                       min_shared_blocks: int = 1) -> SharedPrefixPlan:
    """Plan the shared-prefix decode of a batch from its host tables (int32 [B, W]) and lengths."""
    tables = np.ascontiguousarray(np.asarray(block_tables, dtype=np.int32))
    lens = np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))
    if tables.ndim != 2 or lens.shape != (tables.shape[0],):
        raise ValueError("block_tables must be [B, W] and seq_lens [B]")
    B, W = tables.shape
    groups = np.zeros(2 * max(B, 1), dtype=np.int32)
    pblk = np.zeros(max(B, 1), dtype=np.int32)
    ng, mg, mp = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int32(0)
    check(lib().pa_plan_shared_prefix(tables.ctypes.data_as(P_I32), lens.ctypes.data_as(P_I32), B, W, block_size,
                                      max_group_size, min_shared_blocks, groups.ctypes.data_as(P_I32),
                                      pblk.ctypes.data_as(P_I32), ctypes.byref(ng), ctypes.byref(mg),
                                      ctypes.byref(mp)), "pa_plan_shared_prefix")
    return SharedPrefixPlan(groups[:2 * ng.value].reshape(ng.value, 2).copy(), pblk[:B].copy(), mg.value, mp.value)


def decode_shared_prefix_workspace_bytes(num_seqs: int, num_q_heads: int, head_dim: int, block_size: int,
                                         max_blocks_per_seq: int, max_prefix_blocks: int,
                                         partition_size: int) -> int:
    return int(lib().pa_decode_shared_prefix_workspace_bytes(num_seqs, num_q_heads, head_dim, block_size,
                                                             max_blocks_per_seq, max_prefix_blocks, partition_size))


def decode_shared_prefix(q, k_cache, v_cache, block_tables, seq_lens, num_kv_heads: int, scale: float,
                         plan: SharedPrefixPlan, partition_size: int = 512, out=None, workspace=None, stream=None,
                         max_group_size: Optional[int] = None):
    """Decode attention that reads blocks shared by a plan's groups once per group (pa_decode_shared_prefix).

    ``plan`` must hold device copies (``plan.to(device)``).  Returns ``out``.
    ``max_group_size`` overrides the plan's (to size the launch for a larger bound).
    """
    torch = _torch()
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    if hkv != num_kv_heads:
        raise ValueError("num_kv_heads does not match the cache")
    B, hq, dq = q.shape
    if dq != d or q.dtype != k_cache.dtype:
        raise ValueError("q must be [B, Hq, head_dim] in the cache dtype")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks]")
    if seq_lens.dtype != torch.int32 or seq_lens.numel() != B:
        raise ValueError("seq_lens must be int32 [B]")
    if plan.d_groups is None or plan.d_prefix_blocks is None:
        raise ValueError("plan has no device copies: call plan.to(device)")
    if plan.d_prefix_blocks.numel() != B:
        raise ValueError("plan was made for another batch")
    if out is None:
        with _on_stream(stream):
            out = torch.empty_like(q)
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    mb = block_tables.shape[1]
    mg = plan.max_group if max_group_size is None else int(max_group_size)
    need = decode_shared_prefix_workspace_bytes(B, hq, d, bs, mb, plan.max_prefix_blocks, partition_size) if B else 0
    ws_ptr, ws_bytes = None, 0
    if need:
        if workspace is None:
            with _on_stream(stream):
                workspace = new_workspace(need, q.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    check(lib().pa_decode_shared_prefix(
        _dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(block_tables, "block_tables"),
        _dev(seq_lens, "seq_lens"), hkv, float(scale), _dev(out, "out"), _stream_ptr(stream), B, hq, d, bs, nb, mb,
        _dtype_code(q.dtype), _dev(plan.d_groups, "groups"), _dev(plan.d_prefix_blocks, "prefix_blocks"),
        plan.num_groups, mg, plan.max_prefix_blocks, partition_size, ws_ptr, ws_bytes), "pa_decode_shared_prefix")
    return out


def simulate_memory(arrival, prompt, reply, capacity_slots: int, scheme: int, param: int) -> dict:
    """KV-memory accounting of a request trace (pa_simulate_memory): ``scheme``
    PA_MEM_CONTIGUOUS with ``param`` = reserved reply length, or PA_MEM_PAGED
    with ``param`` = block size.  Returns the pa_mem_stats fields."""
    arrs = [np.ascontiguousarray(np.asarray(x, dtype=np.int32)) for x in (arrival, prompt, reply)]
    n = arrs[0].shape[0]
    if any(a.shape != (n,) for a in arrs):
        raise ValueError("arrival, prompt and reply must be 1-D of one length")
    st = MemStats()
    check(lib().pa_simulate_memory(arrs[0].ctypes.data_as(P_I32), arrs[1].ctypes.data_as(P_I32),
                                   arrs[2].ctypes.data_as(P_I32), n, int(capacity_slots), scheme, param,
                                   ctypes.byref(st)), "pa_simulate_memory")
    return {name: int(getattr(st, name)) for name, _ in MemStats._fields_}


def prefill_workspace_bytes(num_seqs: int, num_query_tokens: int, num_q_heads: int, num_kv_heads: int,
                            head_dim: int, block_size: int, max_blocks_per_seq: int, max_query_len: int) -> int:
    """Workspace for pa_prefill's faster paths, the balanced split or key
    partitions (0: neither applies and the tile kernel runs)."""
    return int(lib().pa_prefill_workspace_bytes(num_seqs, num_query_tokens, num_q_heads, num_kv_heads, head_dim,
                                                block_size, max_blocks_per_seq, max_query_len))


# bfloat16 chunks of at least this many (token, head) columns run on
# workgroups of four query tiles sharing each key/value step through LDS
# (except blocks of 8 with head dim 128)
PREFILL_WORKGROUP_COLUMNS = 128


def prefill_path(num_seqs: int, num_q_heads: int, num_kv_heads: int, max_query_len: int, workspace_bytes: int,
                 bf16: bool = True, head_dim: int = 128, block_size: int = 16, scale: float = 1.0) -> str:
    """Which path pa_prefill takes given a workspace of ``workspace_bytes``
    sized by prefill_workspace_bytes (a description for logs)."""
    if not workspace_bytes:
        # (blocks of 8 with head dim 128, and scales <= 0, keep the query tiles)
        if (bf16 and scale > 0 and not (head_dim == 128 and block_size == 8)
                and max_query_len * (num_q_heads // num_kv_heads) >= PREFILL_WORKGROUP_COLUMNS):
            return "workgroup tiles"
        return "query tiles"
    if max_query_len * (num_q_heads // num_kv_heads) <= 16 and num_seqs <= 1024:
        return "balanced split"
    return "query tiles, key partitions"


def prefill(q, k_cache, v_cache, block_tables, seq_lens, query_start, num_kv_heads: int, scale: float,
            max_query_len: int, out=None, stream=None, workspace=None, balanced: bool = True):
    """Causal multi-token query over the paged cache (pa_prefill): q [T, Hq, D]
    holds each request's new tokens, rows query_start[b] .. query_start[b+1]-1;
    the last M_b of its seq_lens[b] cached tokens are those tokens.  Returns out [T, Hq, D].

    With ``balanced`` (the default) the faster paths run where they apply,
    on ``workspace`` or on a zero-filled one made here: the balanced split for
    verification-sized chunks (max_query_len * G <= 16), key partitions for
    short chunks of a batch.  With ``balanced=False`` (or where neither
    applies) the query-tile kernel runs, or for bfloat16 chunks of at least
    PREFILL_WORKGROUP_COLUMNS (token, head) columns the workgroup kernel."""
    torch = _torch()
    nb, hkv, bs, d = _pool_dims(k_cache, v_cache)
    if hkv != num_kv_heads:
        raise ValueError("num_kv_heads does not match the cache")
    T, hq, dq = q.shape
    if dq != d or q.dtype != k_cache.dtype:
        raise ValueError("q must be [T, Hq, head_dim] in the cache dtype")
    B = seq_lens.numel()
    if block_tables.dtype != torch.int32 or block_tables.dim() != 2 or block_tables.shape[0] != B:
        raise ValueError("block_tables must be int32 [B, max_blocks]")
    if seq_lens.dtype != torch.int32 or query_start.dtype != torch.int32 or query_start.numel() != B + 1:
        raise ValueError("seq_lens must be int32 [B] and query_start int32 [B + 1]")
    if out is None:
        with _on_stream(stream):
            out = torch.empty_like(q)
    if tuple(out.shape) != tuple(q.shape) or out.dtype != q.dtype:
        raise ValueError("out must match q")
    if B == 0 or T == 0:
        return out
    ws_ptr, ws_bytes = None, 0
    need = (prefill_workspace_bytes(B, T, hq, hkv, d, bs, block_tables.shape[1], int(max_query_len))
            if balanced else 0)
    if need:
        if workspace is None:
            with _on_stream(stream):
                workspace = new_workspace(need, q.device)
        ws_ptr, ws_bytes = _dev(workspace, "workspace"), workspace.numel() * workspace.element_size()
    check(lib().pa_prefill(_dev(q, "q"), _dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"),
                           _dev(block_tables, "block_tables"), _dev(seq_lens, "seq_lens"),
                           _dev(query_start, "query_start"), hkv, float(scale), _dev(out, "out"), _stream_ptr(stream),
                           B, T, hq, d, bs, nb, block_tables.shape[1], _dtype_code(q.dtype), int(max_query_len),
                           ws_ptr, ws_bytes), "pa_prefill")
    return out


def swap_blocks(src_k, src_v, dst_k, dst_v, pairs, stream=None) -> None:
    """Copy blocks pairs[i, 0] of (src_k, src_v) to blocks pairs[i, 1] of
    (dst_k, dst_v); pools on the device or in pinned host memory."""
    nb_s, hkv, bs, d = _pool_dims(src_k, src_v)
    nb_d, hkv2, bs2, d2 = _pool_dims(dst_k, dst_v)
    if (hkv, bs, d) != (hkv2, bs2, d2) or src_k.dtype != dst_k.dtype:
        raise ValueError("source and destination pools differ in block shape or dtype")
    if pairs.dtype != _torch().int32 or (pairs.numel() and (pairs.dim() != 2 or pairs.shape[1] != 2)):
        raise ValueError("pairs must be int32 [n, 2]")
    n = pairs.shape[0] if pairs.numel() else 0
    if n == 0:
        return
    for name, t in (("src_k", src_k), ("src_v", src_v), ("dst_k", dst_k), ("dst_v", dst_v), ("pairs", pairs)):
        if not t.is_contiguous() or not (t.is_cuda or t.is_pinned()):
            raise ValueError(f"{name} must be a contiguous device or pinned host tensor")
    check(lib().pa_swap_blocks(src_k.data_ptr(), src_v.data_ptr(), nb_s, dst_k.data_ptr(), dst_v.data_ptr(), nb_d,
                               pairs.data_ptr(), n, hkv, d, bs, _dtype_code(src_k.dtype), _stream_ptr(stream)),
          "pa_swap_blocks")


def stream_read(buf, sink, workgroups: int = 0, stream=None) -> None:
    """Measurement helper: read every byte of device tensor ``buf`` once (pa_bench_stream_read)."""
    if sink.dtype != _torch().int32 or sink.numel() < 1:
        raise ValueError("sink must be a device int32 tensor")
    check(lib().pa_bench_stream_read(_dev(buf, "buf"), buf.numel() * buf.element_size(), _dev(sink, "sink"),
                                     workgroups, _stream_ptr(stream)), "pa_bench_stream_read")


class Allocator:
    """Host block allocator (libpa's pa_alloc_*): on-demand blocks, fork, copy-on-write, free."""

    def __init__(self, num_blocks: int, block_size: int, free_order: Optional[Sequence[int]] = None):
        self._lib = lib()
        self.num_blocks, self.block_size = num_blocks, block_size
        if free_order is not None:
            fo = np.ascontiguousarray(np.asarray(free_order, dtype=np.int32))
            if fo.shape != (num_blocks,):
                raise ValueError("free_order must list every block once")
            ptr = fo.ctypes.data_as(P_I32)
        else:
            ptr = None
        self._h = self._lib.pa_alloc_create(num_blocks, block_size, ptr)
        if not self._h:
            raise ValueError("pa_alloc_create rejected its arguments")
        self._slots = np.zeros(1, dtype=np.int64)
        self._cow = np.zeros(2, dtype=np.int32)
        self._ncow = ctypes.c_int32(0)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h:
            self._lib.pa_alloc_destroy(h)
            self._h = None

    def add_seq(self, seq: int) -> None:
        check(self._lib.pa_alloc_add_seq(self._h, seq), "pa_alloc_add_seq")

    def append(self, seq: int, n: int):
        """Returns (slots int64 [n], copy pairs [(src, dst)])."""
        if self._slots.shape[0] < max(n, 1):
            self._slots = np.zeros(max(n, 2 * self._slots.shape[0]), dtype=np.int64)
        st = self._lib.pa_alloc_append(self._h, seq, n, self._slots.ctypes.data_as(P_I64),
                                       self._cow.ctypes.data_as(P_I32), 1, ctypes.byref(self._ncow))
        check(st, "pa_alloc_append")
        pairs = [(int(self._cow[0]), int(self._cow[1]))] if self._ncow.value else []
        return self._slots[:n].copy(), pairs

    def fork(self, parent: int, child: int) -> None:
        check(self._lib.pa_alloc_fork(self._h, parent, child), "pa_alloc_fork")

    def free(self, seq: int) -> None:
        check(self._lib.pa_alloc_free(self._h, seq), "pa_alloc_free")

    def table(self, seq: int):
        """(table as a list, length in tokens)."""
        nbk, ln = ctypes.c_int32(0), ctypes.c_int32(0)
        check(self._lib.pa_alloc_table(self._h, seq, None, 0, ctypes.byref(nbk), ctypes.byref(ln)), "pa_alloc_table")
        out = np.zeros(max(nbk.value, 1), dtype=np.int32)
        check(self._lib.pa_alloc_table(self._h, seq, out.ctypes.data_as(P_I32), nbk.value, ctypes.byref(nbk),
                                       ctypes.byref(ln)), "pa_alloc_table")
        return out[:nbk.value].tolist(), ln.value

    def batch_tables(self, seqs: Sequence[int], width: Optional[int] = None, pad: int = 0):
        """Dense (block_tables int32 [B, width], seq_lens int32 [B]) for a decode call."""
        seqs = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
        if width is None:
            width = max([len(self.table(int(s))[0]) for s in seqs] + [1])
        tables = np.zeros((len(seqs), width), dtype=np.int32)
        lens = np.zeros(len(seqs), dtype=np.int32)
        check(self._lib.pa_alloc_batch_tables(self._h, seqs.ctypes.data_as(P_I64), len(seqs),
                                              tables.ctypes.data_as(P_I32), width, pad, lens.ctypes.data_as(P_I32)),
              "pa_alloc_batch_tables")
        return tables, lens

    def move(self, to: "Allocator", seqs: Sequence[int]):
        """Move sequences to allocator ``to`` (swap out / in); returns the
        (from block, to block) copy pairs as int32 [n, 2]."""
        seqs = np.ascontiguousarray(np.asarray(list(seqs), dtype=np.int64))
        n = ctypes.c_int32(0)
        cap = max(1, sum(len(self.table(int(s))[0]) for s in seqs)) if len(seqs) else 1
        pairs = np.zeros(2 * cap, dtype=np.int32)
        check(self._lib.pa_alloc_move(self._h, to._h, seqs.ctypes.data_as(P_I64), len(seqs),
                                      pairs.ctypes.data_as(P_I32), cap, ctypes.byref(n)), "pa_alloc_move")
        return pairs[:2 * n.value].reshape(n.value, 2).copy()

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_alloc_refcount(self._h, block))

    def free_list(self):
        n = ctypes.c_int32(0)
        check(self._lib.pa_alloc_free_list(self._h, None, 0, ctypes.byref(n)), "pa_alloc_free_list")
        out = np.zeros(max(n.value, 1), dtype=np.int32)
        check(self._lib.pa_alloc_free_list(self._h, out.ctypes.data_as(P_I32), n.value, ctypes.byref(n)),
              "pa_alloc_free_list")
        return out[:n.value].tolist()

    def num_free(self) -> int:
        return int(self._lib.pa_alloc_num_free(self._h))
