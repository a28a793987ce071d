"""ctypes loader for libpa.so, the package's C-ABI library (include/pa.h).

The library is built in-tree by ``paged_kv_cache_348_amd.build``.  Loading
fails loudly when it is missing: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

c_int32, c_int64, c_size_t, c_float, c_void_p = (ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                                                  ctypes.c_float, ctypes.c_void_p)
P_I32 = ctypes.POINTER(ctypes.c_int32)
P_I64 = ctypes.POINTER(ctypes.c_int64)

PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_OOM, PA_ERR_NOT_FOUND, PA_ERR_LAUNCH, PA_ERR_EXISTS = range(7)
PA_F32, PA_BF16 = 0, 1
PA_PARTITION_BALANCED = -1
PA_MEM_CONTIGUOUS, PA_MEM_PAGED = 0, 1


class MemStats(ctypes.Structure):
    """pa_mem_stats (include/pa.h)."""
    _fields_ = [("steps", c_int64), ("used_slot_steps", c_int64), ("held_slot_steps", c_int64),
                ("peak_used", c_int64), ("peak_held", c_int64), ("max_request_waste", c_int64),
                ("admitted", c_int32), ("rejected", c_int32), ("dropped", c_int32), ("peak_live", c_int32)]

# (name, restype, argtypes) of every symbol include/pa.h and include/pa_bench.h declare
SIGNATURES = [
    ("pa_status_string", ctypes.c_char_p, [c_int32]),
    ("pa_cache_write", c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                 c_int32, c_int32, c_int32, c_void_p]),
    ("pa_check_slots", c_int32, [P_I64, c_int32, c_int64, P_I32]),
    ("pa_copy_blocks", c_int32, [c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                 c_int32, c_void_p]),
    ("pa_decode_workspace_bytes", c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32]),
    ("pa_decode_counter_bytes", c_size_t, []),
    ("pa_decode", c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_void_p,
                            c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                            c_void_p, c_size_t]),
    ("pa_decode_append", c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                   c_int32, c_float, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32,
                                   c_int32, c_int32, c_int32, c_void_p, c_size_t]),
    ("pa_decode_append_noalloc", c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
                                           c_void_p, c_int32, c_float, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                           c_int32, c_int32, c_int32, c_int32]),
    ("pa_decode_shared_prefix_workspace_bytes", c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                                           c_int32]),
    ("pa_decode_shared_prefix", c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float,
                                          c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                          c_int32, c_void_p, c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p,
                                          c_size_t]),
    ("pa_plan_shared_prefix", c_int32, [P_I32, P_I32, c_int32, c_int32, c_int32, c_int32, c_int32, P_I32, P_I32,
                                        P_I32, P_I32, P_I32]),
    ("pa_simulate_memory", c_int32, [P_I32, P_I32, P_I32, c_int32, c_int64, c_int32, c_int32, c_void_p]),
    ("pa_prefill_workspace_bytes", c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                                              c_int32]),
    ("pa_prefill", c_int32, [c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_float, c_void_p,
                             c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32,
                             c_int32, c_void_p, c_size_t]),
    ("pa_swap_blocks", c_int32, [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_void_p, c_int32,
                                 c_int32, c_int32, c_int32, c_int32, c_void_p]),
    ("pa_alloc_move", c_int32, [c_void_p, c_void_p, P_I64, c_int32, P_I32, c_int32, P_I32]),
    ("pa_alloc_create", c_void_p, [c_int32, c_int32, P_I32]),
    ("pa_alloc_destroy", None, [c_void_p]),
    ("pa_alloc_add_seq", c_int32, [c_void_p, c_int64]),
    ("pa_alloc_append", c_int32, [c_void_p, c_int64, c_int32, P_I64, P_I32, c_int32, P_I32]),
    ("pa_alloc_fork", c_int32, [c_void_p, c_int64, c_int64]),
    ("pa_alloc_free", c_int32, [c_void_p, c_int64]),
    ("pa_alloc_table", c_int32, [c_void_p, c_int64, P_I32, c_int32, P_I32, P_I32]),
    ("pa_alloc_batch_tables", c_int32, [c_void_p, P_I64, c_int32, P_I32, c_int32, c_int32, P_I32]),
    ("pa_alloc_refcount", c_int32, [c_void_p, c_int32]),
    ("pa_alloc_free_list", c_int32, [c_void_p, P_I32, c_int32, P_I32]),
    ("pa_alloc_num_free", c_int32, [c_void_p]),
    # include/pa_bench.h
    ("pa_bench_stream_read", c_int32, [c_void_p, c_size_t, c_void_p, c_int32, c_void_p]),
]

_lib = None


class PAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} (status {status})")


# A host-only build of the library's C++ (allocator, planner, simulator,
# slot checker) under the address and undefined-behaviour sanitizers
# (``python -m paged_kv_cache_348_amd.build --sanitize``) is loaded instead
# when this variable names it; its device entry points are absent.
HOST_ONLY_ENV = "PA_HOST_ONLY_LIB"


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        host_only = os.environ.get(HOST_ONLY_ENV)
        path = host_only or LIB_PATH
        if not os.path.exists(path):
            raise ImportError(f"{path} is missing: build it with `python -m paged_kv_cache_348_amd.build`")
        h = ctypes.CDLL(path)
        for name, res, args in SIGNATURES:
            fn = getattr(h, name, None) if host_only else getattr(h, name)
            if fn is None:
                continue
            fn.restype = res
            fn.argtypes = args
        _lib = h
    return _lib


def status_string(status: int) -> str:
    s = lib().pa_status_string(status)
    return s.decode() if s else "?"


def check(status: int, where: str) -> None:
    if status != PA_OK:
        raise PAError(status, where)
