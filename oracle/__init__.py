"""CPU oracle for paged single-query decode attention (test infrastructure).

This package is test infrastructure, not part of the product path.  Only the
tests, the package's smoke check and the benchmark's CPU-baseline leg may
import it.  It shares no code with the HIP path: it reads the same seeded
inputs (``synthetic``) and nothing else.

Every function is a plain, slow, obviously-correct restatement of what the
pages on PagedAttention describe, in float64 for floating point:

* ``allocator``: on-demand block allocation with a free pool, per-request
  block tables, reference-counted sharing after a fork and copy-on-write of
  a shared block, plus slot accounting (held / used / wasted) and the
  contiguous-reservation scheme the pages compare against.
* ``cache``: the KV pool as the pages lay it out (per layer, keys and values
  each ``[num_blocks, num_kv_heads, block_size, head_dim]``), a NaN-poisoned
  pre-image, the slot scatter and whole-block copies, and a sequential replay
  of a workload's operation list.
* ``memsim``: replay of a request trace (arrivals, prompts, replies) under
  contiguous reservation and under paging, with the slot accounting of the
  two allocator models (the pages' waste comparison).
* ``attention``: the block-table walk that gathers K and V per position,
  followed by standard scaled-dot-product attention (dense two-pass softmax),
  a loop-only variant for tiny inputs, and the partition / log-sum-exp merge
  model used for long contexts.

Pins (tests/test_oracle_*.py) tie each function to something other than
itself: values the pages print, invariants they state, closed forms, a
library attention routine, and brute force on tiny inputs.
"""
