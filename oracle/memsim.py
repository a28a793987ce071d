"""KV-memory accounting of a request trace (test infrastructure).

Replays a trace of requests (arrival step, prompt length, reply length)
against the two schemes the pages compare, using the allocator models of
``oracle.allocator``:

* contiguous reservation ("Paged attention in LLMs", section "Why the memory
  gets wasted"): each request reserves its prompt plus the longest reply it
  may produce, in one unbroken run placed first fit
  (``ContiguousReservationModel``); reserved slots the reply never reaches
  and gaps too small for the next reservation are lost;
* paging (same page, "The fix" and "Why this helps so much"; MCQ page,
  comparison table, "Memory waste" row): whole blocks taken one at a time
  from anywhere (``BlockAllocatorModel``), so a request loses at most the
  unfilled tail of its last block.

Reading where the pages are silent (they give no serving loop): time runs in
decode steps; at step t the requests whose reply completed at t - 1 release
their memory, then requests arriving at t are admitted in trace order (the
prompt is stored at once) or rejected when they do not fit, then every
request admitted before t appends one reply token (a paged request that
needs a block when none is free is dropped and frees its blocks), and a
request whose reply is now complete releases at t + 1.  After each step the
slots held and used by the live requests are summed.
"""
from __future__ import annotations

from typing import Dict, Sequence

from .allocator import BlockAllocatorModel, ContiguousReservationModel, OutOfBlocks

CONTIGUOUS, PAGED = 0, 1


def simulate(arrival: Sequence[int], prompt: Sequence[int], reply: Sequence[int], capacity: int, scheme: int,
             param: int) -> Dict[str, int]:
    """Statistics of one replay (the fields of the library's ``pa_mem_stats``)."""
    n = len(arrival)
    assert len(prompt) == n and len(reply) == n
    assert all(arrival[i] <= arrival[i + 1] for i in range(n - 1))
    assert all(p >= 1 for p in prompt) and all(r >= 0 for r in reply)
    paged = scheme == PAGED
    if paged:
        mem = BlockAllocatorModel(capacity // param, param)
    else:
        mem = ContiguousReservationModel(capacity, param)
    st = dict(steps=0, used_slot_steps=0, held_slot_steps=0, peak_used=0, peak_held=0, max_request_waste=0,
              admitted=0, rejected=0, dropped=0, peak_live=0)
    live = []  # request ids holding memory, in admission order
    generated: Dict[int, int] = {}
    done: Dict[int, bool] = {}
    fresh: Dict[int, bool] = {}
    nxt, t = 0, 0
    while nxt < n or live:
        if not live and arrival[nxt] > t:
            t = arrival[nxt]
        # release what completed at the previous step
        for r in [r for r in live if done[r]]:
            if paged:
                mem.free_seq(r)
            else:
                mem.release(r)
            live.remove(r)
        # arrivals
        while nxt < n and arrival[nxt] == t:
            r = nxt
            nxt += 1
            if paged:
                mem.add_seq(r)
                try:
                    mem.append(r, prompt[r])
                    ok = True
                except OutOfBlocks:
                    mem.free_seq(r)
                    ok = False
            else:
                ok = reply[r] <= param and mem.admit(r, prompt[r] + param)
                if ok:
                    mem.grow(r, prompt[r])
            if not ok:
                st["rejected"] += 1
                continue
            st["admitted"] += 1
            live.append(r)
            generated[r] = 0
            done[r] = reply[r] == 0
            fresh[r] = True
        # one decode step
        for r in list(live):
            if fresh[r] or done[r]:
                fresh[r] = False
                continue
            if paged:
                try:
                    mem.append(r, 1)
                except OutOfBlocks:
                    st["dropped"] += 1
                    mem.free_seq(r)
                    live.remove(r)
                    continue
            else:
                mem.grow(r, 1)
            generated[r] += 1
            done[r] = generated[r] == reply[r]
        # accounting
        if paged:  # nothing is shared here: a request holds its table's blocks and stores lens tokens
            held = [len(mem.tables[r]) * param for r in live]
            used = [mem.lens[r] for r in live]
        else:
            held = [mem.held_slots(r) for r in live]
            used = [mem.used_slots(r) for r in live]
        st["steps"] = t + 1
        st["used_slot_steps"] += sum(used)
        st["held_slot_steps"] += sum(held)
        st["peak_used"] = max(st["peak_used"], sum(used))
        st["peak_held"] = max(st["peak_held"], sum(held))
        st["peak_live"] = max(st["peak_live"], len(live))
        st["max_request_waste"] = max([st["max_request_waste"]] + [h - u for h, u in zip(held, used)])
        t += 1
    return st


def waste_fraction(st: Dict[str, int]) -> float:
    """Share of the held slot-steps that held no token."""
    return 1.0 - st["used_slot_steps"] / st["held_slot_steps"] if st["held_slot_steps"] else 0.0
