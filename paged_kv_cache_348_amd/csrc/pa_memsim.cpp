// KV-memory accounting of a request trace under the two schemes the pages
// compare (pa_simulate_memory in include/pa.h).
//
//  - contiguous: each request reserves its prompt plus the largest reply it
//    may produce in one unbroken run of slots, placed first fit; space inside
//    a reservation that the reply never reaches, and free gaps too small for
//    the next reservation, are both lost ("Paged attention in LLMs", "Why the
//    memory gets wasted"; MCQ page, comparison table, "Memory waste" row);
//  - paged: a request holds whole blocks, taken one at a time as it grows
//    from any free place, so it loses at most the unfilled tail of its last
//    block ("Paged attention in LLMs", "The fix", "Why this helps so much").
//
// Time runs in decode steps.  At step t: requests that completed their reply
// at step t - 1 release their memory; requests arriving at t are admitted in
// trace order (their prompt is stored at once) or rejected if they do not fit;
// then every request admitted before t appends one reply token (a paged
// request that needs a block when none is free is dropped and releases its
// memory); a request whose reply is complete is marked to release at t + 1.
// After each step the held and used slots are added up.
//
// Pure host C++, no HIP calls.

#include <algorithm>
#include <cstdint>
#include <map>
#include <vector>

#include "pa.h"

namespace {

struct Req {
    int32_t id;
    int64_t start = 0;  // contiguous: run start
    int64_t run = 0;    // contiguous: run length
    int64_t blocks = 0; // paged: blocks held
    int64_t len = 0;    // tokens stored
    int32_t generated = 0;
    bool done = false;
    bool fresh = true;  // admitted this step: generates from the next step on
};

// First-fit placement in [0, capacity) given the runs in use (start -> length).
bool first_fit(const std::map<int64_t, int64_t>& runs, int64_t capacity, int64_t need, int64_t* at) {
    int64_t cur = 0;
    for (const auto& r : runs) {
        if (r.first - cur >= need) {
            *at = cur;
            return true;
        }
        cur = std::max(cur, r.first + r.second);
    }
    if (capacity - cur >= need) {
        *at = cur;
        return true;
    }
    return false;
}

}  // namespace

extern "C" pa_status pa_simulate_memory(const int32_t* arrival_step, const int32_t* prompt_len,
                                        const int32_t* reply_len, int32_t num_requests, int64_t capacity_slots,
                                        int32_t scheme, int32_t param, pa_mem_stats* out) {
    if (!out || num_requests < 0 || capacity_slots < 0 || param < 0) return PA_ERR_INVALID_ARG;
    if (scheme != PA_MEM_CONTIGUOUS && scheme != PA_MEM_PAGED) return PA_ERR_INVALID_ARG;
    if (scheme == PA_MEM_PAGED && param < 1) return PA_ERR_INVALID_ARG;
    if (num_requests > 0 && (!arrival_step || !prompt_len || !reply_len)) return PA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < num_requests; ++i) {
        if (arrival_step[i] < 0 || prompt_len[i] < 1 || reply_len[i] < 0) return PA_ERR_INVALID_ARG;
        if (i > 0 && arrival_step[i] < arrival_step[i - 1]) return PA_ERR_INVALID_ARG;  // trace order
    }
    *out = pa_mem_stats{};
    const bool paged = scheme == PA_MEM_PAGED;
    const int64_t bs = paged ? param : 1;
    const int64_t nblocks = paged ? capacity_slots / bs : 0;
    int64_t free_blocks = nblocks;
    std::map<int64_t, int64_t> runs;  // contiguous runs in use
    std::vector<Req> live;
    int32_t next = 0;
    for (int64_t t = 0; next < num_requests || !live.empty(); ++t) {
        if (live.empty() && arrival_step[next] > t) t = arrival_step[next];  // idle until the next arrival
        // 1. release the requests that completed at the previous step
        std::vector<Req> keep;
        keep.reserve(live.size());
        for (const Req& r : live) {
            if (!r.done) {
                keep.push_back(r);
                continue;
            }
            if (paged)
                free_blocks += r.blocks;
            else
                runs.erase(r.start);
        }
        live.swap(keep);
        // 2. arrivals, in trace order
        while (next < num_requests && arrival_step[next] == t) {
            const int32_t i = next++;
            Req r;
            r.id = i;
            r.len = prompt_len[i];
            bool ok;
            if (paged) {
                const int64_t need = (r.len + bs - 1) / bs;
                ok = need <= free_blocks;
                if (ok) {
                    free_blocks -= need;
                    r.blocks = need;
                }
            } else {
                const int64_t need = (int64_t)prompt_len[i] + param;
                ok = reply_len[i] <= param && first_fit(runs, capacity_slots, need, &r.start);
                if (ok) {
                    r.run = need;
                    runs[r.start] = need;
                }
            }
            if (!ok) {
                ++out->rejected;
                continue;
            }
            ++out->admitted;
            r.done = reply_len[i] == 0;
            live.push_back(r);
        }
        // 3. one decode step for every request admitted before this step
        keep.clear();
        for (Req& r : live) {
            if (r.fresh || r.done) {
                r.fresh = false;
                keep.push_back(r);
                continue;
            }
            if (paged && r.len == r.blocks * bs) {
                if (free_blocks == 0) {
                    ++out->dropped;
                    free_blocks += r.blocks;
                    continue;
                }
                --free_blocks;
                ++r.blocks;
            }
            ++r.len;
            ++r.generated;
            r.done = r.generated == reply_len[r.id];
            keep.push_back(r);
        }
        live.swap(keep);
        // 4. accounting
        int64_t used = 0, held = 0, tail = 0;
        for (const Req& r : live) {
            const int64_t h = paged ? r.blocks * bs : r.run;
            used += r.len;
            held += h;
            tail = std::max(tail, h - r.len);
        }
        out->steps = t + 1;
        out->used_slot_steps += used;
        out->held_slot_steps += held;
        out->peak_used = std::max(out->peak_used, used);
        out->peak_held = std::max(out->peak_held, held);
        out->peak_live = std::max<int32_t>(out->peak_live, (int32_t)live.size());
        out->max_request_waste = std::max(out->max_request_waste, tail);
    }
    return PA_OK;
}
