// Host block allocator behind pa_alloc_* (see include/pa.h).
//
// The pool of fixed-size physical blocks, per-request block tables,
// reference-counted sharing after a fork and copy-on-write of a shared,
// partially filled last block ("Paged attention in LLMs": "The fix",
// "Keeping track: the block table", "Sharing blocks"; PagedAttention MCQ
// page: comparison table, copy on write for beam search / best of N).
//
// Pure host C++: no HIP calls, so it runs (and is tested) without a GPU.
// The free pool is a FIFO ring so that block placement is deterministic
// for a given initial order; freed blocks join the tail.

#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pa.h"

struct pa_allocator {
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::deque<int32_t> free_q;
    std::vector<int32_t> ref;
    struct Seq {
        std::vector<int32_t> table;
        int64_t len = 0;
    };
    std::unordered_map<int64_t, Seq> seqs;
};

extern "C" const char* pa_status_string(pa_status s) {
    switch (s) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID_ARG: return "invalid argument";
        case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case PA_ERR_OOM: return "out of free blocks";
        case PA_ERR_NOT_FOUND: return "unknown sequence";
        case PA_ERR_LAUNCH: return "kernel launch failed";
        case PA_ERR_EXISTS: return "sequence already exists";
    }
    return "unknown status";
}

extern "C" pa_allocator* pa_alloc_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
    if (num_blocks < 0 || block_size <= 0) return nullptr;
    pa_allocator* a = new (std::nothrow) pa_allocator();
    if (!a) return nullptr;
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->ref.assign(num_blocks, 0);
    if (free_order) {
        std::vector<char> seen(num_blocks, 0);
        for (int32_t i = 0; i < num_blocks; ++i) {
            int32_t b = free_order[i];
            if (b < 0 || b >= num_blocks || seen[b]) {
                delete a;
                return nullptr;
            }
            seen[b] = 1;
            a->free_q.push_back(b);
        }
    } else {
        for (int32_t i = 0; i < num_blocks; ++i) a->free_q.push_back(i);
    }
    return a;
}

extern "C" void pa_alloc_destroy(pa_allocator* a) { delete a; }

extern "C" pa_status pa_alloc_add_seq(pa_allocator* a, int64_t seq) {
    if (!a) return PA_ERR_INVALID_ARG;
    if (a->seqs.count(seq)) return PA_ERR_EXISTS;
    a->seqs.emplace(seq, pa_allocator::Seq{});
    return PA_OK;
}

// Fresh blocks an append of n tokens will pop: one for the copy of a shared
// partial tail (if any), plus one per position that starts a new block.
static int64_t blocks_needed(const pa_allocator* a, const pa_allocator::Seq& s, int64_t n) {
    if (n <= 0) return 0;
    const int64_t bs = a->block_size;
    int64_t need = 0;
    if (s.len % bs != 0 && a->ref[s.table.back()] > 1) need += 1;
    const int64_t held = (s.len + bs - 1) / bs;        // blocks the table already has
    const int64_t last = (s.len + n - 1) / bs;         // logical block of the last new token
    if (last >= held) need += last - held + 1;
    return need;
}

extern "C" pa_status pa_alloc_append(pa_allocator* a, int64_t seq, int32_t n_tokens, int64_t* slots_out,
                                     int32_t* cow_pairs_out, int32_t cow_cap, int32_t* n_cow) {
    if (!a || n_tokens < 0 || (n_tokens > 0 && !slots_out) || !n_cow) return PA_ERR_INVALID_ARG;
    if (cow_cap > 0 && !cow_pairs_out) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
    pa_allocator::Seq& s = it->second;
    if (blocks_needed(a, s, n_tokens) > static_cast<int64_t>(a->free_q.size())) return PA_ERR_OOM;
    // a copy can only happen on the first token, so one pair of room is enough
    if (n_tokens > 0 && s.len % a->block_size != 0 && a->ref[s.table.back()] > 1 && cow_cap < 1)
        return PA_ERR_INVALID_ARG;
    const int64_t bs = a->block_size;
    int32_t copies = 0;
    for (int32_t i = 0; i < n_tokens; ++i) {
        const int64_t pos = s.len;
        if (pos % bs == 0) {
            int32_t b = a->free_q.front();
            a->free_q.pop_front();
            a->ref[b] = 1;
            s.table.push_back(b);
        } else if (a->ref[s.table.back()] > 1) {
            int32_t src = s.table.back();
            int32_t dst = a->free_q.front();
            a->free_q.pop_front();
            a->ref[src] -= 1;
            a->ref[dst] = 1;
            s.table.back() = dst;
            cow_pairs_out[2 * copies] = src;
            cow_pairs_out[2 * copies + 1] = dst;
            ++copies;
        }
        slots_out[i] = static_cast<int64_t>(s.table[pos / bs]) * bs + pos % bs;
        s.len = pos + 1;
    }
    *n_cow = copies;
    return PA_OK;
}

extern "C" pa_status pa_alloc_fork(pa_allocator* a, int64_t parent, int64_t child) {
    if (!a) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(parent);
    if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
    if (a->seqs.count(child)) return PA_ERR_EXISTS;
    pa_allocator::Seq copy = it->second;
    for (int32_t b : copy.table) a->ref[b] += 1;
    a->seqs.emplace(child, std::move(copy));
    return PA_OK;
}

extern "C" pa_status pa_alloc_free(pa_allocator* a, int64_t seq) {
    if (!a) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
    for (int32_t b : it->second.table) {
        if (--a->ref[b] == 0) a->free_q.push_back(b);
    }
    a->seqs.erase(it);
    return PA_OK;
}

extern "C" pa_status pa_alloc_table(const pa_allocator* a, int64_t seq, int32_t* out, int32_t cap,
                                    int32_t* n_blocks, int32_t* seq_len) {
    if (!a || cap < 0 || (cap > 0 && !out) || !n_blocks || !seq_len) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
    const auto& t = it->second.table;
    const int32_t n = static_cast<int32_t>(t.size());
    for (int32_t i = 0; i < n && i < cap; ++i) out[i] = t[i];
    *n_blocks = n;
    *seq_len = static_cast<int32_t>(it->second.len);
    return PA_OK;
}

extern "C" pa_status pa_alloc_batch_tables(const pa_allocator* a, const int64_t* seqs, int32_t n_seqs,
                                           int32_t* tables_out, int32_t width, int32_t pad,
                                           int32_t* seq_lens_out) {
    if (!a || n_seqs < 0 || width < 0 || (n_seqs > 0 && (!seqs || !seq_lens_out)) ||
        (n_seqs > 0 && width > 0 && !tables_out))
        return PA_ERR_INVALID_ARG;
    for (int32_t i = 0; i < n_seqs; ++i) {
        auto it = a->seqs.find(seqs[i]);
        if (it == a->seqs.end()) return PA_ERR_NOT_FOUND;
        if (static_cast<int64_t>(it->second.table.size()) > width) return PA_ERR_INVALID_ARG;
    }
    for (int32_t i = 0; i < n_seqs; ++i) {
        const auto& s = a->seqs.find(seqs[i])->second;
        int32_t* row = tables_out + static_cast<int64_t>(i) * width;
        const int32_t n = static_cast<int32_t>(s.table.size());
        for (int32_t j = 0; j < width; ++j) row[j] = j < n ? s.table[j] : pad;
        seq_lens_out[i] = static_cast<int32_t>(s.len);
    }
    return PA_OK;
}

extern "C" int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block) {
    if (!a || block < 0 || block >= a->num_blocks) return -1;
    return a->ref[block];
}

extern "C" pa_status pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n) {
    if (!a || cap < 0 || (cap > 0 && !out) || !n) return PA_ERR_INVALID_ARG;
    int32_t i = 0;
    for (int32_t b : a->free_q) {
        if (i < cap) out[i] = b;
        ++i;
    }
    *n = i;
    return PA_OK;
}

extern "C" int32_t pa_alloc_num_free(const pa_allocator* a) {
    return a ? static_cast<int32_t>(a->free_q.size()) : -1;
}

// Move sequences between two allocators (device pool <-> host pool for
// preemption by swapping; the MCQ page lists preemption among the things
// paging makes easy).  Every distinct block the moved sequences hold in
// `from` gets one fresh block in `to`, in order of first appearance (the
// sequences in the given order, each table from logical block 0), so
// sharing among the moved sequences is kept; the pairs (from block, to
// block) are what the caller copies.  In `from` the moved sequences are
// freed as pa_alloc_free would, in the given order: a block also held by a
// sequence that stays keeps its data there.
extern "C" pa_status pa_alloc_move(pa_allocator* from, pa_allocator* to, const int64_t* seqs, int32_t n_seqs,
                                   int32_t* pairs_out, int32_t cap, int32_t* n_pairs) {
    if (!from || !to || from == to || n_seqs < 0 || cap < 0 || !n_pairs || (n_seqs > 0 && !seqs) ||
        (cap > 0 && !pairs_out))
        return PA_ERR_INVALID_ARG;
    if (from->block_size != to->block_size) return PA_ERR_INVALID_ARG;
    std::unordered_map<int64_t, int> seen_seq;
    std::unordered_map<int32_t, int32_t> map;  // from block -> index of first appearance
    std::vector<int32_t> order;
    for (int32_t i = 0; i < n_seqs; ++i) {
        if (seen_seq.count(seqs[i])) return PA_ERR_INVALID_ARG;  // a sequence listed twice
        seen_seq[seqs[i]] = 1;
        auto it = from->seqs.find(seqs[i]);
        if (it == from->seqs.end()) return PA_ERR_NOT_FOUND;
        if (to->seqs.count(seqs[i])) return PA_ERR_EXISTS;
        for (int32_t b : it->second.table) {
            if (!map.count(b)) {
                map[b] = static_cast<int32_t>(order.size());
                order.push_back(b);
            }
        }
    }
    const int64_t need = static_cast<int64_t>(order.size());
    if (need > cap) {
        *n_pairs = static_cast<int32_t>(need);  // the room the pairs need; nothing changed
        return PA_ERR_INVALID_ARG;
    }
    if (need > static_cast<int64_t>(to->free_q.size())) return PA_ERR_OOM;
    // destination blocks, one per distinct source block
    std::vector<int32_t> dst(order.size());
    for (size_t k = 0; k < order.size(); ++k) {
        dst[k] = to->free_q.front();
        to->free_q.pop_front();
        to->ref[dst[k]] = 0;
        pairs_out[2 * k] = order[k];
        pairs_out[2 * k + 1] = dst[k];
    }
    for (int32_t i = 0; i < n_seqs; ++i) {
        auto it = from->seqs.find(seqs[i]);
        pa_allocator::Seq moved;
        moved.len = it->second.len;
        moved.table.reserve(it->second.table.size());
        for (int32_t b : it->second.table) {
            const int32_t d = dst[map[b]];
            to->ref[d] += 1;
            moved.table.push_back(d);
        }
        to->seqs.emplace(seqs[i], std::move(moved));
        for (int32_t b : it->second.table) {
            if (--from->ref[b] == 0) from->free_q.push_back(b);
        }
        from->seqs.erase(it);
    }
    *n_pairs = static_cast<int32_t>(order.size());
    return PA_OK;
}
