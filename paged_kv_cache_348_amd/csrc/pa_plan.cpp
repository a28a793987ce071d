// Host planning of the shared-prefix decode (pa_plan_shared_prefix in
// include/pa.h): which consecutive requests of a batch read the same leading
// physical blocks.
//
// Requests forked from one prompt keep pointing their tables at the prompt's
// blocks until they write into one ("Paged attention in LLMs", "Sharing
// blocks"; copy on write in the MCQ page's comparison table), so equal table
// entries mean equal keys and values.  The plan only compares table entries:
// it needs no allocator and works for any caller's tables.
//
// Pure host C++, no HIP calls.

#include <algorithm>
#include <cstdint>

#include "pa.h"

namespace {

// Leading entries two table rows have in common.
int32_t common_prefix(const int32_t* a, const int32_t* b, int32_t n) {
    int32_t k = 0;
    while (k < n && a[k] == b[k]) ++k;
    return k;
}

}  // namespace

extern "C" pa_status pa_plan_shared_prefix(const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                                           int32_t max_blocks_per_seq, int32_t block_size, int32_t max_group_size,
                                           int32_t min_shared_blocks, int32_t* groups, int32_t* prefix_blocks,
                                           int32_t* num_groups, int32_t* max_group, int32_t* max_prefix_blocks) {
    if (num_seqs < 0 || max_blocks_per_seq < 0 || block_size <= 0 || max_group_size < 1 || min_shared_blocks < 1)
        return PA_ERR_INVALID_ARG;
    if (!num_groups || !max_group || !max_prefix_blocks) return PA_ERR_INVALID_ARG;
    if (num_seqs > 0 && (!block_tables || !seq_lens || !groups || !prefix_blocks)) return PA_ERR_INVALID_ARG;
    const int64_t W = max_blocks_per_seq;
    // blocks of request b that lie wholly inside its first L_b tokens
    auto full_blocks = [&](int32_t b) -> int32_t {
        const int32_t L = seq_lens[b];
        if (L <= 0) return 0;
        return (int32_t)std::min<int64_t>(W, L / block_size);
    };
    int32_t ng = 0, mg = 1, mp = 0;
    int32_t s = 0;
    while (s < num_seqs) {
        prefix_blocks[s] = 0;
        // grow a group from s while the blocks every member reads once
        // more than necessary do not decrease: with n members sharing c
        // blocks, (n - 1) * c block reads are saved
        int32_t n = 1;
        int32_t c = full_blocks(s);
        while (s + n < num_seqs && n < max_group_size) {
            const int32_t t = s + n;
            const int32_t c2 = std::min({c, full_blocks(t),
                                        common_prefix(block_tables + (int64_t)s * W, block_tables + (int64_t)t * W,
                                                      (int32_t)W)});
            if (c2 < min_shared_blocks || (int64_t)n * c2 < (int64_t)(n - 1) * c) break;
            c = c2;
            ++n;
        }
        if (n >= 2) {
            groups[2 * ng] = s;
            groups[2 * ng + 1] = n;
            ++ng;
            for (int32_t i = 0; i < n; ++i) prefix_blocks[s + i] = c;
            mg = std::max(mg, n);
            mp = std::max(mp, c);
        } else {
            n = 1;
        }
        s += n;
    }
    *num_groups = ng;
    *max_group = mg;
    *max_prefix_blocks = mp;
    return PA_OK;
}
