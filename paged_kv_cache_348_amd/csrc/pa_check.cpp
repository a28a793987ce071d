// Host check of an append's slot mapping (pa_check_slots in include/pa.h).
//
// One call of the append writes each token to the slot its request's block
// table gives it ("Paged attention in LLMs", "The cache being stored"); the
// device kernels assume the slots of one call are distinct (two tokens on
// one slot race) and skip slots outside the pool.  This finds both before a
// launch.  Pure host C++, no HIP calls.

#include <algorithm>
#include <cstdint>
#include <utility>
#include <vector>

#include "pa.h"

extern "C" pa_status pa_check_slots(const int64_t* slot_mapping, int32_t num_tokens, int64_t num_slots,
                                    int32_t* first_bad) {
    if (first_bad) *first_bad = -1;
    if (num_tokens < 0 || num_slots < 0 || (num_tokens > 0 && !slot_mapping)) return PA_ERR_INVALID_ARG;
    int32_t bad = -1;
    std::vector<std::pair<int64_t, int32_t>> seen;  // (slot, index) of the in-pool entries
    seen.reserve((size_t)num_tokens);
    for (int32_t i = 0; i < num_tokens; ++i) {
        const int64_t s = slot_mapping[i];
        if (s < 0) continue;
        if (s >= num_slots) {
            if (bad < 0) bad = i;
            continue;
        }
        seen.emplace_back(s, i);
    }
    std::sort(seen.begin(), seen.end());
    // within a run of equal slots every index but the first is a repeat
    for (size_t k = 1; k < seen.size(); ++k)
        if (seen[k].first == seen[k - 1].first && (bad < 0 || seen[k].second < bad)) bad = seen[k].second;
    if (first_bad) *first_bad = bad;
    return bad < 0 ? PA_OK : PA_ERR_INVALID_ARG;
}
