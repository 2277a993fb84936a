// mk_capacity.h -- the largest batch a workspace of a given size serves (host code only).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mk_common.h"

namespace mk {

// Bytes of workspace a forward of B tokens needs (B = 0 is sized like B = 1).
inline size_t workspace_bytes_for(const Shape &s, int64_t B) {
    if (B < 1) B = 1;
    return make_layout(s, B).total;
}

// Largest B whose requirement fits in ws_bytes (0 when even B = 1 does not fit), by
// bisection over the monotone requirement.  Nothing shared is written: the last lookup is
// remembered per host thread, keyed by the plan's process-unique id and the size, so
// forwards on one plan from several threads never read each other's entries.
inline int64_t workspace_capacity(const Shape &s, uint64_t plan_id, size_t ws_bytes) {
    struct Entry {
        uint64_t id;
        size_t bytes;
        int64_t cap;
    };
    thread_local Entry last{0, 0, 0};
    if (plan_id != 0 && last.id == plan_id && last.bytes == ws_bytes) return last.cap;
    int64_t lo = 0, hi = ((int64_t)1 << 31) / s.k;  // B*k < 2^31
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo + 1) / 2;
        if (workspace_bytes_for(s, mid) <= ws_bytes)
            lo = mid;
        else
            hi = mid - 1;
    }
    last = Entry{plan_id, ws_bytes, lo};
    return lo;
}

}  // namespace mk
