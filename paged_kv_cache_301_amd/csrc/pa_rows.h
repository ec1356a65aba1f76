// pa_rows.h -- query rows of a multi-token (causal) call.
//
// Sequence s holds n_s = query_start[s+1] - query_start[s] new tokens, the
// last n_s of its L_s = seq_lens[s] context tokens (their K / V are already in
// the cache).  Its query row query_start[s] + k sits at position L_s - n_s + k
// and attends tokens 0 .. L_s - n_s + k: the causal form of the blockwise
// attention equation (glossary "PagedAttention", section "How It Works": query
// i reads logical blocks 1 .. ceil(i / B), the last of them up to i itself).
#pragma once

#include "pa_internal.h"

namespace pa {

struct QueryRow {
    int s;     // sequence
    int lim;   // tokens the row attends: position + 1
};

// Sequence of query row r (binary search over query_start) and its limit.
__device__ __forceinline__ QueryRow query_row(const Args &a, int r) {
    int lo = 0, hi = a.S - 1;            // largest s with query_start[s] <= r
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.query_start[mid] <= r) lo = mid;
        else hi = mid - 1;
    }
    const int n = a.query_start[lo + 1] - a.query_start[lo];
    return {lo, a.seq_lens[lo] - n + (r - a.query_start[lo]) + 1};
}

}  // namespace pa
