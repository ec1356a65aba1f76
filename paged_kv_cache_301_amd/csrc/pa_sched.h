// pa_sched.h -- work-group -> (sequence, kv head, partition) mapping.
//
// Contexts are ragged, so most (sequence, kv head, partition) slots of a
// rectangular grid are past their sequence's end.  If such empty
// work-groups are interleaved with real ones, the dispatcher spends its time
// launching and retiring them while CUs wait for real work (measured: on a
// log-uniform length mix the number of live waves sagged from 2048 to ~1200
// in the middle of the launch).  Instead, every work-group decodes its own
// index into the list of *live* items, ordered partition-major
//     row p = all (sequence, kv head) pairs whose context reaches partition p,
//             kv head fastest,
// so all live items are dispatched first and the surplus work-groups (the
// grid is sized for the worst case) are at the end and exit at once.  Within
// a row, consecutive items are different kv heads of the same sequence and
// (with the dispatcher dealing work-groups round-robin to the 8 XCDs) the
// same (kv head, partition) of different sequences shares an XCD, so a
// prompt prefix shared by the batch is read from that XCD's L2.
//
// The decode is done by one wave from the context lengths alone: every lane
// keeps the partition counts of up to kSchedMaxSeqs / 64 sequences in
// registers, the row is found by a binary search over partition indices and
// the sequence within the row with ballots.  A sequence of length 0 counts as
// one item (its output row must be written as zeros).
#pragma once

#include "pa_device.h"

namespace pa {

constexpr int kSchedMaxSeqs = 1024;
constexpr int kSchedChunks = kSchedMaxSeqs / 64;

struct WorkItem {
    int s, kvh, p;
    bool valid;
};

// Sum of an int over the 64 lanes (DPP within rows of 16, then the four row
// totals through scalar registers); every lane gets the total.
__device__ __forceinline__ int wave_sum_int(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
    x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);  // row_mirror
    return __builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16) +
           __builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48);
}

// Item `item` of the partition-major live list.  Rows shrink with p, so the
// number of items before row p, Hkv * sum_s min(np_s, p), is monotonic in p
// and the row is found by binary search; the sequence is then the
// rank-th one (in order) whose context reaches partition p.
__device__ __forceinline__ WorkItem decode_work_item(const int32_t *seq_lens, int S, int Hkv,
                                                     int part_tokens, int max_parts,
                                                     long long item) {
    const int lane = threadIdx.x & 63;
    int np[kSchedChunks];
#pragma unroll
    for (int c = 0; c < kSchedChunks; ++c) {
        const int s = 64 * c + lane;
        int n = 0;
        if (s < S) {
            const int L = seq_lens[s];
            n = L > 0 ? (L + part_tokens - 1) / part_tokens : 1;
        }
        np[c] = n;
    }
    const int nchunks = (S + 63) >> 6;
    auto items_before_row = [&](int p) -> long long {
        int acc = 0;
#pragma unroll
        for (int c = 0; c < kSchedChunks; ++c)
            if (c < nchunks) acc += min(np[c], p);
        return (long long)Hkv * wave_sum_int(acc);
    };
    if (item >= items_before_row(max_parts)) return WorkItem{0, 0, 0, false};
    int lo = 0, hi = max_parts - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (items_before_row(mid) <= item) lo = mid;
        else hi = mid - 1;
    }
    const int p = lo;
    const long long idx = item - items_before_row(p);
    int rank = (int)(idx / Hkv);
    const int kvh = (int)(idx % Hkv);
#pragma unroll
    for (int c = 0; c < kSchedChunks; ++c) {
        if (c < nchunks) {
            const unsigned long long m = __ballot(np[c] > p);
            const int k = __popcll(m);
            if (rank < k) {
                // the lane whose predicate is set with `rank` set lanes below it
                const unsigned below = __builtin_amdgcn_mbcnt_hi(
                    (unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
                const unsigned long long hm = __ballot((np[c] > p) && (int)below == rank);
                return WorkItem{64 * c + __ffsll((long long)hm) - 1, kvh, p, true};
            }
            rank -= k;
        }
    }
    return WorkItem{0, 0, 0, false};
}

}  // namespace pa
