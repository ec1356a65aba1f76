// pa_sched.h -- work-group -> (sequence, kv head, partition) mapping.
//
// Contexts are ragged, so most (sequence, kv head, partition) slots of a
// rectangular grid are past their sequence's end.  If such empty
// work-groups are interleaved with real ones, the dispatcher spends its time
// launching and retiring them while CUs wait for real work (measured: on a
// log-uniform length mix the number of live waves sagged from 2048 to ~1200
// in the middle of the launch).  Instead, every work-group decodes its own
// index into the list of *live* items, so all live items are dispatched first
// and the surplus work-groups (the grid is sized for the worst case) are at
// the end and exit at once.  The list is ordered longest first, so the last
// items to start are the shortest and the launch ends evenly:
//   1. every full partition (exactly P tokens), partition-major:
//        row p = all (sequence, kv head) pairs with more than p full
//        partitions, kv head fastest;
//   2. then each sequence's last, partly filled partition (and the single
//      empty item of a zero-length sequence), by decreasing token count, ties
//      by sequence index, kv head fastest.
// Within a row of part 1, consecutive items are different kv heads of the
// same sequence and (with the dispatcher dealing work-groups round-robin to
// the 8 XCDs) the same (kv head, partition) of different sequences shares an
// XCD, so a prompt prefix shared by the batch is read from that XCD's L2.
//
// The decode is done by one wave from the context lengths alone: every lane
// keeps the counts of up to kSchedMaxSeqs / 64 sequences in registers; a row
// of part 1 is found by a binary search over partition indices, a rank of
// part 2 by a binary search over token counts, and the sequence with ballots.
#pragma once

#include "pa_args.h"
#include "pa_device.h"

namespace pa {

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

// The sequence holding the rank-th set predicate (in lane / chunk order).
__device__ __forceinline__ int select_rank(const bool (&pred)[kSchedChunks], int nchunks, int rank) {
#pragma unroll
    for (int c = 0; c < kSchedChunks; ++c) {
        if (c < nchunks) {
            const unsigned long long m = __ballot(pred[c]);
            const int k = __popcll(m);
            if (rank < k) {
                // the lane whose predicate is set with `rank` set lanes below it
                const unsigned below = __builtin_amdgcn_mbcnt_hi(
                    (unsigned)(m >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)m, 0u));
                const unsigned long long hm = __ballot(pred[c] && (int)below == rank);
                return 64 * c + __ffsll((long long)hm) - 1;
            }
            rank -= k;
        }
    }
    return -1;
}

// Item `item` of the live list (order above).
__device__ __forceinline__ WorkItem decode_work_item(const int32_t *seq_lens, int S, int Hkv,
                                                     int part_tokens, int max_parts,
                                                     long long item) {
    const int lane = threadIdx.x & 63;
    int nf[kSchedChunks];    // full partitions
    int key[kSchedChunks];   // tokens of the last partial partition; 0: empty sequence; -1: none
#pragma unroll
    for (int c = 0; c < kSchedChunks; ++c) {
        const int s = 64 * c + lane;
        int f = 0, k = -1;
        if (s < S) {
            const int L = seq_lens[s];
            f = L / part_tokens;
            const int r = L - f * part_tokens;
            k = (r > 0 || L == 0) ? r : -1;
        }
        nf[c] = f;
        key[c] = k;
    }
    const int nchunks = (S + 63) >> 6;
    auto full_before_row = [&](int p) -> long long {
        int acc = 0;
#pragma unroll
        for (int c = 0; c < kSchedChunks; ++c)
            if (c < nchunks) acc += min(nf[c], p);
        return (long long)Hkv * wave_sum_int(acc);
    };
    auto count_key_at_least = [&](int v) -> int {
        int acc = 0;
#pragma unroll
        for (int c = 0; c < kSchedChunks; ++c)
            if (c < nchunks) acc += key[c] >= v ? 1 : 0;
        return wave_sum_int(acc);
    };
    const long long n_full = full_before_row(max_parts);
    if (item < n_full) {
        int lo = 0, hi = max_parts - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (full_before_row(mid) <= item) lo = mid;
            else hi = mid - 1;
        }
        const int p = lo;
        const long long idx = item - full_before_row(p);
        bool pred[kSchedChunks];
#pragma unroll
        for (int c = 0; c < kSchedChunks; ++c) pred[c] = nf[c] > p;
        const int s = select_rank(pred, nchunks, (int)(idx / Hkv));
        return WorkItem{s, (int)(idx % Hkv), p, s >= 0};
    }
    const long long idx = item - n_full;
    const int rank = (int)(idx / Hkv);
    if (idx >= (long long)Hkv * count_key_at_least(0)) return WorkItem{0, 0, 0, false};
    // largest v with more than `rank` keys >= v: the key of the rank-th item
    int lo = 0, hi = part_tokens - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (count_key_at_least(mid) > rank) lo = mid;
        else hi = mid - 1;
    }
    const int v = lo;
    const int before = lo + 1 < part_tokens ? count_key_at_least(lo + 1) : 0;
    bool pred[kSchedChunks];
#pragma unroll
    for (int c = 0; c < kSchedChunks; ++c) pred[c] = key[c] == v;
    const int s = select_rank(pred, nchunks, rank - before);
    if (s < 0) return WorkItem{0, 0, 0, false};
    const int L = seq_lens[s];
    return WorkItem{s, (int)(idx % Hkv), L / part_tokens, true};
}

// The sequence that comes rank-th in decreasing length order (ties by
// index; a bijection of [0, S)), found by one wave from the lengths alone,
// as the second part of the live list above: the largest length v with more
// than `rank` sequences at least that long, then the sequence among those of
// length exactly v.  S <= kSchedMaxSeqs; lengths in [0, max_len].
__device__ __forceinline__ int sequence_by_length(const int32_t *seq_lens, int S, int max_len,
                                                  int rank) {
    const int lane = threadIdx.x & 63;
    int key[kSchedChunks];
#pragma unroll
    for (int c = 0; c < kSchedChunks; ++c) {
        const int s = 64 * c + lane;
        key[c] = s < S ? seq_lens[s] : -1;
    }
    const int nchunks = (S + 63) >> 6;
    auto count_at_least = [&](int v) -> int {
        int acc = 0;
#pragma unroll
        for (int c = 0; c < kSchedChunks; ++c)
            if (c < nchunks) acc += key[c] >= v ? 1 : 0;
        return wave_sum_int(acc);
    };
    int lo = 0, hi = max_len;
    while (lo < hi) {
        const int mid = lo + ((hi - lo + 1) >> 1);
        if (count_at_least(mid) > rank) lo = mid;
        else hi = mid - 1;
    }
    const int before = lo < max_len ? count_at_least(lo + 1) : 0;
    bool pred[kSchedChunks];
#pragma unroll
    for (int c = 0; c < kSchedChunks; ++c) pred[c] = key[c] == lo;
    return select_rank(pred, nchunks, rank - before);
}

}  // namespace pa
