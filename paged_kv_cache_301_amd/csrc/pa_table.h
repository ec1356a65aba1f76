// pa_table.h -- block-table translation for the tiled kernels.
//
// Logical token t of a sequence lives in physical block table[t / B] at slot
// t % B ("Paged Attention > The PagedAttention Algorithm", opening section:
// logical block number and within-block offset, then the table lookup; the
// glossary page "PagedAttention", section "How It Works").  With B a power of
// two the division and remainder are a shift and a mask.
//
// Two ways to reach the table entry:
//  * SCALAR (B a multiple of the tokens one load instruction covers): every
//    lane of the instruction is in one block, so the index is wave-uniform and
//    the entry comes through the scalar cache.  Scalar loads count on lgkmcnt,
//    so they never wait behind the wave's outstanding K / V loads.
//  * LDS (smaller B): the partition's slice of the table is copied to LDS once
//    (the first page's "shared memory for block table entries"), and each lane
//    reads its own entry from there -- again off the vmcnt queue.
#pragma once

#include "pa_args.h"
#include "pa_device.h"

namespace pa {


struct TableView {
    const int32_t *row;   // block_tables[s]
    int lb;               // log2(B)
    int j0;               // first logical block of the partition (LDS mode)
};

// Copy the logical blocks covering tokens [t_begin, t_end) into LDS (at most
// kTableLds entries, which the host's partition cap guarantees).  NLANES
// threads share the copy; each issues all of its loads before its first LDS
// write, so the copy costs one memory round trip, not one per entry it
// handles (a one-token-block partition of 1024 tokens is 16 entries per lane
// of a one-wave work-group).
template <int NLANES>
__device__ __forceinline__ void stage_table(int32_t *tbl, const TableView &tv,
                                            int t_begin, int t_end, int lane) {
    constexpr int kPer = (kTableLds + NLANES - 1) / NLANES;
    const int nj = ((t_end - 1) >> tv.lb) - tv.j0 + 1;
    int v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int idx = lane + u * NLANES;
        v[u] = idx < nj ? tv.row[tv.j0 + idx] : 0;
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
        const int idx = lane + u * NLANES;
        if (idx < nj) tbl[idx] = v[u];
    }
}

// Physical block of token t (t must be < the sequence length).
template <bool SCALAR>
__device__ __forceinline__ int phys_block(const TableView &tv, const int32_t *tbl, int t) {
    if constexpr (SCALAR) {
        const int j = __builtin_amdgcn_readfirstlane(t >> tv.lb);
        return __builtin_amdgcn_readfirstlane(tv.row[j]);
    } else {
        return tbl[(t >> tv.lb) - tv.j0];
    }
}

}  // namespace pa
