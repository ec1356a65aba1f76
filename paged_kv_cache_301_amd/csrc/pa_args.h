// pa_args.h -- the argument block every kernel receives and the constants
// the host plan and the kernels share.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

namespace pa {

// Everything one launch needs, passed to kernels by value (kernarg segment).
struct Args {
    const void *query;        // [S][Hq][D]
    const void *key_cache;    // [NB][Hkv][B][D]
    const void *value_cache;  // [NB][Hkv][B][D]
    const int32_t *block_tables;  // [S][max_blocks]
    const int32_t *seq_lens;      // [S]
    void *out;                // [S][Hq][D] (out dtype)
    float *part_o;            // [S][Hq][max_parts][D]   split plans only
    float *part_m;            // [S][Hq][max_parts]      running max, log2 units
    float *part_l;            // [S][Hq][max_parts]      sum of weights
    float scale_log2;         // scale * log2(e): scores live in exp2 units
    int S, Hq, Hkv, D, B, NB, max_blocks;
    int log2B;                // log2(B) when B is a power of two, else -1
    int part_tokens;          // tokens per context partition
    int max_parts;            // partitions per (s, head) in the grid
    int split;                // 1: write partials, 0: write final output
    int stream_kv;            // 1: K / V loads carry the non-temporal hint
    int compact;              // 1: 1-D grid decoded into live items (pa_sched.h)
    int token_waves;          // waves sharing an item's tokens (1, 2 or 4): the VALU
                              // kernel and the matrix-core kernel's one-wave groups
    // Multi-token (causal) calls only; query_start is null for decode.
    const int32_t *query_start;   // [S+1] rows query_start[s] .. query_start[s+1]-1 are sequence s's
    int T;                        // query rows; query / out are [T][Hq][D]
    int q_blocks;                 // query blocks per sequence in the grid
    int prefill_columns;          // (query token, head) columns per work-group
    int by_length;                // 1: (sequence, kv head) pairs in decreasing length
};

// Tokens one loop iteration of the tiled kernels covers; partitions are
// multiples of this.
constexpr int kTileTokens = 32;

// Partitions per (sequence, head): the partition index is grid dimension y.
constexpr int kMaxPartitions = 65535;

// Entries of a partition's block-table slice the tiled kernels copy to LDS
// (blocks of fewer than 4 tokens); the host caps such partitions at
// kTableLds * B tokens.
constexpr int kTableLds = 1024;

// Largest batch whose lengths one wave holds in registers for the live-item
// decode of the tiled decode kernels (pa_sched.h); larger batches use the
// rectangular grid.
constexpr int kSchedMaxSeqs = 1024;

// (query token, head) columns per work-group of the multi-token matrix-core
// kernel: four waves of two 16-column groups; two waves when every
// sequence's rows fit 64 columns (G * max_query_len <= 64), eight when the
// longest chunk fills 256 (G * max_query_len >= 256).
constexpr int kPrefillColumns = 128;
constexpr int kPrefillColumnsNarrow = 64;
constexpr int kPrefillColumnsWide = 256;

// Threads per work-group of the K / V write and block-copy kernels, and
// bytes of one block one copy work-group moves.
constexpr int kKvThreads = 256;
constexpr int kCopyPieceBytes = kKvThreads * 16 * 2;

}  // namespace pa
