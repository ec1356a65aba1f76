// pa_check.hip -- debug check of the device-data preconditions of a call.
//
// The attention kernels trust the caller's lengths and block tables (a
// context of L tokens reads table entries 0 .. ceil(L / B) - 1 and the
// physical blocks they name).  This pass verifies exactly those preconditions
// without touching the K / V pools: 0 <= L <= max_blocks * B and every used
// table entry in [0, NB).  It reads only entries j < min(ceil(L / B),
// max_blocks), so it is safe on any table.  report[0] receives the number of
// offending sequences, report[1] the smallest offending sequence index
// (INT32_MAX when none).
#include <climits>

#include "pa_internal.h"

namespace pa {

namespace {

__global__ __launch_bounds__(64) void check_init(int32_t *report) {
    if (threadIdx.x == 0) {
        report[0] = 0;
        report[1] = INT32_MAX;
    }
}

// one wave per sequence
__global__ __launch_bounds__(64) void check_kernel(const int32_t *block_tables,
                                                   const int32_t *seq_lens, int max_blocks, int B,
                                                   int NB, int32_t *report) {
    const int s = blockIdx.x;
    const int L = seq_lens[s];
    bool bad = L < 0 || (long long)L > (long long)max_blocks * B;
    if (!bad) {
        const int nb = (int)(((long long)L + B - 1) / B);
        const int32_t *row = block_tables + (size_t)s * max_blocks;
        for (int j = threadIdx.x; j < nb; j += 64) {
            const int p = row[j];
            if (p < 0 || p >= NB) bad = true;
        }
    }
    if (__ballot(bad) != 0 && threadIdx.x == 0) {
        atomicAdd(&report[0], 1);
        atomicMin(&report[1], s);
    }
}

}  // namespace

hipError_t launch_check(const int32_t *block_tables, const int32_t *seq_lens, int S,
                        int max_blocks, int B, int NB, int32_t *report, hipStream_t st) {
    hipLaunchKernelGGL(check_init, dim3(1), dim3(64), 0, st, report);
    if (S > 0)
        hipLaunchKernelGGL(check_kernel, dim3(S), dim3(64), 0, st, block_tables, seq_lens,
                           max_blocks, B, NB, report);
    return hipGetLastError();
}

}  // namespace pa
