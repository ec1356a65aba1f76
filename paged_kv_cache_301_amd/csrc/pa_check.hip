// pa_check.hip -- device check of the device-data preconditions of a call.
//
// The attention kernels trust the caller's lengths and block tables (a
// context of L tokens reads table entries 0 .. ceil(L / B) - 1 and the
// physical blocks they name).  This pass verifies exactly those preconditions
// without touching the K / V pools: 0 <= L <= max_blocks * B and every used
// table entry in [0, NB).  It reads only entries j < min(ceil(L / B),
// max_blocks), so it is safe on any table.  For a multi-token call it also
// checks query_start: query_start[0] = 0, query_start[S] = T, and every
// sequence's row count n_s = query_start[s+1] - query_start[s] within
// [0, max_query_len] and at most L_s (the multi-token kernel sizes its grid
// by max_query_len and places row k at position L_s - n_s + k); a sequence
// with no rows reads no context, so only the others' lengths and tables are
// checked.  report[0]
// receives the number of offending sequences, report[1] the smallest
// offending sequence index (INT32_MAX when none).
//
// Checked mode.  The library's own check (PA_CHECK=1) writes its report into
// a per-device array, `g_check_state`, and sets a sticky error word there
// that pa_get_device_error reads and clears.  Host code reaches the array
// only through the address hipGetSymbolAddress returns for the current
// device: in host code the array's name is not a device address.
#include <climits>
#include <mutex>

#include "pa_internal.h"

namespace pa {

namespace {

// [0] offending sequences of the last library check, [1] the first of them,
// [2] sticky error word (1 after a failing check until read), [3] unused.
__device__ __align__(16) int32_t g_check_state[4];

constexpr int kMaxDevices = 64;

__global__ __launch_bounds__(64) void check_init(int32_t *report) {
    if (threadIdx.x == 0) {
        report[0] = 0;
        report[1] = INT32_MAX;
    }
}

__global__ __launch_bounds__(64) void clear_word(int32_t *word) {
    if (threadIdx.x == 0) *word = 0;
}

// one wave per sequence
__global__ __launch_bounds__(64) void check_kernel(const int32_t *block_tables,
                                                   const int32_t *seq_lens,
                                                   const int32_t *query_start, int S, int T,
                                                   int max_query_len, int max_blocks, int B,
                                                   int NB, int32_t *report, int32_t *sticky) {
    const int s = blockIdx.x;
    const int L = seq_lens[s];
    bool bad = false;
    bool uses_context = true;           // a multi-token sequence with no rows reads nothing
    if (query_start) {
        const int q0 = query_start[s], q1 = query_start[s + 1];
        const int n = q1 - q0;
        if (q0 < 0 || q1 > T || n < 0 || n > max_query_len) bad = true;
        if (s == 0 && q0 != 0) bad = true;
        if (s == S - 1 && q1 != T) bad = true;
        if (n > 0 && n > L) bad = true;
        uses_context = n > 0;
    }
    if (uses_context && (L < 0 || (long long)L > (long long)max_blocks * B)) bad = true;
    if (uses_context && !bad) {
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
        if (sticky) atomicOr(sticky, 1);
    }
}

void launch_check_kernels(const int32_t *block_tables, const int32_t *seq_lens,
                          const int32_t *query_start, int S, int T, int max_query_len,
                          int max_blocks, int B, int NB, int32_t *report, int32_t *sticky,
                          hipStream_t st) {
    hipLaunchKernelGGL(check_init, dim3(1), dim3(64), 0, st, report);
    if (S > 0)
        hipLaunchKernelGGL(check_kernel, dim3(S), dim3(64), 0, st, block_tables, seq_lens,
                           query_start, S, T, max_query_len, max_blocks, B, NB, report, sticky);
}

// Device the stream belongs to (the current device for the null stream).
hipError_t stream_device(hipStream_t st, int *dev) {
    if (st) return hipStreamGetDevice(st, dev);
    return hipGetDevice(dev);
}

// Address of g_check_state on device `dev`, looked up once per device with
// that device current.
hipError_t check_state(int dev, int32_t **ptr) {
    static std::mutex mu;
    static int32_t *addr[kMaxDevices] = {};
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        int cur = 0;
        hipError_t e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_check_state));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<int32_t *>(p);
    }
    *ptr = addr[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_check(const int32_t *block_tables, const int32_t *seq_lens, int S,
                        int max_blocks, int B, int NB, int32_t *report, hipStream_t st) {
    launch_check_kernels(block_tables, seq_lens, nullptr, S, 0, 0, max_blocks, B, NB, report,
                         nullptr, st);
    return hipGetLastError();
}

hipError_t library_check(const int32_t *block_tables, const int32_t *seq_lens,
                         const int32_t *query_start, int S, int T, int max_query_len,
                         int max_blocks, int B, int NB, hipStream_t st, int *bad) {
    int dev = 0;
    hipError_t e = stream_device(st, &dev);
    if (e != hipSuccess) return e;
    int32_t *state = nullptr;
    if ((e = check_state(dev, &state)) != hipSuccess) return e;
    launch_check_kernels(block_tables, seq_lens, query_start, S, T, max_query_len, max_blocks, B,
                         NB, state, state + 2, st);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    int32_t report[2] = {0, 0};
    if ((e = hipMemcpyAsync(report, state, sizeof report, hipMemcpyDeviceToHost, st)) != hipSuccess)
        return e;
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
    *bad = report[0];
    return hipSuccess;
}

hipError_t read_device_error(hipStream_t st, int *set, int *first_bad) {
    int dev = 0;
    hipError_t e = stream_device(st, &dev);
    if (e != hipSuccess) return e;
    int32_t *state = nullptr;
    if ((e = check_state(dev, &state)) != hipSuccess) return e;
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
    int32_t words[4] = {0, 0, 0, 0};
    if ((e = hipMemcpyAsync(words, state, sizeof words, hipMemcpyDeviceToHost, st)) != hipSuccess)
        return e;
    if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
    *set = words[2] != 0;
    *first_bad = words[2] != 0 && words[1] != INT32_MAX ? words[1] : -1;
    if (words[2] != 0) {
        hipLaunchKernelGGL(clear_word, dim3(1), dim3(64), 0, st, state + 2);
        if ((e = hipGetLastError()) != hipSuccess) return e;
        if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace pa
