// pa_internal.h -- launcher declarations shared by the host entry points
// (pa_api.cpp) and the kernel files.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "pa_decode.h"
#include "pa_args.h"

namespace pa {

// Launchers return hipErrorInvalidValue when no instantiation covers the
// requested shape / types (the host checks support before calling).
hipError_t launch_generic(const Args &a, pa_dtype dt, pa_dtype odt, hipStream_t st);
hipError_t launch_valu(const Args &a, pa_dtype dt, pa_dtype odt, hipStream_t st);
hipError_t launch_mfma(const Args &a, pa_dtype dt, pa_dtype odt, hipStream_t st);
hipError_t launch_combine(const Args &a, pa_dtype odt, hipStream_t st);
hipError_t launch_prefill(const Args &a, pa_dtype dt, pa_dtype odt, hipStream_t st);
hipError_t launch_check(const int32_t *block_tables, const int32_t *seq_lens, int S,
                        int max_blocks, int B, int NB, int32_t *report, hipStream_t st);

// Checked mode: run the device check into the library's per-device state on
// `st`, wait for it, and return the number of offending sequences in *bad
// (query_start may be null: decode).
hipError_t library_check(const int32_t *block_tables, const int32_t *seq_lens,
                         const int32_t *query_start, int S, int T, int max_query_len,
                         int max_blocks, int B, int NB, hipStream_t st, int *bad);
// Synchronise `st`, read and clear the sticky error word of its device.
hipError_t read_device_error(hipStream_t st, int *set, int *first_bad);

// pa_decode_noalloc: bytes of the static scratch (pa_noalloc.hip) and its
// device address on the stream's device.
constexpr size_t kNoAllocScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(hipStream_t st, void **ptr);

// A 1-D launch of `groups` work-groups of `threads` threads fits the
// hardware: grid.x <= 2^31 - 1 and grid.x * threads < 2^32.
inline bool grid_fits(long long groups, long long threads) {
    return groups >= 0 && groups <= 0x7fffffffLL && groups * threads < (1LL << 32);
}

hipError_t launch_kv_write(const void *key, const void *value, const int32_t *slot_mapping,
                           const int32_t *block_tables, const int32_t *seq_lens,
                           void *key_cache, void *value_cache, int T, int Hkv, int D, int B,
                           int NB, int max_blocks, int esz, hipStream_t st);
hipError_t launch_copy_blocks(void *key_cache, void *value_cache, const int32_t *pairs, int n,
                              long long block_bytes, int NB, hipStream_t st);
hipError_t launch_read(const void *buf, size_t bytes, uint32_t *sink, hipStream_t st);

}  // namespace pa
