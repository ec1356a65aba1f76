// pa_kvwrite.hip -- store new tokens' keys and values into their cache slots.
//
// The step right before decode attention: the current token's key and value
// are written into its slot of the sequence's physical block ("PagedAttention
// by hand", section "Setup", Step 1, and the end of "Forward pass": the next
// token's key and value go into the empty slot of the last block before
// attention runs).  Token t of a batch goes to physical block slot / B, offset
// slot % B, of the [NB][Hkv][B][D] pools; its Hkv rows are scattered one per
// kv head.
//
// Two ways to name the slot:
//  * slot_mapping[t] = block * B + offset (any number of tokens, e.g. a
//    prompt chunk), negative to skip a token;
//  * decode append: sequence s's new token is at position seq_lens[s] - 1
//    (the lengths include it), so slot = block_tables[s][(L-1)/B] * B + (L-1) % B.
// Slots outside the pool (and, for append, empty sequences or table positions
// past the table) are skipped, so a bad index never writes out of bounds.
//
// One 256-thread work-group per token; 16-byte vector copies when a row is a
// multiple of 16 bytes and every pointer is 16-byte aligned, element copies
// otherwise.  The kernel is pure data movement: bits are copied unchanged.
#include "pa_internal.h"
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kThreads = 256;

struct KvWriteArgs {
    const char *key;           // [T][Hkv][D]
    const char *value;
    const int32_t *slot_mapping;   // [T] or null (append mode)
    const int32_t *block_tables;   // [S][max_blocks] (append mode)
    const int32_t *seq_lens;       // [S]             (append mode)
    char *key_cache;           // [NB][Hkv][B][D]
    char *value_cache;
    int T, Hkv, B, NB, max_blocks;
    int row_bytes;             // D * esz
};

__device__ __forceinline__ long long token_slot(const KvWriteArgs &a, int t) {
    if (a.slot_mapping) return a.slot_mapping[t];
    const int L = a.seq_lens[t];
    if (L <= 0) return -1;
    const int pos = L - 1;
    const int j = pos / a.B;
    if (j >= a.max_blocks) return -1;
    const int phys = a.block_tables[(size_t)t * a.max_blocks + j];
    if (phys < 0 || phys >= a.NB) return -1;
    return (long long)phys * a.B + pos % a.B;
}

template <bool VEC16>
__global__ __launch_bounds__(kThreads) void kv_write_kernel(KvWriteArgs a) {
    const int t = blockIdx.x;
    const long long slot = token_slot(a, t);
    if (slot < 0 || slot >= (long long)a.NB * a.B) return;
    const long long block = slot / a.B, offset = slot % a.B;
    const size_t src_row = (size_t)t * a.Hkv;
    const size_t dst_row = (size_t)block * a.Hkv * a.B + offset;   // row of kv head 0
    const size_t head_stride = (size_t)a.B;                        // rows between kv heads
    if constexpr (VEC16) {
        const int chunks = a.row_bytes / 16;
        for (int c = threadIdx.x; c < a.Hkv * chunks; c += kThreads) {
            const int h = c / chunks, k = c % chunks;
            const size_t src = (src_row + h) * a.row_bytes + 16 * (size_t)k;
            const size_t dst = (dst_row + h * head_stride) * a.row_bytes + 16 * (size_t)k;
            *reinterpret_cast<uint4 *>(a.key_cache + dst) = *reinterpret_cast<const uint4 *>(a.key + src);
            *reinterpret_cast<uint4 *>(a.value_cache + dst) = *reinterpret_cast<const uint4 *>(a.value + src);
        }
    } else {
        // element sizes are 2 or 4 bytes; copy 2-byte units
        const int units = a.row_bytes / 2;
        for (int c = threadIdx.x; c < a.Hkv * units; c += kThreads) {
            const int h = c / units, k = c % units;
            const size_t src = (src_row + h) * a.row_bytes + 2 * (size_t)k;
            const size_t dst = (dst_row + h * head_stride) * a.row_bytes + 2 * (size_t)k;
            *reinterpret_cast<u16 *>(a.key_cache + dst) = *reinterpret_cast<const u16 *>(a.key + src);
            *reinterpret_cast<u16 *>(a.value_cache + dst) = *reinterpret_cast<const u16 *>(a.value + src);
        }
    }
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_kv_write(const void *key, const void *value, const int32_t *slot_mapping,
                           const int32_t *block_tables, const int32_t *seq_lens,
                           void *key_cache, void *value_cache, int T, int Hkv, int D, int B,
                           int NB, int max_blocks, int esz, hipStream_t st) {
    if (T == 0) return hipSuccess;
    KvWriteArgs a;
    a.key = static_cast<const char *>(key);
    a.value = static_cast<const char *>(value);
    a.slot_mapping = slot_mapping;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.key_cache = static_cast<char *>(key_cache);
    a.value_cache = static_cast<char *>(value_cache);
    a.T = T;
    a.Hkv = Hkv;
    a.B = B;
    a.NB = NB;
    a.max_blocks = max_blocks;
    a.row_bytes = D * esz;
    const bool vec = a.row_bytes % 16 == 0 && aligned16(key) && aligned16(value) &&
                     aligned16(key_cache) && aligned16(value_cache);
    if (vec)
        hipLaunchKernelGGL(kv_write_kernel<true>, dim3(T), dim3(kThreads), 0, st, a);
    else
        hipLaunchKernelGGL(kv_write_kernel<false>, dim3(T), dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

}  // namespace pa
