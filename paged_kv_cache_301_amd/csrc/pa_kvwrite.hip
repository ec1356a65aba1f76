// pa_kvwrite.hip -- store new tokens' keys and values into their cache slots,
// and copy whole blocks for copy-on-write.
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
// Vector path (a row is a multiple of 16 bytes and every pointer 16-byte
// aligned): grid (token, group of 256 16-byte chunks of the token's Hkv rows);
// each thread moves one K chunk and one V chunk.  The new rows are read once,
// so they are loaded non-temporally; the stores are plain (measured on MI355X:
// non-temporal loads lift the scattered write from ~5.0 to ~6.4 TB/s, the rate
// of a plain device copy, while non-temporal stores lower it again).  Element
// path otherwise: one work-group per token, 2-byte units.  Bits are copied
// unchanged.
#include "pa_internal.h"
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kThreads = kKvThreads;

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

__global__ __launch_bounds__(kThreads) void kv_write_vec16(KvWriteArgs a) {
    const int t = blockIdx.x;
    const int chunks = a.row_bytes / 16;
    const int c = blockIdx.y * kThreads + threadIdx.x;
    if (c >= a.Hkv * chunks) return;
    const long long slot = token_slot(a, t);
    if (slot < 0 || slot >= (long long)a.NB * a.B) return;
    const long long block = slot / a.B, offset = slot % a.B;
    const int h = c / chunks, k = c % chunks;
    const size_t src = ((size_t)t * a.Hkv + h) * a.row_bytes + 16 * (size_t)k;
    const size_t dst = (((size_t)block * a.Hkv + h) * a.B + offset) * a.row_bytes + 16 * (size_t)k;
    const uint4 kv = load_stream16(a.key + src);
    const uint4 vv = load_stream16(a.value + src);
    *reinterpret_cast<uint4 *>(a.key_cache + dst) = kv;
    *reinterpret_cast<uint4 *>(a.value_cache + dst) = vv;
}

__global__ __launch_bounds__(kThreads) void kv_write_u16(KvWriteArgs a) {
    const int t = blockIdx.x;
    const long long slot = token_slot(a, t);
    if (slot < 0 || slot >= (long long)a.NB * a.B) return;
    const long long block = slot / a.B, offset = slot % a.B;
    // element sizes are 2 or 4 bytes; copy 2-byte units
    const int units = a.row_bytes / 2;
    for (int c = threadIdx.x; c < a.Hkv * units; c += kThreads) {
        const int h = c / units, k = c % units;
        const size_t src = ((size_t)t * a.Hkv + h) * a.row_bytes + 2 * (size_t)k;
        const size_t dst = (((size_t)block * a.Hkv + h) * a.B + offset) * a.row_bytes + 2 * (size_t)k;
        *reinterpret_cast<u16 *>(a.key_cache + dst) = *reinterpret_cast<const u16 *>(a.key + src);
        *reinterpret_cast<u16 *>(a.value_cache + dst) = *reinterpret_cast<const u16 *>(a.value + src);
    }
}

// Whole-block copy (page "PagedAttention by hand", section "Memory Sharing
// (Copy-on-Write)": the shared block's contents go to a fresh block before
// the write).  A block of one cache is Hkv * B * D elements, contiguous in the
// [NB][Hkv][B][D] layout.  grid (8 KiB piece of the block, pair): pieces of
// one block run on neighbouring work-groups (measured a few per cent faster
// than pair-fastest order); each thread moves two 16-byte pieces of K and two
// of V, all four loads issued before the stores, when the block size is a
// multiple of 16 bytes and both caches are 16-byte aligned, else 2-byte units.
constexpr int kCopyUnroll = 2;
constexpr int kCopyPiece = kThreads * 16 * kCopyUnroll;
static_assert(kCopyPiece == kCopyPieceBytes, "copy piece size");

template <bool VEC16>
__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(char *kc, char *vc,
                                                               const int32_t *pairs,
                                                               long long block_bytes, int NB) {
    const int i = blockIdx.y;
    const int src = pairs[2 * i], dst = pairs[2 * i + 1];
    if (src < 0 || src >= NB || dst < 0 || dst >= NB || src == dst) return;
    const long long base = (long long)blockIdx.x * kCopyPiece;
    const size_t s0 = (size_t)src * block_bytes, d0 = (size_t)dst * block_bytes;
    if constexpr (VEC16) {
        uint4 kv[kCopyUnroll], vv[kCopyUnroll];
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const long long o = base + 16 * (long long)(u * kThreads + threadIdx.x);
            if (o < block_bytes) {
                kv[u] = load_stream16(kc + s0 + o);
                vv[u] = load_stream16(vc + s0 + o);
            }
        }
#pragma unroll
        for (int u = 0; u < kCopyUnroll; ++u) {
            const long long o = base + 16 * (long long)(u * kThreads + threadIdx.x);
            if (o < block_bytes) {
                *reinterpret_cast<uint4 *>(kc + d0 + o) = kv[u];
                *reinterpret_cast<uint4 *>(vc + d0 + o) = vv[u];
            }
        }
    } else {
        for (long long o = base + 2 * (long long)threadIdx.x; o < base + kCopyPiece && o < block_bytes;
             o += 2 * kThreads) {
            *reinterpret_cast<u16 *>(kc + d0 + o) = *reinterpret_cast<const u16 *>(kc + s0 + o);
            *reinterpret_cast<u16 *>(vc + d0 + o) = *reinterpret_cast<const u16 *>(vc + s0 + o);
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
    if (vec) {
        const long long chunks = (long long)Hkv * (a.row_bytes / 16);
        const long long groups = (chunks + kThreads - 1) / kThreads;
        if (groups > 65535) return hipErrorInvalidValue;
        hipLaunchKernelGGL(kv_write_vec16, dim3(T, (unsigned)groups), dim3(kThreads), 0, st, a);
    } else {
        hipLaunchKernelGGL(kv_write_u16, dim3(T), dim3(kThreads), 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_copy_blocks(void *key_cache, void *value_cache, const int32_t *pairs, int n,
                              long long block_bytes, int NB, hipStream_t st) {
    if (n == 0) return hipSuccess;
    const long long pieces = (block_bytes + kCopyPiece - 1) / kCopyPiece;
    if (n > 65535) {
        // grid.y holds the pair: longer lists go in slices
        for (int first = 0; first < n; first += 65535) {
            const hipError_t e = launch_copy_blocks(key_cache, value_cache, pairs + 2 * (size_t)first,
                                                    n - first < 65535 ? n - first : 65535,
                                                    block_bytes, NB, st);
            if (e != hipSuccess) return e;
        }
        return hipSuccess;
    }
    char *kc = static_cast<char *>(key_cache), *vc = static_cast<char *>(value_cache);
    if (block_bytes % 16 == 0 && aligned16(kc) && aligned16(vc))
        hipLaunchKernelGGL(copy_blocks_kernel<true>, dim3((unsigned)pieces, n), dim3(kThreads), 0,
                           st, kc, vc, pairs, block_bytes, NB);
    else
        hipLaunchKernelGGL(copy_blocks_kernel<false>, dim3((unsigned)pieces, n), dim3(kThreads), 0,
                           st, kc, vc, pairs, block_bytes, NB);
    return hipGetLastError();
}

}  // namespace pa
