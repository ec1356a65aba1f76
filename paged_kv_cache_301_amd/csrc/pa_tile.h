// pa_tile.h -- the K / V tile loader shared by the tiled kernels.
//
// A loop iteration covers 32 consecutive tokens of one (sequence, kv head).
// Each load instruction reads four whole token rows (4 x 256 bytes at D = 128
// in 16-bit types): lane 16 g + c reads the 16-byte chunk c of token 4 k + g,
// so every instruction requests full 128-byte lines.  (Reading a 16 x 64-byte
// slab per instruction instead -- the natural matrix-core operand shape --
// measured 12 % slower on MI355X: 6.0 vs 6.8 TB/s for random 4 KB tiles.)
//
// Tokens past the partition end are clamped to its last token: those lanes
// re-read a line the wave has just read (no HBM traffic) and the caller
// masks their scores, so slots past the context length are never read.
#pragma once

#include "pa_device.h"
#include "pa_table.h"

namespace pa {

constexpr int kHeadDim = 128;      // elements per token row
constexpr int kRowBytes = 256;     // bytes per token row (16-bit elements)
constexpr int kTileLoads = 8;      // load instructions per operand per iteration

// N load instructions per operand: the whole 32-token tile (N = 8), or a
// 1/W share of it when W waves of a work-group load one tile together.
template <int N = kTileLoads>
struct KVTileN {
    uint4 k[N];   // chunk (lane % 16) of token 4 (k0 + k) + lane / 16
    uint4 v[N];
};
using KVTile = KVTileN<>;

template <bool SCALAR, bool STREAM>
struct TileLoader {
    const char *kbase;     // key_cache + kv head offset + 16 * (lane % 16) (bytes)
    const char *vbase;     // value_cache + same offset
    size_t block_bytes;    // bytes between consecutive physical blocks
    int bmask;             // B - 1
    int t_end;             // one past the partition's last token
    int g;                 // token row within a load instruction (lane / 16)
    TableView tv;
    const int32_t *tbl;

    // Rows 4 (k0 + k) + g, k < N, of the tile starting at token t0.
    template <int N>
    __device__ __forceinline__ void load(KVTileN<N> &tile, int t0, int k0 = 0) const {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int t = min(t0 + 4 * (k0 + k) + g, t_end - 1);
            const int phys = phys_block<SCALAR>(tv, tbl, t);
            const size_t off = (size_t)phys * block_bytes + (size_t)(t & bmask) * kRowBytes;
            tile.k[k] = load_kv16<STREAM>(kbase + off);
            tile.v[k] = load_kv16<STREAM>(vbase + off);
        }
    }

    // The two halves of load(), for the LDS table path: the physical blocks
    // of a tile's rows, looked up (LDS reads) an iteration before the loads
    // that use them, so those loads need not wait for the lookups.
    template <int N>
    __device__ __forceinline__ void ids(int (&phys)[N], int t0, int k0 = 0) const {
#pragma unroll
        for (int k = 0; k < N; ++k)
            phys[k] = phys_block<SCALAR>(tv, tbl, min(t0 + 4 * (k0 + k) + g, t_end - 1));
    }
    template <int N>
    __device__ __forceinline__ void load_ids(KVTileN<N> &tile, const int (&phys)[N], int t0,
                                             int k0 = 0) const {
#pragma unroll
        for (int k = 0; k < N; ++k) {
            const int t = min(t0 + 4 * (k0 + k) + g, t_end - 1);
            const size_t off = (size_t)phys[k] * block_bytes + (size_t)(t & bmask) * kRowBytes;
            tile.k[k] = load_kv16<STREAM>(kbase + off);
            tile.v[k] = load_kv16<STREAM>(vbase + off);
        }
    }
};

}  // namespace pa
