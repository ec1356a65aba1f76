// pa_prefill.hip -- several new tokens per sequence, causal, on the matrix cores.
//
// A chunk of new tokens (a chunked prefill, or several tokens appended at
// once) attends the paged cache causally: query row k of sequence s sits at
// position L_s - n_s + k and reads tokens 0 .. L_s - n_s + k (pa_rows.h; the
// blockwise equation of the glossary page "PagedAttention", section "How It
// Works", with the last block cut at the query's own position).  Unlike
// decode, many queries share each K / V tile, so both products are genuinely
// dense:
//     S^T [tokens x (query, head)] = K . Q^T,   O^T += V^T . P^T
//
// One work-group of four waves handles one (sequence, kv head, block of
// query tokens, context partition).  Its 128 columns are (query token, head)
// pairs, column c = token c / G, head c % G of the kv head's group, so a block
// holds 128 / G query tokens; wave w owns columns 32 w .. 32 w + 31 as two
// groups of 16 (the matrix core's column width).  When every sequence's rows
// fit 64 columns (G times the longest query chunk at most 64: a few new
// tokens, or one token of a wide group) the work-group has two waves and 64
// columns instead, so no block is more than half empty by construction
// (measured: 4 new tokens on the 16-sequence batch 104 -> 70 us, on the
// 128-sequence 8-head-group batch 366 -> 334 us), and a 16-column group
// without a query row skips both products and the softmax (that batch's
// kernel 73 -> 63 us).  When the longest chunk
// fills 256 columns it has eight waves and 256 columns: each staged
// sub-tile then serves twice the query rows, which halves the re-reads of
// a sequence's context by its query blocks (HBM reads 2.2 -> 1.4 GB per
// launch on the chunked-prefill batch) and ran 4-9 % faster.  An iteration covers one
// 32-token sub-tile of whole K / V rows (pa_tile.h): each wave loads its
// share of the rows, the shares meet in a double-buffered LDS image (one
// barrier per iteration), and every wave reads the K and V^T fragments of the
// sub-tile once and runs the two products for both of its column groups
// with them -- twice the matrix-core work per LDS byte and per fragment read
// of a one-group wave.  Each column masks the tokens past its own
// position; sub-tiles below the block's first query position need no mask.
// The context loop of a block stops at its last query's position, so early
// query blocks read a shorter context.  Long contexts are cut into
// partitions merged by the same log-sum-exp combine as decode, per query row.
// Measured on MI355X (chunked-prefill workload): four groups per wave (O in
// the accumulation registers, one wave per SIMD) ran at 404 TFLOP/s, one
// group per wave with four sub-tiles per iteration at 440, two groups per
// wave at two waves per SIMD at 529.
#include "pa_internal.h"
#include "pa_device.h"
#include "pa_table.h"
#include "pa_tile.h"
#include "pa_rows.h"
#include "pa_sched.h"
#include "pa_mfma_core.h"

namespace pa {

namespace {

using namespace mfma;

constexpr int kGroups = 2;   // 16-column groups per wave
constexpr int kXcds = 8;     // accelerator dies: consecutive work-group ids alternate between them

template <bool B> struct BoolTag { static constexpr bool value = B; };

// This wave's share of a sub-tile (rows 4 (k0 + k) + g, chunk i, k < NL) to
// the swizzled LDS images.
template <int NL>
__device__ __forceinline__ void stage_part(const KVTileN<NL> &tile, uint4 *klds, uint4 *vlds,
                                           int k0, int g, int i) {
#pragma unroll
    for (int k = 0; k < NL; ++k) {
        const int row = 4 * (k0 + k) + g;
        klds[row * 16 + (i ^ swz_k(row))] = tile.k[k];
        vlds[row * 16 + (i ^ swz_v(row))] = tile.v[k];
    }
}

// One staged 32-token sub-tile starting at t0 for the wave's column groups.
// MASK: some column may not see every token of the sub-tile (lim[j]: tokens
// column group j's lane may see); without it no score is masked, which is
// every sub-tile below the block's first query position.  sc: the score
// scale in exp2 units, positive (see signed_query).  SKIP: a group none of
// whose columns is a query row (live[j] false, wave-uniform) is left out;
// its state stays empty and it writes nothing.
template <typename T, bool MASK, bool SKIP>
__device__ __forceinline__ void subtile_groups(MfmaState<T> (&st)[kGroups],
                                               const typename Mfma<T>::Vec (&qf)[kGroups][4],
                                               const uint4 *klds, const uint4 *vlds, int t0,
                                               const int (&lim)[kGroups], const bool (&live)[kGroups],
                                               int g, int i, float sc) {
    using M = Mfma<T>;
    using Vec = typename M::Vec;
    // K fragments: A operand = chunk 4kk + g of row 16h + i (swizzle swz_k = i)
    Vec kf[2][4];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
            kf[h][kk] = bitcast<Vec>(klds[(16 * h + i) * 16 + ((4 * kk + g) ^ i)]);
    f32x4 acc[kGroups][2];
#pragma unroll
    for (int j = 0; j < kGroups; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            acc[j][h] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (SKIP && !live[j]) continue;          // uniform
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc[j][h] = M::mma(kf[h][kk], qf[j][kk], acc[j][h]);
        }
    // V^T fragments (see swz_v): the same for every group
    const int row_a = 4 * g + (i >> 2);
    const int sw = swz_v(row_a);
    const int lane_off = row_a * kRowBytes + ((i & 3) << 3);
    Vec vf[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int off = lane_off + (((2 * n) ^ sw) << 4);
        struct { i16x4 a, b; } raw = {lds_read_tr16(vlds, off), lds_read_tr16(vlds, off + 16 * kRowBytes)};
        vf[n] = bitcast<Vec>(raw);
    }
    // raw products (masked to -inf) and each column's maximum, scaled once
    float x[kGroups][8];
    float mt[kGroups];
    bool grow[kGroups];
    bool grow_any = false;
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        if (SKIP && !live[j]) {                      // uniform: no query row here
            mt[j] = kNegInf;
            grow[j] = false;
            continue;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float v = acc[j][e >> 2][e & 3];
            x[j][e] = (!MASK || t0 + 16 * (e >> 2) + 4 * g + (e & 3) < lim[j]) ? v : kNegInf;
        }
        float m = x[j][0];
#pragma unroll
        for (int e = 1; e < 8; ++e) m = fmaxf(m, x[j][e]);
        m = fmaxf(m, shfl_xor(m, 16));
        m = fmaxf(m, shfl_xor(m, 32));
        mt[j] = m * sc;
        grow[j] = mt[j] > st[j].m + kRescaleSlack;    // false while mt = -inf
        grow_any = grow_any || grow[j];
    }
    // deferred rescale, as in mfma_tiles: one wave-uniform branch for all the
    // wave's groups, so the straight-line code below lets the matrix core
    // work through one group's P.V while the vector unit computes the next
    // group's probabilities
    if (__builtin_amdgcn_ballot_w64(grow_any) != 0) {
#pragma unroll
        for (int j = 0; j < kGroups; ++j) {
            const float mn = grow[j] ? mt[j] : st[j].m;
            const float alpha = grow[j] ? fast_exp2(st[j].m - mn) : 1.f;
            st[j].l *= alpha;
#pragma unroll
            for (int n = 0; n < 8; ++n) st[j].o[n] *= alpha;
            st[j].m = mn;
        }
    }
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        if (SKIP && !live[j]) continue;              // uniform
        // a column that has seen no token yet keeps zero weights
        const float mneg = st[j].m == kNegInf ? 0.f : -st[j].m;
        float p[8];
        float ps = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            p[e] = fast_exp2(fmaf(x[j][e], sc, mneg));
            ps += p[e];
        }
        st[j].l += ps;
        Vec phi, plo;
        split_probs<T>(p, phi, plo);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            st[j].o[n] = M::mma(vf[n], phi, st[j].o[n]);
            st[j].o[n] = M::mma(vf[n], plo, st[j].o[n]);
        }
    }
}

// NW waves per work-group (2, 4 or 8; see kPrefillColumns): 32 NW columns.
template <typename T, typename OutT, int G, int NW, bool SCALAR, bool STREAM>
__global__ __launch_bounds__(64 * NW, 2) void prefill_kernel(Args a) {
    using Vec = typename Mfma<T>::Vec;
    constexpr int kColumns = 16 * kGroups * NW;
    constexpr int kLoads = kTileLoads / NW;      // load instructions per operand per wave
    constexpr int QPB = kColumns / G;            // query tokens per work-group
    static_assert(QPB * G == kColumns, "G divides the column count");

    // x: work-groups are dealt round-robin to the 8 XCDs (x mod 8); the
    // query blocks of one (sequence, kv head) pair get consecutive slots of
    // one XCD, so they start together and stream the same K / V tiles through
    // that XCD's L2 instead of each reading them from HBM.  y = partition.
    const int xcd = blockIdx.x % kXcds;
    const int slot = blockIdx.x / kXcds;
    // ordered launches also take a pair's query blocks last first: the later
    // rows of a chunk attend the longer causal contexts
    const int qb = a.by_length ? a.q_blocks - 1 - slot % a.q_blocks : slot % a.q_blocks;
    const int pair = (slot / a.q_blocks) * kXcds + xcd;
    if (pair >= a.S * a.Hkv) return;
    // pairs in decreasing context length (kv head fastest) when the launch
    // takes several rounds, so the longest contexts start first and it ends
    // on the short ones
    const int s = a.by_length
                      ? sequence_by_length(a.seq_lens, a.S, a.max_blocks * a.B, pair / a.Hkv)
                      : pair / a.Hkv;
    if (s < 0) return;   // lengths outside [0, max_blocks * B]: nothing to map
    const int kvh = pair % a.Hkv;
    const int p = blockIdx.y;

    const int qs = a.query_start[s];
    const int n = a.query_start[s + 1] - qs;
    const int q_first = qb * QPB;
    if (q_first >= n) return;
    const int q_last = min(n, q_first + QPB) - 1;
    const int L = a.seq_lens[s];
    const int base = L - n;                      // position of the sequence's first new token
    const int lim_min = base + q_first + 1;      // tokens the block's first query attends
    const int lim_max = base + q_last + 1;
    const int t_begin = p * a.part_tokens;
    if (t_begin >= lim_max) return;              // uniform: nothing of this partition is visible
    const int t_end = min(lim_max, t_begin + a.part_tokens);
    const int t_full = min(lim_min, t_end);      // below this every column sees every token

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15;
    const int g = lane >> 4;

    // the wave's column groups: column c = token c / G, head c % G
    int lim[kGroups], lim_eff[kGroups], rows[kGroups], heads[kGroups];
    bool ok[kGroups];
    Vec qf[kGroups][4];
    const float sc = score_scale(a.scale_log2);
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        const int c = 16 * kGroups * w + 16 * j + i;
        const int qi = c / G;
        ok[j] = q_first + qi <= q_last;
        lim[j] = ok[j] ? base + q_first + qi + 1 : 0;
        lim_eff[j] = min(lim[j], t_end);
        rows[j] = qs + q_first + qi;
        heads[j] = kvh * G + c % G;
        const T *qrow = static_cast<const T *>(a.query) +
                        ((size_t)(ok[j] ? rows[j] : qs) * a.Hq + heads[j]) * kHeadDim;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            uint4 v = *reinterpret_cast<const uint4 *>(qrow + 8 * g + 32 * kk);
            if (!ok[j]) v = make_uint4(0, 0, 0, 0);
            qf[j][kk] = signed_query(bitcast<Vec>(v), a.scale_log2);
        }
    }

    // groups with at least one query row (wave-uniform); the two-wave
    // work-groups of few-token calls leave the others out
    bool live[kGroups];
#pragma unroll
    for (int j = 0; j < kGroups; ++j) live[j] = __builtin_amdgcn_ballot_w64(ok[j]) != 0;
    constexpr bool kSkip = NW == 2;

    MfmaState<T> st[kGroups];
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
#pragma unroll
        for (int k = 0; k < 8; ++k) st[j].o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
        st[j].m = kNegInf;
        st[j].l = 0.f;
    }

    __shared__ uint4 klds[2][32 * 16];
    __shared__ uint4 vlds[2][32 * 16];
    __shared__ int32_t tbl[SCALAR ? 1 : kTableLds];

    TileLoader<SCALAR, STREAM> ctx;
    const size_t head_bytes = (size_t)a.B * kRowBytes;
    ctx.kbase = static_cast<const char *>(a.key_cache) + kvh * head_bytes + 16 * i;
    ctx.vbase = static_cast<const char *>(a.value_cache) + kvh * head_bytes + 16 * i;
    ctx.block_bytes = (size_t)a.Hkv * head_bytes;
    ctx.bmask = a.B - 1;
    ctx.t_end = t_end;
    ctx.g = g;
    ctx.tv.row = a.block_tables + (size_t)s * a.max_blocks;
    ctx.tv.lb = a.log2B;
    ctx.tv.j0 = t_begin >> a.log2B;
    ctx.tbl = tbl;
    if constexpr (!SCALAR) {
        stage_table<64 * NW>(tbl, ctx.tv, t_begin, t_end, threadIdx.x);
        __syncthreads();
    }

    // One barrier per sub-tile: a wave writes LDS image b only after the
    // barrier of the previous sub-tile, which every wave reaches after it
    // has finished reading image b (two sub-tiles earlier).  Sub-tiles come
    // in pairs (images 0 and 1, register tiles ra and rb); the leading pairs
    // that lie wholly below t_full run without the causal mask, in a loop of
    // their own (one loop holding both forms needs more registers than two
    // waves per SIMD allow).
    const int niter = (t_end - t_begin + 31) >> 5;
    const int n_full = t_full > t_begin ? (t_full - t_begin) >> 5 : 0;
    const int k0 = kLoads * w;
    KVTileN<kLoads> ra, rb;
    ctx.load(ra, t_begin, k0);
    auto sub_pair = [&](int it, auto mask) {
        constexpr bool MASK = decltype(mask)::value;
        const int t0 = t_begin + 32 * it;
        ctx.load(rb, t0 + 32, k0);
        __builtin_amdgcn_sched_barrier(0);
        stage_part(ra, klds[0], vlds[0], k0, g, i);
        __syncthreads();
        subtile_groups<T, MASK, kSkip>(st, qf, klds[0], vlds[0], t0, lim_eff, live, g, i, sc);
        __builtin_amdgcn_sched_barrier(0);
        ctx.load(ra, t0 + 64, k0);
        __builtin_amdgcn_sched_barrier(0);
        if (it + 1 < niter) {
            stage_part(rb, klds[1], vlds[1], k0, g, i);
            __syncthreads();
            subtile_groups<T, MASK, kSkip>(st, qf, klds[1], vlds[1], t0 + 32, lim_eff, live, g, i,
                                           sc);
        }
        __builtin_amdgcn_sched_barrier(0);
    };
    int it = 0;
    for (; it + 2 <= n_full; it += 2) sub_pair(it, BoolTag<false>{});
    for (; it < niter; it += 2) sub_pair(it, BoolTag<true>{});

#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
        float l = st[j].l;
        l += shfl_xor(l, 16);
        l += shfl_xor(l, 32);
        if (!ok[j]) continue;
        const int np_row = (lim[j] + a.part_tokens - 1) / a.part_tokens;
        if (p >= np_row) continue;               // none of this column's tokens are here
        if (np_row == 1) {
            const float inv = 1.f / l;           // l > 0: token 0 is visible to every row
#pragma unroll
            for (int k = 0; k < 8; ++k)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    store_elem<OutT>(a.out, ((size_t)rows[j] * a.Hq + heads[j]) * kHeadDim + 16 * k + 4 * g + r,
                                     st[j].o[k][r] * inv);
        } else {
            const size_t idx = ((size_t)rows[j] * a.Hq + heads[j]) * a.max_parts + p;
            float *dst = a.part_o + idx * kHeadDim;
#pragma unroll
            for (int k = 0; k < 8; ++k)
                *reinterpret_cast<float4 *>(dst + 16 * k + 4 * g) =
                    make_float4(st[j].o[k][0], st[j].o[k][1], st[j].o[k][2], st[j].o[k][3]);
            if (g == 0) {
                a.part_m[idx] = st[j].m;
                a.part_l[idx] = l;
            }
        }
    }
}

template <typename T, typename OutT, int G, int NW>
void launch_gw(const Args &a, hipStream_t st) {
    const long long pairs = (long long)a.S * a.Hkv;
    const dim3 grid((unsigned)((pairs + kXcds - 1) / kXcds * kXcds * a.q_blocks), a.max_parts);
    const dim3 block(64 * NW);
    const bool scalar = a.B % 4 == 0;
    if (a.stream_kv) {
        if (scalar) hipLaunchKernelGGL((prefill_kernel<T, OutT, G, NW, true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((prefill_kernel<T, OutT, G, NW, false, true>), grid, block, 0, st, a);
    } else {
        if (scalar) hipLaunchKernelGGL((prefill_kernel<T, OutT, G, NW, true, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((prefill_kernel<T, OutT, G, NW, false, false>), grid, block, 0, st, a);
    }
}

template <typename T, typename OutT, int G>
hipError_t launch_g(const Args &a, hipStream_t st) {
    switch (a.prefill_columns) {
    case kPrefillColumnsNarrow: launch_gw<T, OutT, G, 2>(a, st); break;
    case kPrefillColumns: launch_gw<T, OutT, G, 4>(a, st); break;
    case kPrefillColumnsWide: launch_gw<T, OutT, G, 8>(a, st); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <typename T, typename OutT>
hipError_t launch_t(const Args &a, hipStream_t st) {
    switch (a.Hq / a.Hkv) {
    case 1: return launch_g<T, OutT, 1>(a, st);
    case 2: return launch_g<T, OutT, 2>(a, st);
    case 4: return launch_g<T, OutT, 4>(a, st);
    case 8: return launch_g<T, OutT, 8>(a, st);
    case 16: return launch_g<T, OutT, 16>(a, st);
    case 32: return launch_g<T, OutT, 32>(a, st);
    case 64: return launch_g<T, OutT, 64>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill(const Args &a, pa_dtype dt, pa_dtype odt, hipStream_t st) {
    if (a.D != kHeadDim || a.log2B < 0 || !a.query_start) return hipErrorInvalidValue;
    const bool f32out = (odt == PA_F32);
    if (dt == PA_F16) return f32out ? launch_t<_Float16, float>(a, st) : launch_t<_Float16, _Float16>(a, st);
    if (dt == PA_BF16) return f32out ? launch_t<__bf16, float>(a, st) : launch_t<__bf16, __bf16>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace pa
