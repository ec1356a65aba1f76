// pa_mfma.hip -- grouped-query paged decode attention on the matrix cores.
//
// When G = Hq / Hkv query heads share one kv head, each K / V tile read from
// HBM serves all G heads, so the two contractions per tile are small dense
// matrix products:
//     S^T [tokens x heads] = K [tokens x D]   . Q^T [D x heads]
//     O^T [D x heads]     += V^T [D x tokens] . P^T [tokens x heads]
// Both run on v_mfma_f32_16x16x32_{bf16,f16} with the head group padded to 16
// columns per wave.  One work-group handles one (sequence, kv head, context
// partition) with W = ceil(G / 16) waves: wave w owns query heads 16 w .. 16 w
// + 15 of the group (G = Hq with one kv head is multi-query attention).  An
// iteration covers NS 32-token sub-tiles (two 16-row score tiles and one
// 32-deep P.V step each; NS = W, except two for four waves): the waves load
// the sub-tiles' rows between them (one sub-tile each, or half of one at
// four waves) and stage them in LDS, then every wave runs the contractions
// for its own heads over all NS sub-tiles, so each K / V byte is read from
// HBM once for all G heads.  Groups of at most 16 heads (one head wave) can
// also run an item on 2 or 4 token-waves, each streaming its own share of
// the sub-tiles, their softmax states merged in LDS at the end.
//
// The lane layout of both products, the LDS staging and the two-term
// probability split are in pa_mfma_core.h.
#include "pa_internal.h"
#include "pa_device.h"
#include "pa_table.h"
#include "pa_tile.h"
#include "pa_sched.h"
#include "pa_mfma_core.h"

namespace pa {

namespace {

using namespace mfma;

// Sub-tiles per iteration: W (each wave loads one), except for four waves
// (64 heads), which load two sub-tiles between them, half a sub-tile each:
// half the staging registers, score registers and LDS of one sub-tile per
// wave, so 154 VGPRs and 32 KB of LDS give three waves per SIMD instead of
// two (multi-query cold step 83-84 us against 90 at the partition each form
// does best with).  Two waves (32 heads) sharing one sub-tile the same way
// reach three waves per SIMD too (147 VGPRs) but ran slower (75-78 against
// 72 us), so they keep one sub-tile each.
constexpr int sub_tiles(int W) { return W == 4 ? 2 : W; }
constexpr int waves_per_simd(int W) { return W == 4 ? 3 : 2; }

// TW token-waves (groups of at most 16 heads, one head wave): wave t runs
// the item's sub-tiles t, t + TW, ... in an LDS image of its own, with no
// barrier between the waves until their softmax states meet in LDS at the
// end (1, 2 or 4, as the plan decides for the VALU kernel too).
template <typename T, typename OutT, int G, int TW, bool SCALAR, bool STREAM>
__global__ __launch_bounds__(64 * ((G + 15) / 16) * TW, waves_per_simd((G + 15) / 16)) void mfma_kernel(Args a) {
    using Vec = typename Mfma<T>::Vec;
    constexpr int W = (G + 15) / 16;          // head waves per work-group
    static_assert(W == 1 || TW == 1, "token-waves only for groups of at most 16 heads");
    constexpr int NS = sub_tiles(W);          // 32-token sub-tiles per iteration
    constexpr int KL = kTileLoads * NS / W;   // load instructions per operand per wave
    static_assert(KL * W == kTileLoads * NS && KL <= kTileLoads, "whole row quads per wave");
    int s, kvh, p;
    if (a.compact) {
        // 1-D grid over the live items, longest first (see pa_sched.h)
        const WorkItem w = decode_work_item(a.seq_lens, a.S, a.Hkv, a.part_tokens, a.max_parts,
                                            blockIdx.x);
        if (!w.valid) return;
        s = w.s;
        kvh = w.kvh;
        p = w.p;
    } else {
        // x = (sequence, kv head) pairs, y = partition: consecutive work-groups
        // (dealt round-robin to the 8 XCDs) take different (sequence, kv head)
        // pairs of one partition index, spreading ragged contexts over XCDs
        kvh = blockIdx.x % a.Hkv;
        s = blockIdx.x / a.Hkv;
        p = blockIdx.y;
    }
    const int lane = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int w = TW > 1 ? 0 : wv;            // head wave
    const int wt = TW > 1 ? wv : 0;           // token-wave
    const int i = lane & 15;
    const int g = lane >> 4;

    const int L = a.seq_lens[s];
    const int t_begin = p * a.part_tokens;
    if (p > 0 && t_begin >= L) return;
    const int t_end = min(L, t_begin + a.part_tokens);
    const int nparts = (L + a.part_tokens - 1) / a.part_tokens;

    __shared__ uint4 klds[NS * TW][32 * 16];
    __shared__ uint4 vlds[NS * TW][32 * 16];
    __shared__ int32_t tbl[SCALAR ? 1 : kTableLds];

    // Q^T fragments of this wave's heads; columns past the group are zero
    Vec qf[4];
    const int hg = 16 * w + i;                // head within the group
    const bool head_ok = hg < G;
    const T *qrow = static_cast<const T *>(a.query) + ((size_t)s * a.Hq + kvh * G + (head_ok ? hg : 0)) * kD;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        uint4 w = *reinterpret_cast<const uint4 *>(qrow + 8 * g + 32 * kk);
        if (!head_ok) w = make_uint4(0, 0, 0, 0);
        qf[kk] = signed_query(bitcast<Vec>(w), a.scale_log2);
    }
    const float sc = score_scale(a.scale_log2);

    MfmaState<T> st;
#pragma unroll
    for (int n = 0; n < 8; ++n) st.o[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = kNegInf;
    st.l = 0.f;

    if (L > 0) {
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
            stage_table<64 * W * TW>(tbl, ctx.tv, t_begin, t_end, threadIdx.x);
            __syncthreads();
        }

        // iterations of this wave: tokens base + kIter it .. + kIter - 1
        constexpr int kIter = 32 * NS * TW;    // tokens between a wave's iterations
        const int base = t_begin + 32 * NS * wt;
        const int niter = TW == 1 || base < t_end ? (t_end - base + kIter - 1) / kIter : 0;
        // this wave's rows: quads KL w .. KL w + KL - 1 of the iteration, i.e.
        // quads k0 .. k0 + KL - 1 of sub-tile u
        const int u = KL * w / kTileLoads;
        const int k0 = KL * w % kTileLoads;
        const int tw = base + 32 * u;          // this wave's sub-tile of iteration 0
        // the wave's LDS images (its own when there are several token-waves)
        uint4 (*const kimg)[32 * 16] = klds + NS * wt;
        uint4 (*const vimg)[32 * 16] = vlds + NS * wt;
        // One sub-tile of registers: as soon as this wave's sub-tile is in
        // LDS its registers take the loads of the next one, which stay in
        // flight through the barrier and both products.  (Holding two
        // register tiles and prefetching before the compute needs 223 VGPRs
        // instead of 184 and was 1-4 % slower.)  The scheduling barriers keep
        // the compiler from sinking that prefetch below the products.
        // Several token-waves share no image, and one wave's LDS accesses
        // are served in order, so they need no barrier inside the loop.
        auto sync = [] {
            if constexpr (TW == 1) __syncthreads();
        };
        KVTileN<KL> tile;
        if constexpr (SCALAR) {
            ctx.load(tile, tw, k0);
            for (int it = 0; it < niter; ++it) {
                const int t0 = base + kIter * it;
                mfma_stage(tile, kimg[u], vimg[u], g, i, k0);
                __builtin_amdgcn_sched_barrier(0);
                if (it + 1 < niter) ctx.load(tile, tw + kIter * (it + 1), k0);   // uniform
                __builtin_amdgcn_sched_barrier(0);
                sync();   // every wave's rows visible
                const int nsub = min(NS, (t_end - t0 + 31) >> 5);   // >= 1: t0 < t_end
                mfma_tiles<T, NS>(st, qf, kimg, vimg, t0, nsub, t_end, g, i, sc);
                sync();   // reads done before the next stage overwrites LDS
            }
        } else {
            // table in LDS (blocks of fewer than 4 tokens, one per row): the
            // next-but-one sub-tile's block ids are looked up while this one
            // is computed
            int ids[KL];
            ctx.ids(ids, tw, k0);
            ctx.load_ids(tile, ids, tw, k0);
            ctx.ids(ids, tw + kIter, k0);
            for (int it = 0; it < niter; ++it) {
                const int t0 = base + kIter * it;
                mfma_stage(tile, kimg[u], vimg[u], g, i, k0);
                __builtin_amdgcn_sched_barrier(0);
                if (it + 1 < niter) ctx.load_ids(tile, ids, tw + kIter * (it + 1), k0);   // uniform
                __builtin_amdgcn_sched_barrier(0);
                ctx.ids(ids, tw + kIter * (it + 2), k0);
                sync();   // every wave's rows visible
                const int nsub = min(NS, (t_end - t0 + 31) >> 5);   // >= 1: t0 < t_end
                mfma_tiles<T, NS>(st, qf, kimg, vimg, t0, nsub, t_end, g, i, sc);
                sync();   // reads done before the next stage overwrites LDS
            }
        }
        if constexpr (TW == 1) {
            st.l += shfl_xor(st.l, 16);
            st.l += shfl_xor(st.l, 32);
        }
    }

    if constexpr (TW > 1) {
        // token-waves 1 .. TW - 1 leave their states in their own images
        // (o in the K image, m and l in the V image), wave 0 merges them
        if (wt > 0) {
#pragma unroll
            for (int n = 0; n < 8; ++n)
                klds[wt][64 * n + lane] = bitcast<uint4>(st.o[n]);
            vlds[wt][lane] = make_uint4(__float_as_uint(st.m), __float_as_uint(st.l), 0u, 0u);
        }
        __syncthreads();
        if (wt > 0) return;
#pragma unroll
        for (int v = 1; v < TW; ++v) {
            const uint4 ml = vlds[v][lane];
            const float m2 = __uint_as_float(ml.x), l2 = __uint_as_float(ml.y);
            const float mn = fmaxf(st.m, m2);
            const float ms = mn == kNegInf ? 0.f : mn;   // neither wave saw a token
            const float ca = fast_exp2(st.m - ms), cb = fast_exp2(m2 - ms);
            st.l = st.l * ca + l2 * cb;
#pragma unroll
            for (int n = 0; n < 8; ++n) st.o[n] = st.o[n] * ca + bitcast<f32x4>(klds[v][64 * n + lane]) * cb;
            st.m = mn;
        }
        st.l += shfl_xor(st.l, 16);
        st.l += shfl_xor(st.l, 32);
    }

    if (!head_ok) return;
    const int head = kvh * G + hg;
    if (nparts <= 1) {
        const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
#pragma unroll
        for (int n = 0; n < 8; ++n) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                store_elem<OutT>(a.out, ((size_t)s * a.Hq + head) * kD + 16 * n + 4 * g + r, st.o[n][r] * inv);
        }
    } else {
        const size_t idx = ((size_t)s * a.Hq + head) * a.max_parts + p;
        float *dst = a.part_o + idx * kD;
#pragma unroll
        for (int n = 0; n < 8; ++n)
            *reinterpret_cast<float4 *>(dst + 16 * n + 4 * g) =
                make_float4(st.o[n][0], st.o[n][1], st.o[n][2], st.o[n][3]);
        if (g == 0) {
            a.part_m[idx] = st.m;
            a.part_l[idx] = st.l;
        }
    }
}

template <typename T, typename OutT, int G, int TW, bool STREAM>
void launch_gs(const Args &a, hipStream_t st) {
    const dim3 grid = a.compact ? dim3((unsigned)((long long)a.Hkv * a.S * a.max_parts))
                                : dim3(a.Hkv * a.S, a.max_parts);
    const dim3 block(64 * ((G + 15) / 16) * TW);
    if (a.B % 4 == 0)
        hipLaunchKernelGGL((mfma_kernel<T, OutT, G, TW, true, STREAM>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((mfma_kernel<T, OutT, G, TW, false, STREAM>), grid, block, 0, st, a);
}

template <typename T, typename OutT, int G, int TW>
void launch_gt(const Args &a, hipStream_t st) {
    if (a.stream_kv) launch_gs<T, OutT, G, TW, true>(a, st);
    else launch_gs<T, OutT, G, TW, false>(a, st);
}

template <typename T, typename OutT, int G>
hipError_t launch_g(const Args &a, hipStream_t st) {
    if constexpr (G <= 16) {
        switch (a.token_waves) {
        case 4: launch_gt<T, OutT, G, 4>(a, st); break;
        case 2: launch_gt<T, OutT, G, 2>(a, st); break;
        default: launch_gt<T, OutT, G, 1>(a, st); break;
        }
    } else {
        launch_gt<T, OutT, G, 1>(a, st);
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

hipError_t launch_mfma(const Args &a, pa_dtype dt, pa_dtype odt, hipStream_t st) {
    if (a.D != kD || a.log2B < 0) return hipErrorInvalidValue;
    const bool f32out = (odt == PA_F32);
    if (dt == PA_F16) return f32out ? launch_t<_Float16, float>(a, st) : launch_t<_Float16, _Float16>(a, st);
    if (dt == PA_BF16) return f32out ? launch_t<__bf16, float>(a, st) : launch_t<__bf16, __bf16>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace pa
