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
// iteration covers 32 W tokens: wave u loads the 32-token sub-tile u (two
// 16-row score tiles, one 32-deep P.V step) and stages it in LDS; then every
// wave runs the contractions for its own heads over all W sub-tiles, so each
// K / V byte is read from HBM once for all G heads and each wave keeps a whole
// sub-tile of loads in flight, as in the one-wave case.
//
// K and V arrive as whole token rows (pa_tile.h: full 128-byte lines per load
// instruction) and are staged through LDS, from where each operand is read in
// the matrix core's lane layout (lane = 16 g + i):
//  * QK, A = K rows: lane holds token i of a 16-token sub-tile, elements
//    8g + 32kk .. +7 (16-byte chunk 4kk + g), read with ds_read_b128.
//    B = Q^T: lane holds q[head i] at the same elements, loaded once.
//  * The result lane holds S^T[4g + r][i], r = 0..3: scores of four tokens for
//    head i.  The two sub-tiles give the lane tokens {4g+r} and {16+4g+r}.
//  * PV, B = P^T: lane holds P[head i] at exactly those eight tokens, so the
//    contraction index k = (g, j) maps to token 4g + j (j < 4) or
//    16 + 4g + j - 4 (j >= 4) and no probability moves between lanes.
//  * PV, A = V^T: lane holds V[token(g, j)][16n + i] for d-chunk n, read with
//    ds_read_b64_tr_b16 (see swz_v below).
//  * The PV result lane holds O^T[16n + 4g + r][i]: four consecutive output
//    elements of head i, and the softmax rescale factor of head i is lane-local.
//
// Softmax is online over iterations (running max per head, made uniform over
// the four lane groups by two cross-lane max steps).  The probabilities enter
// the matrix core as a two-term split in the input type (p = hi + lo, both
// rounded to bf16 / fp16), with fp32 accumulation: one rounding of p to 16
// bits would cost up to 2^-9 (bf16) or 2^-12 (fp16) relative per weight.
#include "pa_internal.h"
#include "pa_device.h"
#include "pa_table.h"
#include "pa_tile.h"
#include "pa_sched.h"

namespace pa {

namespace {

constexpr int kD = kHeadDim;
constexpr float kRescaleSlack = 8.f;   // see mfma_subtile

template <typename T> struct Mfma;
template <> struct Mfma<__bf16> {
    using Vec = bf16x8;
    __device__ static f32x4 mma(Vec a, Vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
};
template <> struct Mfma<_Float16> {
    using Vec = f16x8;
    __device__ static f32x4 mma(Vec a, Vec b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
};

// Two-term split of the probabilities for the 16-bit matrix-core operand:
// hi = round(p), lo = round(p - hi), so hi + lo carries 2 * (mantissa + 1)
// bits of p and the P.V product keeps fp32-level accuracy.
template <typename T, typename Vec>
__device__ __forceinline__ void split_probs(const float (&p)[8], Vec &hi, Vec &lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const T h = (T)p[j];
        hi[j] = h;
        lo[j] = (T)(p[j] - (float)h);
    }
}

// LDS images of one iteration: 32 token rows of 256 bytes (16 chunks of 16
// bytes) for K and for V; chunk c of row r is stored at c ^ swz(r).
//
// K: swz_k(r) = r % 16.  A QK operand read (fixed kk) has the 16 lanes of a
// group on 16 rows at one logical chunk, which the swizzle spreads over all 16
// chunk positions, i.e. all 64 banks.
//
// V: read with ds_read_b64_tr_b16.  Within each 16-lane group, lane q
// addresses 8 bytes (4 consecutive elements) and receives, in result slot r,
// element (q % 4) of the 4-vector addressed by lane 4r + q / 4.  Lane q of
// group g therefore addresses row 4g + q / 4 (the second read: 16 rows
// further), elements 16n + 4 (q % 4) .. +3, and receives V[4g + r][16n + q]
// (second read: V[16 + 4g + r][16n + q]) for r = 0..3: exactly the A-operand
// slots k = (g, r) and (g, 4 + r).  swz_v(r) = 2 ((r / 2) % 8) spreads the 16
// rows one such read touches over 8 even chunk offsets, so its 64 eight-byte
// accesses fill all 64 banks twice (the minimum for 512 bytes).
//
// The 16-byte row writes of both images are conflict free (each row is a
// permutation of its 16 chunks).
__device__ __forceinline__ int swz_k(int row) { return row & 15; }
__device__ __forceinline__ int swz_v(int row) { return 2 * ((row >> 1) & 7); }

using i16x4 = short __attribute__((ext_vector_type(4)));
using lds_i16x4 = __attribute__((address_space(3))) i16x4;
using lds_char = __attribute__((address_space(3))) char;

__device__ __forceinline__ i16x4 lds_read_tr16(const uint4 *lds_base, int byte_off) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4 *)((lds_char *)lds_base + byte_off));
}

template <typename T>
struct MfmaState {
    f32x4 o[8];   // O^T, d-chunk n: rows 16n + 4g + r, column = head i
    float m;      // running max of head i (exp2 units), uniform over g
    float l;      // this lane's share of head i's weight sum
};

// This wave's tile rows 4k + g, chunk i, to its swizzled LDS images.
__device__ __forceinline__ void mfma_stage(const KVTile &tile, uint4 *klds, uint4 *vlds, int g,
                                           int i) {
#pragma unroll
    for (int k = 0; k < kTileLoads; ++k) {
        const int row = 4 * k + g;
        klds[row * 16 + (i ^ swz_k(row))] = tile.k[k];
        vlds[row * 16 + (i ^ swz_v(row))] = tile.v[k];
    }
}

// Scores, online softmax update and P.V for one staged 32-token sub-tile
// starting at token t0 (which is < t_end).
template <typename T>
__device__ __forceinline__ void mfma_subtile(MfmaState<T> &st, const typename Mfma<T>::Vec (&qf)[4],
                                             const uint4 *klds, const uint4 *vlds, int t0,
                                             int t_end, int g, int i, float scale_log2) {
    using M = Mfma<T>;
    using Vec = typename M::Vec;
    // scores: A operand = chunk 4kk + g of row 16u + i (swizzle swz_k = i)
    f32x4 acc[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const uint4 a = klds[(16 * u + i) * 16 + ((4 * kk + g) ^ i)];
            acc[u] = M::mma(bitcast<Vec>(a), qf[kk], acc[u]);
        }
    }
    float x[8];
    if (t0 + 32 <= t_end) {   // uniform: the whole sub-tile is inside the context
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = acc[j >> 2][j & 3] * scale_log2;
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j)
            x[j] = (t0 + 16 * (j >> 2) + 4 * g + (j & 3) < t_end) ? acc[j >> 2][j & 3] * scale_log2
                                                                  : kNegInf;
    }
    float mt = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mt = fmaxf(mt, x[j]);
    mt = fmaxf(mt, shfl_xor(mt, 16));
    mt = fmaxf(mt, shfl_xor(mt, 32));
    // The reference point st.m moves only when a head's maximum exceeds it by
    // more than kRescaleSlack (log2 units; always on the first sub-tile, where
    // st.m = -inf): otherwise the weights are taken against the stale value
    // (p <= 2^kRescaleSlack, exact in fp32) and the rescale of O, which is most
    // of a sub-tile's vector work, is skipped for the whole wave.  o / l and
    // the partial triple (m, l, o) are the same quantities either way.
    const bool grow = mt > st.m + kRescaleSlack;     // finite mt: token t0 is valid
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {    // uniform branch
        const float mn = grow ? mt : st.m;
        const float alpha = fast_exp2(st.m - mn);
        st.l *= alpha;
#pragma unroll
        for (int n = 0; n < 8; ++n) st.o[n] *= alpha;
        st.m = mn;
    }
    float p[8];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        p[j] = fast_exp2(x[j] - st.m);
        ps += p[j];
    }
    st.l += ps;
    Vec phi, plo;
    split_probs<T>(p, phi, plo);

    const int row_a = 4 * g + (i >> 2);
    const int sw = swz_v(row_a);
    const int lane_off = row_a * kRowBytes + ((i & 3) << 3);
#pragma unroll
    for (int n = 0; n < 8; ++n) {
        const int off = lane_off + (((2 * n) ^ sw) << 4);
        struct { i16x4 a, b; } raw = {lds_read_tr16(vlds, off), lds_read_tr16(vlds, off + 16 * kRowBytes)};
        const Vec va = bitcast<Vec>(raw);
        st.o[n] = M::mma(va, phi, st.o[n]);
        st.o[n] = M::mma(va, plo, st.o[n]);
    }
}

// One iteration: every wave stages its sub-tile, then runs all W sub-tiles
// that start before t_end.  t0 = first token of the iteration.
template <typename T, int W>
__device__ __forceinline__ void mfma_compute(MfmaState<T> &st, const KVTile &tile,
                                             const typename Mfma<T>::Vec (&qf)[4],
                                             uint4 (*klds)[32 * 16], uint4 (*vlds)[32 * 16],
                                             int w, int t0, int t_end, int g, int i,
                                             float scale_log2) {
    mfma_stage(tile, klds[w], vlds[w], g, i);
    __syncthreads();   // rows visible to every lane of every wave
#pragma unroll
    for (int u = 0; u < W; ++u) {
        if (t0 + 32 * u >= t_end) break;   // uniform: the rest of the iteration is past the end
        mfma_subtile<T>(st, qf, klds[u], vlds[u], t0 + 32 * u, t_end, g, i, scale_log2);
    }
    __syncthreads();   // reads done before the next iteration overwrites LDS
}

template <typename T, typename OutT, int G, bool SCALAR, bool STREAM>
__global__ __launch_bounds__(64 * ((G + 15) / 16), 2) void mfma_kernel(Args a) {
    using Vec = typename Mfma<T>::Vec;
    constexpr int W = (G + 15) / 16;          // waves per work-group = 32-token sub-tiles per iteration
    int s, kvh, p;
    if (a.compact) {
        // 1-D grid over the live items, partition-major (see pa_sched.h)
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
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15;
    const int g = lane >> 4;

    const int L = a.seq_lens[s];
    const int t_begin = p * a.part_tokens;
    if (p > 0 && t_begin >= L) return;
    const int t_end = min(L, t_begin + a.part_tokens);
    const int nparts = (L + a.part_tokens - 1) / a.part_tokens;

    __shared__ uint4 klds[W][32 * 16];
    __shared__ uint4 vlds[W][32 * 16];
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
        qf[kk] = bitcast<Vec>(w);
    }

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
            stage_table(tbl, ctx.tv, t_begin, t_end, threadIdx.x, 64 * W);
            __syncthreads();
        }

        constexpr int kIter = 32 * W;          // tokens per iteration
        const int niter = (t_end - t_begin + kIter - 1) / kIter;
        const int tw = t_begin + 32 * w;       // this wave's sub-tile of iteration 0
        KVTile ta, tb;
        ctx.load(ta, tw);
        // The scheduling barriers keep each prefetch ahead of the wait for
        // the tile computed next; without them the compiler sinks the loads
        // below that wait and the wave never has two tiles in flight.
        for (int it = 0; it < niter; it += 2) {
            const int t0 = t_begin + kIter * it;
            ctx.load(tb, tw + kIter * (it + 1));
            __builtin_amdgcn_sched_barrier(0);
            mfma_compute<T, W>(st, ta, qf, klds, vlds, w, t0, t_end, g, i, a.scale_log2);
            __builtin_amdgcn_sched_barrier(0);
            ctx.load(ta, tw + kIter * (it + 2));
            __builtin_amdgcn_sched_barrier(0);
            if (it + 1 < niter)
                mfma_compute<T, W>(st, tb, qf, klds, vlds, w, t0 + kIter, t_end, g, i, a.scale_log2);
            __builtin_amdgcn_sched_barrier(0);
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

template <typename T, typename OutT, int G, bool STREAM>
void launch_gs(const Args &a, hipStream_t st) {
    const dim3 grid = a.compact ? dim3((unsigned)((long long)a.Hkv * a.S * a.max_parts))
                                : dim3(a.Hkv * a.S, a.max_parts);
    const dim3 block(64 * ((G + 15) / 16));
    if (a.B % 4 == 0)
        hipLaunchKernelGGL((mfma_kernel<T, OutT, G, true, STREAM>), grid, block, 0, st, a);
    else
        hipLaunchKernelGGL((mfma_kernel<T, OutT, G, false, STREAM>), grid, block, 0, st, a);
}

template <typename T, typename OutT, int G>
hipError_t launch_g(const Args &a, hipStream_t st) {
    if (a.stream_kv) launch_gs<T, OutT, G, true>(a, st);
    else launch_gs<T, OutT, G, false>(a, st);
    return hipGetLastError();
}

template <typename T, typename OutT>
hipError_t launch_t(const Args &a, hipStream_t st) {
    switch (a.Hq / a.Hkv) {
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
