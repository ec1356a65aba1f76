// pa_mfma_core.h -- matrix-core building blocks shared by the decode kernel
// (pa_mfma.hip) and the multi-token causal kernel (pa_prefill.hip).
//
// A 32-token sub-tile of K and V (whole token rows, pa_tile.h) is staged in
// LDS and consumed by two small dense products on
// v_mfma_f32_16x16x32_{bf16,f16}, with 16 query columns per wave:
//     S^T [tokens x columns] = K [tokens x D]   . Q^T [D x columns]
//     O^T [D x columns]     += V^T [D x tokens] . P^T [tokens x columns]
// Lane layout (lane = 16 g + i; column i):
//  * QK, A = K rows: lane holds token i of a 16-token half, elements
//    8g + 32kk .. +7 (16-byte chunk 4kk + g), read with ds_read_b128.
//    B = Q^T: lane holds the query of column i at the same elements.
//  * The result lane holds S^T[4g + r][i], r = 0..3: scores of four tokens for
//    column i.  The two halves give the lane tokens {4g+r} and {16+4g+r}.
//  * PV, B = P^T: lane holds P[column i] at exactly those eight tokens, so the
//    contraction index k = (g, j) maps to token 4g + j (j < 4) or
//    16 + 4g + j - 4 (j >= 4) and no probability moves between lanes.
//  * PV, A = V^T: lane holds V[token(g, j)][16n + i] for d-chunk n, read with
//    ds_read_b64_tr_b16 (see swz_v below).
//  * The PV result lane holds O^T[16n + 4g + r][i]: four consecutive output
//    elements of column i; the softmax rescale factor of column i is
//    lane-local.
//
// Softmax is online (running max per column, made uniform over the four lane
// groups by two cross-lane max steps).  The probabilities enter the matrix
// core as a two-term split in the input type (p = hi + lo, both rounded to
// bf16 / fp16), with fp32 accumulation: one rounding of p to 16 bits would
// cost up to 2^-9 (bf16) or 2^-12 (fp16) relative per weight.
#pragma once

#include "pa_device.h"
#include "pa_tile.h"

namespace pa {
namespace mfma {

constexpr int kD = kHeadDim;
constexpr float kRescaleSlack = 8.f;   // see mfma_tiles

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
// bits of p and the P.V product keeps fp32-level accuracy.  Each pair is
// rounded once with a packed conversion (v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32) and hi is read back from those bits, so no element is
// converted twice.
template <typename T> struct Split;
template <> struct Split<__bf16> {
    __device__ static void run(const float (&p)[8], bf16x8 &hi, bf16x8 &lo) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x2 hv = {(__bf16)p[2 * j], (__bf16)p[2 * j + 1]};
            h[j] = bitcast<uint32_t>(hv);
            // a bfloat16 widens to fp32 by appending 16 zero bits: element 0
            // moves to the upper half (byte select), element 1 is masked
            const float h0 = bitcast<float>(__builtin_amdgcn_perm(h[j], h[j], 0x01000c0cu));
            const float h1 = bitcast<float>(h[j] & 0xffff0000u);
            const bf16x2 lv = {(__bf16)(p[2 * j] - h0), (__bf16)(p[2 * j + 1] - h1)};
            l[j] = bitcast<uint32_t>(lv);
        }
        hi = bitcast<bf16x8>(make_uint4(h[0], h[1], h[2], h[3]));
        lo = bitcast<bf16x8>(make_uint4(l[0], l[1], l[2], l[3]));
    }
};
template <> struct Split<_Float16> {
    __device__ static void run(const float (&p)[8], f16x8 &hi, f16x8 &lo) {
        uint32_t h[4], l[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const f16x2 hv = {(_Float16)p[2 * j], (_Float16)p[2 * j + 1]};
            h[j] = bitcast<uint32_t>(hv);
            // an identity byte select keeps the compiler from converting the
            // two elements again one by one
            const f16x2 hb = bitcast<f16x2>(__builtin_amdgcn_perm(h[j], h[j], 0x07060504u));
            const f16x2 lv = {(_Float16)(p[2 * j] - (float)hb[0]),
                              (_Float16)(p[2 * j + 1] - (float)hb[1])};
            l[j] = bitcast<uint32_t>(lv);
        }
        hi = bitcast<f16x8>(make_uint4(h[0], h[1], h[2], h[3]));
        lo = bitcast<f16x8>(make_uint4(l[0], l[1], l[2], l[3]));
    }
};

template <typename T, typename Vec>
__device__ __forceinline__ void split_probs(const float (&p)[8], Vec &hi, Vec &lo) {
    Split<T>::run(p, hi, lo);
}

// Scores enter the softmax as fma(acc, sc, -m) with sc = |scale * log2(e)|:
// the query fragments carry the sign of the scale (flipping a 16-bit sign bit
// is exact), and a zero scale becomes a zero query with sc = 1 (every score
// exactly 0).  The raw products then order like the scores, so maxima are
// taken on them and scaled once.
template <typename Vec>
__device__ __forceinline__ Vec signed_query(Vec q, float scale_log2) {
    const uint4 u = bitcast<uint4>(q);
    if (scale_log2 == 0.f) return bitcast<Vec>(make_uint4(0, 0, 0, 0));
    if (scale_log2 < 0.f)
        return bitcast<Vec>(make_uint4(u.x ^ 0x80008000u, u.y ^ 0x80008000u, u.z ^ 0x80008000u,
                                       u.w ^ 0x80008000u));
    return q;
}
__device__ __forceinline__ float score_scale(float scale_log2) {
    return scale_log2 == 0.f ? 1.f : fabsf(scale_log2);
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
// slots k = (g, r) and (g, 4 + r).  The four lanes of a row read 32
// contiguous bytes (one chunk pair), and the LDS serves the read half a wave
// (eight rows, 256 bytes) per cycle, so the eight rows of each half-wave must
// land on eight different chunk pairs: swz_v(r) = 2 (r % 8).  (The earlier
// 2 ((r / 2) % 8) gave two rows of each half-wave the same pair: rocprofv3
// counted 2 bank-conflict cycles in every 4 of these reads.)  Rows r and
// r + 16 share the swizzle, so the second read uses the same chunk offset.
//
// The 16-byte row writes of both images are conflict free (each row is a
// permutation of its 16 chunks).
__device__ __forceinline__ int swz_k(int row) { return row & 15; }
__device__ __forceinline__ int swz_v(int row) { return 2 * (row & 7); }

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

// This wave's tile rows 4 (k0 + k) + g, chunk i, k < N, to the swizzled LDS
// images of their sub-tile.
template <int N>
__device__ __forceinline__ void mfma_stage(const KVTileN<N> &tile, uint4 *klds, uint4 *vlds,
                                           int g, int i, int k0 = 0) {
#pragma unroll
    for (int k = 0; k < N; ++k) {
        const int row = 4 * (k0 + k) + g;
        klds[row * 16 + (i ^ swz_k(row))] = tile.k[k];
        vlds[row * 16 + (i ^ swz_v(row))] = tile.v[k];
    }
}

// Scores, online softmax update and P.V for NS staged 32-token sub-tiles
// (LDS images klds[u] / vlds[u]) starting at tokens t0 + 32 u, of which the
// first nsub (wave-uniform, 1 <= nsub <= NS) are inside the partition.  All
// score products are issued before the softmax and all P.V products after
// it, so the matrix core has independent work while the vector unit waits,
// and one maximum / rescale step serves all NS sub-tiles.  Tokens at or past
// t_end (the partition end, wave-uniform; t0 < t_end) are masked; sub-tiles
// that end before it need no mask.  sc: the score scale in exp2 units,
// positive (the query fragments carry its sign, see signed_query).
template <typename T, int NS>
__device__ __forceinline__ void mfma_tiles(MfmaState<T> &st, const typename Mfma<T>::Vec (&qf)[4],
                                           const uint4 (*klds)[32 * 16], const uint4 (*vlds)[32 * 16],
                                           int t0, int nsub, int t_end, int g, int i, float sc) {
    using M = Mfma<T>;
    using Vec = typename M::Vec;
    // scores: A operand = chunk 4kk + g of row 16h + i (swizzle swz_k = i)
    f32x4 acc[NS][2];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        if (u >= nsub) break;                        // uniform
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            acc[u][h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const uint4 a = klds[u][(16 * h + i) * 16 + ((4 * kk + g) ^ i)];
                acc[u][h] = M::mma(bitcast<Vec>(a), qf[kk], acc[u][h]);
            }
        }
    }
    // raw products, masked to -inf past the partition
    float x[NS][8];
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        const int tu = t0 + 32 * u;
        if (u >= nsub) {                              // uniform: past the partition
#pragma unroll
            for (int j = 0; j < 8; ++j) x[u][j] = kNegInf;
        } else if (tu + 32 <= t_end) {                // uniform: no token masked
#pragma unroll
            for (int j = 0; j < 8; ++j) x[u][j] = acc[u][j >> 2][j & 3];
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                x[u][j] = (tu + 16 * (j >> 2) + 4 * g + (j & 3) < t_end) ? acc[u][j >> 2][j & 3]
                                                                         : kNegInf;
        }
    }
    float mr = x[0][0];
#pragma unroll
    for (int u = 0; u < NS; ++u)
#pragma unroll
        for (int j = 0; j < 8; ++j) mr = fmaxf(mr, x[u][j]);
    mr = fmaxf(mr, shfl_xor(mr, 16));
    mr = fmaxf(mr, shfl_xor(mr, 32));
    const float mt = mr * sc;                        // the column's maximum score
    // The reference point st.m moves only when a column's maximum exceeds it
    // by more than kRescaleSlack (log2 units; always on the first sub-tile,
    // where st.m = -inf): otherwise the weights are taken against the stale
    // value (p <= 2^kRescaleSlack, exact in fp32) and the rescale of O, which
    // is most of a sub-tile's vector work, is skipped for the whole wave.
    // o / l and the partial triple (m, l, o) are the same quantities either way.
    const bool grow = mt > st.m + kRescaleSlack;     // false while mt = -inf
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {    // uniform branch
        const float mn = grow ? mt : st.m;
        // lanes that keep their reference scale by exactly 1 (also when it is
        // still -inf, where st.m - mn would be NaN)
        const float alpha = grow ? fast_exp2(st.m - mn) : 1.f;
        st.l *= alpha;
#pragma unroll
        for (int n = 0; n < 8; ++n) st.o[n] *= alpha;
        st.m = mn;
    }
    // st.m is finite here: the first sub-tile (t0 < t_end) has a valid token
    const float mneg = -st.m;

    const int row_a = 4 * g + (i >> 2);
    const int sw = swz_v(row_a);
    const int lane_off = row_a * kRowBytes + ((i & 3) << 3);
    float ps = 0.f;
#pragma unroll
    for (int u = 0; u < NS; ++u) {
        if (u >= nsub) break;                        // uniform
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = fast_exp2(fmaf(x[u][j], sc, mneg));
            ps += p[j];
        }
        Vec phi, plo;
        split_probs<T>(p, phi, plo);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int off = lane_off + (((2 * n) ^ sw) << 4);
            struct { i16x4 a, b; } raw = {lds_read_tr16(vlds[u], off),
                                          lds_read_tr16(vlds[u], off + 16 * kRowBytes)};
            const Vec va = bitcast<Vec>(raw);
            st.o[n] = M::mma(va, phi, st.o[n]);
            st.o[n] = M::mma(va, plo, st.o[n]);
        }
    }
    st.l += ps;
}

}  // namespace mfma
}  // namespace pa
