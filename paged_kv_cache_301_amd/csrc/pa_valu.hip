// pa_valu.hip -- tiled paged decode attention on the vector ALUs.
//
// For head size 128 in fp16 / bf16 and groups of 1, 2, 4 or 8 query heads per
// kv head.  One wave64 handles one (sequence, kv head, context partition).
//
// Data movement.  A (block, kv head) tile is B rows of 128 elements, 256
// contiguous bytes per token in the [NB][Hkv][B][D] pools.  Each load
// instruction reads four whole token rows with one 16-byte load per lane:
// lane = 16 * g + c reads elements 8c .. 8c+7 of token 4k + g.  A loop
// iteration covers 32 tokens (8 K and 8 V loads per lane), and the loads for
// the next iteration are issued before the current one is computed, so every
// wave keeps 16-32 KB in flight.  Slots past the context length are never
// read: such lanes re-read the last valid token (a cache hit) and their
// scores are forced to -inf by selection, so neither the data nor NaN in
// unused slots reaches the result ("PagedAttention by hand", Step 2: the
// unfilled slot is masked, and ideally never read).
//
// Arithmetic.  q.K per token is four v_dot2 (two 16-bit products each, fp32
// accumulate) per lane and a 16-lane DPP sum; every lane of the row then
// holds its token's score, which is exactly the weight it needs for the V row
// it loaded.  Softmax is online per 16-lane row group (running max in exp2
// units, rescale on a new max: "Optimized CUDA Kernels", the online softmax
// of the first page), and the four row groups merge at the end.
//
// Output.  A sequence that fits one partition writes its normalised result;
// otherwise the partition writes (max, sum, unnormalised o) for the combine
// kernel.
#include "pa_internal.h"
#include "pa_device.h"
#include "pa_table.h"
#include "pa_tile.h"
#include "pa_sched.h"

namespace pa {

namespace {

constexpr int kD = kHeadDim;
constexpr int kLoads = kTileLoads;

template <typename T, int G>
struct ValuState {
    float o[G][8];
    float m[G];
    float l[G];
};

template <typename T, int G>
__device__ __forceinline__ void valu_compute(ValuState<T, G> &st, const KVTile &tile,
                                             const uint4 (&q)[G], int t0, int t_end, int g,
                                             float scale_log2) {
    float x[G][kLoads];
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        const bool valid = t0 + 4 * k + g < t_end;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            float acc = Elem<T>::dot2(tile.k[k].x, q[i].x, 0.f);
            acc = Elem<T>::dot2(tile.k[k].y, q[i].y, acc);
            acc = Elem<T>::dot2(tile.k[k].z, q[i].z, acc);
            acc = Elem<T>::dot2(tile.k[k].w, q[i].w, acc);
            acc = row16_sum(acc);
            x[i][k] = valid ? acc * scale_log2 : kNegInf;
        }
    }
    float p[G][kLoads];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        float mt = x[i][0];
#pragma unroll
        for (int k = 1; k < kLoads; ++k) mt = fmaxf(mt, x[i][k]);
        const float mn = fmaxf(st.m[i], mt);
        const float ms = (mn == kNegInf) ? 0.f : mn;   // row group saw no token yet
        const float alpha = fast_exp2(st.m[i] - ms);
        float ps = 0.f;
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            p[i][k] = fast_exp2(x[i][k] - ms);
            ps += p[i][k];
        }
        st.l[i] = st.l[i] * alpha + ps;
        st.m[i] = mn;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.o[i][e] *= alpha;
    }
#pragma unroll
    for (int k = 0; k < kLoads; ++k) {
        float v[8];
        const uint32_t w[4] = {tile.v[k].x, tile.v[k].y, tile.v[k].z, tile.v[k].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            v[2 * e] = Elem<T>::lo(w[e]);
            v[2 * e + 1] = Elem<T>::hi(w[e]);
        }
#pragma unroll
        for (int i = 0; i < G; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) st.o[i][e] = fmaf(p[i][k], v[e], st.o[i][e]);
    }
}

// NW waves per item (1, 2 or 4, as the plan decides): wave w runs the
// item's 32-token tiles w, w + NW, ..., and the waves' softmax states meet
// in LDS at the end.  Long partitions on several waves need a quarter of the
// partial results of short ones on one, or none when a partition covers the
// whole context.
template <typename T, typename OutT, int G, int NW, bool SCALAR, bool STREAM>
__global__ __launch_bounds__(64 * NW) void valu_kernel(Args a) {
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
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15;
    const int g = lane >> 4;

    const int L = a.seq_lens[s];
    const int t_begin = p * a.part_tokens;
    if (p > 0 && t_begin >= L) return;            // partition past the context
    const int t_end = min(L, t_begin + a.part_tokens);
    const int nparts = (L + a.part_tokens - 1) / a.part_tokens;

    __shared__ int32_t tbl[SCALAR ? 1 : kTableLds];
    // the other waves' states, lanes 0..15 of each: m, l and 8 output columns
    __shared__ float xst[NW > 1 ? NW - 1 : 1][G][16][10];

    uint4 q[G];
#pragma unroll
    for (int i = 0; i < G; ++i)
        q[i] = *reinterpret_cast<const uint4 *>(
            static_cast<const T *>(a.query) + ((size_t)s * a.Hq + kvh * G + i) * kD + 8 * c);

    ValuState<T, G> st;
#pragma unroll
    for (int i = 0; i < G; ++i) {
        st.m[i] = kNegInf;
        st.l[i] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.o[i][e] = 0.f;
    }

    if (L > 0) {
        TileLoader<SCALAR, STREAM> ctx;
        const size_t head_bytes = (size_t)a.B * kD * 2;
        ctx.kbase = static_cast<const char *>(a.key_cache) + kvh * head_bytes + 16 * c;
        ctx.vbase = static_cast<const char *>(a.value_cache) + kvh * head_bytes + 16 * c;
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

        // this wave's tiles: w, w + NW, ... of the partition's 32-token tiles
        const int ntiles = (t_end - t_begin + 31) >> 5;
        const int niter = (ntiles - w + NW - 1) / NW;
        constexpr int kStep = 32 * NW;
        const int tw = t_begin + 32 * w;
        KVTile ta, tb;
        ctx.load(ta, tw);
        // The scheduling barriers keep each prefetch ahead of the wait for
        // the tile computed next; without them the compiler sinks the loads
        // below that wait and the wave never has two tiles in flight.  The
        // loads past the partition's last tile are left unconditional (they
        // re-read rows just read, see TileLoader): guarding them raised the
        // kernel from 159 to 206 VGPRs, two waves per SIMD instead of three,
        // and was slower.
        for (int it = 0; it < niter; it += 2) {
            const int t0 = tw + kStep * it;
            ctx.load(tb, t0 + kStep);
            __builtin_amdgcn_sched_barrier(0);
            valu_compute<T, G>(st, ta, q, t0, t_end, g, a.scale_log2);
            __builtin_amdgcn_sched_barrier(0);
            ctx.load(ta, t0 + 2 * kStep);
            __builtin_amdgcn_sched_barrier(0);
            if (it + 1 < niter) valu_compute<T, G>(st, tb, q, t0 + kStep, t_end, g, a.scale_log2);
            __builtin_amdgcn_sched_barrier(0);
        }

        // merge the four row groups (lanes c, c+16, c+32, c+48 hold the same columns)
#pragma unroll
        for (int msk = 16; msk <= 32; msk <<= 1) {
#pragma unroll
            for (int i = 0; i < G; ++i) {
                float o2[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) o2[e] = shfl_xor(st.o[i][e], msk);
                const float m2 = shfl_xor(st.m[i], msk);
                const float l2 = shfl_xor(st.l[i], msk);
                merge_state(st.m[i], st.l[i], st.o[i], 8, m2, l2, o2);
            }
        }
    }

    if constexpr (NW > 1) {
        // the other waves hand their states to wave 0 (L and the partition
        // are the work-group's, so every wave reaches the barrier)
        if (w > 0 && g == 0) {
#pragma unroll
            for (int i = 0; i < G; ++i) {
                float *x = xst[w - 1][i][c];
                x[0] = st.m[i];
                x[1] = st.l[i];
#pragma unroll
                for (int e = 0; e < 8; ++e) x[2 + e] = st.o[i][e];
            }
        }
        __syncthreads();
        if (w > 0) return;
        if (g == 0) {
#pragma unroll
            for (int u = 0; u < NW - 1; ++u) {
#pragma unroll
                for (int i = 0; i < G; ++i) {
                    const float *x = xst[u][i][c];
                    float o2[8];
#pragma unroll
                    for (int e = 0; e < 8; ++e) o2[e] = x[2 + e];
                    merge_state(st.m[i], st.l[i], st.o[i], 8, x[0], x[1], o2);
                }
            }
        }
    }
    if (g != 0) return;
    if (nparts <= 1) {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const float inv = st.l[i] > 0.f ? 1.f / st.l[i] : 0.f;
            float r[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) r[e] = st.o[i][e] * inv;
            OutT *dst = static_cast<OutT *>(a.out) + ((size_t)s * a.Hq + kvh * G + i) * kD + 8 * c;
            store8<OutT>(dst, r);
        }
    } else {
#pragma unroll
        for (int i = 0; i < G; ++i) {
            const size_t idx = ((size_t)s * a.Hq + kvh * G + i) * a.max_parts + p;
            store8<float>(a.part_o + idx * kD + 8 * c, st.o[i]);
            if (c == 0) {
                a.part_m[idx] = st.m[i];
                a.part_l[idx] = st.l[i];
            }
        }
    }
}

template <typename T, typename OutT, int G, int NW>
void launch_gw(const Args &a, hipStream_t st) {
    const dim3 grid = a.compact ? dim3((unsigned)((long long)a.Hkv * a.S * a.max_parts))
                                : dim3(a.Hkv * a.S, a.max_parts);
    const dim3 block(64 * NW);
    const bool scalar = a.B % 4 == 0;
    if (a.stream_kv) {
        if (scalar) hipLaunchKernelGGL((valu_kernel<T, OutT, G, NW, true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((valu_kernel<T, OutT, G, NW, false, true>), grid, block, 0, st, a);
    } else {
        if (scalar) hipLaunchKernelGGL((valu_kernel<T, OutT, G, NW, true, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((valu_kernel<T, OutT, G, NW, false, false>), grid, block, 0, st, a);
    }
}

template <typename T, typename OutT, int G>
hipError_t launch_g(const Args &a, hipStream_t st) {
    if (a.token_waves == 4) launch_gw<T, OutT, G, 4>(a, st);
    else if (a.token_waves == 2) launch_gw<T, OutT, G, 2>(a, st);
    else launch_gw<T, OutT, G, 1>(a, st);
    return hipGetLastError();
}

template <typename T, typename OutT>
hipError_t launch_t(const Args &a, hipStream_t st) {
    switch (a.Hq / a.Hkv) {
    case 1: return launch_g<T, OutT, 1>(a, st);
    case 2: return launch_g<T, OutT, 2>(a, st);
    case 4: return launch_g<T, OutT, 4>(a, st);
    case 8: return launch_g<T, OutT, 8>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_valu(const Args &a, pa_dtype dt, pa_dtype odt, hipStream_t st) {
    if (a.D != kD || a.log2B < 0) return hipErrorInvalidValue;
    const bool f32out = (odt == PA_F32);
    if (dt == PA_F16) return f32out ? launch_t<_Float16, float>(a, st) : launch_t<_Float16, _Float16>(a, st);
    if (dt == PA_BF16) return f32out ? launch_t<__bf16, float>(a, st) : launch_t<__bf16, __bf16>(a, st);
    return hipErrorInvalidValue;
}

}  // namespace pa
