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
// query tokens, context partition).  Its 64 columns are (query token, head)
// pairs, column c = token c / G, head c % G of the kv head's group, so a block
// holds 64 / G query tokens (64 for G = 1, 1 for G = 64) and wave w owns
// columns 16 w .. 16 w + 15.  An iteration covers 128 tokens: each wave loads
// one 32-token sub-tile of whole K / V rows (pa_tile.h), stages it in LDS,
// and every wave runs the two products for its columns over the four
// sub-tiles (pa_mfma_core.h).  Each column masks the tokens past its own
// position; sub-tiles below the block's first query position need no mask.
// The context loop of a block stops at its last query's position, so early
// query blocks read a shorter context.  Long contexts are cut into
// partitions merged by the same log-sum-exp combine as decode, per query row.
#include "pa_internal.h"
#include "pa_device.h"
#include "pa_table.h"
#include "pa_tile.h"
#include "pa_rows.h"
#include "pa_mfma_core.h"

namespace pa {

namespace {

using namespace mfma;

constexpr int kWaves = kPrefillColumns / 16;
constexpr int kXcds = 8;   // accelerator dies: consecutive work-group ids alternate between them

template <typename T, typename OutT, int G, bool SCALAR, bool STREAM>
__global__ __launch_bounds__(64 * kWaves, 2) void prefill_kernel(Args a) {
    using Vec = typename Mfma<T>::Vec;
    constexpr int QPB = kPrefillColumns / G;     // query tokens per work-group
    static_assert(QPB * G == kPrefillColumns, "G divides the column count");

    // x: work-groups are dealt round-robin to the 8 XCDs (x mod 8); the
    // query blocks of one (sequence, kv head) pair get consecutive slots of
    // one XCD, so they start together and stream the same K / V tiles through
    // that XCD's L2 instead of each reading them from HBM.  y = partition.
    const int xcd = blockIdx.x % kXcds;
    const int slot = blockIdx.x / kXcds;
    const int qb = slot % a.q_blocks;
    const int pair = (slot / a.q_blocks) * kXcds + xcd;
    if (pair >= a.S * a.Hkv) return;
    const int s = pair / a.Hkv;
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

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int i = lane & 15;
    const int g = lane >> 4;
    const int c = 16 * w + i;                    // column: (query token c / G, head c % G)
    const int qi = c / G;
    const int hg = c % G;
    const bool col_ok = q_first + qi <= q_last;
    const int lim = col_ok ? base + q_first + qi + 1 : 0;   // this column's visible tokens
    const int lim_eff = min(lim, t_end);
    const int t_full = min(lim_min, t_end);      // below this every column sees every token
    const int row = qs + q_first + qi;           // query row
    const int head = kvh * G + hg;

    __shared__ uint4 klds[kWaves][32 * 16];
    __shared__ uint4 vlds[kWaves][32 * 16];
    __shared__ int32_t tbl[SCALAR ? 1 : kTableLds];

    Vec qf[4];
    const T *qrow = static_cast<const T *>(a.query) + ((size_t)(col_ok ? row : qs) * a.Hq + head) * kHeadDim;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        uint4 v = *reinterpret_cast<const uint4 *>(qrow + 8 * g + 32 * kk);
        if (!col_ok) v = make_uint4(0, 0, 0, 0);
        qf[kk] = bitcast<Vec>(v);
    }

    MfmaState<T> st;
#pragma unroll
    for (int k = 0; k < 8; ++k) st.o[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    st.m = kNegInf;
    st.l = 0.f;

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
        stage_table(tbl, ctx.tv, t_begin, t_end, threadIdx.x, 64 * kWaves);
        __syncthreads();
    }

    constexpr int kIter = 32 * kWaves;
    const int niter = (t_end - t_begin + kIter - 1) / kIter;
    const int tw = t_begin + 32 * w;
    KVTile ta, tb;
    ctx.load(ta, tw);
    for (int it = 0; it < niter; it += 2) {
        const int t0 = t_begin + kIter * it;
        ctx.load(tb, tw + kIter * (it + 1));
        __builtin_amdgcn_sched_barrier(0);
        mfma_compute<T, kWaves, true>(st, ta, qf, klds, vlds, w, t0, t_end, lim_eff, t_full, g, i,
                                      a.scale_log2);
        __builtin_amdgcn_sched_barrier(0);
        ctx.load(ta, tw + kIter * (it + 2));
        __builtin_amdgcn_sched_barrier(0);
        if (it + 1 < niter)
            mfma_compute<T, kWaves, true>(st, tb, qf, klds, vlds, w, t0 + kIter, t_end, lim_eff,
                                          t_full, g, i, a.scale_log2);
        __builtin_amdgcn_sched_barrier(0);
    }
    st.l += shfl_xor(st.l, 16);
    st.l += shfl_xor(st.l, 32);

    if (!col_ok) return;
    const int np_row = (lim + a.part_tokens - 1) / a.part_tokens;
    if (p >= np_row) return;                     // none of this column's tokens are here
    if (np_row == 1) {
        const float inv = 1.f / st.l;            // l > 0: token 0 is visible to every row
#pragma unroll
        for (int k = 0; k < 8; ++k) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                store_elem<OutT>(a.out, ((size_t)row * a.Hq + head) * kHeadDim + 16 * k + 4 * g + r,
                                 st.o[k][r] * inv);
        }
    } else {
        const size_t idx = ((size_t)row * a.Hq + head) * a.max_parts + p;
        float *dst = a.part_o + idx * kHeadDim;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            *reinterpret_cast<float4 *>(dst + 16 * k + 4 * g) =
                make_float4(st.o[k][0], st.o[k][1], st.o[k][2], st.o[k][3]);
        if (g == 0) {
            a.part_m[idx] = st.m;
            a.part_l[idx] = st.l;
        }
    }
}

template <typename T, typename OutT, int G>
hipError_t launch_g(const Args &a, hipStream_t st) {
    const long long pairs = (long long)a.S * a.Hkv;
    const dim3 grid((unsigned)((pairs + kXcds - 1) / kXcds * kXcds * a.q_blocks), a.max_parts);
    const dim3 block(64 * kWaves);
    const bool scalar = a.B % 4 == 0;
    if (a.stream_kv) {
        if (scalar) hipLaunchKernelGGL((prefill_kernel<T, OutT, G, true, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((prefill_kernel<T, OutT, G, false, true>), grid, block, 0, st, a);
    } else {
        if (scalar) hipLaunchKernelGGL((prefill_kernel<T, OutT, G, true, false>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((prefill_kernel<T, OutT, G, false, false>), grid, block, 0, st, a);
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
