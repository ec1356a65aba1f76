// pa_combine.hip -- merge per-partition softmax states into the output.
//
// A split plan cuts each context into partitions of P tokens; partition p of
// (sequence s, head h) leaves m_p (its max score, exp2 units), l_p (sum of
// exp2(x - m_p)) and o_p (sum of exp2(x - m_p) * V).  The exact result is
//     M = max_p m_p,   out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p,
// the same rescaling the online softmax applies block by block ("Paged
// Attention > The PagedAttention Algorithm", section "Optimized CUDA
// Kernels": running maximum and running sum, combined without a contiguous
// buffer).  Sequences that fit one partition were written directly by the
// partition kernel and are skipped here.
//
// Rows of up to 8 partitions (most decode plans): one wave per (sequence,
// head) row, four rows per 256-thread work-group; lane l owns output columns
// 4 (l % 32) .. +3 and every other partition (l / 32, l / 32 + 2, ...),
// merged online with a running max, and the two halves of the wave merge
// through a cross-lane exchange.  Longer rows: one 256-thread work-group per
// row, thread t owns columns 4 (t % 32) .. +3 and partitions t / 32,
// t / 32 + 8, ..., and the eight group states meet in LDS, so eight partial
// rows are in flight at once.  Either way every partial row is read with
// full-width 16-byte loads.  (Measured: the one-wave form cut the combine
// from 8.4 to 6.9 us on gqa_70b and from 13 to 9.7 us on multi-query, and
// was slower on gqa_long's 32-partition rows, 9.9 against 6.8 us.)
//
// Multi-token (causal) calls combine per query row: row r attends lim tokens
// (pa_rows.h) and has ceil(lim / P) partitions.
#include "pa_internal.h"
#include "pa_device.h"
#include "pa_rows.h"

namespace pa {

namespace {

constexpr int kD = 128;
constexpr int kRowsPerGroup = 4;              // one wave per row
constexpr int kCols = kD / 4;                 // float4 columns per row (32)
constexpr int kWideThreads = 256;             // long rows: one work-group per row
constexpr int kWideGroups = kWideThreads / kCols;
constexpr int kWideFrom = 16;                 // max partitions from which rows go wide

template <typename OutT>
__global__ __launch_bounds__(64 * kRowsPerGroup) void combine_kernel(Args a) {
    const int h = blockIdx.x;
    const int qrow = blockIdx.y * kRowsPerGroup + (threadIdx.x >> 6);   // sequence or query row
    const int nrows = a.query_start ? a.T : a.S;
    if (qrow >= nrows) return;                 // uniform per wave
    const int L = a.query_start ? query_row(a, qrow).lim : a.seq_lens[qrow];
    const int np = (L + a.part_tokens - 1) / a.part_tokens;
    if (np <= 1) return;                       // finished by the partition kernel

    const int lane = threadIdx.x & 63;
    const int c = lane & (kCols - 1);
    const int half = lane >> 5;
    const size_t row = (size_t)qrow * a.Hq + h;
    const float *pm = a.part_m + row * a.max_parts;
    const float *pl = a.part_l + row * a.max_parts;
    const float4 *po = reinterpret_cast<const float4 *>(a.part_o + row * a.max_parts * kD);

    float m = kNegInf, z = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = half; p < np; p += 2) {
        const float mp = pm[p];
        const float lp = pl[p];
        const float4 o = po[(size_t)p * kCols + c];
        const float mn = fmaxf(m, mp);          // finite: every partition holds a token
        const float wa = fast_exp2(m - mn);     // 0 on the first partition
        const float wb = fast_exp2(mp - mn);
        z = z * wa + lp * wb;
        acc.x = acc.x * wa + o.x * wb;
        acc.y = acc.y * wa + o.y * wb;
        acc.z = acc.z * wa + o.z * wb;
        acc.w = acc.w * wa + o.w * wb;
        m = mn;
    }
    // merge the two halves (np >= 2: both hold at least one partition)
    const float m2 = shfl_xor(m, 32);
    const float z2 = shfl_xor(z, 32);
    const float4 acc2 = make_float4(shfl_xor(acc.x, 32), shfl_xor(acc.y, 32),
                                    shfl_xor(acc.z, 32), shfl_xor(acc.w, 32));
    if (half != 0) return;
    const float M = fmaxf(m, m2);
    const float wa = fast_exp2(m - M), wb = fast_exp2(m2 - M);
    const float inv = 1.f / (z * wa + z2 * wb);
    const size_t base = row * kD + 4 * c;
    store_elem<OutT>(a.out, base + 0, (acc.x * wa + acc2.x * wb) * inv);
    store_elem<OutT>(a.out, base + 1, (acc.y * wa + acc2.y * wb) * inv);
    store_elem<OutT>(a.out, base + 2, (acc.z * wa + acc2.z * wb) * inv);
    store_elem<OutT>(a.out, base + 3, (acc.w * wa + acc2.w * wb) * inv);
}

template <typename OutT>
__global__ __launch_bounds__(kWideThreads) void combine_wide_kernel(Args a) {
    const int h = blockIdx.x;
    const int qrow = blockIdx.y;               // sequence (decode) or query row
    const int t = threadIdx.x;
    const int L = a.query_start ? query_row(a, qrow).lim : a.seq_lens[qrow];
    const int np = (L + a.part_tokens - 1) / a.part_tokens;
    if (np <= 1) return;

    const size_t row = (size_t)qrow * a.Hq + h;
    const float *pm = a.part_m + row * a.max_parts;
    const float *pl = a.part_l + row * a.max_parts;
    const float4 *po = reinterpret_cast<const float4 *>(a.part_o + row * a.max_parts * kD);

    __shared__ float4 acc_s[kWideGroups][kCols];
    __shared__ float m_s[kWideGroups];
    __shared__ float z_s[kWideGroups];

    // Each group of 32 threads merges partitions grp, grp + 8, ... online
    // (running max), so no pass over the maxima precedes the loads.
    const int c = t % kCols;
    const int grp = t / kCols;
    float m = kNegInf, z = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = grp; p < np; p += kWideGroups) {
        const float mp = pm[p];
        const float lp = pl[p];
        const float4 o = po[(size_t)p * kCols + c];
        const float mn = fmaxf(m, mp);          // finite: every partition holds a token
        const float wa = fast_exp2(m - mn);     // 0 on the first partition
        const float wb = fast_exp2(mp - mn);
        z = z * wa + lp * wb;
        acc.x = acc.x * wa + o.x * wb;
        acc.y = acc.y * wa + o.y * wb;
        acc.z = acc.z * wa + o.z * wb;
        acc.w = acc.w * wa + o.w * wb;
        m = mn;
    }
    acc_s[grp][c] = acc;
    if (c == 0) {
        m_s[grp] = m;
        z_s[grp] = z;
    }
    __syncthreads();
    if (grp != 0) return;
    float M = kNegInf;
#pragma unroll
    for (int k = 0; k < kWideGroups; ++k) M = fmaxf(M, m_s[k]);
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    float Z = 0.f;
#pragma unroll
    for (int k = 0; k < kWideGroups; ++k) {
        const float w = fast_exp2(m_s[k] - M);  // groups without partitions: m = -inf, w = 0
        const float4 o = acc_s[k][c];
        r.x += w * o.x;
        r.y += w * o.y;
        r.z += w * o.z;
        r.w += w * o.w;
        Z += w * z_s[k];
    }
    const float inv = 1.f / Z;
    const size_t base = row * kD + 4 * c;
    store_elem<OutT>(a.out, base + 0, r.x * inv);
    store_elem<OutT>(a.out, base + 1, r.y * inv);
    store_elem<OutT>(a.out, base + 2, r.z * inv);
    store_elem<OutT>(a.out, base + 3, r.w * inv);
}

}  // namespace

hipError_t launch_combine(const Args &a, pa_dtype odt, hipStream_t st) {
    if (a.D != kD) return hipErrorInvalidValue;
    const int nrows = a.query_start ? a.T : a.S;
    if (a.max_parts >= kWideFrom) {
        const dim3 grid(a.Hq, nrows);
        switch (odt) {
        case PA_F32: hipLaunchKernelGGL(combine_wide_kernel<float>, grid, dim3(kWideThreads), 0, st, a); break;
        case PA_F16: hipLaunchKernelGGL(combine_wide_kernel<_Float16>, grid, dim3(kWideThreads), 0, st, a); break;
        case PA_BF16: hipLaunchKernelGGL(combine_wide_kernel<__bf16>, grid, dim3(kWideThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
    const dim3 grid(a.Hq, (nrows + kRowsPerGroup - 1) / kRowsPerGroup);
    const dim3 block(64 * kRowsPerGroup);
    switch (odt) {
    case PA_F32: hipLaunchKernelGGL(combine_kernel<float>, grid, block, 0, st, a); break;
    case PA_F16: hipLaunchKernelGGL(combine_kernel<_Float16>, grid, block, 0, st, a); break;
    case PA_BF16: hipLaunchKernelGGL(combine_kernel<__bf16>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pa
