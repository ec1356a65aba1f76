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
// One 256-thread work-group per (sequence, head): thread t owns output
// columns 4 (t % 32) .. +3 and partitions t / 32, t / 32 + 8, ..., merged
// online, so every partial row is read with full-width 16-byte loads and all
// partitions are in flight at once; the eight group states meet in LDS.
//
// Multi-token (causal) calls combine per query row: row r attends lim tokens
// (pa_rows.h) and has ceil(lim / P) partitions.
#include "pa_internal.h"
#include "pa_device.h"
#include "pa_rows.h"

namespace pa {

namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;
constexpr int kCols = kD / 4;                 // float4 columns per row
constexpr int kGroups = kThreads / kCols;     // partitions handled in parallel

template <typename OutT>
__global__ __launch_bounds__(kThreads) void combine_kernel(Args a) {
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

    __shared__ float4 acc_s[kGroups][kCols];
    __shared__ float m_s[kGroups];
    __shared__ float z_s[kGroups];

    // Each group of 32 threads merges partitions grp, grp + 8, ... online
    // (running max), so no pass over the maxima precedes the loads.
    const int c = t % kCols;
    const int grp = t / kCols;
    float m = kNegInf, z = 0.f;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p = grp; p < np; p += kGroups) {
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
    for (int k = 0; k < kGroups; ++k) M = fmaxf(M, m_s[k]);
    float4 r = make_float4(0.f, 0.f, 0.f, 0.f);
    float Z = 0.f;
#pragma unroll
    for (int k = 0; k < kGroups; ++k) {
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
    dim3 grid(a.Hq, a.query_start ? a.T : a.S);
    switch (odt) {
    case PA_F32: hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(kThreads), 0, st, a); break;
    case PA_F16: hipLaunchKernelGGL(combine_kernel<_Float16>, grid, dim3(kThreads), 0, st, a); break;
    case PA_BF16: hipLaunchKernelGGL(combine_kernel<__bf16>, grid, dim3(kThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pa
