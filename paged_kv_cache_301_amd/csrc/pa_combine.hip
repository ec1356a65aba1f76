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
// columns 4 (t % 32) .. +3 and partitions t / 32, t / 32 + 8, ..., so every
// partial row is read with full-width 16-byte loads and all partitions are in
// flight at once; the eight partial sums meet in LDS.
#include "pa_internal.h"
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kD = 128;
constexpr int kThreads = 256;
constexpr int kCols = kD / 4;                 // float4 columns per row
constexpr int kGroups = kThreads / kCols;     // partitions handled in parallel

template <typename OutT>
__global__ __launch_bounds__(kThreads) void combine_kernel(Args a) {
    const int h = blockIdx.x;
    const int s = blockIdx.y;
    const int t = threadIdx.x;
    const int L = a.seq_lens[s];
    const int np = (L + a.part_tokens - 1) / a.part_tokens;
    if (np <= 1) return;

    const size_t row = (size_t)s * a.Hq + h;
    const float *pm = a.part_m + row * a.max_parts;
    const float *pl = a.part_l + row * a.max_parts;
    const float4 *po = reinterpret_cast<const float4 *>(a.part_o + row * a.max_parts * kD);

    __shared__ float red[kThreads / 64];
    __shared__ float4 acc_s[kGroups][kCols];
    __shared__ float z_s[kGroups];

    // M = max over partitions
    float M = kNegInf;
    for (int p = t; p < np; p += kThreads) M = fmaxf(M, pm[p]);
    M = wave_max(M);
    if ((t & 63) == 0) red[t >> 6] = M;
    __syncthreads();
    M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

    const int c = t % kCols;
    const int grp = t / kCols;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float z = 0.f;
    for (int p = grp; p < np; p += kGroups) {
        const float w = fast_exp2(pm[p] - M);
        const float4 o = po[(size_t)p * kCols + c];
        acc.x = fmaf(w, o.x, acc.x);
        acc.y = fmaf(w, o.y, acc.y);
        acc.z = fmaf(w, o.z, acc.z);
        acc.w = fmaf(w, o.w, acc.w);
        z = fmaf(w, pl[p], z);
    }
    acc_s[grp][c] = acc;
    if (c == 0) z_s[grp] = z;
    __syncthreads();
    if (grp != 0) return;
#pragma unroll
    for (int g = 1; g < kGroups; ++g) {
        const float4 o = acc_s[g][c];
        acc.x += o.x;
        acc.y += o.y;
        acc.z += o.z;
        acc.w += o.w;
    }
    float Z = 0.f;
#pragma unroll
    for (int g = 0; g < kGroups; ++g) Z += z_s[g];
    const float inv = 1.f / Z;
    const size_t base = row * kD + 4 * c;
    store_elem<OutT>(a.out, base + 0, acc.x * inv);
    store_elem<OutT>(a.out, base + 1, acc.y * inv);
    store_elem<OutT>(a.out, base + 2, acc.z * inv);
    store_elem<OutT>(a.out, base + 3, acc.w * inv);
}

}  // namespace

hipError_t launch_combine(const Args &a, pa_dtype odt, hipStream_t st) {
    if (a.D != kD) return hipErrorInvalidValue;
    dim3 grid(a.Hq, a.S);
    switch (odt) {
    case PA_F32: hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(kThreads), 0, st, a); break;
    case PA_F16: hipLaunchKernelGGL(combine_kernel<_Float16>, grid, dim3(kThreads), 0, st, a); break;
    case PA_BF16: hipLaunchKernelGGL(combine_kernel<__bf16>, grid, dim3(kThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pa
