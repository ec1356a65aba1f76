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
// One wave64 per (sequence, head): lanes first own partitions (max and
// weights, staged in LDS 64 at a time), then own head dimensions for the
// weighted sum of the o_p rows.
#include "pa_internal.h"
#include "pa_device.h"

namespace pa {

namespace {

constexpr int kMaxD = 512;

template <typename OutT>
__global__ __launch_bounds__(64) void combine_kernel(Args a) {
    const int h = blockIdx.x;
    const int s = blockIdx.y;
    const int lane = threadIdx.x;
    const int D = a.D;
    const int L = a.seq_lens[s];
    const int np = (L + a.part_tokens - 1) / a.part_tokens;
    if (np <= 1) return;

    const size_t row = (size_t)s * a.Hq + h;
    const float *pm = a.part_m + row * a.max_parts;
    const float *pl = a.part_l + row * a.max_parts;
    const float *po = a.part_o + row * a.max_parts * D;

    float M = kNegInf;
    for (int p = lane; p < np; p += 64) M = fmaxf(M, pm[p]);
    M = wave_max(M);

    __shared__ float w_s[64];
    float acc[kMaxD / 64];
#pragma unroll
    for (int k = 0; k < kMaxD / 64; ++k) acc[k] = 0.f;
    float Z = 0.f;
    for (int p0 = 0; p0 < np; p0 += 64) {
        const int p = p0 + lane;
        float w = 0.f;
        if (p < np) {
            w = fast_exp2(pm[p] - M);
            Z += w * pl[p];
        }
        w_s[lane] = w;
        __syncthreads();
        const int n = min(64, np - p0);
#pragma unroll
        for (int k = 0; k < kMaxD / 64; ++k) {
            const int d = lane + 64 * k;
            if (d < D) {
                float sum = acc[k];
#pragma unroll 8
                for (int j = 0; j < n; ++j) sum = fmaf(w_s[j], po[(size_t)(p0 + j) * D + d], sum);
                acc[k] = sum;
            }
        }
        __syncthreads();
    }
    Z = wave_sum(Z);
    const float inv = 1.f / Z;
#pragma unroll
    for (int k = 0; k < kMaxD / 64; ++k) {
        const int d = lane + 64 * k;
        if (d < D) store_elem<OutT>(a.out, row * D + d, acc[k] * inv);
    }
}

}  // namespace

hipError_t launch_combine(const Args &a, pa_dtype odt, hipStream_t st) {
    if (a.D > kMaxD) return hipErrorInvalidValue;
    dim3 grid(a.Hq, a.S);
    switch (odt) {
    case PA_F32: hipLaunchKernelGGL(combine_kernel<float>, grid, dim3(64), 0, st, a); break;
    case PA_F16: hipLaunchKernelGGL(combine_kernel<_Float16>, grid, dim3(64), 0, st, a); break;
    case PA_BF16: hipLaunchKernelGGL(combine_kernel<__bf16>, grid, dim3(64), 0, st, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace pa
