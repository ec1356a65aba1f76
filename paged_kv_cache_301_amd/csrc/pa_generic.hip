// pa_generic.hip -- the plain paged decode-attention kernel.
//
// One wave64 per (sequence, query head).  Covers every shape the library
// accepts (D <= 512, any block size, any group size, fp32 / fp16 / bf16) and
// is the fallback where the tiled kernels do not apply.  It follows the
// incremental scheme of "Paged Attention > The PagedAttention Algorithm",
// section "Optimized CUDA Kernels": walk the context in logical order,
// translate each token through the block table, and keep a running maximum
// and running sum (online softmax) so no contiguous K / V copy is built.
//
// Per chunk of 64 tokens: lane i scores token c + i (dot product over D read
// straight from its physical slot), the chunk's max / weights update the
// running state, the weights go to LDS, and lanes then own head dimensions
// (d = lane + 64 k) to accumulate the weighted value rows.
//
// Multi-token (causal) calls run the same kernel over query rows: row r of
// sequence s attends the first lim tokens of s (pa_rows.h).
#include "pa_internal.h"
#include "pa_device.h"
#include "pa_rows.h"

namespace pa {

constexpr int kGenericMaxD = 512;

template <typename T, typename OutT>
__global__ __launch_bounds__(64) void generic_kernel(Args a) {
    const int h = blockIdx.x;
    const int r = blockIdx.y;                 // query row: sequence (decode) or token
    const int lane = threadIdx.x;
    const int D = a.D, B = a.B;
    const int kvh = h / (a.Hq / a.Hkv);
    int s = r, L;
    if (a.query_start) {
        const QueryRow qr = query_row(a, r);
        s = qr.s;
        L = qr.lim;
    } else {
        L = a.seq_lens[s];
    }
    const int32_t *table = a.block_tables + (size_t)s * a.max_blocks;
    const size_t head_stride = (size_t)B * D;             // one (block, kv head) tile
    const size_t block_stride = (size_t)a.Hkv * head_stride;

    __shared__ float q_s[kGenericMaxD];
    __shared__ float p_s[64];
    for (int d = lane; d < D; d += 64)
        q_s[d] = Elem<T>::load(a.query, ((size_t)r * a.Hq + h) * D + d);
    __syncthreads();

    float o[kGenericMaxD / 64];
#pragma unroll
    for (int k = 0; k < kGenericMaxD / 64; ++k) o[k] = 0.f;
    float m = kNegInf, l = 0.f;

    for (int c = 0; c < L; c += 64) {
        const int t = c + lane;
        float x = kNegInf;
        if (t < L) {
            const int phys = table[t / B];
            const size_t base = (size_t)phys * block_stride + kvh * head_stride + (size_t)(t % B) * D;
            float acc = 0.f;
            for (int d = 0; d < D; ++d) acc += q_s[d] * Elem<T>::load(a.key_cache, base + d);
            x = acc * a.scale_log2;
        }
        const float mn = fmaxf(m, wave_max(x));      // finite: token c is valid
        const float alpha = fast_exp2(m - mn);
        const float p = (t < L) ? fast_exp2(x - mn) : 0.f;
        l = l * alpha + wave_sum(p);
        m = mn;
        p_s[lane] = p;
        __syncthreads();
        const int n = min(64, L - c);
#pragma unroll
        for (int k = 0; k < kGenericMaxD / 64; ++k) {
            const int d = lane + 64 * k;
            if (d < D) {
                float acc = o[k] * alpha;
                for (int j = 0; j < n; ++j) {
                    const int tt = c + j;
                    const int phys = table[tt / B];
                    const size_t base = (size_t)phys * block_stride + kvh * head_stride + (size_t)(tt % B) * D;
                    acc += p_s[j] * Elem<T>::load(a.value_cache, base + d);
                }
                o[k] = acc;
            }
        }
        __syncthreads();
    }

    const float inv = (L > 0) ? 1.f / l : 0.f;
#pragma unroll
    for (int k = 0; k < kGenericMaxD / 64; ++k) {
        const int d = lane + 64 * k;
        if (d < D) store_elem<OutT>(a.out, ((size_t)r * a.Hq + h) * D + d, o[k] * inv);
    }
}

template <typename T, typename OutT>
static hipError_t launch_generic_t(const Args &a, hipStream_t st) {
    dim3 grid(a.Hq, a.query_start ? a.T : a.S);
    hipLaunchKernelGGL((generic_kernel<T, OutT>), grid, dim3(64), 0, st, a);
    return hipGetLastError();
}

hipError_t launch_generic(const Args &a, pa_dtype dt, pa_dtype odt, hipStream_t st) {
    if (a.D > kGenericMaxD) return hipErrorInvalidValue;
    const bool f32out = (odt == PA_F32);
    switch (dt) {
    case PA_F32:
        return launch_generic_t<float, float>(a, st);
    case PA_F16:
        return f32out ? launch_generic_t<_Float16, float>(a, st)
                      : launch_generic_t<_Float16, _Float16>(a, st);
    case PA_BF16:
        return f32out ? launch_generic_t<__bf16, float>(a, st)
                      : launch_generic_t<__bf16, __bf16>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace pa
