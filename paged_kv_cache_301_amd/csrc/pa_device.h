// pa_device.h -- device-side helpers for the gfx950 kernels: element types,
// conversions, wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace pa {

using u16 = unsigned short;
using f16x2 = _Float16 __attribute__((ext_vector_type(2)));
using bf16x2 = __bf16 __attribute__((ext_vector_type(2)));
using f16x8 = _Float16 __attribute__((ext_vector_type(8)));
using bf16x8 = __bf16 __attribute__((ext_vector_type(8)));
using f32x4 = float __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

template <typename To, typename From>
__device__ __forceinline__ To bitcast(From x) {
    static_assert(sizeof(To) == sizeof(From), "size mismatch");
    return __builtin_bit_cast(To, x);
}

using u32x4 = unsigned __attribute__((ext_vector_type(4)));

// 16-byte load with the non-temporal hint: K / V rows are read once per call,
// so they should not displace other lines in L2 / MALL (on MI355X this also
// lifts the attainable streaming read rate from about 6.1 to 7.0 TB/s).
__device__ __forceinline__ uint4 load_stream16(const void *p) {
    const u32x4 v = __builtin_nontemporal_load(static_cast<const u32x4 *>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// 16-byte load of K / V: streamed (non-temporal) or cached.
template <bool STREAM>
__device__ __forceinline__ uint4 load_kv16(const void *p) {
    if constexpr (STREAM) return load_stream16(p);
    else return *static_cast<const uint4 *>(p);
}

// exp2 on the transcendental unit (v_exp_f32): exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- elements
// Per-type operations on one 32-bit word holding two packed 16-bit values
// (element 2i in the low half, 2i+1 in the high half).
template <typename T> struct Elem;

template <> struct Elem<_Float16> {
    __device__ static float lo(uint32_t w) { return (float)bitcast<f16x2>(w)[0]; }
    __device__ static float hi(uint32_t w) { return (float)bitcast<f16x2>(w)[1]; }
    // c + a.lo * b.lo + a.hi * b.hi, fp32 accumulate (v_dot2_f32_f16)
    __device__ static float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2(bitcast<f16x2>(a), bitcast<f16x2>(b), c, false);
    }
    __device__ static float load(const void *p, size_t i) {
        return (float)static_cast<const _Float16 *>(p)[i];
    }
    __device__ static uint32_t pack(float a, float b) {  // round to nearest even
        f16x2 v = {(_Float16)a, (_Float16)b};
        return bitcast<uint32_t>(v);
    }
};

template <> struct Elem<__bf16> {
    // a bfloat16 is the upper half of an fp32
    __device__ static float lo(uint32_t w) { return bitcast<float>(w << 16); }
    __device__ static float hi(uint32_t w) { return bitcast<float>(w & 0xffff0000u); }
    // c + a.lo * b.lo + a.hi * b.hi, fp32 accumulate (v_dot2_f32_bf16)
    __device__ static float dot2(uint32_t a, uint32_t b, float c) {
        return __builtin_amdgcn_fdot2_f32_bf16(bitcast<bf16x2>(a), bitcast<bf16x2>(b), c, false);
    }
    __device__ static float load(const void *p, size_t i) {
        return bitcast<float>((uint32_t)static_cast<const u16 *>(p)[i] << 16);
    }
    __device__ static uint32_t pack(float a, float b) {  // round to nearest even
        bf16x2 v = {(__bf16)a, (__bf16)b};
        return bitcast<uint32_t>(v);
    }
};

template <> struct Elem<float> {
    __device__ static float load(const void *p, size_t i) {
        return static_cast<const float *>(p)[i];
    }
};

// Store one float as element i of an array of OutT.
template <typename OutT> __device__ __forceinline__ void store_elem(void *p, size_t i, float v);
template <> __device__ __forceinline__ void store_elem<float>(void *p, size_t i, float v) {
    static_cast<float *>(p)[i] = v;
}
template <> __device__ __forceinline__ void store_elem<_Float16>(void *p, size_t i, float v) {
    static_cast<_Float16 *>(p)[i] = (_Float16)v;
}
template <> __device__ __forceinline__ void store_elem<__bf16>(void *p, size_t i, float v) {
    static_cast<__bf16 *>(p)[i] = (__bf16)v;
}

// Store 8 consecutive floats (16-byte aligned destination for 16-bit types,
// 32-byte for fp32) as OutT.
template <typename OutT> __device__ __forceinline__ void store8(void *p, const float (&v)[8]);
template <> __device__ __forceinline__ void store8<float>(void *p, const float (&v)[8]) {
    float4 *d = static_cast<float4 *>(p);
    d[0] = make_float4(v[0], v[1], v[2], v[3]);
    d[1] = make_float4(v[4], v[5], v[6], v[7]);
}
template <typename OutT> __device__ __forceinline__ void store8(void *p, const float (&v)[8]) {
    uint4 w;
    w.x = Elem<OutT>::pack(v[0], v[1]);
    w.y = Elem<OutT>::pack(v[2], v[3]);
    w.z = Elem<OutT>::pack(v[4], v[5]);
    w.w = Elem<OutT>::pack(v[6], v[7]);
    *static_cast<uint4 *>(p) = w;
}

// ------------------------------------------------------------- cross-lane
// DPP move: lane i reads `x` from the lane the control word names.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return bitcast<float>(__builtin_amdgcn_update_dpp(0, bitcast<int>(x), CTRL, 0xF, 0xF, false));
}
constexpr int kQuadXor1 = 0xB1;      // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;      // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over each row of 16 lanes; every lane of the row receives the total.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp<kQuadXor1>(x);
    x += dpp<kQuadXor2>(x);
    x += dpp<kRowHalfMirror>(x);   // lane i <-> 7-i within each half row
    x += dpp<kRowMirror>(x);       // lane i <-> 15-i within the row
    return x;
}

__device__ __forceinline__ float shfl_xor(float x, int m) {
    return __shfl_xor(x, m, 64);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, shfl_xor(x, m));
    return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += shfl_xor(x, m);
    return x;
}

// Merge two online-softmax states (m: running max in exp2 units, l: sum of
// weights, o: weighted value sum), either of which may be empty (m = -inf).
__device__ __forceinline__ void merge_state(float &m, float &l, float *o, int n,
                                            float m2, float l2, const float *o2) {
    const float mn = fmaxf(m, m2);
    const float ms = (mn == kNegInf) ? 0.f : mn;
    const float a = fast_exp2(m - ms);
    const float b = fast_exp2(m2 - ms);
    l = l * a + l2 * b;
    for (int i = 0; i < n; ++i) o[i] = o[i] * a + o2[i] * b;
    m = mn;
}

}  // namespace pa
