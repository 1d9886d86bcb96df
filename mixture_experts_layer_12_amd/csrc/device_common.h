// Device-side helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace colibri {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// bf16 <-> fp32.  Widening is exact; narrowing rounds to nearest, ties to even.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// Narrowing uses gfx950's v_cvt_pk_bf16_f32 (round to nearest, ties to even;
// a NaN stays a quiet NaN): checked on the GPU against the integer rounding
// u + 0x7fff + (bit 16 of u), truncated, with NaN quieted by setting bit 6 of
// the result, over all 2^32 inputs -- identical bits everywhere.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) { return pack_bf16x2(f, 0.0f) & 0xffffu; }

// Element load/store for the two storage types.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float *p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void store(float *p, size_t i, float v) { p[i] = v; }
};
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t *p, size_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void store(uint16_t *p, size_t i, float v) {
        p[i] = (uint16_t)f32_to_bf16_bits(v);
    }
};

// 16-byte vector of a row: 4 fp32 or 8 bf16, widened to fp32.
template <typename T> struct Vec16;
template <> struct Vec16<float> {
    static constexpr int N = 4;
    static __device__ __forceinline__ void load(const float *p, float (&o)[4]) {
        f32x4 v = *reinterpret_cast<const f32x4 *>(p);
        o[0] = v[0]; o[1] = v[1]; o[2] = v[2]; o[3] = v[3];
    }
};
template <> struct Vec16<uint16_t> {
    static constexpr int N = 8;
    static __device__ __forceinline__ void load(const uint16_t *p, float (&o)[8]) {
        u32x4 v = *reinterpret_cast<const u32x4 *>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) { o[2 * i] = bf16_lo(v[i]); o[2 * i + 1] = bf16_hi(v[i]); }
    }
};

enum Act { ACT_RELU = 0, ACT_GELU = 1, ACT_SWIGLU = 2 };

__device__ __forceinline__ float gelu_erf(float z) { return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f)); }
__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }
// silu for results stored in bf16: 2^(-z log2 e) on v_exp_f32 and one
// v_rcp_f32 instead of the library exp and an IEEE division (relative error
// about 1e-6, far below the 2^-9 rounding step of the bf16 store)
__device__ __forceinline__ float silu_bf16out(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

// GELU for results stored in bf16: erf from Hastings' rational approximation
// (Abramowitz & Stegun, Handbook of Mathematical Functions, 7.1.26; absolute
// error at most 1.5e-7), with 1 + erf(z / sqrt 2) formed as q or 2 - q from
// q = erfc(|z| / sqrt 2), so negative z loses nothing to cancellation; one
// v_rcp_f32 and one v_exp_f32, about half the instructions of the library
// erff and far below the 2^-9 rounding step of the bf16 store.
__device__ __forceinline__ float gelu_bf16out(float z) {
    constexpr double kInvSqrt2 = 0.70710678118654752;
    constexpr float p = (float)(0.3275911 * kInvSqrt2);  // t = 1 / (1 + p x), x = |z| / sqrt 2
    constexpr float a1 = 0.254829592f, a2 = -0.284496736f, a3 = 1.421413741f, a4 = -1.453152027f,
                    a5 = 1.061405429f;
    constexpr float c = -0.72134752044448170f;  // exp(-x^2) = 2^(c z^2), c = -log2(e) / 2
    const float t = __builtin_amdgcn_rcpf(fmaf(p, fabsf(z), 1.0f));
    const float poly = t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, a5, a4), a3), a2), a1);
    const float q = poly * __builtin_amdgcn_exp2f(c * z * z);  // erfc(|z| / sqrt 2)
    return 0.5f * z * (z >= 0.0f ? 2.0f - q : q);
}

template <int ACT>
__device__ __forceinline__ float apply_act(float z) {
    if (ACT == ACT_RELU) return z > 0.0f ? z : 0.0f;
    return gelu_erf(z);
}
// the same for results stored in bf16
template <int ACT>
__device__ __forceinline__ float apply_act_bf16out(float z) {
    if (ACT == ACT_RELU) return z > 0.0f ? z : 0.0f;
    return gelu_bf16out(z);
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace colibri
