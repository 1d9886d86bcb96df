// Epilogues shared by the grouped expert GEMM kernels.
#pragma once

#include "device_common.h"

namespace colibri {

// What the GEMM's epilogue does with an accumulated value u (and, for SwiGLU,
// the matching W3 product v) at output column n of expert e.
enum Epi { EPI_ACT_RELU = 0, EPI_ACT_GELU = 1, EPI_SWIGLU = 2, EPI_BIAS_ONLY = 3 };

// (bf16 outputs only: the callers store the value rounded to bf16)
template <int EPI>
__device__ __forceinline__ float epi_value(float u, float v, const uint16_t *__restrict__ bias, int e, int N, int n) {
    if (EPI == EPI_SWIGLU) return silu_bf16out(u) * v;
    const float b = bias ? bf16_to_f32(bias[(size_t)e * N + n]) : 0.0f;
    if (EPI == EPI_ACT_RELU) return apply_act_bf16out<ACT_RELU>(u + b);
    if (EPI == EPI_ACT_GELU) return apply_act_bf16out<ACT_GELU>(u + b);
    return u + b;
}

// 8 consecutive output columns n..n+7 -> one 16-byte bf16 store (dst 16-byte aligned).
template <int EPI>
__device__ __forceinline__ void store_epilogue8(uint16_t *dst, const float (&u)[8], const float (&v)[8],
                                                const uint16_t *__restrict__ bias, int e, int N, int n) {
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q)
        o[q] = pack_bf16x2(epi_value<EPI>(u[2 * q], v[2 * q], bias, e, N, n + 2 * q),
                           epi_value<EPI>(u[2 * q + 1], v[2 * q + 1], bias, e, N, n + 2 * q + 1));
    *reinterpret_cast<u32x4 *>(dst) = o;
}

// CPL (2 or 4) consecutive output columns -> one 4- or 8-byte bf16 store.
template <int EPI, int CPL>
__device__ __forceinline__ void store_epilogue(uint16_t *dst, const float (&u)[CPL], const float (&v)[CPL],
                                               const uint16_t *__restrict__ bias, int e, int N, int n) {
    uint32_t w[CPL / 2];
#pragma unroll
    for (int q = 0; q < CPL / 2; ++q)
        w[q] = pack_bf16x2(epi_value<EPI>(u[2 * q], v[2 * q], bias, e, N, n + 2 * q),
                           epi_value<EPI>(u[2 * q + 1], v[2 * q + 1], bias, e, N, n + 2 * q + 1));
    if constexpr (CPL == 2) {
        *reinterpret_cast<uint32_t *>(dst) = w[0];
    } else {
        *reinterpret_cast<u32x2 *>(dst) = u32x2{w[0], w[1]};
    }
}

// i-th set bit of a 64-bit mask (wave-uniform loop)
__device__ __forceinline__ int nth_set_bit(uint64_t m, int i) {
    for (int q = 0; q < i; ++q) m &= m - 1;
    return __ffsll((unsigned long long)m) - 1;
}

// Live expert `slot` (experts with rows, in index order): e, first row, row count.
// Returns false when fewer experts are live.  Whole-wave call.
__device__ __forceinline__ bool live_expert(const int32_t *__restrict__ offsets, int E, int A_total, int slot,
                                            int &e, int &r0, int &count) {
    const int lane = threadIdx.x & (kWave - 1);
    int lo_l = 0, cnt_l = 0;
    if (lane < E) {
        lo_l = min(max(offsets[lane], 0), A_total);
        const int hi = min(max(offsets[lane + 1], lo_l), A_total);
        cnt_l = hi - lo_l;
    }
    const uint64_t live = __ballot(cnt_l > 0);
    if (__popcll(live) <= slot) return false;
    e = nth_set_bit(live, slot);
    r0 = __shfl(lo_l, e);
    count = __shfl(cnt_l, e);
    return true;
}

}  // namespace colibri
