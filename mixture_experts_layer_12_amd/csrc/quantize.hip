// Per-column int8 quantization of expert weights.
//
// Colibri write-up [zskr] http://www.zskr.cn/news/2272131 section 5.3: the
// expert weights are quantized to INT8 per channel, with the scales stored
// beside them, halving the weight bytes the layer streams.  Here a channel is
// an output column n of one expert e (the dimension the layer's sums run
// along is k), and the scale is symmetric:
//   amax = max_k |w[e][k][n]|,  s = amax / 127 (1 for an all-zero column),
//   q = round_to_nearest_even(w / s), clamped to [-127, 127],
// all in fp32 (IEEE division, as the reference quantizer does it).
//
// One thread owns 4 adjacent columns of one expert: a first pass over k finds
// the 4 maxima, a second writes the codes as one 32-bit store per k-row.
// Neighbouring threads own neighbouring columns, so every k-row is read and
// written in contiguous runs.
//
// 4-bit codes with a zero point ([rkmt] http://news.rkmt.cn/news/2271114
// section 4.2: AWQ 4-bit weights, quantization group 128, zero point): a group
// is 128 consecutive k of one column n; in fp32, with the group's largest and
// smallest weight mx, mn:
//   s = max(mx - mn, 1e-5) / 15,  z = -rint(mn / s) clamped to [0, 15],
//   q = rint(w / s) + z clamped to [0, 15]   (rint: ties to even).
// One thread owns 4 adjacent columns of one group: a first pass finds the
// extremes, a second writes the codes packed 8 k to a 32-bit word (word j: the
// code of k = 8j + 2m in bits 4m .. 4m+3, of k = 8j + 2m + 1 in bits 16 + 4m ..
// 16 + 4m + 3), one 16-byte store per 8 k-rows.
#include "device_common.h"
#include "launchers.h"

namespace colibri {
namespace {

template <typename TI>
__device__ __forceinline__ void load4(const TI *p, float (&v)[4]);
template <>
__device__ __forceinline__ void load4<float>(const float *p, float (&v)[4]) {
    const f32x4 x = *reinterpret_cast<const f32x4 *>(p);
    v[0] = x[0], v[1] = x[1], v[2] = x[2], v[3] = x[3];
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t *p, float (&v)[4]) {
    const u32x2 x = *reinterpret_cast<const u32x2 *>(p);
    v[0] = bf16_to_f32((uint16_t)(x[0] & 0xffffu)), v[1] = bf16_to_f32((uint16_t)(x[0] >> 16));
    v[2] = bf16_to_f32((uint16_t)(x[1] & 0xffffu)), v[3] = bf16_to_f32((uint16_t)(x[1] >> 16));
}

template <typename TI>
__global__ __launch_bounds__(256) void quantize_q8_kernel(const TI *__restrict__ w, int E, int K, int N,
                                                          int8_t *__restrict__ q, float *__restrict__ scale) {
    const int NG = N / 4;
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)E * NG) return;
    const int e = (int)(i / NG), n = (int)(i % NG) * 4;
    const size_t base = (size_t)e * K * N + n;
    float amax[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < K; ++k) {
        float v[4];
        load4<TI>(w + base + (size_t)k * N, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) amax[j] = fmaxf(amax[j], fabsf(v[j]));
    }
    float s[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s[j] = amax[j] > 0.0f ? amax[j] / 127.0f : 1.0f;
        scale[(size_t)e * N + n + j] = s[j];
    }
    for (int k = 0; k < K; ++k) {
        float v[4];
        load4<TI>(w + base + (size_t)k * N, v);
        uint32_t packed = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float r = fminf(fmaxf(rintf(v[j] / s[j]), -127.0f), 127.0f);
            packed |= ((uint32_t)(int32_t)r & 0xffu) << (8 * j);
        }
        *reinterpret_cast<uint32_t *>(q + base + (size_t)k * N) = packed;
    }
}

template <typename TI>
__global__ __launch_bounds__(256) void quantize_q4_kernel(const TI *__restrict__ w, int E, int K, int N,
                                                          uint32_t *__restrict__ q, float *__restrict__ scale,
                                                          uint8_t *__restrict__ zero) {
    constexpr int GK = 128;  // k per group
    const int NG = N / 4, G = K / GK;
    const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (long)E * G * NG) return;
    const int e = (int)(i / ((long)G * NG)), g = (int)((i / NG) % G), n = (int)(i % NG) * 4;
    const TI *src = w + (size_t)e * K * N + (size_t)g * GK * N + n;
    float mx[4], mn[4];
    load4<TI>(src, mx);
#pragma unroll
    for (int j = 0; j < 4; ++j) mn[j] = mx[j];
    for (int k = 1; k < GK; ++k) {
        float v[4];
        load4<TI>(src + (size_t)k * N, v);
#pragma unroll
        for (int j = 0; j < 4; ++j) mx[j] = fmaxf(mx[j], v[j]), mn[j] = fminf(mn[j], v[j]);
    }
    float s[4], z[4];
    uint32_t zw = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        s[j] = fmaxf(mx[j] - mn[j], 1e-5f) / 15.0f;
        z[j] = fminf(fmaxf(-rintf(mn[j] / s[j]), 0.0f), 15.0f);
        zw |= (uint32_t)z[j] << (8 * j);
    }
    const size_t gi = ((size_t)e * G + g) * N + n;
    *reinterpret_cast<f32x4 *>(scale + gi) = f32x4{s[0], s[1], s[2], s[3]};
    *reinterpret_cast<uint32_t *>(zero + gi) = zw;
    for (int kb = 0; kb < GK / 8; ++kb) {
        u32x4 words = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            float v[4];
            load4<TI>(src + (size_t)(8 * kb + t) * N, v);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float r = fminf(fmaxf(rintf(v[j] / s[j]) + z[j], 0.0f), 15.0f);
                words[j] |= (uint32_t)r << (4 * (t >> 1) + 16 * (t & 1));
            }
        }
        *reinterpret_cast<u32x4 *>(q + ((size_t)e * (K / 8) + (size_t)g * (GK / 8) + kb) * N + n) = words;
    }
}

}  // namespace

hipError_t launch_quantize_q8(const void *w, colibri_dtype_t dtype, int E, int K, int N, int8_t *q, float *scale,
                              hipStream_t st) {
    const long threads = (long)E * (N / 4);
    const int blocks = (int)((threads + 255) / 256);
    if (dtype == COLIBRI_F32)
        quantize_q8_kernel<float><<<blocks, 256, 0, st>>>(static_cast<const float *>(w), E, K, N, q, scale);
    else
        quantize_q8_kernel<uint16_t><<<blocks, 256, 0, st>>>(static_cast<const uint16_t *>(w), E, K, N, q, scale);
    return hipGetLastError();
}

hipError_t launch_quantize_q4(const void *w, colibri_dtype_t dtype, int E, int K, int N, uint32_t *q, float *scale,
                              uint8_t *zero, hipStream_t st) {
    const long threads = (long)E * (K / 128) * (N / 4);
    const int blocks = (int)((threads + 255) / 256);
    if (dtype == COLIBRI_F32)
        quantize_q4_kernel<float><<<blocks, 256, 0, st>>>(static_cast<const float *>(w), E, K, N, q, scale, zero);
    else
        quantize_q4_kernel<uint16_t><<<blocks, 256, 0, st>>>(static_cast<const uint16_t *>(w), E, K, N, q, scale,
                                                             zero);
    return hipGetLastError();
}

}  // namespace colibri
