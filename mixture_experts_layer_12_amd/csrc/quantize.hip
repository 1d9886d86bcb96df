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

}  // namespace colibri
