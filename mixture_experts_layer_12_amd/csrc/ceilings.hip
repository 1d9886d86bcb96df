// Two measurement kernels that give the achieved ceilings the layer's kernels
// are compared against (they are not part of the layer):
//   * a streaming read: every lane reads 16-byte vectors of a large buffer,
//     grid-stride, and folds them into one word so the loads stay live;
//   * an MFMA loop: every wave issues independent v_mfma_f32_32x32x16_bf16 on
//     register operands, no memory traffic, so the chip's matrix-core issue
//     rate under full load (and its clock under that load) sets the time.
// Built as a library of its own (libcolibri_ceilings.so) and called by the
// benchmark only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "colibri_ceilings.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ src, size_t n, uint32_t *sink) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    // four independent loads in flight per lane
    for (; i + 3 * stride < n; i += 4 * stride) {
        const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3] ^ b[0] ^ b[1] ^ b[2] ^ b[3] ^ c[0] ^ c[1] ^ c[2] ^ c[3] ^ d[0] ^ d[1] ^ d[2] ^
               d[3];
    }
    for (; i < n; i += stride) {
        const u32x4 a = src[i];
        acc ^= a[0] ^ a[1] ^ a[2] ^ a[3];
    }
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

constexpr int kAcc = 8;  // independent accumulators per wave

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float *sink) {
    const int lane = threadIdx.x & 63;
    bf16x8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        a[i] = (__bf16)(float)((lane + i) & 7);
        b[i] = (__bf16)(float)((lane * 3 + i) & 7);
    }
    f32x16 acc[kAcc];
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kAcc; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < kAcc; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) s += acc[j][r];
    sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace

extern "C" {

int colibri_ceiling_stream_read(const void *src, size_t bytes, uint32_t *sink, int blocks, hipStream_t stream) {
    if (!src || !sink || bytes % 16 || blocks < 1 || ((uintptr_t)src % 16)) return -1;
    stream_read_kernel<<<blocks, 256, 0, stream>>>(static_cast<const u32x4 *>(src), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

int colibri_ceiling_mfma_loop(int iters, float *sink, int blocks, hipStream_t stream) {
    if (!sink || iters < 1 || blocks < 1) return -1;
    mfma_loop_kernel<<<blocks, 256, 0, stream>>>(iters, sink);
    return hipGetLastError() == hipSuccess ? 0 : -4;
}

double colibri_ceiling_mfma_flops(int iters, int blocks) {
    // 4 waves per block, kAcc MFMAs of 2 * 32 * 32 * 16 flops per iteration
    return (double)blocks * 4.0 * kAcc * iters * 2.0 * 32 * 32 * 16;
}

}  // extern "C"
