// Dispatch: per-expert histogram, offsets and the stable expert-sorted
// permutation of the 2T assignments, plus an optional row gather.
//
// Colibri write-ups: [zskr] http://www.zskr.cn/news/2272131 section 3.2 (count
// the top-k indices per expert, then build dispatch offsets) and 3.3 (one
// contiguous buffer region per expert); [hnwysp] https://www.hnwysp.cn/news/30485
// section 2.2 (hand the expert kernel row offsets instead of copying rows).
//
// Design (gfx950): one workgroup of 16 waves runs dispatch_block
// (dispatch_block.h: ballot/popcount histogram, scan, stable placement).
#include "device_common.h"
#include "dispatch_block.h"
#include "launchers.h"

namespace colibri {
namespace {

constexpr int kDispatchWaves = 16;
constexpr int kDispatchThreads = kDispatchWaves * kWave;

__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(const int32_t *__restrict__ idx, int A, int E,
                                                                    int32_t *__restrict__ counts,
                                                                    int32_t *__restrict__ offsets,
                                                                    int32_t *__restrict__ sorted_assign,
                                                                    int32_t *__restrict__ assign_pos) {
    __shared__ DispatchShared<kDispatchWaves> sh;
    dispatch_block<kDispatchWaves>([&](int a) { return idx[a]; }, A, E, counts, offsets, sorted_assign, assign_pos,
                                   sh);
}

template <typename TE>
__global__ __launch_bounds__(256) void gather_rows_kernel(const TE *__restrict__ x, const int32_t *__restrict__ sa,
                                                          int A, int T, int d, TE *__restrict__ xs) {
    constexpr int VEC = 16 / sizeof(TE);
    const int vecs_per_row = d / VEC;
    const size_t total = (size_t)A * vecs_per_row;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
        const int p = (int)(i / vecs_per_row);
        const int v = (int)(i % vecs_per_row);
        const int a = sa[p];
        u32x4 val = {0u, 0u, 0u, 0u};
        if (a >= 0 && (a >> 1) < T) val = *reinterpret_cast<const u32x4 *>(x + (size_t)(a >> 1) * d + v * VEC);
        *reinterpret_cast<u32x4 *>(xs + (size_t)p * d + v * VEC) = val;
    }
}

}  // namespace

hipError_t launch_dispatch(const colibri_moe_shape_t &s, const int32_t *topk_idx, int32_t *counts,
                           int32_t *offsets, int32_t *sorted_assign, int32_t *assign_pos, hipStream_t st) {
    dispatch_kernel<<<1, kDispatchThreads, 0, st>>>(topk_idx, 2 * s.T, s.E, counts, offsets, sorted_assign,
                                                    assign_pos);
    return hipGetLastError();
}

hipError_t launch_gather_rows(const colibri_moe_shape_t &s, const void *x, const int32_t *sorted_assign,
                              void *x_sorted, hipStream_t st) {
    const int A = 2 * s.T;
    const int vec = s.dtype == COLIBRI_F32 ? 4 : 8;
    const size_t total = (size_t)A * (s.d / vec);
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 4096);
    if (s.dtype == COLIBRI_F32)
        gather_rows_kernel<float><<<blocks, 256, 0, st>>>((const float *)x, sorted_assign, A, s.T, s.d,
                                                          (float *)x_sorted);
    else
        gather_rows_kernel<uint16_t><<<blocks, 256, 0, st>>>((const uint16_t *)x, sorted_assign, A, s.T, s.d,
                                                             (uint16_t *)x_sorted);
    return hipGetLastError();
}

}  // namespace colibri
