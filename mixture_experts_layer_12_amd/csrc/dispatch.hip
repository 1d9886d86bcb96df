// Dispatch: per-expert histogram, offsets and the stable expert-sorted
// permutation of the 2T assignments, plus an optional row gather.
//
// Colibri write-ups: [zskr] http://www.zskr.cn/news/2272131 section 3.2 (count
// the top-k indices per expert, then build dispatch offsets) and 3.3 (one
// contiguous buffer region per expert); [hnwysp] https://www.hnwysp.cn/news/30485
// section 2.2 (hand the expert kernel row offsets instead of copying rows).
//
// Design (gfx950): one workgroup of 16 waves.  The assignments are cut into
// 64-wide chunks and each wave owns a contiguous run of chunks.
//   pass 1  per wave and expert, the number of its assignments, from ballots;
//   scan    wave 0 turns those into counts, offsets and each wave's starting
//           position per expert (exclusive scan over waves, then over experts);
//   pass 2  each wave walks its chunks in order; an assignment's position is
//           its wave's running position for its expert plus the number of
//           lower lanes in the chunk with the same expert (ballot + popcount).
// Positions never depend on atomic order, so the result is the stable order
// (expert ascending, assignment ascending) and is identical on every run.
// Inside a chunk only the experts that occur are visited (a leader lane's
// expert is peeled off per step).
#include "device_common.h"
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
    __shared__ int wave_cnt[kDispatchWaves][kWave];
    __shared__ int wave_base[kDispatchWaves][kWave];
    __shared__ int total_valid;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int nchunks = ceil_div(A, kWave);
    const int per = ceil_div(nchunks, kDispatchWaves);
    const int c_begin = min(nchunks, w * per);
    const int c_end = min(nchunks, c_begin + per);
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

    // pass 1: lane e accumulates this wave's count of expert e
    int my_cnt = 0;
    for (int c = c_begin; c < c_end; ++c) {
        const int a = c * kWave + lane;
        int e = (a < A) ? idx[a] : -1;
        if (e < 0 || e >= E) e = -1;
        uint64_t rem = __ballot(e >= 0);
        while (rem) {
            const int leader = __ffsll((unsigned long long)rem) - 1;
            const int ee = __shfl(e, leader);
            const uint64_t m = __ballot(e == ee);
            if (lane == ee) my_cnt += __popcll(m);
            rem &= ~m;
        }
    }
    wave_cnt[w][lane] = my_cnt;
    __syncthreads();

    if (w == 0) {
        int run = 0;
        for (int v = 0; v < kDispatchWaves; ++v) {
            wave_base[v][lane] = run;
            run += wave_cnt[v][lane];
        }
        // run = total count of expert `lane`; exclusive scan over experts
        const int tot = (lane < E) ? run : 0;
        int incl = tot;
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const int o = __shfl_up(incl, s);
            if (lane >= s) incl += o;
        }
        const int excl = incl - tot;
        for (int v = 0; v < kDispatchWaves; ++v) wave_base[v][lane] += excl;
        if (lane < E) {
            counts[lane] = tot;
            offsets[lane] = excl;
        }
        if (lane == E - 1) {
            offsets[E] = incl;
            total_valid = incl;
        }
    }
    __syncthreads();

    // pass 2: stable positions
    int run = wave_base[w][lane];  // lane e: next free position of expert e for this wave
    for (int c = c_begin; c < c_end; ++c) {
        const int a = c * kWave + lane;
        int e = (a < A) ? idx[a] : -1;
        if (e < 0 || e >= E) e = -1;
        int pos = -1;
        uint64_t rem = __ballot(e >= 0);
        while (rem) {
            const int leader = __ffsll((unsigned long long)rem) - 1;
            const int ee = __shfl(e, leader);
            const uint64_t m = __ballot(e == ee);
            const int base = __shfl(run, ee);
            if (e == ee) pos = base + __popcll(m & lt_mask);
            if (lane == ee) run += __popcll(m);
            rem &= ~m;
        }
        if (a < A) {
            assign_pos[a] = pos;
            if (pos >= 0) sorted_assign[pos] = a;
        }
    }
    // positions past the valid assignments (only when some index was out of range)
    for (int p = total_valid + threadIdx.x; p < A; p += kDispatchThreads) sorted_assign[p] = -1;
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
