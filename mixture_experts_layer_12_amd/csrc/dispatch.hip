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
// Large batches, given scratch, spread the same three passes over the chip:
// a count kernel (one wave per 64-assignment chunk writes the chunk's
// per-expert counts), a one-workgroup scan (each chunk's starting position
// per expert, the counts and offsets) and a scatter kernel (one wave per
// chunk places its assignments at the chunk's start + the number of lower
// lanes with the same expert).  Every position is a function of the indices
// alone, so both paths give the same stable order.
#include "device_common.h"
#include "dispatch_block.h"
#include "launchers.h"

namespace colibri {
namespace {

constexpr int kDispatchWaves = 16;
constexpr int kDispatchThreads = kDispatchWaves * kWave;

// zero[0 .. n) = 0 by the whole grid (zero: 16-byte aligned or nullptr), with
// 16-byte vector stores.
__device__ __forceinline__ void zero_words(int32_t *zero, size_t n) {
    if (zero == nullptr) return;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    const size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    u32x4 *z4 = reinterpret_cast<u32x4 *>(zero);
    for (size_t i = i0; i < n / 4; i += stride) z4[i] = u32x4{0u, 0u, 0u, 0u};
    for (size_t i = n / 4 * 4 + i0; i < n; i += stride) zero[i] = 0;
}

__global__ __launch_bounds__(kDispatchThreads) void dispatch_kernel(const int32_t *__restrict__ idx, int A, int E,
                                                                    int32_t *__restrict__ counts,
                                                                    int32_t *__restrict__ offsets,
                                                                    int32_t *__restrict__ sorted_assign,
                                                                    int32_t *__restrict__ assign_pos,
                                                                    int32_t *__restrict__ zero, size_t nzero) {
    zero_words(zero, nzero);
    __shared__ DispatchShared<kDispatchWaves> sh;
    dispatch_block<kDispatchWaves>([&](int a) { return idx[a]; }, A, E, counts, offsets, sorted_assign, assign_pos,
                                   sh);
}

// Lane e of the calling wave gets the number of assignments of expert e in
// chunk c (64 assignments); out-of-range indices are skipped.
__device__ __forceinline__ int chunk_count(const int32_t *__restrict__ idx, int A, int E, int c) {
    const int lane = threadIdx.x & (kWave - 1);
    const int a = c * kWave + lane;
    int e = (a < A) ? idx[a] : -1;
    if (e < 0 || e >= E) e = -1;
    int cnt = 0;
    uint64_t rem = __ballot(e >= 0);
    while (rem) {
        const int leader = __ffsll((unsigned long long)rem) - 1;
        const int ee = __shfl(e, leader);
        const uint64_t m = __ballot(e == ee);
        if (lane == ee) cnt = __popcll(m);
        rem &= ~m;
    }
    return cnt;
}

constexpr int kChunkWaves = 4;  // chunks (waves) per workgroup of the count and scatter kernels

__global__ __launch_bounds__(kChunkWaves *kWave) void dispatch_count_kernel(const int32_t *__restrict__ idx, int A,
                                                                            int E, int nchunks,
                                                                            int32_t *__restrict__ hist,
                                                                            int32_t *__restrict__ zero,
                                                                            size_t nzero) {
    zero_words(zero, nzero);
    const int c = (int)blockIdx.x * kChunkWaves + (int)(threadIdx.x / kWave);
    if (c >= nchunks) return;  // uniform per wave
    const int lane = threadIdx.x & (kWave - 1);
    const int cnt = chunk_count(idx, A, E, c);
    if (lane < E) hist[(size_t)c * E + lane] = cnt;
}

// One workgroup: thread (part p, expert e) covers chunks [p L, (p + 1) L);
// base[c][e] = offsets[e] + (assignments of expert e in chunks before c).
constexpr int kScanParts = 16;
__global__ __launch_bounds__(kScanParts *kWave) void dispatch_scan_kernel(const int32_t *__restrict__ hist,
                                                                          int nchunks, int E,
                                                                          int32_t *__restrict__ base,
                                                                          int32_t *__restrict__ counts,
                                                                          int32_t *__restrict__ offsets) {
    __shared__ int psum[kScanParts][kWave];
    __shared__ int pbase[kScanParts][kWave];
    const int e = threadIdx.x & (kWave - 1);
    const int part = threadIdx.x / kWave;
    const int L = ceil_div(nchunks, kScanParts);
    const int c0 = min(nchunks, part * L), c1 = min(nchunks, c0 + L);
    // up to kScanRegs chunk counts per thread are loaded once, all in flight
    // (one after another the loads left the scan bound by their latency)
    constexpr int kScanRegs = 32;
    int v[kScanRegs];
#pragma unroll
    for (int q = 0; q < kScanRegs; ++q) v[q] = (e < E && c0 + q < c1) ? hist[(size_t)(c0 + q) * E + e] : 0;
    int sum = 0;
#pragma unroll
    for (int q = 0; q < kScanRegs; ++q) sum += v[q];
    if (e < E)
        for (int c = c0 + kScanRegs; c < c1; ++c) sum += hist[(size_t)c * E + e];
    psum[part][e] = sum;
    __syncthreads();
    if (part == 0) {
        int run = 0;
        for (int q = 0; q < kScanParts; ++q) {
            pbase[q][e] = run;
            run += psum[q][e];
        }
        const int tot = (e < E) ? run : 0;
        int incl = tot;
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const int o = __shfl_up(incl, s);
            if (e >= s) incl += o;
        }
        const int excl = incl - tot;
        for (int q = 0; q < kScanParts; ++q) pbase[q][e] += excl;
        if (e < E) {
            counts[e] = tot;
            offsets[e] = excl;
        }
        if (e == E - 1) offsets[E] = incl;
    }
    __syncthreads();
    if (e < E) {
        int run = pbase[part][e];
#pragma unroll
        for (int q = 0; q < kScanRegs; ++q) {
            if (c0 + q < c1) base[(size_t)(c0 + q) * E + e] = run;
            run += v[q];
        }
        for (int c = c0 + kScanRegs; c < c1; ++c) {
            base[(size_t)c * E + e] = run;
            run += hist[(size_t)c * E + e];
        }
    }
}

__global__ __launch_bounds__(kChunkWaves *kWave) void dispatch_scatter_kernel(
    const int32_t *__restrict__ idx, int A, int E, int nchunks, const int32_t *__restrict__ base,
    const int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_assign, int32_t *__restrict__ assign_pos) {
    const int lane = threadIdx.x & (kWave - 1);
    // positions past the valid assignments (only when some index was out of range)
    const int valid = offsets[E];
    for (int p = valid + (int)(blockIdx.x * blockDim.x + threadIdx.x); p < A; p += (int)(gridDim.x * blockDim.x))
        sorted_assign[p] = -1;
    const int c = (int)blockIdx.x * kChunkWaves + (int)(threadIdx.x / kWave);
    if (c >= nchunks) return;  // uniform per wave
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    const int a = c * kWave + lane;
    int e = (a < A) ? idx[a] : -1;
    if (e < 0 || e >= E) e = -1;
    const int my_base = (lane < E) ? base[(size_t)c * E + lane] : 0;  // lane e: chunk start of expert e
    int pos = -1;
    uint64_t rem = __ballot(e >= 0);
    while (rem) {
        const int leader = __ffsll((unsigned long long)rem) - 1;
        const int ee = __shfl(e, leader);
        const uint64_t m = __ballot(e == ee);
        const int b = __shfl(my_base, ee);
        if (e == ee) pos = b + __popcll(m & lt_mask);
        rem &= ~m;
    }
    if (a < A) {
        assign_pos[a] = pos;
        if (pos >= 0) sorted_assign[pos] = a;
    }
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

#ifndef COLIBRI_DISPATCH_MULTI_MIN_A
#define COLIBRI_DISPATCH_MULTI_MIN_A 4096
#endif
constexpr int kMultiMinA = COLIBRI_DISPATCH_MULTI_MIN_A;  // assignments from which the multi-workgroup path pays

size_t dispatch_scratch_bytes(const colibri_moe_shape_t &s) {
    const long A = 2L * s.T;
    if (A < kMultiMinA) return 0;
    const size_t table = (size_t)ceil_div((int)A, kWave) * s.E * 4;
    return 2 * align256(table);
}

hipError_t launch_dispatch(const colibri_moe_shape_t &s, const int32_t *topk_idx, int32_t *counts,
                           int32_t *offsets, int32_t *sorted_assign, int32_t *assign_pos, hipStream_t st,
                           void *scratch, int32_t *zero, size_t nzero) {
    const int A = 2 * s.T;
    const size_t need = dispatch_scratch_bytes(s);
    if (need == 0 || scratch == nullptr) {
        dispatch_kernel<<<1, kDispatchThreads, 0, st>>>(topk_idx, A, s.E, counts, offsets, sorted_assign,
                                                        assign_pos, zero, nzero);
        return hipGetLastError();
    }
    const int nchunks = ceil_div(A, kWave);
    int32_t *hist = static_cast<int32_t *>(scratch);
    int32_t *base = reinterpret_cast<int32_t *>(static_cast<char *>(scratch) + need / 2);
    const int blocks = ceil_div(nchunks, kChunkWaves);
    dispatch_count_kernel<<<blocks, kChunkWaves * kWave, 0, st>>>(topk_idx, A, s.E, nchunks, hist, zero, nzero);
    dispatch_scan_kernel<<<1, kScanParts * kWave, 0, st>>>(hist, nchunks, s.E, base, counts, offsets);
    dispatch_scatter_kernel<<<blocks, kChunkWaves * kWave, 0, st>>>(topk_idx, A, s.E, nchunks, base, offsets,
                                                                    sorted_assign, assign_pos);
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
