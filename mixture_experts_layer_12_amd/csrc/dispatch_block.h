// Dispatch of the 2T assignments by one workgroup of NW waves: per-expert
// counts, offsets, the stable expert-sorted permutation and its inverse.
// Shared by the dispatch kernel and the fused route + dispatch kernel.
//
// Colibri write-ups: [zskr] http://www.zskr.cn/news/2272131 section 3.2 (count
// the top-k indices per expert, then build dispatch offsets) and 3.3 (one
// contiguous buffer region per expert).
//
// The assignments are cut into 64-wide chunks and each wave owns a contiguous
// run of chunks.
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
#pragma once

#include "device_common.h"

namespace colibri {

template <int NW>
struct DispatchShared {
    int wave_cnt[NW][kWave];
    int wave_base[NW][kWave];
    int total_valid;
};

// idx_at(a): expert index of assignment a (0 <= a < A); out-of-range values are
// skipped.  Must be called by all NW * 64 threads of the workgroup.  The result
// does not depend on NW (it is the unique stable order).
template <int NW, class IdxAt>
__device__ __forceinline__ void dispatch_block(IdxAt idx_at, int A, int E, int32_t *__restrict__ counts,
                                               int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_assign,
                                               int32_t *__restrict__ assign_pos, DispatchShared<NW> &sh) {
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    if (A <= kWave) {
        // one chunk: wave 0 alone, in registers, with no barrier (decode batches)
        if (w != 0) return;
        int e = (lane < A) ? idx_at(lane) : -1;
        if (e < 0 || e >= E) e = -1;
        int cnt = 0;  // lane x: assignments of expert x
        uint64_t rem = __ballot(e >= 0);
        while (rem) {
            const int leader = __ffsll((unsigned long long)rem) - 1;
            const int ee = __shfl(e, leader);
            const uint64_t m = __ballot(e == ee);
            if (lane == ee) cnt = __popcll(m);
            rem &= ~m;
        }
        const int tot = (lane < E) ? cnt : 0;
        int incl = tot;
#pragma unroll
        for (int s = 1; s < kWave; s <<= 1) {
            const int o = __shfl_up(incl, s);
            if (lane >= s) incl += o;
        }
        const int excl = incl - tot;
        if (lane < E) {
            counts[lane] = tot;
            offsets[lane] = excl;
        }
        if (lane == E - 1) offsets[E] = incl;
        const int total_valid = __shfl(incl, E - 1);
        int pos = -1;
        rem = __ballot(e >= 0);
        while (rem) {
            const int leader = __ffsll((unsigned long long)rem) - 1;
            const int ee = __shfl(e, leader);
            const uint64_t m = __ballot(e == ee);
            const int base = __shfl(excl, ee);
            if (e == ee) pos = base + __popcll(m & lt_mask);
            rem &= ~m;
        }
        if (lane < A) {
            assign_pos[lane] = pos;
            if (pos >= 0) sorted_assign[pos] = lane;
            if (lane >= total_valid) sorted_assign[lane] = -1;
        }
        return;
    }
    const int nchunks = ceil_div(A, kWave);
    const int per = ceil_div(nchunks, NW);
    const int c_begin = min(nchunks, w * per);
    const int c_end = min(nchunks, c_begin + per);

    // pass 1: lane e accumulates this wave's count of expert e
    int my_cnt = 0;
    for (int c = c_begin; c < c_end; ++c) {
        const int a = c * kWave + lane;
        int e = (a < A) ? idx_at(a) : -1;
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
    sh.wave_cnt[w][lane] = my_cnt;
    __syncthreads();

    if (w == 0) {
        int run = 0;
        for (int v = 0; v < NW; ++v) {
            sh.wave_base[v][lane] = run;
            run += sh.wave_cnt[v][lane];
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
        for (int v = 0; v < NW; ++v) sh.wave_base[v][lane] += excl;
        if (lane < E) {
            counts[lane] = tot;
            offsets[lane] = excl;
        }
        if (lane == E - 1) {
            offsets[E] = incl;
            sh.total_valid = incl;
        }
    }
    __syncthreads();

    // pass 2: stable positions
    int run = sh.wave_base[w][lane];  // lane e: next free position of expert e for this wave
    for (int c = c_begin; c < c_end; ++c) {
        const int a = c * kWave + lane;
        int e = (a < A) ? idx_at(a) : -1;
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
    for (int p = sh.total_valid + threadIdx.x; p < A; p += NW * kWave) sorted_assign[p] = -1;
}

}  // namespace colibri
