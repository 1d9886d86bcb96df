// Weight-streaming grouped expert GEMM for decode-sized batches (few rows per
// expert), used for both FFN layers when T <= 64.
//
// Colibri write-ups: [zskr] http://www.zskr.cn/news/2272131 section 2.1 (the
// Compute stage: a grouped GEMM over the experts' token groups), section 2.2
// (top-2 activates 2 of the experts: only their weights need to move);
// [nxbn] http://m.nxbn.cn/news/48047 section 2.1 (matmul + activation fused
// in one kernel).
//
// At decode sizes the layer is a stream of expert weights: every weight
// element of a live expert is used by only a handful of rows.  The design
// keeps HBM busy and nothing else in the way:
//   * a wave owns one (live expert, column block, K split) unit: 128 weight
//     columns, or 64 W1 + 64 W3 columns for SwiGLU; only experts with rows
//     get waves (found from the device-side offsets); the 4 waves of a
//     workgroup take 4 adjacent column blocks over the same K range (waves
//     of one workgroup that split K instead lose about a quarter of the
//     stream bandwidth on this memory system: measured 5.2-5.7 against
//     6.7-7.0 TB/s for the same read pattern);
//   * each wave streams weights straight from HBM into registers: a lane loads an 8 (k) x 8 (n) bf16
//     block with eight 16-byte non-temporal loads, transposes it in
//     registers and feeds it as the B operand of eight
//     v_mfma_f32_16x16x32_bf16 instructions (lane l's columns are
//     n0 + 8(l%16) + j, j = 0..7, so MFMA j covers a strided set of 16
//     columns and a lane owns 8 consecutive output columns); the few token
//     rows (A operand) are read from L2; two k-steps (16 KB per wave) are
//     always in flight;
//   * int8 weights (one fp32 scale per output column): with 16-row tiles a
//     lane loads an 8 (k) x 16 (n) block of codes with eight 16-byte loads
//     (256 columns per wave, the same 8 KB per k-step as bf16); with 32-row
//     tiles an 8 x 8 block with 8-byte loads (128 columns, four k-steps in
//     flight), which keeps the accumulators within the register budget.  The
//     codes become exact bf16 values in registers and each column's sum is
//     multiplied by its scale before the epilogue or the partial store;
//   * with one K split, the epilogue (bias + activation, silu(u) * v, or bias
//     only) runs on the accumulators and rounds once to bf16;
//   * when the live experts' column blocks alone cannot fill the chip, the K
//     range is split S ways: each wave writes its partial sums
//     (fp32) to scratch, and the next kernel on the stream adds the S parts
//     in order 0..S-1 and applies the epilogue (a separate reduce kernel, or
//     the combine kernel for the second layer inside the layer call).
#include "device_common.h"
#include "ffn_common.h"
#include "launchers.h"

#include <type_traits>

namespace colibri {
namespace {

constexpr int kDecWaves = 4;  // waves (adjacent column blocks) per workgroup

// The 8 x 8 bf16 block in rows r[0..7] (r[i] = columns c..c+7 of k-row i)
// becomes eight B fragments: frag[j] = (k-rows 0..7 of column c + j).
__device__ __forceinline__ void transpose8x8(const u32x4 (&r)[8], bf16x8 (&frag)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int q = j >> 1;
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const uint32_t a = r[2 * p][q], b = r[2 * p + 1][q];
            o[p] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        frag[j] = __builtin_bit_cast(bf16x8, o);
    }
}

// int8 weights: the 8 x 16 block in rows r[0..7] (r[i] = bytes of columns
// c..c+15 of k-row i) becomes sixteen B fragments of exact bf16 values.  A byte
// is sign-extended and converted exactly to fp32 (one conversion with a byte
// select), and its bf16 pattern is the fp32 pattern's upper half (|q| < 2^8:
// no bits are lost); two such halves are packed per 32-bit word.
__device__ __forceinline__ uint32_t q8_f32_bits(uint32_t w, int b) {
    return __builtin_bit_cast(uint32_t, (float)(int32_t)(int8_t)(w >> (8 * b)));
}
// The same for an 8 x 8 block (r[i] = bytes of columns c..c+7 of k-row i).
__device__ __forceinline__ void transpose8x8_q8(const u32x2 (&r)[8], bf16x8 (&frag)[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            o[p] = __builtin_amdgcn_perm(q8_f32_bits(r[2 * p + 1][j >> 2], j & 3),
                                         q8_f32_bits(r[2 * p][j >> 2], j & 3), 0x07060302u);
        frag[j] = __builtin_bit_cast(bf16x8, o);
    }
}
// (H selects columns 8H .. 8H+7: the fragments are built eight at a time.)
template <int H>
__device__ __forceinline__ void transpose8x16_q8(const u32x4 (&r)[8], bf16x8 (&frag)[8]) {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
        const int j = 8 * H + jj;
        u32x4 o;
#pragma unroll
        for (int p = 0; p < 4; ++p)
            // bytes 2, 3 of the even row's fp32 bits, then bytes 2, 3 of the odd row's
            o[p] = __builtin_amdgcn_perm(q8_f32_bits(r[2 * p + 1][j >> 2], j & 3),
                                         q8_f32_bits(r[2 * p][j >> 2], j & 3), 0x07060302u);
        frag[jj] = __builtin_bit_cast(bf16x8, o);
    }
}

// HEPI >= 0: second layer whose A rows (H) are rebuilt by the workgroup from
// the first layer's hS split partials hpart [hS][2T][K or 2K], in split order
// with the first layer's epilogue HEPI (bias hbias) and bf16 rounding, exactly
// as the split reduce would store them; the slice for the workgroup's rows and
// K range is staged in LDS (dynamic shared memory) before the weight stream.
//
// QW: int8 weights (B0, B1 hold int8 codes) with one fp32 scale per output
// column (Sc0 for B0's columns, Sc1 for B1's): the codes enter the MFMAs as
// exact bf16 values and each column's sum is multiplied by its scale before
// the epilogue (or before it is written as a partial).
template <int MB, int EPI, bool GATHER, int HEPI, bool QW>
__global__ __launch_bounds__(kDecWaves *kWave) void ffn_decode_kernel(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ sorted_assign, int T,
    const int32_t *__restrict__ offsets, int E, const void *__restrict__ B0, const void *__restrict__ B1,
    const float *__restrict__ Sc0, const float *__restrict__ Sc1, const uint16_t *__restrict__ bias,
    uint16_t *__restrict__ C, int K, int N, int NCB, int S, float *__restrict__ part,
    const float *__restrict__ hpart, int hS, const uint16_t *__restrict__ hbias) {
    using WT = std::conditional_t<QW, int8_t, uint16_t>;  // weight element
    // weight columns per lane: 8 (bf16: one 16-byte run; int8 with 32-row tiles:
    // one 8-byte run, which keeps the registers within budget) or 16 (int8, 16-row tiles)
    constexpr int CPL = (QW && MB == 1) ? 16 : 8;
    using BRow = std::conditional_t<QW && CPL == 8, u32x2, u32x4>;  // one k-row of the lane's columns
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    constexpr bool HFROMP = HEPI >= 0;
    constexpr int WCOLS = (DUAL ? 8 : 16) * CPL;  // output columns per wave
    constexpr int ROWS = MB * 16;
    extern __shared__ __attribute__((aligned(16))) uint8_t hlds[];

    const int lane = threadIdx.x & (kWave - 1);
    const int ncbg = (NCB + kDecWaves - 1) / kDecWaves;  // groups of 4 column blocks
    const int cbg = blockIdx.x % ncbg;
    const int rest = blockIdx.x / ncbg;
    const int split = rest % S;
    const int slot = rest / S;
    const int cb = cbg * kDecWaves + (int)(threadIdx.x / kWave);
    const bool active = cb < NCB;       // waves past the last column block only help stage H
    if (!HFROMP && !active) return;

    const int A_total = 2 * T;
    int e, r0, count;
    if (!live_expert(offsets, E, A_total, slot, e, r0, count)) return;

    const int n0 = cb * WCOLS;
    const int c = lane & 15;  // column group of this lane
    const int g = lane >> 4;  // k group: k 8g..8g+7 of a 32-deep step
    // this lane's 8 consecutive weight columns and the matrix they come from;
    // out-of-range columns load column block 0 instead (never stored)
    const WT *Bm = static_cast<const WT *>((DUAL && c >= 8) ? B1 : B0);
    const int ccol = n0 + CPL * (DUAL ? (c & 7) : c);
    const bool col_ok = ccol < N;
    const WT *b_base = Bm + (size_t)e * K * N + (size_t)(8 * g) * N + (col_ok ? ccol : 0);
    // QW: the scales of this lane's 8 columns (column block 0's for padding lanes)
    float wscale[CPL];
    if constexpr (QW) {
        const float *sc = ((DUAL && c >= 8) ? Sc1 : Sc0) + (size_t)e * N + (col_ok ? ccol : 0);
#pragma unroll
        for (int j = 0; j < CPL; ++j) wscale[j] = sc[j];
    }

    // k-steps of this split
    const int ksteps = K / 32;
    const int s_begin = (int)((long)ksteps * split / S);
    const int s_end = (int)((long)ksteps * (split + 1) / S);

    // staged H slice (HFROMP): ROWS rows x klen k, rows padded by 16 bytes so the
    // 16 rows one A-fragment read touches fall in different banks
    const int klen = (s_end - s_begin) * 32;
    const int hstride = klen * 2 + 16;

    for (int rc = 0; rc < count; rc += ROWS) {
        const int rows = min(ROWS, count - rc);
        if constexpr (HFROMP) {
            constexpr bool HDUAL = (HEPI == EPI_SWIGLU);
            constexpr int U = 8;  // splits loaded per batch (the first layer's S is mostly <= 8)
            const int NCU = HDUAL ? 2 * K : K;  // columns of a first-layer partial row
            const size_t split_stride = (size_t)A_total * NCU;
            __syncthreads();  // the previous chunk's H reads are done
            const int vq = klen / 4;
            for (int i = threadIdx.x; i < rows * vq; i += blockDim.x) {
                const int r = i / vq;
                const int kq = (i - r * vq) * 4;
                const int col = s_begin * 32 + kq;  // first-layer output column
                const float *src0 = hpart + (size_t)(r0 + rc + r) * NCU + col;
                float u[4] = {0.0f, 0.0f, 0.0f, 0.0f}, v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                for (int sp = 0; sp < hS; sp += U) {
                    f32x4 a[U], b[U];
#pragma unroll
                    for (int k = 0; k < U; ++k) {
                        const float *p = src0 + min(sp + k, hS - 1) * split_stride;
                        a[k] = *reinterpret_cast<const f32x4 *>(p);
                        if (HDUAL) b[k] = *reinterpret_cast<const f32x4 *>(p + K);
                    }
#pragma unroll
                    for (int k = 0; k < U; ++k) {
                        if (sp + k < hS) {  // split order, as the reduce adds them
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                u[q] += a[k][q];
                                if (HDUAL) v[q] += b[k][q];
                            }
                        }
                    }
                }
                const uint32_t lo = pack_bf16x2(epi_value<HEPI>(u[0], v[0], hbias, e, K, col),
                                                epi_value<HEPI>(u[1], v[1], hbias, e, K, col + 1));
                const uint32_t hi = pack_bf16x2(epi_value<HEPI>(u[2], v[2], hbias, e, K, col + 2),
                                                epi_value<HEPI>(u[3], v[3], hbias, e, K, col + 3));
                *reinterpret_cast<u32x2 *>(hlds + (size_t)r * hstride + kq * 2) = u32x2{lo, hi};
            }
            __syncthreads();
            if (!active) continue;
        }
        // A rows of this lane: row (lane % 16) of each 16-row subtile; rows past
        // the segment read row r0 instead (never stored)
        const uint16_t *a_src[MB];
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            const int r = mi * 16 + c;
            const int p = r0 + rc + (r < rows ? r : 0);
            long src = p;
            if (GATHER && !HFROMP) {
                const int a = sorted_assign[p];
                src = (a >= 0 && (a >> 1) < T) ? (a >> 1) : 0;
            }
            a_src[mi] = A + (size_t)src * K + 8 * g;
        }

        f32x4 acc[MB][CPL];
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int j = 0; j < CPL; ++j) acc[mi][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

        // one k-step of operands: the lane's 8 x 8 weight block and its A fragments
        struct Stage {
            BRow b[8];
            u32x4 a[MB];
        };
        auto load_stage = [&](Stage &sg, int step) {
            const WT *p = b_base + (size_t)step * 32 * N;
#pragma unroll
            for (int i = 0; i < 8; ++i)
                sg.b[i] = __builtin_nontemporal_load(reinterpret_cast<const BRow *>(p + (size_t)i * N));
            if constexpr (!HFROMP) {
#pragma unroll
                for (int mi = 0; mi < MB; ++mi) sg.a[mi] = *reinterpret_cast<const u32x4 *>(a_src[mi] + step * 32);
            } else {
                // A fragment from the staged H slice: row mi*16 + c, k 8g..8g+7 of this step
#pragma unroll
                for (int mi = 0; mi < MB; ++mi)
                    sg.a[mi] = *reinterpret_cast<const u32x4 *>(hlds + (size_t)(mi * 16 + c) * hstride +
                                                                 ((step - s_begin) * 32 + 8 * g) * 2);
            }
        };
        // MFMAs of one k-step, eight weight columns at a time (int8: two halves,
        // so that only eight converted fragments are live at once)
        auto mma_half = [&](const Stage &sg, auto hv) {
            constexpr int H = decltype(hv)::value;
            bf16x8 bfrag[8];
            if constexpr (QW && CPL == 16) transpose8x16_q8<H>(sg.b, bfrag);
            else if constexpr (QW) transpose8x8_q8(sg.b, bfrag);
            else transpose8x8(sg.b, bfrag);
#pragma unroll
            for (int mi = 0; mi < MB; ++mi) {
                const bf16x8 afrag = __builtin_bit_cast(bf16x8, sg.a[mi]);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    acc[mi][8 * H + j] =
                        __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag[j], acc[mi][8 * H + j], 0, 0, 0);
            }
        };
        auto mma = [&](const Stage &sg) {
            mma_half(sg, std::integral_constant<int, 0>{});
            if constexpr (CPL == 16) mma_half(sg, std::integral_constant<int, 1>{});
        };

        if constexpr (QW && CPL == 8) {
            // narrow int8 layout: a k-step is 4 KB per wave, so four k-steps stay
            // in flight.  Stage i holds the steps st + i; the steady-state loop
            // issues every prefetch unconditionally.
            constexpr int NST = 4;
            Stage sg[NST];
#pragma unroll
            for (int i = 0; i < NST; ++i)
                if (s_begin + i < s_end) load_stage(sg[i], s_begin + i);
            int st = s_begin;
            for (; st + 2 * NST <= s_end; st += NST) {
#pragma unroll
                for (int i = 0; i < NST; ++i) {
                    mma(sg[i]);
                    load_stage(sg[i], st + NST + i);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
            // fewer than 2 NST steps left: the stages hold st .. st + NST - 1 (those below s_end)
#pragma unroll
            for (int i = 0; i < NST; ++i) {
                if (st + i < s_end) {
                    mma(sg[i]);
                    if (st + NST + i < s_end) load_stage(sg[i], st + NST + i);
                }
            }
#pragma unroll
            for (int i = 0; i < NST; ++i)
                if (st + NST + i < s_end) mma(sg[i]);
        } else {
            // two k-steps in flight (8 KB per wave: 8 k-rows x 16 bytes x 64 lanes):
            // stage 0 holds even steps, stage 1 odd steps.
            // The steady-state loop issues both prefetches unconditionally; the
            // scheduling barriers keep each stage's loads together.
            Stage sg0, sg1;
            const int nsteps = s_end - s_begin;
            if (nsteps > 0) load_stage(sg0, s_begin);
            if (nsteps > 1) load_stage(sg1, s_begin + 1);
            int st = s_begin;
            for (; st + 3 < s_end; st += 2) {
                mma(sg0);
                load_stage(sg0, st + 2);
                __builtin_amdgcn_sched_barrier(0);
                mma(sg1);
                load_stage(sg1, st + 3);
                __builtin_amdgcn_sched_barrier(0);
            }
            const int left = s_end - st;  // 0 (no steps), 1, 2 or 3
            if (left == 3) {
                mma(sg0);
                load_stage(sg0, st + 2);
                mma(sg1);
                mma(sg0);
            } else if (left == 2) {
                mma(sg0);
                mma(sg1);
            } else if (left == 1) {
                mma(sg0);
            }
        }

        // accumulator register r of MFMA j, subtile mi: row mi*16 + 4g + r,
        // weight column ccol + j (for SwiGLU, lanes c >= 8 hold the W3 product)
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = mi * 16 + 4 * g + r;
                float u[CPL], v[CPL];
#pragma unroll
                for (int j = 0; j < CPL; ++j) {
                    u[j] = QW ? acc[mi][j][r] * wscale[j] : acc[mi][j][r];
                    v[j] = DUAL ? __shfl_xor(u[j], 8) : 0.0f;
                }
                if (row >= rows || !col_ok) continue;
                if (S == 1) {
                    if (DUAL && c >= 8) continue;
#pragma unroll
                    for (int h8 = 0; h8 < CPL; h8 += 8) {
                        float uh[8], vh[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j) uh[j] = u[h8 + j], vh[j] = v[h8 + j];
                        store_epilogue8<EPI>(C + (size_t)(r0 + rc + row) * N + ccol + h8, uh, vh, bias, e, N,
                                             ccol + h8);
                    }
                } else {
                    // partial sums of this split: [split][row][NC], W3 products at column N + n
                    const int NC = DUAL ? 2 * N : N;
                    const int pcol = (DUAL && c >= 8) ? N + ccol : ccol;
                    float *dst = part + ((size_t)split * A_total + (r0 + rc + row)) * NC + pcol;
#pragma unroll
                    for (int q = 0; q < CPL; q += 4)
                        *reinterpret_cast<f32x4 *>(dst + q) = f32x4{u[q], u[q + 1], u[q + 2], u[q + 3]};
                }
            }
    }
}

// Adds the S split partials of every row in order 0..S-1 and applies the
// epilogue: H (first layer) or Y (second layer) in bf16.  One thread per 4
// output columns.  U: splits loaded per batch (a multiple of 8, or S <= U < 8:
// one batch).
template <int EPI, int U>
__global__ __launch_bounds__(256) void split_reduce_kernel(const float *__restrict__ part, int S, int T,
                                                           const int32_t *__restrict__ offsets, int E,
                                                           const uint16_t *__restrict__ bias,
                                                           uint16_t *__restrict__ C, int N) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    const int A_total = 2 * T;
    const int NC = DUAL ? 2 * N : N;
    const int q_per_row = N / 4;
    const size_t total = (size_t)A_total * q_per_row;
    const int rows_valid = min(max(offsets[E], 0), A_total);
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (size_t)gridDim.x * blockDim.x) {
        const int row = (int)(i / q_per_row);
        const int col = (int)(i % q_per_row) * 4;
        if (row >= rows_valid) continue;
        int e = 0;  // expert of this row: the last e with offsets[e] <= row
        for (int k = 1; k < E; ++k)
            if (offsets[k] <= row) e = k;
        // First-layer splits are added in order s = 0 .. S-1 (the second layer's
        // rebuild of H from them uses the same order).  Second-layer splits
        // (bias only) go into 8 interleaved sums, sum j taking s = j, j + 8, ...
        // in order, and the 8 sums are then added in order j = 0 .. 7: the order
        // the combine uses, which spreads a row's splits over 8 lanes (for S <= 8
        // it is the plain order).  Loads are issued U at a time so a thread waits
        // on memory ceil(S / U) times.
        static_assert(U % 8 == 0 || U < 8, "a batch keeps split s in interleaved sum s % 8");
        constexpr bool IL = (EPI == EPI_BIAS_ONLY);
        constexpr int NJ = IL ? 8 : 1;
        float u8[NJ][4], v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) u8[j][q] = 0.0f;
        const size_t split_stride = (size_t)A_total * NC;
        const float *src0 = part + (size_t)row * NC + col;
        // batches of U splits; a last, partial batch loads split S-1 in its unused
        // slots and skips their additions, so the order of additions is unchanged
        for (int sp = 0; sp < S; sp += U) {
            f32x4 a[U], b[U];
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const float *src = src0 + min(sp + k, S - 1) * split_stride;
                a[k] = *reinterpret_cast<const f32x4 *>(src);
                if (DUAL) b[k] = *reinterpret_cast<const f32x4 *>(src + N);
            }
#pragma unroll
            for (int k = 0; k < U; ++k) {
                if (sp + k < S) {  // uniform; no break, so every index stays a constant
                    const int kj = IL ? k % 8 : 0;  // sp + k = k (mod 8): U % 8 == 0, or sp = 0
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        u8[kj][q] += a[k][q];
                        if (DUAL) v[q] += b[k][q];
                    }
                }
            }
        }
        float u[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) u[q] = IL ? u[q] + u8[j][q] : u8[j][q];
        store_epilogue<EPI, 4>(C + (size_t)row * N + col, u, v, bias, e, N, col);
    }
}

}  // namespace

bool ffn_decode_eligible(const colibri_moe_shape_t &s) { return s.dtype == COLIBRI_BF16 && s.T <= 64; }

DecodePlan decode_plan(const colibri_moe_shape_t &s, bool up, bool q8) {
    DecodePlan p;
    const bool dual = up && s.act == COLIBRI_ACT_SWIGLU;
    const int K = up ? s.d : s.h;
    const int N = up ? s.h : s.d;
    // 16-row tiles when the expected rows per expert (2T/E) leave a 2x margin
    p.MB = (2 * s.T <= 8 * s.E) ? 1 : 2;
    // columns per wave: 128 (SwiGLU: 64 of W1 and W3); int8 weights with 16-row
    // tiles take 16 columns per lane, twice that
    const int wcols = (dual ? 64 : 128) * ((q8 && p.MB == 1) ? 2 : 1);
    p.NCB = (N + wcols - 1) / wcols;
    p.slots = std::min(s.E, 2 * s.T);
    const int ksteps = K / 32;
    // S minimises an estimate of the layer's time.  The kernel runs one wave
    // per SIMD, so 256 workgroups (one per CU) make one round; a wave streams
    // one k-step per ~1.15 us (two k-steps in flight, measured with bf16
    // weights; an int8 k-step moves as many bytes over twice the columns) plus ~3 k-steps of
    // start-up and epilogue; the stream cannot beat ~6.5 TB/s; S > 1 adds the
    // partials' write and read (~5 TB/s) and a ~4 us reduce launch.  A larger
    // S must win by 3% (the estimate is rough; fewer splits mean fewer partials).
    const long wg_per_split = (long)p.slots * ((p.NCB + kDecWaves - 1) / kDecWaves);
    const double cols = (double)N * (dual ? 2 : 1);
    const double weight_bytes = (double)p.slots * K * cols * (q8 ? 1 : 2);
    const double step_us = 1.15;
    p.S = 1;
    double best = 1e300;
    for (int S = 1; S <= std::max(1, ksteps / 2); ++S) {
        const double rounds = (double)((wg_per_split * S + 255) / 256);
        double us = std::max(rounds * ((double)ksteps / S + 3.0) * step_us, weight_bytes / 6.5e6);
        if (S > 1) us += 4.0 + 2.0 * S * (2.0 * s.T) * cols * 4 / 5.0e6;
        if (us < best * 0.97) best = us, p.S = S;
    }
    p.W = kDecWaves;
    p.part_bytes = p.S > 1 ? align256((size_t)p.S * 2 * s.T * (dual ? 2 : 1) * N * 4) : 0;
    return p;
}

// The second layer rebuilds H from the first layer's split partials (instead
// of a separate reduce launch) when the first layer is split, the staged H
// slice fits in 64 KB of LDS, and the partial reads -- repeated once per column
// group of the second layer -- stay within 5% of the second layer's weights,
// or 25% with 16-row tiles (a handful of rows per expert: each workgroup then
// stages a few KB, and the saved launch is worth more; measured on the
// 15-expert layer at T = 1: 34.5 -> 32.4 us; at 32-row tiles the same rule
// slowed the 8-expert layer at T = 64 from 94 to 110 us).
bool decode_fuse_h(const colibri_moe_shape_t &s, bool q8) {
    if (!ffn_decode_eligible(s)) return false;
    const DecodePlan up = decode_plan(s, true, q8), down = decode_plan(s, false, q8);
    if (up.S <= 1) return false;
    const int ksteps = s.h / 32;
    const size_t klen_max = (size_t)((ksteps + down.S - 1) / down.S) * 32;
    if ((size_t)16 * down.MB * (klen_max * 2 + 16) > 64 * 1024) return false;
    const double reads = (double)((down.NCB + kDecWaves - 1) / kDecWaves) * up.part_bytes;
    const double down_weights = (double)down.slots * s.h * s.d * (q8 ? 1 : 2);
#ifndef COLIBRI_FUSE_H_READS
#define COLIBRI_FUSE_H_READS 0.05
#endif
#ifndef COLIBRI_FUSE_H_READS_MB1
#define COLIBRI_FUSE_H_READS_MB1 0.25
#endif
    return reads <= (down.MB == 1 ? COLIBRI_FUSE_H_READS_MB1 : COLIBRI_FUSE_H_READS) * down_weights;
}

size_t ffn_decode_scratch_bytes(const colibri_moe_shape_t &s) {
    size_t need = 0;
    for (int q8 = 0; q8 < 2; ++q8) {
        const size_t up = decode_plan(s, true, q8).part_bytes, down = decode_plan(s, false, q8).part_bytes;
        need = std::max(need, decode_fuse_h(s, q8) ? align256(up) + down : std::max(up, down));
    }
    return std::max(need, ffn_decode_q4_scratch_bytes(s));  // 4-bit weights
}

namespace {
// HEPI >= 0: A is not read from memory; each workgroup rebuilds its K slice of
// the rows from the first layer's partials (hpart, hS splits) with activation
// HEPI and bias hbias, in dynamic LDS.  QW: int8 weights with scales Sc0, Sc1.
template <int EPI, int HEPI, bool QW>
hipError_t launch_decode_t(const colibri_moe_shape_t &s, const DecodePlan &p, bool gather, const void *Am,
                           const int32_t *sa, const int32_t *offsets, const void *B0, const void *B1,
                           const float *Sc0, const float *Sc1, const void *bias, void *C, int K, int N, void *scratch,
                           hipStream_t st, const float *hpart, int hS, const void *hbias) {
    float *part = static_cast<float *>(scratch);
    const int blocks = p.slots * p.S * ((p.NCB + kDecWaves - 1) / kDecWaves);
    size_t lds = 0;
    if (HEPI >= 0) {
        const int ksteps = K / 32;
        lds = (size_t)16 * p.MB * ((size_t)((ksteps + p.S - 1) / p.S) * 32 * 2 + 16);
    }
#define COLIBRI_DEC_LAUNCH(MBV, G)                                                                              \
    ffn_decode_kernel<MBV, EPI, G, HEPI, QW><<<blocks, kDecWaves * kWave, lds, st>>>(                          \
        (const uint16_t *)Am, sa, s.T, offsets, s.E, B0, B1, Sc0, Sc1, (const uint16_t *)bias, (uint16_t *)C, K, N, \
        p.NCB, p.S, part, hpart, hS, (const uint16_t *)hbias)
    if (p.MB == 1) {
        if (gather) COLIBRI_DEC_LAUNCH(1, true);
        else COLIBRI_DEC_LAUNCH(1, false);
    } else {
        if (gather) COLIBRI_DEC_LAUNCH(2, true);
        else COLIBRI_DEC_LAUNCH(2, false);
    }
#undef COLIBRI_DEC_LAUNCH
    return hipGetLastError();
}

template <int EPI>
hipError_t launch_reduce_t(const colibri_moe_shape_t &s, int S, const int32_t *offsets, const void *bias, void *C,
                           int N, const void *scratch, hipStream_t st) {
    const size_t total = (size_t)2 * s.T * (N / 4);
    const int blocks = (int)std::min<size_t>((total + 255) / 256, 4096);
    // batches no larger than S: a thread loads only the splits it adds
#define COLIBRI_REDUCE_LAUNCH(UV)                                                                             \
    split_reduce_kernel<EPI, UV><<<blocks, 256, 0, st>>>((const float *)scratch, S, s.T, offsets, s.E,        \
                                                         (const uint16_t *)bias, (uint16_t *)C, N)
    if (S <= 2) COLIBRI_REDUCE_LAUNCH(2);
    else if (S <= 4) COLIBRI_REDUCE_LAUNCH(4);
    else if (S <= 8) COLIBRI_REDUCE_LAUNCH(8);
    else COLIBRI_REDUCE_LAUNCH(16);
#undef COLIBRI_REDUCE_LAUNCH
    return hipGetLastError();
}

template <int EPI, bool QW>
hipError_t up_t(const colibri_moe_shape_t &s, const DecodePlan &p, bool gather, const void *x_rows,
                const int32_t *sa, const int32_t *offsets, const DecodeWeights &w, const void *B1, const float *S1,
                const void *bias, void *H, void *scratch, bool reduce, hipStream_t st) {
    hipError_t err = launch_decode_t<EPI, -1, QW>(s, p, gather, x_rows, sa, offsets, w.w1, B1, w.s1, S1, bias, H, s.d,
                                                  s.h, scratch, st, nullptr, 0, nullptr);
    if (err == hipSuccess && p.S > 1 && reduce) err = launch_reduce_t<EPI>(s, p.S, offsets, bias, H, s.h, scratch, st);
    return err;
}

template <bool QW>
hipError_t up_q(const colibri_moe_shape_t &s, const DecodePlan &p, bool gather, const void *x_rows,
                const int32_t *sa, const int32_t *offsets, const DecodeWeights &w, void *H, void *scratch,
                bool reduce, hipStream_t st) {
    switch (s.act) {
        case COLIBRI_ACT_RELU:
            return up_t<EPI_ACT_RELU, QW>(s, p, gather, x_rows, sa, offsets, w, nullptr, nullptr, w.b1, H, scratch,
                                          reduce, st);
        case COLIBRI_ACT_GELU:
            return up_t<EPI_ACT_GELU, QW>(s, p, gather, x_rows, sa, offsets, w, nullptr, nullptr, w.b1, H, scratch,
                                          reduce, st);
        default:
            return up_t<EPI_SWIGLU, QW>(s, p, gather, x_rows, sa, offsets, w, w.w3, w.s3, nullptr, H, scratch,
                                        reduce, st);
    }
}

template <int HEPI, bool QW>
hipError_t down_t(const colibri_moe_shape_t &s, const DecodePlan &p, const void *H, const int32_t *offsets,
                  const DecodeWeights &w, const void *b2, void *y, void *scratch, hipStream_t st, const float *hpart,
                  int hS, const void *hbias) {
    return launch_decode_t<EPI_BIAS_ONLY, HEPI, QW>(s, p, false, H, nullptr, offsets, w.w2, nullptr, w.s2, nullptr,
                                                     b2, y, s.h, s.d, scratch, st, hpart, hS, hbias);
}

template <bool QW>
hipError_t down_q(const colibri_moe_shape_t &s, const DecodePlan &p, const void *H, const int32_t *offsets,
                  const DecodeWeights &w, const void *b2, void *y, void *scratch, hipStream_t st,
                  const float *h_partials) {
    if (h_partials == nullptr) return down_t<-1, QW>(s, p, H, offsets, w, b2, y, scratch, st, nullptr, 0, nullptr);
    const int hS = decode_plan(s, true, QW).S;
    switch (s.act) {
        case COLIBRI_ACT_RELU:
            return down_t<EPI_ACT_RELU, QW>(s, p, H, offsets, w, b2, y, scratch, st, h_partials, hS, w.b1);
        case COLIBRI_ACT_GELU:
            return down_t<EPI_ACT_GELU, QW>(s, p, H, offsets, w, b2, y, scratch, st, h_partials, hS, w.b1);
        default: return down_t<EPI_SWIGLU, QW>(s, p, H, offsets, w, b2, y, scratch, st, h_partials, hS, nullptr);
    }
}
}  // namespace

hipError_t launch_decode_up(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                            const int32_t *offsets, const DecodeWeights &w, void *H, void *scratch, hipStream_t st,
                            bool reduce) {
    const DecodePlan p = decode_plan(s, true, w.q8);
    const bool gather = sorted_assign != nullptr;
    return w.q8 ? up_q<true>(s, p, gather, x_rows, sorted_assign, offsets, w, H, scratch, reduce, st)
                : up_q<false>(s, p, gather, x_rows, sorted_assign, offsets, w, H, scratch, reduce, st);
}

hipError_t launch_decode_down(const colibri_moe_shape_t &s, const void *H, const int32_t *offsets,
                              const DecodeWeights &w, void *y, void *scratch, bool reduce, hipStream_t st,
                              const float *h_partials) {
    const DecodePlan p = decode_plan(s, false, w.q8);
    const void *b2 = s.act == COLIBRI_ACT_SWIGLU ? nullptr : w.b2;
    hipError_t err = w.q8 ? down_q<true>(s, p, H, offsets, w, b2, y, scratch, st, h_partials)
                          : down_q<false>(s, p, H, offsets, w, b2, y, scratch, st, h_partials);
    if (err == hipSuccess && p.S > 1 && reduce)
        err = launch_reduce_t<EPI_BIAS_ONLY>(s, p.S, offsets, b2, y, s.d, scratch, st);
    return err;
}

hipError_t launch_split_reduce(const colibri_moe_shape_t &s, bool up, int S, const int32_t *offsets,
                               const colibri_moe_experts_t &w, void *C, const float *part, hipStream_t st) {
    if (!up)
        return launch_reduce_t<EPI_BIAS_ONLY>(s, S, offsets, s.act == COLIBRI_ACT_SWIGLU ? nullptr : w.b2, C, s.d,
                                              part, st);
    switch (s.act) {
        case COLIBRI_ACT_RELU: return launch_reduce_t<EPI_ACT_RELU>(s, S, offsets, w.b1, C, s.h, part, st);
        case COLIBRI_ACT_GELU: return launch_reduce_t<EPI_ACT_GELU>(s, S, offsets, w.b1, C, s.h, part, st);
        default: return launch_reduce_t<EPI_SWIGLU>(s, S, offsets, nullptr, C, s.h, part, st);
    }
}

}  // namespace colibri
