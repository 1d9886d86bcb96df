// Weight-streaming expert FFN for decode-sized batches with 4-bit expert
// weights (zero point, groups of 128 input channels).
//
// Colibri write-ups: [rkmt] http://news.rkmt.cn/news/2271114 section 4.2
// (4-bit AWQ expert weights, quantization group 128, zero point: the weight
// bytes a decode step streams drop to a quarter); [zskr]
// http://www.zskr.cn/news/2272131 section 2.2 (top-2 activates 2 of the
// experts: only their weights need to move).
//
//   W[e][k][n] = s[e][k/128][n] * (q[e][k][n] - z[e][k/128][n]),  q, z in [0, 15]
//
// Layout: word (e, j, n) of q [E][K/8][N] packs the codes of k = 8j .. 8j+7 of
// column n, the code of k = 8j + 2m in bits 4m .. 4m+3 and of k = 8j + 2m + 1
// in bits 16 + 4m .. 16 + 4m + 3 (m = 0..3).  One word is the eight k a lane
// feeds to one column of v_mfma_f32_16x16x32_bf16, a lane's four columns of a
// k-step are one 16-byte load, and k-pair m of the word is the halfword pair
// (word >> 4m) & 0x000f000f.
//
// Design (as the bf16 weight-streaming kernel, with the weights 4x smaller):
//   * a wave owns (live expert, 64 columns -- SwiGLU: 32 of W1 and 32 of W3 --,
//     K split); 4 waves of a workgroup take adjacent column blocks; few
//     registers per wave, so several workgroups share a CU;
//   * a code becomes an exact bf16 operand with no conversion: the bit
//     pattern 0x4300 | q is the bf16 value 128 + q (bf16 has 7 fraction bits,
//     so 128 .. 143 are exact), built for two k at once with one shift and one
//     AND-OR.  The MFMAs accumulate x * (128 + q) over a group, and one
//     more MFMA per k-step against a B operand of ones accumulates the rows'
//     sums of x over the group, so that at the end of every group
//       total += s * (acc - (128 + z) * rowsum_x)
//     is the group's exact contribution (up to fp32 rounding);
//   * the rows (A operand) of a group -- 128 k of every row of the tile -- are
//     loaded once per workgroup, a share per thread, and staged in LDS (two
//     buffers, one barrier per group), where the four waves read their
//     fragments: a wave's global loads are its codes only;
//   * the codes of the next group's four k-steps are in flight during a group
//     (each k-step is 1 KB per wave); the group scales and zero points (20
//     bytes per lane and group) are read at each group's start and used at
//     its end;
//   * K splits run along whole groups; split partials (fp32) are added by
//     the split reduce or, for the second layer inside the layer call, by the
//     combine.
#include "device_common.h"
#include "ffn_common.h"
#include "launchers.h"

namespace colibri {
namespace {

constexpr int kQ4Waves = 4;   // waves (adjacent column blocks) per workgroup
constexpr int kQ4Group = 128; // k per scale / zero point

// The four words of a lane's four columns (w[j] = column j, k 0..7) -> four B
// fragments holding 128 + q: fragment dword m (k 2m, 2m + 1) is the halfword
// pair (w[j] >> 4m) & 0x000f000f over the pattern of 128.0 in both halves.
__device__ __forceinline__ void unpack_q4(const u32x4 &w, bf16x8 (&frag)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        u32x4 o;
#pragma unroll
        for (int m = 0; m < 4; ++m) o[m] = ((w[j] >> (4 * m)) & 0x000f000fu) | 0x43004300u;
        frag[j] = __builtin_bit_cast(bf16x8, o);
    }
}

template <int MB, int EPI, bool GATHER>
__global__ __launch_bounds__(kQ4Waves *kWave) void ffn_decode_q4_kernel(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ sorted_assign, int T,
    const int32_t *__restrict__ offsets, int E, const uint32_t *__restrict__ Q0, const uint32_t *__restrict__ Q1,
    const float *__restrict__ S0, const float *__restrict__ S1, const uint8_t *__restrict__ Z0,
    const uint8_t *__restrict__ Z1, const uint16_t *__restrict__ bias, uint16_t *__restrict__ C, int K, int N,
    int NCB, int S, float *__restrict__ part) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    constexpr int WCOLS = DUAL ? 32 : 64;  // output columns per wave (per matrix)
    constexpr int ROWS = MB * 16;
    // the rows of one group staged in LDS, row pitch 136 bf16 (272 bytes: the
    // 16 rows one fragment read touches start in distinct banks); two buffers
    constexpr int APITCH = kQ4Group + 8;
    __shared__ __attribute__((aligned(16))) uint16_t arows[2][ROWS * APITCH];
    const int lane = threadIdx.x & (kWave - 1);
    const int ncbg = (NCB + kQ4Waves - 1) / kQ4Waves;
    const int cbg = blockIdx.x % ncbg;
    const int rest = blockIdx.x / ncbg;
    const int split = rest % S;
    const int slot = rest / S;
    const int cb = cbg * kQ4Waves + (int)(threadIdx.x / kWave);
    const bool active = cb < NCB;  // waves past the last column block only help stage the rows

    const int A_total = 2 * T;
    int e, r0, count;
    if (!live_expert(offsets, E, A_total, slot, e, r0, count)) return;  // the same for every wave

    const int c = lane & 15;  // column group: columns ccol .. ccol + 3
    const int g = lane >> 4;  // k group: k 8g .. 8g+7 of a 32-deep step
    const bool third = DUAL && c >= 8;  // SwiGLU: lanes 8..15 hold W3's columns
    const uint32_t *Qm = third ? Q1 : Q0;
    const float *Sm = third ? S1 : S0;
    const uint8_t *Zm = third ? Z1 : Z0;
    const int ccol = cb * WCOLS + 4 * (DUAL ? (c & 7) : c);
    const bool col_ok = ccol < N;
    const int col = col_ok ? ccol : 0;  // padding lanes read column block 0 (never stored)
    const int G = K / kQ4Group;
    // word (k-step st, k group g) of this lane's columns: row 4 st + g of [K/8][N]
    const uint32_t *q_base = Qm + (size_t)e * (K / 8) * N + (size_t)g * N + col;
    const float *s_base = Sm + (size_t)e * G * N + col;
    const uint8_t *z_base = Zm + (size_t)e * G * N + col;

    // whole groups per split: groups [g_begin, g_end), k-steps 4 g_begin ..
    const int g_begin = (int)((long)G * split / S), g_end = (int)((long)G * (split + 1) / S);
    const u32x4 ones = {0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u};  // bf16 1.0 x 8
    // this thread's share of a staged group: 16-byte chunk q of rows ar0 + 16 m
    const int aq = threadIdx.x & 15, ar0 = (threadIdx.x >> 4) & 15;

    for (int rc = 0; rc < count; rc += ROWS) {
        const int rows = min(ROWS, count - rc);
        const uint16_t *asrc[MB];  // rows past the segment read row r0 instead (never stored)
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            const int r = ar0 + 16 * m;
            const int p = r0 + rc + (r < rows ? r : 0);
            long src = p;
            if (GATHER) {
                const int a = sorted_assign[p];
                src = (a >= 0 && (a >> 1) < T) ? (a >> 1) : 0;
            }
            asrc[m] = A + (size_t)src * K + 8 * aq;
        }
        u32x4 ra[MB];
        auto load_rows = [&](int grp) {
#pragma unroll
            for (int m = 0; m < MB; ++m) ra[m] = *reinterpret_cast<const u32x4 *>(asrc[m] + (size_t)grp * kQ4Group);
        };
        auto store_rows = [&](int buf) {
#pragma unroll
            for (int m = 0; m < MB; ++m)
                *reinterpret_cast<u32x4 *>(&arows[buf][(ar0 + 16 * m) * APITCH + 8 * aq]) = ra[m];
        };

        f32x4 acc[MB][4], rsum[MB], tot[MB][4];
#pragma unroll
        for (int mi = 0; mi < MB; ++mi) {
            rsum[mi] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[mi][j] = tot[mi][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
        u32x4 wb[4];  // the codes of the group's four k-steps
        auto load_codes = [&](int kk, int step) {
            wb[kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(q_base + (size_t)step * 4 * N));
        };
        // k-step kk of the group in buffer buf: rows mi*16 + c, k 32 kk + 8g .. + 7
        auto mma = [&](int kk, int buf) {
            bf16x8 bfrag[4];
            unpack_q4(wb[kk], bfrag);
#pragma unroll
            for (int mi = 0; mi < MB; ++mi) {
                const bf16x8 afrag = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(&arows[buf][(mi * 16 + c) * APITCH + 32 * kk + 8 * g]));
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[mi][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag[j], acc[mi][j], 0, 0, 0);
                rsum[mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, __builtin_bit_cast(bf16x8, ones), rsum[mi],
                                                                  0, 0, 0);
            }
        };
        // the group's scales and zero points (read at its start) fold its sums into the totals
        f32x4 gs;
        uint32_t gz;
        auto load_group = [&](int grp) {
            gs = *reinterpret_cast<const f32x4 *>(s_base + (size_t)grp * N);
            gz = *reinterpret_cast<const uint32_t *>(z_base + (size_t)grp * N);
        };
        auto finish_group = [&]() {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float sj = gs[j];
                const float zj = 128.0f + (float)((gz >> (8 * j)) & 0xffu);
#pragma unroll
                for (int mi = 0; mi < MB; ++mi)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        tot[mi][j][r] = fmaf(sj, fmaf(-zj, rsum[mi][r], acc[mi][j][r]), tot[mi][j][r]);
                        acc[mi][j][r] = 0.0f;
                    }
            }
#pragma unroll
            for (int mi = 0; mi < MB; ++mi) rsum[mi] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        };

        // group g_begin + j sits in buffer j % 2; the rows of the next group are
        // loaded during a group and stored at its end, behind one barrier; the
        // codes of the next group's four k-steps are in flight during a group
        __syncthreads();  // the previous row chunk's reads are done
        load_rows(g_begin);
        store_rows(0);
        __syncthreads();
        if (g_begin + 1 < g_end) load_rows(g_begin + 1);
        if (active)
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) load_codes(kk, 4 * g_begin + kk);
        int grp = g_begin;
        for (; grp + 1 < g_end; ++grp) {
            const int buf = (grp - g_begin) & 1;
            if (active) {
                load_group(grp);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    mma(kk, buf);
                    load_codes(kk, 4 * (grp + 1) + kk);
                    __builtin_amdgcn_sched_barrier(0);
                }
                finish_group();
            }
            store_rows(buf ^ 1);  // its last reads were before the previous barrier
            __syncthreads();
            load_rows(min(grp + 2, g_end - 1));
        }
        if (active) {  // the last group
            load_group(grp);
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) mma(kk, (grp - g_begin) & 1);
            finish_group();
        }
        if (!active) continue;

        // accumulator register r of column j, subtile mi: row mi*16 + 4g + r,
        // column ccol + j (SwiGLU: lanes c >= 8 hold the W3 product)
#pragma unroll
        for (int mi = 0; mi < MB; ++mi)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = mi * 16 + 4 * g + r;
                float u[4], v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    u[j] = tot[mi][j][r];
                    v[j] = DUAL ? __shfl_xor(u[j], 8) : 0.0f;
                }
                if (row >= rows || !col_ok) continue;
                if (S == 1) {
                    if (DUAL && c >= 8) continue;
                    store_epilogue<EPI, 4>(C + (size_t)(r0 + rc + row) * N + ccol, u, v, bias, e, N, ccol);
                } else {
                    // partial sums of this split: [split][row][NC], W3 products at column N + n
                    const int NC = DUAL ? 2 * N : N;
                    const int pcol = third ? N + ccol : ccol;
                    float *dst = part + ((size_t)split * A_total + (r0 + rc + row)) * NC + pcol;
                    *reinterpret_cast<f32x4 *>(dst) = f32x4{u[0], u[1], u[2], u[3]};
                }
            }
    }
}

struct Q4Plan {
    int NCB, slots, S, MB;
    size_t part_bytes;
};

// Column blocks, live-expert slots, row tile and K split of one layer.  S
// minimises an estimate of the layer's time, as for the bf16 kernel: a round
// is 256 CUs times the workgroups one CU holds (4 with 16-row tiles, 2 with
// 32: the kernel's register budget); a wave streams one k-step (1 KB of codes)
// per ~0.5 us plus ~3 k-steps of start-up and epilogue; the stream cannot beat
// ~6 TB/s; S > 1 adds the partials' write and read and a reduce launch.
Q4Plan q4_plan(const colibri_moe_shape_t &s, bool up) {
    Q4Plan p;
    const bool dual = up && s.act == COLIBRI_ACT_SWIGLU;
    const int K = up ? s.d : s.h;
    const int N = up ? s.h : s.d;
    p.MB = (2 * s.T <= 8 * s.E) ? 1 : 2;
    p.NCB = (N + (dual ? 32 : 64) - 1) / (dual ? 32 : 64);
    p.slots = std::min(s.E, 2 * s.T);
    const int G = K / kQ4Group;
    const long wg_per_split = (long)p.slots * ((p.NCB + kQ4Waves - 1) / kQ4Waves);
    const double cols = (double)N * (dual ? 2 : 1);
    const double weight_bytes = (double)p.slots * K * cols * 0.5;
#ifndef COLIBRI_Q4_STEP_US
#define COLIBRI_Q4_STEP_US 0.5
#endif
    const double step_us = COLIBRI_Q4_STEP_US;
    p.S = 1;
    double best = 1e300;
    for (int S = 1; S <= G; ++S) {
        const long per_round = 256L * (p.MB == 1 ? 4 : 2);
        const double rounds = (double)((wg_per_split * S + per_round - 1) / per_round);
        const double steps = 4.0 * ((G + S - 1) / S);
        double us = std::max(rounds * (steps + 3.0) * step_us, weight_bytes / 6.0e6);
        if (S > 1) us += 4.0 + 2.0 * S * (2.0 * s.T) * cols * 4 / 5.0e6;
        if (us < best * 0.97) best = us, p.S = S;
    }
    p.part_bytes = p.S > 1 ? align256((size_t)p.S * 2 * s.T * (dual ? 2 : 1) * N * 4) : 0;
    return p;
}

template <int EPI>
hipError_t launch_q4_t(const colibri_moe_shape_t &s, const Q4Plan &p, bool gather, const void *Am, const int32_t *sa,
                       const int32_t *offsets, const uint32_t *Q0, const uint32_t *Q1, const float *S0,
                       const float *S1, const uint8_t *Z0, const uint8_t *Z1, const void *bias, void *C, int K, int N,
                       void *scratch, hipStream_t st) {
    float *part = static_cast<float *>(scratch);
    const int blocks = p.slots * p.S * ((p.NCB + kQ4Waves - 1) / kQ4Waves);
#define COLIBRI_Q4_LAUNCH(MBV, G)                                                                                    \
    ffn_decode_q4_kernel<MBV, EPI, G><<<blocks, kQ4Waves * kWave, 0, st>>>(                                          \
        (const uint16_t *)Am, sa, s.T, offsets, s.E, Q0, Q1, S0, S1, Z0, Z1, (const uint16_t *)bias, (uint16_t *)C, K, \
        N, p.NCB, p.S, part)
    if (p.MB == 1) {
        if (gather) COLIBRI_Q4_LAUNCH(1, true);
        else COLIBRI_Q4_LAUNCH(1, false);
    } else {
        if (gather) COLIBRI_Q4_LAUNCH(2, true);
        else COLIBRI_Q4_LAUNCH(2, false);
    }
#undef COLIBRI_Q4_LAUNCH
    return hipGetLastError();
}

// bias-only view of the 4-bit weights for the split reduce
colibri_moe_experts_t bias_view(const colibri_moe_experts_q4_t &w) {
    colibri_moe_experts_t b{};
    b.b1 = w.b1;
    b.b2 = w.b2;
    return b;
}

}  // namespace

bool ffn_q4_eligible(const colibri_moe_shape_t &s) {
    return ffn_decode_eligible(s) && s.d % kQ4Group == 0 && s.h % kQ4Group == 0;
}

size_t ffn_decode_q4_scratch_bytes(const colibri_moe_shape_t &s) {
    if (!ffn_q4_eligible(s)) return 0;
    return std::max(q4_plan(s, true).part_bytes, q4_plan(s, false).part_bytes);
}

int ffn_down_splits_q4(const colibri_moe_shape_t &s) { return q4_plan(s, false).S; }

hipError_t launch_ffn_layers_q4(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                                const int32_t *offsets, const colibri_moe_experts_q4_t &w, void *y_sorted, void *ws,
                                bool reduce, hipStream_t st, const float **down_partials) {
    if (!ffn_q4_eligible(s)) return hipErrorInvalidValue;  // the callers check the shape first
    char *H = static_cast<char *>(ws);
    char *scratch = H + align256((size_t)2 * s.T * s.h * 2);
    const bool gather = sorted_assign != nullptr;
    const Q4Plan up = q4_plan(s, true), down = q4_plan(s, false);
    hipError_t e;
    switch (s.act) {
        case COLIBRI_ACT_RELU:
            e = launch_q4_t<EPI_ACT_RELU>(s, up, gather, x_rows, sorted_assign, offsets, w.q1, nullptr, w.s1, nullptr,
                                          w.z1, nullptr, w.b1, H, s.d, s.h, scratch, st);
            break;
        case COLIBRI_ACT_GELU:
            e = launch_q4_t<EPI_ACT_GELU>(s, up, gather, x_rows, sorted_assign, offsets, w.q1, nullptr, w.s1, nullptr,
                                          w.z1, nullptr, w.b1, H, s.d, s.h, scratch, st);
            break;
        default:
            e = launch_q4_t<EPI_SWIGLU>(s, up, gather, x_rows, sorted_assign, offsets, w.q1, w.q3, w.s1, w.s3, w.z1,
                                        w.z3, nullptr, H, s.d, s.h, scratch, st);
    }
    const colibri_moe_experts_t bv = bias_view(w);
    if (e == hipSuccess && up.S > 1)
        e = launch_split_reduce(s, true, up.S, offsets, bv, H, reinterpret_cast<const float *>(scratch), st);
    if (e != hipSuccess) return e;
    const void *b2 = s.act == COLIBRI_ACT_SWIGLU ? nullptr : w.b2;
    e = launch_q4_t<EPI_BIAS_ONLY>(s, down, false, H, nullptr, offsets, w.q2, nullptr, w.s2, nullptr, w.z2, nullptr,
                                   b2, y_sorted, s.h, s.d, scratch, st);
    if (down_partials) *down_partials = reinterpret_cast<const float *>(scratch);
    if (e == hipSuccess && down.S > 1 && reduce)
        e = launch_split_reduce(s, false, down.S, offsets, bv, y_sorted, reinterpret_cast<const float *>(scratch),
                                st);
    return e;
}

}  // namespace colibri
