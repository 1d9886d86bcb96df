// Combine: gate-weighted sum of each token's two expert outputs, fused with
// the un-permute from expert-sorted order back to token order.
//
// Colibri write-up [nxbn] http://m.nxbn.cn/news/48047 section 3.3 (output
// aggregation: the expert outputs are summed weighted by their gating scores).
//
//   out[t] = g[t,0] * Y[assign_pos[2t]] + g[t,1] * Y[assign_pos[2t+1]]
//            (+ shared[t], a shared expert's output, + residual[t], when given)
//
// The optional addends follow [rkmt] http://news.rkmt.cn/news/2271114 section
// 5.2 (a shared expert applied to every token beside the routed ones) and
// [nxbn] section 2.1 (residual add fused into the expert computation): both
// are added in fp32 after the gated pair, in that order, before the one
// rounding.
//
// Design: a pure streaming kernel (reads 2 rows, writes 1 row per token).
// Each thread handles one 16-byte vector of a token row; rows are read with
// 16-byte loads and the sum is formed in fp32, then rounded once to the
// storage type.  A slot whose assign_pos is negative (an out-of-range expert
// index upstream) contributes nothing.
#include "combine_common.h"

namespace colibri {
namespace {

// A thread takes kCombineUnroll vectors, gridDim * blockDim apart, per pass
// and issues the loads of all of them before any arithmetic, so each thread
// keeps several rows' loads in flight (one vector per thread left the kernel
// bound by the latency of its dependent index and row loads).
constexpr int kCombineUnroll = 4;

template <typename TE>
__global__ __launch_bounds__(256) void combine_kernel(const TE *__restrict__ y, const int32_t *__restrict__ pos,
                                                      const float *__restrict__ gate, TE *out, int T, int d,
                                                      const TE *shared, const TE *residual, SharedPartials sp) {
    constexpr int VEC = 16 / sizeof(TE), U = kCombineUnroll;
    const int vpr = d / VEC;  // vectors per row
    const size_t total = (size_t)T * vpr;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    if (sp.part) {  // the shared row is formed from its partials inside the finish: one vector at a time
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride)
            combine_rows_vec<TE>(y, pos, gate, out, T, d, shared, residual, sp, (int)(i / vpr), (int)(i % vpr) * VEC);
        return;
    }
    for (size_t i0 = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i0 < total; i0 += U * stride) {
        RowsVec r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = i0 + u * stride;
            if (i < total)
                rows_vec_load<TE>(r[u], y, pos, gate, T, d, shared, residual, (int)(i / vpr), (int)(i % vpr) * VEC);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = i0 + u * stride;
            if (i < total)
                rows_vec_finish<TE>(r[u], shared != nullptr, residual != nullptr, out, sp, d, (int)(i / vpr),
                                    (int)(i % vpr) * VEC);
        }
    }
}

// Same combine, but each expert row Y[p] is first formed from the second
// layer's S split partial sums: Y[p] = bf16(sum of part[s][p] + b2[e]), the
// value the separate reduce would have stored, in the reduce's order (see
// combine_partials_vec).  L = 1: a thread forms both rows of its VEC output
// columns, loading U splits of each at a time; L = 8: the 8 lanes of a group
// each form one interleaved sum and lane 0 adds the 8 through shuffles and
// finishes the output (few outputs, many splits: decode sizes).
template <int VEC, int U, int L>
__global__ __launch_bounds__(256) void combine_partials_kernel(const float *__restrict__ part, int S,
                                                               const int32_t *__restrict__ pos,
                                                               const int32_t *__restrict__ idx,
                                                               const float *__restrict__ gate,
                                                               const uint16_t *__restrict__ b2, int E,
                                                               uint16_t *out, int T, int d, const uint16_t *shared,
                                                               const uint16_t *residual, SharedPartials sp) {
    typedef float fv __attribute__((ext_vector_type(VEC)));
    static_assert(L == 1 || L == 8, "lanes per output");
    const int vpr = d / VEC;
    const size_t total = (size_t)T * vpr;
    if constexpr (L == 1) {
        for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
             i += (size_t)gridDim.x * blockDim.x)
            combine_partials_vec<VEC, U>(part, S, pos, idx, gate, b2, E, out, T, d, shared, residual, sp,
                                         (int)(i / vpr), (int)(i % vpr) * VEC);
        return;
    }
    const int A = 2 * T;
    const size_t split_stride = (size_t)A * d;
    const int j0 = (int)(threadIdx.x & (L - 1));  // this lane's interleaved sum
    const int base = (int)(threadIdx.x & (kWave - 1)) & ~(L - 1);
    for (size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) / L; i < total;
         i += (size_t)gridDim.x * blockDim.x / L) {
        const int t = (int)(i / vpr);
        const int c = (int)(i % vpr) * VEC;
        int p[2], e[2];
        bool live[2];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            p[sl] = pos[2 * t + sl];
            e[sl] = idx[2 * t + sl];
            live[sl] = p[sl] >= 0 && p[sl] < A && e[sl] >= 0 && e[sl] < E;
        }
        float y8[2][VEC];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
            for (int q = 0; q < VEC; ++q) y8[sl][q] = 0.0f;
        // loads are unconditional (a dead slot reads row 0, then contributes
        // nothing), so no branch separates a load from its use
        auto load = [&](int s, int sl) {
            const int row = live[sl] ? p[sl] : 0;
            return *reinterpret_cast<const fv *>(part + s * split_stride + (size_t)row * d + c);
        };
        // this lane's splits: s = j0 + L m; batches of U of them; a last, partial
        // batch loads the lane's last split in its unused slots and skips their
        // additions, so the order of additions is unchanged
        const int nmine = S > j0 ? (S - j0 + L - 1) / L : 0;
        for (int mb = 0; mb < nmine; mb += U) {
            fv a[2][U];
#pragma unroll
            for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                for (int u = 0; u < U; ++u) a[sl][u] = load(j0 + L * min(mb + u, nmine - 1), sl);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (mb + u < nmine) {  // no break, so every index stays a constant
#pragma unroll
                    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                        for (int q = 0; q < VEC; ++q) y8[sl][q] += a[sl][u][q];
                }
            }
        }
        // the 8 interleaved sums in order
        float y[2][VEC];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl)
#pragma unroll
            for (int q = 0; q < VEC; ++q) {
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc += __shfl(y8[sl][q], base + j);
                y[sl][q] = acc;
            }
        // the shared expert's row from its own split partials: this lane's
        // interleaved sum, added over the 8 lanes in order by lane 0
        float ysh[VEC];
        if (sp.part) {
            float a8[VEC];
#pragma unroll
            for (int q = 0; q < VEC; ++q) a8[q] = 0.0f;
            const int nsh = sp.S > j0 ? (sp.S - j0 + L - 1) / L : 0;
            for (int mb = 0; mb < nsh; mb += U) {
                fv a[U];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    a[u] = *reinterpret_cast<const fv *>(sp.part + (size_t)(j0 + L * min(mb + u, nsh - 1)) * sp.stride +
                                                         (size_t)t * d + c);
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (mb + u < nsh)
#pragma unroll
                        for (int q = 0; q < VEC; ++q) a8[q] += a[u][q];
            }
#pragma unroll
            for (int q = 0; q < VEC; ++q) {
                float acc = 0.0f;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc += __shfl(a8[q], base + j);
                const float yb = acc + (sp.b2 ? bf16_to_f32(sp.b2[c + q]) : 0.0f);
                ysh[q] = bf16_to_f32((uint16_t)f32_to_bf16_bits(yb));
            }
        }
        if (j0 != 0) continue;
        float o[VEC];
        gate_partial_sums<VEC>(o, y, live, e, gate, b2, d, t, c);
        if (sp.part)
#pragma unroll
            for (int q = 0; q < VEC; ++q) o[q] += ysh[q];
        if (shared || residual) {
            const size_t at = (size_t)t * d + c;
#pragma unroll
            for (int q = 0; q < VEC; ++q) {
                if (shared && !sp.part) o[q] += bf16_to_f32(shared[at + q]);
                if (residual) o[q] += bf16_to_f32(residual[at + q]);
            }
        }
        static_assert(VEC == 4, "4 columns per output");
        *reinterpret_cast<u32x2 *>(out + (size_t)t * d + c) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    }
}

}  // namespace

hipError_t launch_combine(const colibri_moe_shape_t &s, const void *y_sorted, const int32_t *assign_pos,
                          const float *topk_gate, void *out, hipStream_t st, const void *shared,
                          const void *residual, SharedPartials sp) {
    const int vec = s.dtype == COLIBRI_F32 ? 4 : 8;
    const size_t total = (size_t)s.T * (s.d / vec);
    const size_t per_block = sp.part ? 256 : 256 * kCombineUnroll;  // vectors a block takes per pass
    const int blocks = (int)std::min<size_t>((total + per_block - 1) / per_block, 8192);
    if (s.dtype == COLIBRI_F32)
        combine_kernel<float><<<blocks, 256, 0, st>>>((const float *)y_sorted, assign_pos, topk_gate, (float *)out,
                                                      s.T, s.d, (const float *)shared, (const float *)residual,
                                                      SharedPartials{});  // fp32 layers have no split partials
    else
        combine_kernel<uint16_t><<<blocks, 256, 0, st>>>((const uint16_t *)y_sorted, assign_pos, topk_gate,
                                                         (uint16_t *)out, s.T, s.d, (const uint16_t *)shared,
                                                         (const uint16_t *)residual, sp);
    return hipGetLastError();
}

#ifndef COLIBRI_COMBINE_LANES_MIN_S
#define COLIBRI_COMBINE_LANES_MIN_S 9
#endif
hipError_t launch_combine_partials(const colibri_moe_shape_t &s, const float *part, int S, const int32_t *assign_pos,
                                   const int32_t *topk_idx, const float *topk_gate, const void *b2, void *out,
                                   hipStream_t st, const void *shared, const void *residual, SharedPartials sp) {
    const size_t total = (size_t)s.T * (s.d / 4);
    if (S >= COLIBRI_COMBINE_LANES_MIN_S && total <= 65536) {  // few outputs, several splits: 8 lanes per output
        // a lane adds ceil(S / 8) splits, loaded in batches no larger than that
        const int blocks = (int)std::min<size_t>((total * 8 + 255) / 256, 8192);
        const int per_lane = (S + 7) / 8;
#define COLIBRI_COMBINE_LANES(UV)                                                                              \
    combine_partials_kernel<4, UV, 8><<<blocks, 256, 0, st>>>(part, S, assign_pos, topk_idx, topk_gate,        \
                                                              (const uint16_t *)b2, s.E, (uint16_t *)out, s.T, \
                                                              s.d, (const uint16_t *)shared,                   \
                                                              (const uint16_t *)residual, sp)
        if (per_lane <= 2) COLIBRI_COMBINE_LANES(2);
        else if (per_lane <= 4) COLIBRI_COMBINE_LANES(4);
        else COLIBRI_COMBINE_LANES(8);
#undef COLIBRI_COMBINE_LANES
    } else {
        // one thread per output vector; batches no larger than S, so a thread
        // loads only the splits it adds
        const int blocks = (int)std::min<size_t>((total + 255) / 256, 8192);
#define COLIBRI_COMBINE_PARTIALS(UV)                                                                           \
    combine_partials_kernel<4, UV, 1><<<blocks, 256, 0, st>>>(part, S, assign_pos, topk_idx, topk_gate,        \
                                                              (const uint16_t *)b2, s.E, (uint16_t *)out, s.T, \
                                                              s.d, (const uint16_t *)shared,                   \
                                                              (const uint16_t *)residual, sp)
        if (S <= 2) COLIBRI_COMBINE_PARTIALS(2);
        else if (S <= 4) COLIBRI_COMBINE_PARTIALS(4);
        else if (S <= 8) COLIBRI_COMBINE_PARTIALS(8);
        else COLIBRI_COMBINE_PARTIALS(16);
#undef COLIBRI_COMBINE_PARTIALS
    }
    return hipGetLastError();
}

namespace {
__global__ void pair_offsets_kernel(int32_t *o, int n) {
    if (threadIdx.x == 0) o[0] = 0;
    if (threadIdx.x == 1) o[1] = n;
}
}  // namespace

hipError_t launch_pair_offsets(int32_t *offsets, int n, hipStream_t st) {
    pair_offsets_kernel<<<1, 64, 0, st>>>(offsets, n);
    return hipGetLastError();
}

}  // namespace colibri
