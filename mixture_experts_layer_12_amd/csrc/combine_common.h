// The combine of one token's output vector, shared by the combine kernels
// (combine.hip) and the combine folded into the second layer's grouped GEMM
// (ffn_gemm.hip), so both form every output element with the same arithmetic
// in the same order.
//
// Colibri write-up [nxbn] http://m.nxbn.cn/news/48047 section 3.3 (output
// aggregation: the expert outputs are summed weighted by their gating scores);
// [rkmt] http://news.rkmt.cn/news/2271114 section 5.2 (a shared expert beside
// the routed ones) and [nxbn] section 2.1 (residual add fused into the expert
// computation).
//
//   out[t] = g[t,0] * Y[assign_pos[2t]] + g[t,1] * Y[assign_pos[2t+1]]
//            (+ shared[t], + residual[t], when given)
//
// in fp32: the second product is fused into the sum (fmaf), the addends follow
// in that order, and the result is rounded once to the storage type.
#pragma once

#include "device_common.h"
#include "ffn_common.h"
#include "launchers.h"

namespace colibri {

// The shared expert's row t, columns c .. c + VEC - 1, from its second layer's
// S split partials (part[s][t][...], rows `stride` floats apart per split),
// formed as the reduce forms it (8 interleaved sums in order, + b2, rounded to
// bf16), then added to o.
template <int VEC>
__device__ __forceinline__ void add_shared_partials(float (&o)[VEC], const SharedPartials &sp, size_t at, int c) {
    constexpr int U = 8;
    float y8[8][VEC];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int q = 0; q < VEC; ++q) y8[j][q] = 0.0f;
    for (int s0 = 0; s0 < sp.S; s0 += U) {
        float a[U][VEC];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float *src = sp.part + (size_t)min(s0 + u, sp.S - 1) * sp.stride + at;
#pragma unroll
            for (int q4 = 0; q4 < VEC; q4 += 4) {
                const f32x4 v = *reinterpret_cast<const f32x4 *>(src + q4);
#pragma unroll
                for (int r = 0; r < 4; ++r) a[u][q4 + r] = v[r];
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (s0 + u < sp.S)  // s0 is a multiple of 8: split s0 + u goes to sum u
#pragma unroll
                for (int q = 0; q < VEC; ++q) y8[u][q] += a[u][q];
    }
#pragma unroll
    for (int q = 0; q < VEC; ++q) {
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc += y8[j][q];
        const float yb = acc + (sp.b2 ? bf16_to_f32(sp.b2[c + q]) : 0.0f);
        o[q] += bf16_to_f32((uint16_t)f32_to_bf16_bits(yb));
    }
}

// out[t][c .. c + VEC) from the expert rows Y (dtype TE, sorted order), VEC =
// one 16-byte vector, in two steps -- the loads, then the arithmetic and the
// store -- so that a caller may keep several vectors' loads in flight.  A slot
// whose assign_pos is outside [0, 2T) contributes nothing.  The residual may
// be the output buffer itself (an in-place layer): each element is read by the
// thread that stores it afterwards, so neither pointer is restrict.
struct RowsVec {
    u32x4 y0, y1, sh, res;  // raw 16-byte vectors (4 fp32 or 8 bf16)
    float g0, g1;
};

template <typename TE>
__device__ __forceinline__ void rows_vec_load(RowsVec &r, const TE *y, const int32_t *pos, const float *gate, int T,
                                              int d, const TE *shared, const TE *residual, int t, int c) {
    const int A = 2 * T;
    const int p0 = pos[2 * t], p1 = pos[2 * t + 1];
    r.g0 = gate[2 * t];
    r.g1 = gate[2 * t + 1];
    const u32x4 z = {0u, 0u, 0u, 0u};
    r.y0 = (p0 >= 0 && p0 < A) ? *reinterpret_cast<const u32x4 *>(y + (size_t)p0 * d + c) : z;
    r.y1 = (p1 >= 0 && p1 < A) ? *reinterpret_cast<const u32x4 *>(y + (size_t)p1 * d + c) : z;
    const size_t at = (size_t)t * d + c;
    r.sh = shared ? *reinterpret_cast<const u32x4 *>(shared + at) : z;
    r.res = residual ? *reinterpret_cast<const u32x4 *>(residual + at) : z;
}

template <typename TE>
__device__ __forceinline__ void rows_vec_widen(const u32x4 &v, float (&o)[16 / sizeof(TE)]) {
    if constexpr (sizeof(TE) == 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(v[i]);
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) { o[2 * i] = bf16_lo(v[i]); o[2 * i + 1] = bf16_hi(v[i]); }
    }
}

// o = fmaf(g1, y1, g0 * y0), then (+ the shared row formed from its split
// partials, or + shared) and + residual, rounded once and stored.
template <typename TE>
__device__ __forceinline__ void rows_vec_finish(const RowsVec &r, bool has_shared, bool has_res, TE *out,
                                                const SharedPartials &sp, int d, int t, int c) {
    constexpr int VEC = 16 / sizeof(TE);
    float y0[VEC], y1[VEC], o[VEC];
    rows_vec_widen<TE>(r.y0, y0);
    rows_vec_widen<TE>(r.y1, y1);
#pragma unroll
    for (int q = 0; q < VEC; ++q) o[q] = fmaf(r.g1, y1[q], r.g0 * y0[q]);
    if (sp.part) {
        add_shared_partials<VEC>(o, sp, (size_t)t * d + c, c);  // bf16 layers only
    } else if (has_shared) {
        float v[VEC];
        rows_vec_widen<TE>(r.sh, v);
#pragma unroll
        for (int q = 0; q < VEC; ++q) o[q] += v[q];
    }
    if (has_res) {
        float v[VEC];
        rows_vec_widen<TE>(r.res, v);
#pragma unroll
        for (int q = 0; q < VEC; ++q) o[q] += v[q];
    }
    if constexpr (sizeof(TE) == 4) {
        *reinterpret_cast<f32x4 *>(out + (size_t)t * d + c) = f32x4{o[0], o[1], o[2], o[3]};
    } else {
        u32x4 ov;
#pragma unroll
        for (int q = 0; q < 4; ++q) ov[q] = pack_bf16x2(o[2 * q], o[2 * q + 1]);
        *reinterpret_cast<u32x4 *>(out + (size_t)t * d + c) = ov;
    }
}

template <typename TE>
__device__ __forceinline__ void combine_rows_vec(const TE *y, const int32_t *pos, const float *gate, TE *out, int T,
                                                 int d, const TE *shared, const TE *residual,
                                                 const SharedPartials &sp, int t, int c) {
    RowsVec r;
    rows_vec_load<TE>(r, y, pos, gate, T, d, sp.part ? nullptr : shared, residual, t, c);
    rows_vec_finish<TE>(r, shared != nullptr && sp.part == nullptr, residual != nullptr, out, sp, d, t, c);
}

// The gated sum of the expert row's two terms once each is formed from the
// second layer's S split partials: yb = (sum of the splits) + b2[e], rounded to
// bf16 (the value the split reduce would have stored), then
// o = g0 * y0, o = fmaf(g1, y1, o) over the live slots.
template <int VEC>
__device__ __forceinline__ void gate_partial_sums(float (&o)[VEC], const float (&y)[2][VEC], const bool (&live)[2],
                                                  const int (&e)[2], const float *gate, const uint16_t *b2, int d,
                                                  int t, int c) {
#pragma unroll
    for (int q = 0; q < VEC; ++q) o[q] = 0.0f;
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
        if (!live[sl]) continue;
        const float g = gate[2 * t + sl];
#pragma unroll
        for (int q = 0; q < VEC; ++q) {
            const float yb = y[sl][q] + (b2 ? bf16_to_f32(b2[(size_t)e[sl] * d + c + q]) : 0.0f);
            const float yr = bf16_to_f32((uint16_t)f32_to_bf16_bits(yb));  // Y is a bf16 value
            o[q] = sl == 0 ? g * yr : fmaf(g, yr, o[q]);
        }
    }
}

// out[t][c .. c + VEC) (bf16) straight from the second layer's S split partial
// sums part[s][p][.] (split stride 2T * d floats), one thread per vector.  The
// splits of each expert row are added in the split reduce's order: 8
// interleaved sums (sum j takes s = j, j + 8, ... in order), then those 8 in
// order j = 0 .. 7.  Splits are loaded U at a time (U a multiple of 8, or
// S <= U < 8).
template <int VEC, int U>
__device__ __forceinline__ void combine_partials_vec(const float *part, int S, const int32_t *pos,
                                                     const int32_t *idx, const float *gate, const uint16_t *b2, int E,
                                                     uint16_t *out, int T, int d, const uint16_t *shared,
                                                     const uint16_t *residual, const SharedPartials &sp, int t,
                                                     int c) {
    typedef float fv __attribute__((ext_vector_type(VEC)));
    static_assert(U % 8 == 0 || U < 8, "batch size");
    const int A = 2 * T;
    const size_t split_stride = (size_t)A * d;
    int p[2], e[2];
    bool live[2];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
        p[sl] = pos[2 * t + sl];
        e[sl] = idx[2 * t + sl];
        live[sl] = p[sl] >= 0 && p[sl] < A && e[sl] >= 0 && e[sl] < E;
    }
    float y8[2][8][VEC];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
            for (int q = 0; q < VEC; ++q) y8[sl][j][q] = 0.0f;
    // loads are unconditional (a dead slot reads row 0, then contributes
    // nothing), so no branch separates a load from its use; a last, partial
    // batch loads split S - 1 in its unused slots and skips their additions
    for (int mb = 0; mb < S; mb += U) {
        fv a[2][U];
#pragma unroll
        for (int sl = 0; sl < 2; ++sl) {
            const int row = live[sl] ? p[sl] : 0;
#pragma unroll
            for (int u = 0; u < U; ++u)
                a[sl][u] = *reinterpret_cast<const fv *>(part + min(mb + u, S - 1) * split_stride + (size_t)row * d + c);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (mb + u < S) {  // mb % 8 == 0 (U < 8: mb = 0), so split mb + u goes to sum u % 8
#pragma unroll
                for (int sl = 0; sl < 2; ++sl)
#pragma unroll
                    for (int q = 0; q < VEC; ++q) y8[sl][u % 8][q] += a[sl][u][q];
            }
        }
    }
    float y[2][VEC];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl)
#pragma unroll
        for (int q = 0; q < VEC; ++q) {
            float acc = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += y8[sl][j][q];
            y[sl][q] = acc;
        }
    float o[VEC];
    gate_partial_sums<VEC>(o, y, live, e, gate, b2, d, t, c);
    if (sp.part) add_shared_partials<VEC>(o, sp, (size_t)t * d + c, c);
    if (shared || residual) {
        const size_t at = (size_t)t * d + c;
#pragma unroll
        for (int q = 0; q < VEC; ++q) {
            if (shared && !sp.part) o[q] += bf16_to_f32(shared[at + q]);
            if (residual) o[q] += bf16_to_f32(residual[at + q]);
        }
    }
    uint16_t *dst = out + (size_t)t * d + c;
    static_assert(VEC == 4, "4 columns per thread");
    *reinterpret_cast<u32x2 *>(dst) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
}

}  // namespace colibri
