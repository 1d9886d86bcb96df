// Grouped per-expert two-layer FFN over the expert-sorted rows.
//
// Colibri write-ups: [zskr] http://www.zskr.cn/news/2272131 section 1 (each
// expert is a two-layer FFN) and 2.1 (the Compute stage is a grouped GEMM);
// [nxbn] http://m.nxbn.cn/news/48047 section 2.1 (matmul and activation fused in
// one per-expert kernel) and 3.1 (per-expert W1 | b1 | W2 | b2);
// [hnwysp] https://www.hnwysp.cn/news/30485 section 2.2 (feed the expert kernel
// row offsets instead of copying token rows) and 3.2 (affine layer per expert).
//
//   GEMM1: H[p] = act(X[tok(p)] W1[e] + b1[e])       (SwiGLU: silu(X W1) * (X W3))
//   GEMM2: Y[p] = H[p] W2[e] + b2[e]
// for every row p of expert e's segment [offsets[e], offsets[e+1]).
//
// Both GEMMs use one kernel template.  A workgroup owns one (row tile of one
// expert, column tile) pair; the row tiles of all experts are numbered
// expert by expert from the device-side offsets, so the host never reads the
// counts back: the grid is sized for the worst case and surplus workgroups
// exit.  GEMM1 gathers its A rows through sorted_assign (no copy of X).
//
// bf16 layers run the MFMA kernels of ffn_gemm.hip (T > 64) and
// ffn_decode.hip (T <= 64); this file holds the fp32 path -- a plain
// LDS-tiled FMA GEMM (64 x 64 tiles, 4 x 4 per thread) -- and the entry
// points that pick the kernel.
#include "device_common.h"
#include "ffn_common.h"
#include "launchers.h"

namespace colibri {
namespace {

// ------------------------------------------------------------------ tiles
struct TileInfo {
    int e, row0, rows;
};

// Locate row tile `mt` among the experts' tiles (ceil(count_e / BM) each, in
// expert order).  Executed by a whole wave; every lane gets the same answer.
// Offsets are clamped to [0, A] so that no offsets array can move a row
// outside the [A, *] buffers.
template <int BM>
__device__ __forceinline__ bool find_row_tile(const int32_t *__restrict__ offsets, int E, int A, int mt,
                                              TileInfo &ti) {
    const int lane = threadIdx.x & (kWave - 1);
    int lo = 0, hi = 0;
    if (lane < E) {
        lo = min(max(offsets[lane], 0), A);
        hi = min(max(offsets[lane + 1], lo), A);
    }
    const int cnt = hi > lo ? hi - lo : 0;
    const int nt = (cnt + BM - 1) / BM;
    int incl = nt;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) {
        const int o = __shfl_up(incl, s);
        if (lane >= s) incl += o;
    }
    const int excl = incl - nt;
    const uint64_t m = __ballot(lane < E && mt >= excl && mt < incl);
    if (m == 0) return false;
    const int l = __ffsll((unsigned long long)m) - 1;
    ti.e = l;
    ti.row0 = __shfl(lo, l) + (mt - __shfl(excl, l)) * BM;
    ti.rows = min(BM, __shfl(hi, l) - ti.row0);
    return true;
}

// Source row of A for tile row `p` (global row index in sorted order).
template <bool GATHER>
__device__ __forceinline__ long a_source_row(const int32_t *__restrict__ sa, int p, int T) {
    if (!GATHER) return p;
    const int a = sa[p];
    if (a < 0 || (a >> 1) >= T) return -1;
    return a >> 1;
}

// ------------------------------------------------------------------ fp32 FMA GEMM
template <int EPI, bool GATHER>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float *__restrict__ A,
                                                       const int32_t *__restrict__ sorted_assign, int T,
                                                       const int32_t *__restrict__ offsets, int E,
                                                       const float *__restrict__ B0, const float *__restrict__ B1,
                                                       const float *__restrict__ bias, float *__restrict__ C, int K,
                                                       int N, int max_m_tiles) {
    constexpr int BM = 64, BN = 64, BK = 16;
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    constexpr int NB = DUAL ? 2 : 1;
    __shared__ float As[BK][BM];
    __shared__ float Bs[NB][BK][BN];

    const int tid = threadIdx.x;
    const int mt = blockIdx.x % max_m_tiles;
    const int n0 = (blockIdx.x / max_m_tiles) * BN;
    TileInfo ti;
    if (!find_row_tile<BM>(offsets, E, 2 * T, mt, ti)) return;
    const int e = ti.e;

    const int ar = tid / 4, aq = tid % 4;
    long src = -1;
    if (ar < ti.rows) src = a_source_row<GATHER>(sorted_assign, ti.row0 + ar, T);
    const float *a_ptr = (src >= 0) ? A + (size_t)src * K + aq * 4 : nullptr;
    const int br = tid / 16, bq = tid % 16;
    const float *b_ptr[NB];
    b_ptr[0] = B0 + (size_t)e * K * N + (size_t)br * N + n0 + bq * 4;
    if (DUAL) b_ptr[NB - 1] = B1 + (size_t)e * K * N + (size_t)br * N + n0 + bq * 4;

    const int ty = tid / 16, tx = tid % 16;
    float acc[NB][4][4] = {};
    // the next k-tile's operands are loaded into registers while the current
    // one is multiplied, so each k-tile does not wait a full load latency
    f32x4 av, bv[NB];
    auto load = [&](int k0) {
        av = a_ptr ? *reinterpret_cast<const f32x4 *>(a_ptr + k0) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < NB; ++b) bv[b] = *reinterpret_cast<const f32x4 *>(b_ptr[b] + (size_t)k0 * N);
    };
    load(0);
    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
        for (int q = 0; q < 4; ++q) As[aq * 4 + q][ar] = av[q];
#pragma unroll
        for (int b = 0; b < NB; ++b) *reinterpret_cast<f32x4 *>(&Bs[b][br][bq * 4]) = bv[b];
        __syncthreads();
        if (k0 + BK < K) load(k0 + BK);
#pragma unroll
        for (int k = 0; k < BK; ++k) {
            const f32x4 a4 = *reinterpret_cast<const f32x4 *>(&As[k][ty * 4]);
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(&Bs[b][k][tx * 4]);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[b][i][j] = fmaf(a4[i], b4[j], acc[b][i][j]);
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = ty * 4 + i;
        if (m >= ti.rows) continue;
        f32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            const float bv = (EPI != EPI_SWIGLU && bias != nullptr) ? bias[(size_t)e * N + n] : 0.0f;
            float v;
            if (EPI == EPI_SWIGLU) v = silu(acc[0][i][j]) * acc[NB - 1][i][j];
            else if (EPI == EPI_ACT_RELU) v = apply_act<ACT_RELU>(acc[0][i][j] + bv);
            else if (EPI == EPI_ACT_GELU) v = apply_act<ACT_GELU>(acc[0][i][j] + bv);
            else v = acc[0][i][j] + bv;
            o[j] = v;
        }
        *reinterpret_cast<f32x4 *>(&C[(size_t)(ti.row0 + m) * N + n0 + tx * 4]) = o;
    }
}

// ------------------------------------------------------------------ launch
inline int max_row_tiles(int A, int E, int BM) { return (A + BM - 1) / BM + std::min(E, A); }

template <int EPI>
hipError_t launch_gemm_f32(bool gather, const void *Am, const int32_t *sa, int T, const int32_t *offsets, int E,
                           const void *B0, const void *B1, const void *bias, void *C, int K, int N, int A_rows,
                           hipStream_t st) {
    const int mtiles = max_row_tiles(A_rows, E, 64);
    const dim3 grid(mtiles * (N / 64));
    if (gather)
        gemm_f32_kernel<EPI, true><<<grid, 256, 0, st>>>((const float *)Am, sa, T, offsets, E, (const float *)B0,
                                                         (const float *)B1, (const float *)bias, (float *)C, K, N,
                                                         mtiles);
    else
        gemm_f32_kernel<EPI, false><<<grid, 256, 0, st>>>((const float *)Am, sa, T, offsets, E, (const float *)B0,
                                                          (const float *)B1, (const float *)bias, (float *)C, K, N,
                                                          mtiles);
    return hipGetLastError();
}

}  // namespace

size_t ffn_up_scratch_bytes(const colibri_moe_shape_t &s) {
    if (ffn_decode_eligible(s)) return ffn_decode_scratch_bytes(s);
    return s.dtype == COLIBRI_BF16 ? gemm_scratch_bytes(s, true) : 0;
}
size_t ffn_down_scratch_bytes(const colibri_moe_shape_t &s) {
    if (ffn_decode_eligible(s)) return ffn_decode_scratch_bytes(s);
    return s.dtype == COLIBRI_BF16 ? gemm_scratch_bytes(s, false) : 0;
}

int ffn_down_splits(const colibri_moe_shape_t &s, bool q8) {
    if (ffn_decode_eligible(s)) return decode_plan(s, false, q8).S;
    return s.dtype == COLIBRI_BF16 ? gemm_splits(s, false) : 1;
}

size_t ffn_workspace_bytes(const colibri_moe_shape_t &s) {
    const size_t el = s.dtype == COLIBRI_F32 ? 4 : 2;
    return align256((size_t)2 * s.T * s.h * el) + std::max(ffn_up_scratch_bytes(s), ffn_down_scratch_bytes(s));
}

hipError_t launch_ffn_up(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                         const int32_t *offsets, const colibri_moe_experts_t &w, void *H, void *scratch,
                         hipStream_t st) {
    if (ffn_decode_eligible(s))
        return launch_decode_up(s, x_rows, sorted_assign, offsets, decode_weights(w), H, scratch, st);
    const int A = 2 * s.T;
    const bool gather = sorted_assign != nullptr;
    if (s.dtype == COLIBRI_F32) {
        switch (s.act) {
            case COLIBRI_ACT_RELU:
                return launch_gemm_f32<EPI_ACT_RELU>(gather, x_rows, sorted_assign, s.T, offsets, s.E, w.w1,
                                                     nullptr, w.b1, H, s.d, s.h, A, st);
            case COLIBRI_ACT_GELU:
                return launch_gemm_f32<EPI_ACT_GELU>(gather, x_rows, sorted_assign, s.T, offsets, s.E, w.w1,
                                                     nullptr, w.b1, H, s.d, s.h, A, st);
            default:
                return launch_gemm_f32<EPI_SWIGLU>(gather, x_rows, sorted_assign, s.T, offsets, s.E, w.w1, w.w3,
                                                   nullptr, H, s.d, s.h, A, st);
        }
    }
    return launch_gemm_up(s, x_rows, sorted_assign, offsets, w, H, scratch, st);
}

size_t combine_fold_counts(const colibri_moe_shape_t &s) {
    if (s.dtype != COLIBRI_BF16 || s.T <= 0 || ffn_decode_eligible(s) || !gemm_fold_ok(s)) return 0;
    const GemmPlan p = gemm_plan(s, false);
    return (size_t)s.T * (size_t)ceil_div(s.d, p.BNC);
}

// The fold pays one L2 write-back and one L2 invalidation per tile of the
// second layer (cross-XCD visibility of the rows it reads), atomics and its
// tail work; measured on MI355X it does not beat the separate combine at the
// benchmarked shapes, so the default keeps the kernel.
bool combine_fold_preferred(const colibri_moe_shape_t &s) {
    (void)s;
    return false;
}

hipError_t launch_ffn_down(const colibri_moe_shape_t &s, const void *H, const int32_t *offsets,
                           const colibri_moe_experts_t &w, void *y_sorted, void *scratch, hipStream_t st,
                           bool reduce, const CombineFold *fold) {
    if (fold && combine_fold_counts(s) == 0) return hipErrorInvalidValue;  // no fold at this shape
    if (ffn_decode_eligible(s)) return launch_decode_down(s, H, offsets, decode_weights(w), y_sorted, scratch, reduce, st);
    const int A = 2 * s.T;
    const void *b2 = s.act == COLIBRI_ACT_SWIGLU ? nullptr : w.b2;
    if (s.dtype == COLIBRI_F32)
        return launch_gemm_f32<EPI_BIAS_ONLY>(false, H, nullptr, s.T, offsets, s.E, w.w2, nullptr, b2, y_sorted, s.h,
                                              s.d, A, st);
    return launch_gemm_down(s, H, offsets, w, y_sorted, scratch, reduce, st, fold);
}

namespace {
// Both decode-size layers (bf16 or int8 weights).  H first in ws, then the scratch.
hipError_t decode_layers(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                         const int32_t *offsets, const DecodeWeights &w, void *y_sorted, void *ws, bool reduce,
                         hipStream_t st, const float **down_partials) {
    char *H = static_cast<char *>(ws);
    char *scratch = H + align256((size_t)2 * s.T * s.h * 2);
    if (decode_fuse_h(s, w.q8)) {
        // the first layer leaves its split partials; the second layer rebuilds H from them
        char *down_scratch = scratch + align256(decode_plan(s, true, w.q8).part_bytes);
        if (down_partials) *down_partials = reinterpret_cast<const float *>(down_scratch);
        hipError_t e = launch_decode_up(s, x_rows, sorted_assign, offsets, w, H, scratch, st, false);
        if (e != hipSuccess) return e;
        return launch_decode_down(s, H, offsets, w, y_sorted, down_scratch, reduce, st,
                                  reinterpret_cast<const float *>(scratch));
    }
    if (down_partials) *down_partials = reinterpret_cast<const float *>(scratch);
    hipError_t e = launch_decode_up(s, x_rows, sorted_assign, offsets, w, H, scratch, st);
    if (e != hipSuccess) return e;
    return launch_decode_down(s, H, offsets, w, y_sorted, scratch, reduce, st);
}
}  // namespace

hipError_t launch_ffn_layers(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                             const int32_t *offsets, const colibri_moe_experts_t &w, void *y_sorted, void *ws,
                             bool reduce, hipStream_t st, const float **down_partials, const CombineFold *fold) {
    if (fold && combine_fold_counts(s) == 0) return hipErrorInvalidValue;  // no fold at this shape
    if (ffn_decode_eligible(s))
        return decode_layers(s, x_rows, sorted_assign, offsets, decode_weights(w), y_sorted, ws, reduce, st,
                             down_partials);
    const size_t el = s.dtype == COLIBRI_F32 ? 4 : 2;
    char *H = static_cast<char *>(ws);
    char *scratch = H + align256((size_t)2 * s.T * s.h * el);
    if (down_partials) *down_partials = reinterpret_cast<const float *>(scratch);
    hipError_t e = launch_ffn_up(s, x_rows, sorted_assign, offsets, w, H, scratch, st);
    if (e != hipSuccess) return e;
    return launch_ffn_down(s, H, offsets, w, y_sorted, scratch, st, reduce, fold);
}

hipError_t launch_ffn_layers_q8(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                                const int32_t *offsets, const colibri_moe_experts_q8_t &w, void *y_sorted, void *ws,
                                bool reduce, hipStream_t st, const float **down_partials) {
    if (!ffn_decode_eligible(s)) return hipErrorInvalidValue;  // the callers check the shape first
    return decode_layers(s, x_rows, sorted_assign, offsets, decode_weights(w), y_sorted, ws, reduce, st,
                         down_partials);
}

hipError_t launch_expert_ffn(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                             const int32_t *offsets, const colibri_moe_experts_t &w, void *y_sorted, void *ws,
                             hipStream_t st) {
    return launch_ffn_layers(s, x_rows, sorted_assign, offsets, w, y_sorted, ws, true, st, nullptr);
}

}  // namespace colibri
