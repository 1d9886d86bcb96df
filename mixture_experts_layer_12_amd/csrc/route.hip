// Router: logits, deterministic top-2 and gates, one launch.
//
// Colibri write-ups: [zskr] http://www.zskr.cn/news/2272131 section 3.2 (logits
// = input x routing weights, then a fixed-sequence top-k that is
// deterministic), [hnwysp] https://www.hnwysp.cn/news/30485 section 3.1
// (softmax over experts, top-k indices strictly descending by score) and 4.3
// (printed gate pairs sum to one), [rkmt] http://news.rkmt.cn/news/2271114
// section 3.1 (router bias [E]).
//
// Design (gfx950): one wavefront handles TPW = 64 / EP tokens, EP = E rounded
// up to a power of two.  Each lane streams 16-byte slices of the tokens' rows
// of X and the matching rows of W_r and accumulates TPW * EP = 64 partial dot
// products in fp32.  A six-step butterfly reduce-scatter (fixed order, so the
// result is reproducible) leaves lane l holding the full logit of token
// l / EP, expert l % EP.  The top-2 is then an argmax over the EP lanes of a
// token under the total order (logit desc, index asc; NaN below -inf),
// taken twice with xor-shuffles, which is deterministic by construction.
// Small batches (few token groups) split d over the W waves of a workgroup
// instead: each wave reduce-scatters its slice's partial logits and wave 0
// adds the W partials in wave order before the top-2.
#include "device_common.h"
#include "dispatch_block.h"
#include "launchers.h"

namespace colibri {
namespace {

constexpr int kRouteThreads = 128;  // 2 waves per block

// rank class: 2 = a number, 1 = NaN, 0 = padding lane / already chosen
__device__ __forceinline__ bool route_beats(int ca, float va, int ia, int cb, float vb, int ib) {
    if (ca != cb) return ca > cb;
    if (ca == 2 && va != vb) return va > vb;
    return ia < ib;
}

template <int EP>
__device__ __forceinline__ void segment_argmax(int &c, float &v, int &i) {
#pragma unroll
    for (int s = 1; s < EP; s <<= 1) {
        int oc = __shfl_xor(c, s);
        float ov = __shfl_xor(v, s);
        int oi = __shfl_xor(i, s);
        if (route_beats(oc, ov, oi, c, v, i)) { c = oc; v = ov; i = oi; }
    }
}

template <typename TI, int EP, bool FULL>
__device__ __forceinline__ void load_router_row(const TI *row, int E, float (&wv)[EP]) {
    if constexpr (FULL && EP * sizeof(TI) >= 16) {
#pragma unroll
        for (int q = 0; q < EP; q += Vec16<TI>::N) {
            float tmp[Vec16<TI>::N];
            Vec16<TI>::load(row + q, tmp);
#pragma unroll
            for (int r = 0; r < Vec16<TI>::N; ++r) wv[q + r] = tmp[r];
        }
    } else {
#pragma unroll
        for (int e = 0; e < EP; ++e) wv[e] = (FULL || e < E) ? Elem<TI>::load(row, e) : 0.0f;
    }
}

constexpr int kRouteMaxW = 8;   // waves sharing one token group (split of d)
constexpr int kFusedWaves = 8;  // waves of the fused route + dispatch workgroup
constexpr int kFusedGroups = 2; // token groups up to which routing and dispatch are fused

// One wave's partial logits of token group t0 over its slice of d (16-byte
// chunks j_first + i * j_stride).  Returns, in lane l, the sum for value index l
// (token t0 + l / EP, expert l % EP), reduced over the wave by a fixed
// butterfly reduce-scatter.
template <typename TI, int EP, bool FULL>
__device__ __forceinline__ float route_wave_partial(const TI *__restrict__ x, const TI *__restrict__ w_r, int T, int d,
                                                    int E, int t0, int j_first, int j_stride) {
    constexpr int TPW = kWave / EP;
    constexpr int VEC = Vec16<TI>::N;
    const int lane = threadIdx.x & (kWave - 1);
    float acc[TPW * EP];
#pragma unroll
    for (int i = 0; i < TPW * EP; ++i) acc[i] = 0.0f;

    for (int j0 = j_first + lane * VEC; j0 < d; j0 += j_stride) {
        if constexpr (EP <= 8) {
            // few experts: keep the VEC router rows in registers, stream the tokens
            float wv[VEC][EP];
#pragma unroll
            for (int jj = 0; jj < VEC; ++jj) load_router_row<TI, EP, FULL>(w_r + (size_t)(j0 + jj) * E, E, wv[jj]);
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                if (t0 + tt >= T) break;
                float xv[VEC];
                Vec16<TI>::load(x + (size_t)(t0 + tt) * d + j0, xv);
#pragma unroll
                for (int jj = 0; jj < VEC; ++jj)
#pragma unroll
                    for (int e = 0; e < EP; ++e) acc[tt * EP + e] += xv[jj] * wv[jj][e];
            }
        } else {
            // many experts: keep the tokens' slices in registers, stream the router rows
            float xv[TPW][VEC];
#pragma unroll
            for (int tt = 0; tt < TPW; ++tt) {
                if (t0 + tt < T) {
                    Vec16<TI>::load(x + (size_t)(t0 + tt) * d + j0, xv[tt]);
                } else {
#pragma unroll
                    for (int q = 0; q < VEC; ++q) xv[tt][q] = 0.0f;
                }
            }
#pragma unroll
            for (int jj = 0; jj < VEC; ++jj) {
                float wv[EP];
                load_router_row<TI, EP, FULL>(w_r + (size_t)(j0 + jj) * E, E, wv);
#pragma unroll
                for (int tt = 0; tt < TPW; ++tt)
#pragma unroll
                    for (int e = 0; e < EP; ++e) acc[tt * EP + e] += xv[tt][jj] * wv[e];
            }
        }
    }

    // Butterfly reduce-scatter over the 64 lanes: after the step on lane bit b
    // a lane keeps the half of its values selected by that bit, so at the end
    // lane l holds the complete sum for value index l.
#pragma unroll
    for (int b = 5; b >= 0; --b) {
        const int half = 1 << b;
        const bool up = (lane >> b) & 1;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            float send = up ? acc[i] : acc[i + half];
            float keep = up ? acc[i + half] : acc[i];
            acc[i] = keep + __shfl_xor(send, half);
        }
    }
    return acc[0];
}

// Top-2 and gates of token group t0 from the full logits (lane l: token
// t0 + l / EP, expert l % EP; bias not yet added).  sidx, when given, receives
// the chosen experts at [2 (t - t_base)] (an LDS copy for a fused dispatch).
// Gates (colibri_gate_t): softmax over the chosen pair, g0 = 1 / (1 + e^(l1 - l0))
// and g1 = 1 - g0; softmax over all experts, the pair taken unnormalised
// (DeepSeek-MoE, [rkmt] section 5.2): g = e^(l - l0) / sum_e e^(l_e - l0), the
// sum formed by a fixed xor-shuffle tree over the expert lanes; or the two
// logits themselves (LINEAR_SCORE, [zskr] section 2.3: no softmax).
template <int EP>
__device__ __forceinline__ void route_select(float lg, const float *__restrict__ b_r, int T, int E, int t0,
                                             int32_t *__restrict__ topk_idx, float *__restrict__ topk_gate,
                                             float *__restrict__ logits, int32_t *sidx, int gate_mode) {
    const int lane = threadIdx.x & (kWave - 1);
    const int tt = lane / EP;
    const int e = lane % EP;
    const int t = t0 + tt;
    const bool valid = (e < E) && (t < T);
    if (b_r != nullptr && e < E) lg += b_r[e];
    if (valid && logits != nullptr) logits[(size_t)t * E + e] = lg;

    int c1 = valid ? (__builtin_isnan(lg) ? 1 : 2) : 0;
    float v1 = lg;
    int i1 = e;
    segment_argmax<EP>(c1, v1, i1);
    int c2 = (valid && e != i1) ? (__builtin_isnan(lg) ? 1 : 2) : 0;
    float v2 = lg;
    int i2 = e;
    segment_argmax<EP>(c2, v2, i2);

    float g0, g1;
    if (gate_mode == COLIBRI_GATE_SOFTMAX) {
        float z = (valid && !__builtin_isnan(lg)) ? expf(lg - v1) : 0.0f;
#pragma unroll
        for (int s = 1; s < EP; s <<= 1) z += __shfl_xor(z, s);
        g0 = 1.0f / z;
        g1 = expf(v2 - v1) / z;
    } else if (gate_mode == COLIBRI_GATE_LINEAR) {
        g0 = v1;
        g1 = v2;
    } else {
        g0 = 1.0f / (1.0f + expf(v2 - v1));
        g1 = 1.0f - g0;
    }
    if (e == 0 && t < T) {
        topk_idx[2 * t] = i1;
        topk_idx[2 * t + 1] = i2;
        topk_gate[2 * t] = g0;
        topk_gate[2 * t + 1] = g1;
        if (sidx != nullptr) {
            sidx[2 * t] = i1;
            sidx[2 * t + 1] = i2;
        }
    }
}

// SPLITD: the block's W = blockDim.x / 64 waves share token group blockIdx.x
// and take interleaved slices of d; else every wave owns its own token group.
template <typename TI, int EP, bool FULL, bool SPLITD>
__global__ __launch_bounds__(SPLITD ? kRouteMaxW * kWave : kRouteThreads) void route_kernel(
    const TI *__restrict__ x, const TI *__restrict__ w_r, const float *__restrict__ b_r, int T, int d, int E,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_gate, float *__restrict__ logits, int gate_mode) {
    constexpr int TPW = kWave / EP;
    constexpr int VEC = Vec16<TI>::N;
    const int lane = threadIdx.x & (kWave - 1);
    const int W = SPLITD ? (int)(blockDim.x / kWave) : 1;
    const int wib = threadIdx.x / kWave;  // wave in block
    const int wave = SPLITD ? (int)blockIdx.x : (int)((blockIdx.x * blockDim.x + threadIdx.x) / kWave);
    const int t0 = wave * TPW;
    if (t0 >= T) return;  // uniform per wave (per block when SPLITD)
    __shared__ float red[SPLITD ? kRouteMaxW : 1][kWave];

    float lg = route_wave_partial<TI, EP, FULL>(x, w_r, T, d, E, t0, (SPLITD ? wib : 0) * kWave * VEC,
                                                W * kWave * VEC);
    if constexpr (SPLITD) {
        red[wib][lane] = lg;
        __syncthreads();
        if (wib != 0) return;
        float sum = red[0][lane];
        for (int q = 1; q < W; ++q) sum += red[q][lane];
        lg = sum;
    }
    route_select<EP>(lg, b_r, T, E, t0, topk_idx, topk_gate, logits, nullptr, gate_mode);
}

// Small batches: routing and dispatch in one workgroup of 8 waves.  The token
// groups' logits are formed exactly as route_kernel forms them (W waves per
// group split d and are added in wave order), the chosen experts stay in LDS,
// and dispatch_block runs on them after a barrier: one launch instead of two.
template <typename TI, int EP, bool FULL>
__global__ __launch_bounds__(kFusedWaves *kWave) void route_dispatch_kernel(
    const TI *__restrict__ x, const TI *__restrict__ w_r, const float *__restrict__ b_r, int T, int d, int E, int W,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_gate, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_assign, int32_t *__restrict__ assign_pos,
    int gate_mode) {
    constexpr int TPW = kWave / EP;
    constexpr int VEC = Vec16<TI>::N;
    constexpr int kMaxA = 2 * kFusedWaves * TPW;  // assignments of kFusedWaves token groups
    __shared__ float red[kFusedWaves][kWave];
    __shared__ int32_t sidx[kMaxA];
    __shared__ DispatchShared<kFusedWaves> dsh;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int gi = w / W, wib = w % W;  // token group and wave within it
    const int G = ceil_div(T, TPW);
    if (gi < G)
        red[w][lane] = route_wave_partial<TI, EP, FULL>(x, w_r, T, d, E, gi * TPW, wib * kWave * VEC, W * kWave * VEC);
    __syncthreads();
    if (gi < G && wib == 0) {
        float sum = red[w][lane];
        for (int q = 1; q < W; ++q) sum += red[w + q][lane];
        route_select<EP>(sum, b_r, T, E, gi * TPW, topk_idx, topk_gate, nullptr, sidx, gate_mode);
    }
    __syncthreads();
    dispatch_block<kFusedWaves>([&](int a) { return sidx[a]; }, 2 * T, E, counts, offsets, sorted_assign, assign_pos,
                                dsh);
}

// Waves per token group: with few groups, split d over W (a power of two, one
// 16-byte slice of d per lane at most) so that about 256 waves run; with at
// most kFusedGroups groups, also G * W <= 8 so that one workgroup holds them
// all (the fused route + dispatch kernel uses the same W, so both paths form
// every logit identically).  With more groups, fusing would leave each group
// too few waves: its d-stream costs more than the launch it saves.
inline int route_waves(int T, int d, int EP, int VEC) {
    const int G = ceil_div(T, kWave / EP);
    int W = 1;
    while (W < kRouteMaxW && G * W * 2 <= 256 && (W * 2) * kWave * VEC <= d && (G > kFusedGroups || G * W * 2 <= kFusedWaves))
        W *= 2;
    return W;
}

template <typename TI, int EP>
hipError_t launch_ep(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r, int32_t *idx,
                     float *gate, float *logits, int gate_mode, hipStream_t st) {
    constexpr int TPW = kWave / EP;
    constexpr int VEC = Vec16<TI>::N;
    const int groups = ceil_div(s.T, TPW);
    const int W = route_waves(s.T, s.d, EP, VEC);
#define COLIBRI_ROUTE_LAUNCH(FULLV, SPLITV, BLOCKS, THREADS)                                      \
    route_kernel<TI, EP, FULLV, SPLITV><<<BLOCKS, THREADS, 0, st>>>((const TI *)x, (const TI *)w_r, b_r, s.T, s.d, \
                                                                  s.E, idx, gate, logits, gate_mode)
    if (W > 1) {
        if (s.E == EP) COLIBRI_ROUTE_LAUNCH(true, true, groups, W * kWave);
        else COLIBRI_ROUTE_LAUNCH(false, true, groups, W * kWave);
    } else {
        const int blocks = ceil_div(groups, kRouteThreads / kWave);
        if (s.E == EP) COLIBRI_ROUTE_LAUNCH(true, false, blocks, kRouteThreads);
        else COLIBRI_ROUTE_LAUNCH(false, false, blocks, kRouteThreads);
    }
#undef COLIBRI_ROUTE_LAUNCH
    return hipGetLastError();
}

template <typename TI, int EP>
hipError_t launch_fused_ep(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r,
                           int32_t *idx, float *gate, int32_t *counts, int32_t *offsets, int32_t *sorted,
                           int32_t *pos, int gate_mode, hipStream_t st) {
    constexpr int VEC = Vec16<TI>::N;
    const int W = route_waves(s.T, s.d, EP, VEC);
#define COLIBRI_FUSED_LAUNCH(FULLV)                                                                          \
    route_dispatch_kernel<TI, EP, FULLV><<<1, kFusedWaves * kWave, 0, st>>>((const TI *)x, (const TI *)w_r, b_r, s.T, \
                                                                       s.d, s.E, W, idx, gate, counts, offsets,    \
                                                                       sorted, pos, gate_mode)
    if (s.E == EP) COLIBRI_FUSED_LAUNCH(true);
    else COLIBRI_FUSED_LAUNCH(false);
#undef COLIBRI_FUSED_LAUNCH
    return hipGetLastError();
}

template <typename TI>
hipError_t launch_t(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r, int32_t *idx,
                    float *gate, float *logits, int gm, hipStream_t st) {
    if (s.E <= 2) return launch_ep<TI, 2>(s, x, w_r, b_r, idx, gate, logits, gm, st);
    if (s.E <= 4) return launch_ep<TI, 4>(s, x, w_r, b_r, idx, gate, logits, gm, st);
    if (s.E <= 8) return launch_ep<TI, 8>(s, x, w_r, b_r, idx, gate, logits, gm, st);
    if (s.E <= 16) return launch_ep<TI, 16>(s, x, w_r, b_r, idx, gate, logits, gm, st);
    if (s.E <= 32) return launch_ep<TI, 32>(s, x, w_r, b_r, idx, gate, logits, gm, st);
    return launch_ep<TI, 64>(s, x, w_r, b_r, idx, gate, logits, gm, st);
}

template <typename TI>
hipError_t launch_fused_t(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r,
                          int32_t *idx, float *gate, int32_t *counts, int32_t *offsets, int32_t *sorted, int32_t *pos,
                          int gm, hipStream_t st) {
    if (s.E <= 2) return launch_fused_ep<TI, 2>(s, x, w_r, b_r, idx, gate, counts, offsets, sorted, pos, gm, st);
    if (s.E <= 4) return launch_fused_ep<TI, 4>(s, x, w_r, b_r, idx, gate, counts, offsets, sorted, pos, gm, st);
    return launch_fused_ep<TI, 8>(s, x, w_r, b_r, idx, gate, counts, offsets, sorted, pos, gm, st);
}

}  // namespace

hipError_t launch_route(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r,
                        int32_t *topk_idx, float *topk_gate, float *logits, hipStream_t st, int gate_mode) {
    if (s.dtype == COLIBRI_F32) return launch_t<float>(s, x, w_r, b_r, topk_idx, topk_gate, logits, gate_mode, st);
    return launch_t<uint16_t>(s, x, w_r, b_r, topk_idx, topk_gate, logits, gate_mode, st);
}

// E <= 8 and at most kFusedGroups token groups (T <= 16 for E = 8)
bool route_dispatch_fusable(const colibri_moe_shape_t &s) {
    if (s.E > 8 || s.T <= 0) return false;
    const int EP = s.E <= 2 ? 2 : s.E <= 4 ? 4 : 8;
    return ceil_div(s.T, kWave / EP) <= kFusedGroups;
}

hipError_t launch_route_dispatch(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r,
                                 int32_t *topk_idx, float *topk_gate, int32_t *counts, int32_t *offsets,
                                 int32_t *sorted_assign, int32_t *assign_pos, hipStream_t st, int gate_mode) {
    if (s.dtype == COLIBRI_F32)
        return launch_fused_t<float>(s, x, w_r, b_r, topk_idx, topk_gate, counts, offsets, sorted_assign, assign_pos,
                                     gate_mode, st);
    return launch_fused_t<uint16_t>(s, x, w_r, b_r, topk_idx, topk_gate, counts, offsets, sorted_assign, assign_pos,
                                    gate_mode, st);
}

}  // namespace colibri
