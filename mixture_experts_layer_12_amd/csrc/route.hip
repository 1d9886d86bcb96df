// Router: logits, deterministic top-2 and gates, one launch.
//
// Colibri write-ups: [zskr] http://www.zskr.cn/news/2272131 section 3.2 (logits
// = input x routing weights, then a fixed-sequence top-k that is
// deterministic), [hnwysp] https://www.hnwysp.cn/news/30485 section 3.1
// (softmax over experts, top-k indices strictly descending by score) and 4.3
// (printed gate pairs sum to one), [rkmt] http://news.rkmt.cn/news/2271114
// section 3.1 (router bias [E]).
//
// Design (gfx950).  bf16 layers: the logits are a skinny GEMM (E <= 64
// columns) on the matrix cores: a wave owns 16 tokens and a share of the
// k-steps of 32 rows, feeds v_mfma_f32_16x16x32_bf16 with 16 bytes of each
// token row and the k-step's W_r block (copied through LDS, since W_r is
// stored expert-minor and the B operand wants 8 consecutive rows of one
// expert), and the W waves of a tile add their sums in wave order.  fp32
// layers use VALU dot products: up to 64 tokens, lanes are (k-group, expert)
// pairs over a token group of TW tokens; beyond that, lanes stream 16-byte
// slices of d with every expert's weights of the slice in registers (the
// "wide" kernel), reduced by a butterfly.  Every path ends in the same select:
// lanes (token, expert), EP = E rounded up to a power of two, an argmax over
// the EP lanes of a token under the total order (logit desc, index asc; NaN
// below -inf), taken twice with xor-shuffles, deterministic by construction.
// Small batches (at most two tiles) fuse routing with the dispatch in one
// workgroup.
#include "device_common.h"
#include "dispatch_block.h"
#include "launchers.h"

namespace colibri {
namespace {

#ifndef COLIBRI_ROUTE_SMALL_T
#define COLIBRI_ROUTE_SMALL_T 64
#endif
// fp32 batches of at most kRouteSmallT tokens take route_kernel (lanes over
// (k-group, expert), few k-steps per wave); larger ones route_wide_kernel (lanes
// over 16-byte slices of d, every expert's weights of a slice in registers:
// fewer load instructions per token once there are enough tokens to share them).
constexpr int kRouteSmallT = COLIBRI_ROUTE_SMALL_T;
constexpr int kRouteMaxW = 16;   // waves sharing one token group (split of the k-steps)
constexpr int kFusedWaves = 16;  // waves of the fused route + dispatch workgroup
constexpr int kFusedGroups = 2;  // token groups up to which fp32 routing and dispatch are fused
// bf16 (MFMA router): one 16-token tile.  At 17..32 tokens the two launches,
// whose router spreads each tile's k-steps over more waves, were faster
// (Mixtral-shaped T = 24 / 32: 449.1 -> 447.1, 452.4 -> 449.7 us per layer;
// 8-expert T = 32: 94.0 -> 93.1 us).
constexpr int kFusedGroupsMfma = 1;

template <int EP> constexpr int route_tw() { return EP == 2 ? 32 : 16; }  // tokens per group (a multiple of 64 / EP)

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

// 8 consecutive values of a row, widened to fp32 (16 bytes of bf16, 32 of fp32)
template <typename TI>
__device__ __forceinline__ void load8(const TI *p, float (&o)[8]) {
    if constexpr (sizeof(TI) == 2) {
        Vec16<TI>::load(p, o);
    } else {
        float a[4], b[4];
        Vec16<TI>::load(p, a);
        Vec16<TI>::load(p + 4, b);
#pragma unroll
        for (int i = 0; i < 4; ++i) { o[i] = a[i]; o[4 + i] = b[i]; }
    }
}

// Partial logits of token group t0 over the k-steps ks0, ks0 + kstride, ...
// acc[t] (t < TW) is the sum for token t0 + t and expert lane % EP, complete
// over the wave's k-steps in every lane of that expert.  Within a lane the
// products are added in row order, k-step after k-step; the k-groups are then
// added by a fixed xor tree (every lane of an expert gets the same bits).
template <typename TI, int EP, bool FULL, int TW>
__device__ __forceinline__ void route_group_partial(const TI *__restrict__ x, const TI *__restrict__ w_r, int T,
                                                    int d, int E, int t0, int ks0, int kstride, float (&acc)[TW]) {
    constexpr int KG = kWave / EP;
    constexpr int KS = 8 * KG;  // rows of W_r per k-step
    const int lane = threadIdx.x & (kWave - 1);
    const int e = lane % EP, g = lane / EP;
    const bool live = FULL || e < E;
    const int col = live ? e : 0;  // padding lanes read column 0 and weight it by zero
    const int nt = min(TW, T - t0);
#pragma unroll
    for (int t = 0; t < TW; ++t) acc[t] = 0.0f;
    for (int ks = ks0; ks * KS < d; ks += kstride) {
        const int j = ks * KS + 8 * g;  // d is a multiple of 64, so a k-group's 8 rows are all in or all out
        if (j >= d) continue;
        float w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float v = Elem<TI>::load(w_r, (size_t)(j + i) * E + col);
            w[i] = live ? v : 0.0f;
        }
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            if (t < nt) {  // uniform
                float xv[8];
                load8<TI>(x + (size_t)(t0 + t) * d + j, xv);
                float a = acc[t];
#pragma unroll
                for (int i = 0; i < 8; ++i) a = fmaf(xv[i], w[i], a);
                acc[t] = a;
            }
        }
    }
#pragma unroll
    for (int s = EP; s < kWave; s <<= 1)
#pragma unroll
        for (int t = 0; t < TW; ++t) acc[t] += __shfl_xor(acc[t], s);
}

// acc[r * TPW + g] for this lane's k-group g (TPW = 64 / EP tokens per select round)
template <int EP, int TW>
__device__ __forceinline__ float round_value(const float (&acc)[TW], int r) {
    constexpr int TPW = kWave / EP;
    const int g = (threadIdx.x & (kWave - 1)) / EP;
    float v = acc[0];
#pragma unroll
    for (int q = 0; q < TW; ++q)
        if (q / TPW == r && q % TPW == g) v = acc[q];
    return v;
}

constexpr int kRouteThreads = 128;  // wide path: 2 waves per block
constexpr int kWideMaxW = 8;        // wide path: waves sharing one token group

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

// Larger batches (route_wide_kernel): one wave's partial logits of token
// group t0 (TPW = 64 / EP tokens) over its slice of d (16-byte
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

// One token group per block: W waves split its k-steps; their sums are added
// in wave order (through LDS when W > 1), then the select rounds (TW / TPW of
// them, TPW = 64 / EP tokens each) are spread over the waves.
template <typename TI, int EP, bool FULL>
__global__ __launch_bounds__(kRouteMaxW *kWave) void route_kernel(
    const TI *__restrict__ x, const TI *__restrict__ w_r, const float *__restrict__ b_r, int T, int d, int E,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_gate, float *__restrict__ logits, int gate_mode) {
    constexpr int TW = route_tw<EP>();
    constexpr int TPW = kWave / EP;
    constexpr int R = TW / TPW;
    const int lane = threadIdx.x & (kWave - 1);
    const int W = (int)(blockDim.x / kWave);
    const int w = threadIdx.x / kWave;
    const int t0 = (int)blockIdx.x * TW;
    __shared__ float red[kRouteMaxW][TW][EP];
    float acc[TW];
    route_group_partial<TI, EP, FULL, TW>(x, w_r, T, d, E, t0, w, W, acc);
    if (W == 1) {
#pragma unroll
        for (int r = 0; r < R; ++r)
            route_select<EP>(round_value<EP, TW>(acc, r), b_r, T, E, t0 + r * TPW, topk_idx, topk_gate, logits,
                             nullptr, gate_mode);
        return;
    }
    if (lane < EP)
#pragma unroll
        for (int t = 0; t < TW; ++t) red[w][t][lane] = acc[t];
    __syncthreads();
    const int e = lane % EP, g = lane / EP;
    for (int r = w; r < R; r += W) {
        float sum = red[0][r * TPW + g][e];
        for (int q = 1; q < W; ++q) sum += red[q][r * TPW + g][e];
        route_select<EP>(sum, b_r, T, E, t0 + r * TPW, topk_idx, topk_gate, logits, nullptr, gate_mode);
    }
}

// Wide path.  SPLITD: the block's W = blockDim.x / 64 waves share token group blockIdx.x
// and take interleaved slices of d; else every wave owns its own token group.
template <typename TI, int EP, bool FULL, bool SPLITD>
__global__ __launch_bounds__(SPLITD ? kWideMaxW * kWave : kRouteThreads) void route_wide_kernel(
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
    __shared__ float red[SPLITD ? kWideMaxW : 1][kWave];

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

// Waves per token group of the wide path: split d over W (a power of two, one
// 16-byte slice of d per lane at most) so that about 256 waves run.
inline int wide_waves(int T, int d, int EP, int VEC) {
    const int G = ceil_div(T, kWave / EP);
    int W = 1;
    while (W < kWideMaxW && G * W * 2 <= 256 && (W * 2) * kWave * VEC <= d)
        W *= 2;
    return W;
}

// ---- bf16: the logits as MFMA products (v_mfma_f32_16x16x32_bf16).
// A wave owns a tile of 16 tokens and the k-steps ks0, ks0 + kstride, ... of
// 32 rows of W_r each.  Per k-step a lane loads 16 bytes of its token's row of
// X (the A operand: token l % 16, rows 8 (l / 16) .. + 7) and up to EP / 16
// 16-byte pieces of the k-step's W_r block (32 rows x E, contiguous and
// 16-byte aligned whatever E is); the block is copied into the wave's own LDS
// slot and each lane gathers its B operand (rows 8 (l / 16) .. + 7 of expert
// 16 j + l % 16, zero past E) from there.  The next k-step's loads are issued
// before the current one is consumed.  The MFMA sums each 32-row k-step in
// fp32 and the k-steps are added in order; a wave's 16 x EP sums leave through
// LDS.
template <int EP> constexpr int mfma_nt() { return EP >= 16 ? EP / 16 : 1; }  // 16-expert column tiles
template <int EP> constexpr int mfma_nv() { return EP >= 16 ? EP / 16 : 1; }  // 16-byte W_r pieces per lane per k-step
template <int EP> constexpr int mfma_maxw() { return EP == 64 ? 8 : 16; }      // waves per token tile (LDS budget)

template <int EP>
__device__ __forceinline__ void route_mfma_partial(const uint16_t *__restrict__ x, const uint16_t *__restrict__ w_r,
                                                   int T, int d, int E, int t0, int ks0, int kstride,
                                                   uint16_t *__restrict__ wblk, f32x4 (&acc)[mfma_nt<EP>()]) {
    constexpr int NT = mfma_nt<EP>(), NV = mfma_nv<EP>();
    const int lane = threadIdx.x & (kWave - 1);
    const int c = lane & 15, g = lane >> 4;
    const uint16_t *arow = x + (size_t)min(t0 + c, T - 1) * d + 8 * g;  // rows past T repeat row T - 1 (unused)
    const int nvec = 4 * E;                                             // 16-byte pieces of one k-step block
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int nks = d / 32;
    if (ks0 >= nks) return;
    auto load = [&](int ks, u32x4 &a, u32x4 (&w)[NV]) {
        a = *reinterpret_cast<const u32x4 *>(arow + (size_t)ks * 32);
        const uint16_t *blk = w_r + (size_t)ks * 32 * E;
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int v = lane + kWave * q;
            w[q] = v < nvec ? *reinterpret_cast<const u32x4 *>(blk + 8 * v) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    u32x4 a_nx, w_nx[NV];
    load(ks0, a_nx, w_nx);
    for (int ks = ks0; ks < nks; ks += kstride) {
        const u32x4 a = a_nx;
        u32x4 w[NV];
#pragma unroll
        for (int q = 0; q < NV; ++q) w[q] = w_nx[q];
        if (ks + kstride < nks) load(ks + kstride, a_nx, w_nx);
        // the k-step block into this wave's LDS slot, then the B operands out of it
#pragma unroll
        for (int q = 0; q < NV; ++q) {
            const int v = lane + kWave * q;
            if (v < nvec) *reinterpret_cast<u32x4 *>(wblk + 8 * v) = w[q];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const bf16x8 afrag = __builtin_bit_cast(bf16x8, a);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const int e = 16 * j + c;
            const bool live = e < E;
            const int col = live ? e : 0;
            u32x4 b;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t lo = wblk[(8 * g + 2 * r) * E + col];
                const uint32_t hi = wblk[(8 * g + 2 * r + 1) * E + col];
                b[r] = live ? (lo | (hi << 16)) : 0u;
            }
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, __builtin_bit_cast(bf16x8, b), acc[j], 0, 0, 0);
        }
        // this step's LDS reads are issued before the next step's writes (a wave's
        // LDS operations run in order)
        __builtin_amdgcn_wave_barrier();
    }
}

// acc (D layout: token 4 (l / 16) + r, expert 16 j + l % 16) -> red[token][expert]
template <int EP>
__device__ __forceinline__ void mfma_store(const f32x4 (&acc)[mfma_nt<EP>()], float (*red)[EP]) {
    const int lane = threadIdx.x & (kWave - 1);
    const int c = lane & 15, g = lane >> 4;
#pragma unroll
    for (int j = 0; j < mfma_nt<EP>(); ++j)
        if (16 * j + c < EP)
#pragma unroll
            for (int r = 0; r < 4; ++r) red[4 * g + r][16 * j + c] = acc[j][r];
}

// The select rounds of one 16-token tile whose W partial sums are in red[0..W-1]
// (added in wave order): round r (TPW = 64 / EP tokens) by wave r mod W.
template <int EP>
__device__ __forceinline__ void mfma_select(float (*red)[16][EP], int W, int wib, const float *__restrict__ b_r,
                                            int T, int E, int t0, int32_t *__restrict__ topk_idx,
                                            float *__restrict__ topk_gate, float *__restrict__ logits,
                                            int32_t *sidx, int gate_mode) {
    constexpr int TPW = kWave / EP;
    constexpr int R = TPW >= 16 ? 1 : 16 / TPW;
    const int lane = threadIdx.x & (kWave - 1);
    const int tt = lane / EP, e = lane % EP;
    const int Tt = min(T, t0 + 16);  // tokens of this tile
    for (int r = wib; r < R; r += W) {
        const int tok = min(r * TPW + tt, 15);
        float sum = red[0][tok][e];
        for (int q = 1; q < W; ++q) sum += red[q][tok][e];
        route_select<EP>(sum, b_r, Tt, E, t0 + r * TPW, topk_idx, topk_gate, logits, sidx, gate_mode);
    }
}

template <int EP>
__global__ __launch_bounds__(mfma_maxw<EP>() * kWave) void route_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w_r, const float *__restrict__ b_r, int T, int d,
    int E, int32_t *__restrict__ topk_idx, float *__restrict__ topk_gate, float *__restrict__ logits,
    int gate_mode) {
    constexpr int MW = mfma_maxw<EP>();
    __shared__ __align__(16) uint16_t wblk[MW][32 * EP];
    __shared__ float red[MW][16][EP];
    const int W = (int)(blockDim.x / kWave);
    const int w = threadIdx.x / kWave;
    const int t0 = (int)blockIdx.x * 16;
    f32x4 acc[mfma_nt<EP>()];
    route_mfma_partial<EP>(x, w_r, T, d, E, t0, w, W, wblk[w], acc);
    mfma_store<EP>(acc, red[w]);
    __syncthreads();
    mfma_select<EP>(red, W, w, b_r, T, E, t0, topk_idx, topk_gate, logits, nullptr, gate_mode);
}

// Routing and dispatch in one workgroup of 16 waves for at most kFusedGroupsMfma
// tiles of 16 tokens; W waves per tile as in route_mfma_kernel, so the logits
// are identical.
template <int EP>
__global__ __launch_bounds__(kFusedWaves *kWave) void route_dispatch_mfma_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ w_r, const float *__restrict__ b_r, int T, int d,
    int E, int W, int32_t *__restrict__ topk_idx, float *__restrict__ topk_gate, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_assign, int32_t *__restrict__ assign_pos,
    int gate_mode) {
    constexpr int MW = mfma_maxw<EP>();
    __shared__ __align__(16) uint16_t wblk[MW][32 * EP];
    __shared__ float red[MW][16][EP];
    __shared__ int32_t sidx[2 * kFusedGroupsMfma * 16];
    __shared__ DispatchShared<kFusedWaves> dsh;
    const int w = threadIdx.x / kWave;
    const int gi = w / W, wib = w % W;
    const int G = ceil_div(T, 16);
    if (gi < G && w < MW) {
        f32x4 acc[mfma_nt<EP>()];
        route_mfma_partial<EP>(x, w_r, T, d, E, gi * 16, wib, W, wblk[w], acc);
        mfma_store<EP>(acc, red[w]);
    }
    __syncthreads();
    if (gi < G && w < MW)
        mfma_select<EP>(red + gi * W, W, wib, b_r, T, E, gi * 16, topk_idx, topk_gate, nullptr, sidx, gate_mode);
    __syncthreads();
    dispatch_block<kFusedWaves>([&](int a) { return sidx[a]; }, 2 * T, E, counts, offsets, sorted_assign, assign_pos,
                                dsh);
}

// Waves per 16-token tile of the MFMA router: a power of two up to
// mfma_maxw<EP>, each wave keeping at least 4 k-steps of 32 rows, G W <=
// kMfmaMaxWaves in all; with at most kFusedGroupsMfma tiles also G W <= the fused
// kernel's wave slots, min(kFusedWaves, mfma_maxw<EP>) (it uses the same W, so
// both paths form every logit identically).
#ifndef COLIBRI_MFMA_MAX_WAVES
#define COLIBRI_MFMA_MAX_WAVES 8192
#endif
constexpr int kMfmaMaxWaves = COLIBRI_MFMA_MAX_WAVES;  // waves of one launch at most
inline int mfma_waves(int T, int d, int EP) {
    const int G = ceil_div(T, 16);
    const int nks = d / 32;
    const int maxw = EP == 64 ? mfma_maxw<64>() : mfma_maxw<32>();
    int W = 1;
    const int fused = kFusedWaves < maxw ? kFusedWaves : maxw;
    while (W < maxw && nks >= 8 * W && G * W * 2 <= kMfmaMaxWaves && (G > kFusedGroupsMfma || G * W * 2 <= fused))
        W *= 2;
    return W;
}

// Small batches: routing and dispatch in one workgroup of 16 waves.  Each of
// the G <= 2 token groups gets W waves (G W <= 16, the W of route_kernel), so
// the logits are formed exactly as route_kernel forms them; the chosen experts
// stay in LDS, and dispatch_block runs on them after a barrier: one launch
// instead of two.
template <typename TI, int EP, bool FULL>
__global__ __launch_bounds__(kFusedWaves *kWave) void route_dispatch_kernel(
    const TI *__restrict__ x, const TI *__restrict__ w_r, const float *__restrict__ b_r, int T, int d, int E, int W,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_gate, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_assign, int32_t *__restrict__ assign_pos,
    int gate_mode) {
    constexpr int TW = route_tw<EP>();
    constexpr int TPW = kWave / EP;
    constexpr int R = TW / TPW;
    constexpr int kMaxA = 2 * kFusedGroups * TW;
    __shared__ float red[kFusedWaves][TW][EP];
    __shared__ int32_t sidx[kMaxA];
    __shared__ DispatchShared<kFusedWaves> dsh;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    const int gi = w / W, wib = w % W;  // token group and wave within it
    const int G = ceil_div(T, TW);
    if (gi < G) {
        float acc[TW];
        route_group_partial<TI, EP, FULL, TW>(x, w_r, T, d, E, gi * TW, wib, W, acc);
        if (lane < EP)
#pragma unroll
            for (int t = 0; t < TW; ++t) red[w][t][lane] = acc[t];
    }
    __syncthreads();
    if (gi < G) {
        const int e = lane % EP, g = lane / EP;
        for (int r = wib; r < R; r += W) {
            float sum = red[gi * W][r * TPW + g][e];
            for (int q = 1; q < W; ++q) sum += red[gi * W + q][r * TPW + g][e];
            route_select<EP>(sum, b_r, T, E, gi * TW + r * TPW, topk_idx, topk_gate, nullptr, sidx, gate_mode);
        }
    }
    __syncthreads();
    dispatch_block<kFusedWaves>([&](int a) { return sidx[a]; }, 2 * T, E, counts, offsets, sorted_assign, assign_pos,
                                dsh);
}

// Waves per token group: a power of two, at most kRouteMaxW, each wave keeping
// at least 2 k-steps, and G W <= 1024 waves in all; with at most kFusedGroups
// groups also G W <= kFusedWaves, so that one workgroup holds them all (the
// fused route + dispatch kernel uses the same W, so both paths form every logit
// identically).
inline int route_waves(int T, int d, int EP) {
    const int TW = EP == 2 ? 32 : 16;
    const int G = ceil_div(T, TW);
    const int nks = ceil_div(d, 8 * (kWave / EP));
    int W = 1;
    while (W < kRouteMaxW && nks >= 4 * W && G * W * 2 <= 1024 && (G > kFusedGroups || G * W * 2 <= kFusedWaves))
        W *= 2;
    return W;
}

template <typename TI, int EP>
hipError_t launch_wide(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r, int32_t *idx,
                       float *gate, float *logits, int gate_mode, hipStream_t st) {
    constexpr int TPW = kWave / EP;
    constexpr int VEC = Vec16<TI>::N;
    const int groups = ceil_div(s.T, TPW);
    const int W = wide_waves(s.T, s.d, EP, VEC);
#define COLIBRI_ROUTE_LAUNCH(FULLV, SPLITV, BLOCKS, THREADS)                                                      \
    route_wide_kernel<TI, EP, FULLV, SPLITV><<<BLOCKS, THREADS, 0, st>>>((const TI *)x, (const TI *)w_r, b_r, s.T, \
                                                                       s.d, s.E, idx, gate, logits, gate_mode)
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
hipError_t launch_ep(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r, int32_t *idx,
                     float *gate, float *logits, int gate_mode, hipStream_t st) {
    if constexpr (sizeof(TI) == 2) {
        const int W = mfma_waves(s.T, s.d, EP);
        route_mfma_kernel<EP><<<ceil_div(s.T, 16), W * kWave, 0, st>>>(
            (const uint16_t *)x, (const uint16_t *)w_r, b_r, s.T, s.d, s.E, idx, gate, logits, gate_mode);
        return hipGetLastError();
    }
    if (s.T > kRouteSmallT) return launch_wide<TI, EP>(s, x, w_r, b_r, idx, gate, logits, gate_mode, st);
    const int groups = ceil_div(s.T, route_tw<EP>());
    const int W = route_waves(s.T, s.d, EP);
    if (s.E == EP)
        route_kernel<TI, EP, true><<<groups, W * kWave, 0, st>>>((const TI *)x, (const TI *)w_r, b_r, s.T, s.d, s.E,
                                                                  idx, gate, logits, gate_mode);
    else
        route_kernel<TI, EP, false><<<groups, W * kWave, 0, st>>>((const TI *)x, (const TI *)w_r, b_r, s.T, s.d,
                                                                   s.E, idx, gate, logits, gate_mode);
    return hipGetLastError();
}

template <typename TI, int EP>
hipError_t launch_fused_ep(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r,
                           int32_t *idx, float *gate, int32_t *counts, int32_t *offsets, int32_t *sorted,
                           int32_t *pos, int gate_mode, hipStream_t st) {
    if constexpr (sizeof(TI) == 2) {
        const int W = mfma_waves(s.T, s.d, EP);
        route_dispatch_mfma_kernel<EP><<<1, kFusedWaves * kWave, 0, st>>>(
            (const uint16_t *)x, (const uint16_t *)w_r, b_r, s.T, s.d, s.E, W, idx, gate, counts, offsets, sorted,
            pos, gate_mode);
        return hipGetLastError();
    }
    const int W = route_waves(s.T, s.d, EP);
    if (s.E == EP)
        route_dispatch_kernel<TI, EP, true><<<1, kFusedWaves * kWave, 0, st>>>(
            (const TI *)x, (const TI *)w_r, b_r, s.T, s.d, s.E, W, idx, gate, counts, offsets, sorted, pos, gate_mode);
    else
        route_dispatch_kernel<TI, EP, false><<<1, kFusedWaves * kWave, 0, st>>>(
            (const TI *)x, (const TI *)w_r, b_r, s.T, s.d, s.E, W, idx, gate, counts, offsets, sorted, pos, gate_mode);
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
    if (s.E <= 8) return launch_fused_ep<TI, 8>(s, x, w_r, b_r, idx, gate, counts, offsets, sorted, pos, gm, st);
    if (s.E <= 16) return launch_fused_ep<TI, 16>(s, x, w_r, b_r, idx, gate, counts, offsets, sorted, pos, gm, st);
    if (s.E <= 32) return launch_fused_ep<TI, 32>(s, x, w_r, b_r, idx, gate, counts, offsets, sorted, pos, gm, st);
    return launch_fused_ep<TI, 64>(s, x, w_r, b_r, idx, gate, counts, offsets, sorted, pos, gm, st);
}

}  // namespace

hipError_t launch_route(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r,
                        int32_t *topk_idx, float *topk_gate, float *logits, hipStream_t st, int gate_mode) {
    if (s.dtype == COLIBRI_F32) return launch_t<float>(s, x, w_r, b_r, topk_idx, topk_gate, logits, gate_mode, st);
    return launch_t<uint16_t>(s, x, w_r, b_r, topk_idx, topk_gate, logits, gate_mode, st);
}

// bf16: one 16-token tile (T <= 16); fp32: at most kFusedGroups token groups
// (T <= 32; with E <= 2: T <= 64)
bool route_dispatch_fusable(const colibri_moe_shape_t &s) {
    if (s.T <= 0) return false;
    if (s.dtype != COLIBRI_F32) return ceil_div(s.T, 16) <= kFusedGroupsMfma;
    const int TW = s.E <= 2 ? 32 : 16;
    return ceil_div(s.T, TW) <= kFusedGroups;
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
