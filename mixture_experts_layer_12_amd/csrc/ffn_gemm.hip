// Grouped expert GEMM for prefill and mid-sized batches (T > 64), bf16 MFMA.
//
// Colibri write-ups: [zskr] http://www.zskr.cn/news/2272131 section 2.1 (the
// Compute stage: a grouped GEMM over token groups) and 3.3 (every expert's
// weights share one stride so every tile's shared-memory load pattern is the
// same); [nxbn] http://m.nxbn.cn/news/48047 section 2.1 (matmul + activation
// fused in one kernel); [hnwysp] https://www.hnwysp.cn/news/30485 section 2.2
// (feed the expert kernel row offsets instead of copying rows).
//
//   GEMM1: H[p] = act(X[tok(p)] W1[e] + b1[e])  or  silu(X W1[e]) * (X W3[e])
//   GEMM2: Y[p] = H[p] W2[e] + b2[e]
//
// Structure (gfx950):
//   * tiles: up to 320 rows of one expert x 256 weight columns (SwiGLU: 128
//     of W1 and the same 128 of W3), 8 waves in a 2 x 4 grid, two per SIMD;
//     the tile's 32-row subtiles are split evenly over the two wave rows,
//     each wave owning up to 5 x 2 v_mfma_f32_32x32x16_bf16 accumulators;
//   * tile order: row tiles are numbered expert by expert from the
//     device-side offsets (the grid is sized for the worst case; surplus
//     workgroups exit); inside an expert, column tiles go in groups with all
//     of the expert's row tiles, sized to fit one XCD's 32 CUs, so tiles that
//     share a weight panel or token rows run side by side; consecutive tiles
//     are kept on one XCD
//     (workgroups are dealt to the 8 XCDs round-robin) so they share its L2;
//   * operands: both go global -> LDS with 16-byte-per-lane copies that skip
//     the register file (global_load_lds_dwordx4); A rows are gathered
//     through sorted_assign (GEMM1) or read in place (GEMM2) into
//     XOR-swizzled rows; the row-major [K, N] weights land as 4 x 16 blocks
//     that ds_read_b64_tr_b16 turns into k-contiguous MFMA B operands, so no
//     transposes run in registers;
//   * pipeline: a ring of two LDS stages; the operands of k-step ks+1 are
//     read from LDS while k-step ks is multiplied, and the one workgroup
//     barrier per k-tile sits before the tile's last k-step; the copies of a
//     k-tile are issued two k-steps apart (weights right after the barrier
//     that frees their stage, A rows one k-step later), each placed between
//     MFMAs;
//   * epilogue: bias + ReLU/GELU, silu(u)*v (the W1 and W3 tiles of a column
//     block live in the same wave and lane), or bias only; the bf16 tile is
//     staged through LDS and written back with 16-byte row stores;
//   * combine folded into GEMM2 ([nxbn] section 2.1 fuses the stages that
//     follow the matmul into its kernel; section 3.3 defines the gated sum):
//     after storing its rows, a tile counts itself in per (token, column
//     tile), and the tile that completes a token's two slots writes that
//     token's output columns (see CombineFold).
#include "combine_common.h"
#include "device_common.h"
#include "ffn_common.h"
#include "launchers.h"

#include <type_traits>

namespace colibri {
namespace {

constexpr int kXcds = 8;
constexpr int kCusPerXcd = 32;  // a scheduling group fits the CUs of one XCD

constexpr int kCus = kXcds * kCusPerXcd;

struct Tile {
    int e, row0, rows, n0, split, S;  // S: K splits of this tile
    int tpos, ntail;                  // tail split: this tile's place among the ntail tail tiles, else -1
};

// Row tiles of expert e.  Two rules, both giving every tile at most BM rows:
//  * big tiles (BMB = 256, BM = 320; two wave rows of up to five 32-row
//    subtiles): the expert's ceil(count_e / 64) row pairs -- one subtile for
//    each wave row -- are dealt out as evenly as possible over
//    ceil(count_e / BM) tiles, so that every tile's two wave rows carry the
//    same number of subtiles (an expert of 1025 rows runs as 320 + 256 + 256 +
//    193 rows: 5 + 4 + 4 + 4 subtile pairs, where equal tiles of 257 rows
//    would split 9 subtiles 5 / 4 and run every tile at the pace of 5);
//  * mid tiles: ceil(count_e / BMB) tiles of (nearly) equal size, except that
//    a tail of at most BMB / 4 rows is spread over the other tiles when they
//    stay within BM rows (a small tail tile would stream the whole weight
//    panel for a few rows).
// A tile m of expert e starts at lo + m * u + min(m, r) * g and holds up to
// u + (m < r ? g : 0) rows (the expert's last tile: what is left).
template <int BMB, int BM>
struct RowSplit {
    static constexpr bool kPairs = (BMB == 256);
    int mt, u, r, g;
    __device__ __forceinline__ RowSplit(int rows) {
        if (rows <= 0) {
            mt = u = r = g = 0;
        } else if (kPairs) {
            const int P = (rows + 63) / 64;  // subtile pairs
            mt = (rows + BM - 1) / BM;
            u = 64 * (P / mt), r = P % mt, g = 64;
        } else {
            mt = (rows + BMB - 1) / BMB;
            const int tail = rows % BMB;
            if (mt > 1 && tail != 0 && tail <= BMB / 4 && rows <= BM * (mt - 1)) mt -= 1;
            u = (rows + mt - 1) / mt, r = 0, g = 0;
        }
    }
};

// Row tiles of every expert (lane e holds expert e's) and their prefix sums.
// Whole-wave call; every lane gets the same total.
struct TileTable {
    int lo, hi, mt, u, r, g, tiles, incl, total;
};
template <int BMB, int BM>
__device__ __forceinline__ TileTable tile_table(const int32_t *__restrict__ offsets, int E, int A, int NT) {
    const int lane = threadIdx.x & (kWave - 1);
    TileTable tt;
    tt.lo = 0, tt.hi = 0;
    if (lane < E) {
        tt.lo = min(max(offsets[lane], 0), A);
        tt.hi = min(max(offsets[lane + 1], tt.lo), A);
    }
    const RowSplit<BMB, BM> rs(tt.hi - tt.lo);  // row tiles of expert `lane`
    tt.mt = rs.mt, tt.u = rs.u, tt.r = rs.r, tt.g = rs.g;
    tt.tiles = tt.mt * NT;
    tt.incl = tt.tiles;
#pragma unroll
    for (int s = 1; s < kWave; s <<= 1) {
        const int o = __shfl_up(tt.incl, s);
        if (lane >= s) tt.incl += o;
    }
    tt.total = __shfl(tt.incl, kWave - 1);
    return tt;
}

// Tail split: tiles fill some rounds of one workgroup per CU and a last,
// partial round.  The full rounds run whole; the last round's tail tiles run
// as f K parts each (f * tail <= kCus, so the parts take one round of about
// 1/f the length), f = the largest of 2 .. kTailMax that fits and leaves each
// part at least 4 k-tiles; a tail of more than half the CUs runs whole.  The
// parts write fp32 partials [part][tail tile][tile row][tile column] and
// tail_reduce_kernel adds them.  Both kernels derive the plan from the actual
// tile count.
constexpr int kTailMax = 4;
struct TailPlan {
    int F, f;  // tiles that run whole; K parts of each tail tile (1: none)
};
__host__ __device__ __forceinline__ TailPlan tail_plan(int total, int kts, bool tail_split) {
    TailPlan p{total, 1};
    if (!tail_split || total <= kCus) return p;
    const int tail = total % kCus;
    if (tail == 0) return p;
    int f = kCus / tail;
    f = f < kTailMax ? f : kTailMax;
    while (f > 1 && kts / f < 4) --f;
    if (f > 1) p = {total - tail, f};
    return p;
}

// Logical tile L -> expert, row range and first column.  Inside an expert,
// column tiles go in groups of gn, each with all mte row tiles, gn * mte <= one
// XCD's CUs so that a group's tiles are resident together.
template <int BN>
__device__ __forceinline__ void tile_at(const TileTable &tt, int E, int NT, int L, Tile &t) {
    const int lane = threadIdx.x & (kWave - 1);
    const int excl = tt.incl - tt.tiles;
    const uint64_t m = __ballot(lane < E && L >= excl && L < tt.incl);
    const int e = __ffsll((unsigned long long)m) - 1;
    const int mte = __shfl(tt.mt, e);
    const int local = L - __shfl(excl, e);
    const int gn = max(1, kCusPerXcd / mte);
    const int ng = local / (mte * gn);
    const int gs = min(gn, NT - ng * gn);
    const int rr = local - ng * mte * gn;
    const int mi = rr / gs;
    const int ni = ng * gn + rr % gs;
    t.e = e;
    const int u = __shfl(tt.u, e), r = __shfl(tt.r, e), g = __shfl(tt.g, e);
    t.row0 = __shfl(tt.lo, e) + mi * u + min(mi, r) * g;
    t.rows = min(u + (mi < r ? g : 0), __shfl(tt.hi, e) - t.row0);
    t.n0 = ni * BN;
}

// Block b -> (expert, row range, first column, K split); column tiles: NT,
// K splits: S (or a tail split, see whole_tiles).  Whole-wave call; every lane
// gets the same answer.  Returns false for surplus blocks (the grid is sized
// for the worst case).
template <int BMB, int BM, int BN>
__device__ __forceinline__ bool locate_tile(const int32_t *__restrict__ offsets, int E, int A, int NT, int S,
                                            bool tail_split, int kts, int b, Tile &t) {
    const TileTable tt = tile_table<BMB, BM>(offsets, E, A, NT);
    const int total = tt.total;
    const TailPlan tp = tail_plan(total, kts, tail_split && S == 1);
    if (b >= (S > 1 ? total * S : tp.F + tp.f * (total - tp.F))) return false;
    // logical tiles [base, base + cnt), SS splits each; blocks bb = 0 .. cnt * SS - 1
    int base = 0, cnt = S == 1 ? tp.F : total, SS = S, bb = b;
    const bool tail = S == 1 && b >= tp.F;
    if (tail) base = tp.F, cnt = total - tp.F, SS = tp.f, bb = b - tp.F;  // F is a multiple of 8
    // Block b runs on XCD b % 8.  Whole rounds of kCus blocks: XCD x takes the
    // chunks x, x + 8, x + 16, ... of kCusPerXcd consecutive logical indices,
    // so neighbouring tiles (a group sharing weight panels and token rows) run
    // side by side on one XCD while every XCD gets chunks of every expert (one
    // contiguous range per XCD gave each XCD one expert of the Mixtral-shaped
    // prefill, and the XCD with the most rows set the kernel's time); the
    // last, partial round is cut into 8 contiguous ranges.  The index is
    // split-major, so a chunk is one K range of neighbouring tiles.
    const int xcd = bb % kXcds, i = bb / kXcds;
    const int n = cnt * SS, nfull = n / kCus;
    int LS;
    if (i < nfull * kCusPerXcd) {
        LS = (i / kCusPerXcd) * kCus + xcd * kCusPerXcd + i % kCusPerXcd;
    } else {
        const int rem = n - nfull * kCus, i2 = i - nfull * kCusPerXcd;
        LS = nfull * kCus + xcd * (rem / kXcds) + min(xcd, rem % kXcds) + i2;
    }
    t.split = LS / cnt;
    t.S = SS;
    t.tpos = tail ? LS - t.split * cnt : -1;
    t.ntail = tail ? cnt : 0;
    tile_at<BN>(tt, E, NT, base + LS - t.split * cnt, t);
    return true;
}

template <int N, class F>
__device__ __forceinline__ void with_live_count(int n, F &&f) {
    if constexpr (N > 0) {
        if (n < N) {
            with_live_count<N - 1>(n, f);
            return;
        }
    }
    f(std::integral_constant<int, N>{});
}

// 16-byte chunk swizzle inside an A row of BK bf16 (BK/8 chunks): the 16 rows
// that one ds_read_b128 phase touches land on 16 distinct 16-byte bank slots
// of the 256-byte bank window.
template <int BK>
__device__ __forceinline__ int swz(int row) {
    if (BK == 64) return (row ^ (row >> 3)) & 7;  // 128-byte rows: 2 per window
    return (row >> 2) & 3;                        // 64-byte rows: 4 per window
}

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_byte;
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// Global -> LDS copy of 16 bytes per lane that bypasses registers
// (global_load_lds_dwordx4): lane i fills LDS bytes [dst + 16 i, dst + 16 i + 16);
// dst is wave-uniform and goes through M0 (nothing else in these kernels uses
// M0).  Issued from inline assembly so that the waits for the copies are
// placed by hand (wait_vmcnt) rather than before every LDS read.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"  // M0 in the clobber list
__device__ __forceinline__ void dma16(const void *src, uint32_t dst) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "s"(dst) : "memory", "m0");
}
// same, from a wave-uniform base plus a per-lane 32-bit byte offset
__device__ __forceinline__ void dma16_s(uint32_t voff, const void *sbase, uint32_t dst) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(dst)
                 : "memory", "m0");
}
#pragma clang diagnostic pop
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// vmcnt(n * PER) for a runtime n in [0, MAXN] (larger n waits for MAXN * PER)
template <int PER, int MAXN>
__device__ __forceinline__ void wait_groups(int n) {
    if constexpr (MAXN >= 0) {
        if (n >= MAXN) {
            wait_vmcnt<MAXN * PER>();
            return;
        }
        if constexpr (MAXN > 0) wait_groups<PER, MAXN - 1>(n);
    }
}

// vmcnt(n_a + NB) for a runtime count n_a of A copies per stage (0 .. NA)
template <int NA, int NB>
__device__ __forceinline__ void wait_live_stage(int n_a) {
    if constexpr (NA >= 0) {
        if (n_a >= NA) {
            wait_vmcnt<NA + NB>();
            return;
        }
        if constexpr (NA > 0) wait_live_stage<NA - 1, NB>(n_a);
    }
}

// One BM x BNC output tile of one expert.  NW = WM x WN waves, each owning a
// (BM/WM) x (BNC/WN) block (for SwiGLU: that block of both W1 and W3).
//
// LDS stage (STAGES of them, a ring):
//   A: BM rows x BK k, 16-byte chunks XOR-swizzled per row (swz);
//   B: BK k x BN columns (SwiGLU: W1's BNC columns then W3's), stored as
//      128-byte blocks of 4 k rows x 16 columns, block (kq, n16) at
//      (kq * BN/16 + n16) * 128, row-major inside.  ds_read_b64_tr_b16 turns
//      a block into 4 consecutive k of one column per lane, so two of them
//      give a 32x32x16 MFMA B operand with no register transposes.
// Both are filled with 1 KB global->LDS copies: an A copy is RPD whole rows,
// a B copy is 4 k rows x 128 columns (16-byte runs of one weight row).
//
// BLD > 0 (loader waves): BLD extra waves copy the weight tiles into a ring of
// BST B stages of their own, and the NW compute waves copy only the A tiles
// (two A stages).  A wave's copies retire in issue order, so when one wave
// copies both operands, waiting for the next A tile also waits for every
// weight tile issued before it, and the weight ring can be no deeper than the
// A ring.  Split over waves, the weights run BST - 1 tiles ahead while A
// (rows already in L2) runs one tile ahead.  All waves meet at the same
// barriers; the loader waves leave after the last one.
// ---- the combine folded into GEMM2's epilogue (CombineFold).  Called by every
// wave of the workgroup (NWT waves) once the tile's Y rows (SK == 1) or split
// partials (SK > 1) are stored.  Lane l of wave w counts in tile row w + NWT l;
// a lane whose count completes its token's 2 SK arrivals marks it, and the
// wave then forms the marked tokens' output columns n0 .. n0 + BNC - 1, RPP
// tokens at a time, with the combine kernels' own per-vector code.
template <int RPP, int LPR, class F>
__device__ __forceinline__ void fold_marked(uint64_t m, int t, F &&fn) {
    static_assert(RPP * LPR == kWave, "lane groups");
    const int lane = threadIdx.x & (kWave - 1);
    const int q = lane / LPR, cv = lane % LPR;
    while (m) {  // m is the same in every lane
        int src = -1;
#pragma unroll
        for (int r = 0; r < RPP; ++r) {
            const int b = m ? __builtin_ctzll(m) : -1;
            if (r == q) src = b;
            if (m) m &= m - 1;
        }
        const int tt = __shfl(t, src < 0 ? 0 : src);
        if (src >= 0) fn(tt, cv);
    }
}

// 4 columns per lane, LPR lanes per token
template <int U, int LPR>
__device__ __forceinline__ void fold_partials(uint64_t m, int t, const CombineFold &f, const float *part, int S, int E,
                                              int T, int N, int n0) {
    fold_marked<kWave / LPR, LPR>(m, t, [&](int tt, int cv) {
        const int c = n0 + 4 * cv;
        if (c < N)
            combine_partials_vec<4, U>(part, S, f.pos, f.idx, f.gate, f.b2, E, f.out, T, N, f.shared, f.residual,
                                       SharedPartials{}, tt, c);
    });
}

constexpr int kFoldMaxSplits = 4;  // more splits: the separate combine (registers)

template <int NWT, int BNC>
__device__ __forceinline__ void fold_combine(const CombineFold &f, const uint16_t *Y, const float *part, int T, int E,
                                             int N, int NT, int n0, int row0, int rows, int SK, uint8_t *lds) {
    static_assert(BNC == 256 || BNC == 128, "column tile");
    const int lane = threadIdx.x & (kWave - 1);
    const int w = (int)(threadIdx.x / kWave);
    volatile int *any = reinterpret_cast<volatile int *>(lds);  // the LDS tile is free from here on
    // Release: every wave's stores have reached the L2 (vmcnt counts stores
    // on this chip) before the barrier; then one agent-scope release fence, a
    // write-back of the XCD's L2, covers the whole tile.  Fences here cost an
    // L2 scan each, so the tile issues one per direction, not one per wave.
    wait_vmcnt<0>();
    __syncthreads();
    if (w == 0) {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (lane == 0) *any = 0;
    }
    __syncthreads();
    const int rl = w + NWT * lane;  // rows <= NWT * 64
    int t = 0;
    bool fin = false;
    if (rl < rows) {
        t = f.sorted[row0 + rl] >> 1;
        fin = atomicAdd(f.arrive + (size_t)t * NT + n0 / BNC, 1) == 2 * SK - 1;
    }
    const uint64_t m = __ballot(fin);
    if (m != 0 && lane == 0) *any = 1;
    __syncthreads();
    if (*any == 0) return;  // the same in every wave
    // Acquire: one agent-scope acquire fence (invalidates this CU's L1 and the
    // XCD's L2) orders every wave's reads below after the counts it observed.
    if (w == 0) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    __syncthreads();
    if (m == 0) return;
    if (SK == 1) {
        // one 16-byte vector (8 bf16 columns) per lane, RPP tokens per pass,
        // the loads of UNR passes in flight together
        constexpr int LPR = BNC / 8, RPP = kWave / LPR, UNR = 2;
        const int q = lane / LPR;
        const int c = n0 + 8 * (lane % LPR);
        uint64_t mm = m;
        while (mm) {  // the same in every lane
            int tt[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u) {
                int src = -1;
#pragma unroll
                for (int r = 0; r < RPP; ++r) {
                    const int b = mm ? __builtin_ctzll(mm) : -1;
                    if (r == q) src = b;
                    if (mm) mm &= mm - 1;
                }
                const int v = __shfl(t, src < 0 ? 0 : src);
                tt[u] = (src >= 0 && c < N) ? v : -1;
            }
            RowsVec rv[UNR];
#pragma unroll
            for (int u = 0; u < UNR; ++u)
                if (tt[u] >= 0) rows_vec_load<uint16_t>(rv[u], Y, f.pos, f.gate, T, N, f.shared, f.residual, tt[u], c);
#pragma unroll
            for (int u = 0; u < UNR; ++u)
                if (tt[u] >= 0)
                    rows_vec_finish<uint16_t>(rv[u], f.shared != nullptr, f.residual != nullptr, f.out,
                                              SharedPartials{}, N, tt[u], c);
        }
        return;
    }
    // 4 columns per lane
    constexpr int LPR = BNC / 4 < kWave ? BNC / 4 : kWave;
#pragma unroll
    for (int h = 0; h < BNC; h += 4 * LPR) {
        if (SK <= 2) fold_partials<2, LPR>(m, t, f, part, SK, E, T, N, n0 + h);
        else fold_partials<4, LPR>(m, t, f, part, SK, E, T, N, n0 + h);  // SK <= kFoldMaxSplits
    }
}

template <int BMB, int BM, int BN, int BK, int WM, int WN, int STAGES, int EPI, bool GATHER, int WPE, int BLD = 0,
          int BST = 2>
__global__ __launch_bounds__((WM * WN + BLD) * kWave, WPE) void ffn_gemm_kernel(
    const uint16_t *__restrict__ A, const int32_t *__restrict__ sorted_assign, int T,
    const int32_t *__restrict__ offsets, int E, const uint16_t *__restrict__ B0, const uint16_t *__restrict__ B1,
    const uint16_t *__restrict__ bias, uint16_t *__restrict__ C, int K, int N, int NT, int S, int tail_split,
    float *__restrict__ part, CombineFold fold) {
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    // the combine folds into GEMM2 only (bias-only epilogue); fold.arrive is the same in every thread
    const bool folded = EPI == EPI_BIAS_ONLY && fold.arrive != nullptr;
    constexpr int NB = DUAL ? 2 : 1;             // weight matrices per tile
    constexpr int NW = WM * WN;
    constexpr int BNC = DUAL ? BN / 2 : BN;      // output columns per tile
    constexpr int WTM = BM / WM;                 // wave tile rows
    constexpr int WNC = BNC / WN;                // wave tile columns (per matrix)
    constexpr int SM = WTM / 32, SJ = WNC / 32;  // 32x32 subtiles per wave (per matrix)
    constexpr bool SPEC = BLD > 0;               // weight tiles copied by loader waves
    constexpr int CW = SPEC ? BLD : NW;          // waves copying B
    constexpr int A_BYTES = BM * BK * 2, B_BYTES = BK * BN * 2, STAGE_BYTES = A_BYTES + B_BYTES;
    constexpr int A_PW = A_BYTES / 1024 / NW, B_PW = B_BYTES / 1024 / CW;  // 1 KB copies per wave per stage
    constexpr int CPR = BK / 8;                  // 16-byte chunks per A row
    constexpr int RPD = 64 / CPR;                // A rows per copy
    constexpr int KQ_ROW = (BN / 16) * 128;      // bytes per 4-k-row band of the B tile
    constexpr int HPB = BN / 128;                // B copies per band
    static_assert(SM >= 1 && SJ >= 1, "wave tile too small");
    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(A_PW * NW * 1024 == A_BYTES && B_PW * CW * 1024 == B_BYTES, "whole copies per wave");
    static_assert(CW % HPB == 0, "a wave's B copies share one column range");
    static_assert(!SPEC || (STAGES == 2 && BST >= 3 && (BST - 1) * B_PW <= 63), "loader-wave ring");
    static_assert(!DUAL || BNC % 128 == 0, "a B copy covers one matrix");
    static_assert(STAGES >= 2 && (STAGES - 2) * (A_PW + B_PW) <= 63, "vmcnt range");
    // LDS: the shared ring of STAGES (A, B) stages, or (SPEC) two A stages then BST B stages
    constexpr int LDS_MAIN = SPEC ? 2 * A_BYTES + BST * B_BYTES : STAGES * STAGE_BYTES;
    constexpr int LDS_EPI = BM * BNC * 2;  // bf16 output tile
    __shared__ __attribute__((aligned(1024))) uint8_t lds[LDS_MAIN > LDS_EPI ? LDS_MAIN : LDS_EPI];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int w = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wm = w / WN, wn = w % WN;

    Tile tl;
    if (!locate_tile<BMB, BM, BNC>(offsets, E, 2 * T, NT, S, tail_split != 0, K / BK, blockIdx.x, tl))
        return;  // uniform per block
    const int e = __builtin_amdgcn_readfirstlane(tl.e);
    const int row0 = __builtin_amdgcn_readfirstlane(tl.row0);
    const int rows = __builtin_amdgcn_readfirstlane(tl.rows);
    const int n0 = __builtin_amdgcn_readfirstlane(tl.n0);
    const int split = __builtin_amdgcn_readfirstlane(tl.split);
    const int SK = __builtin_amdgcn_readfirstlane(tl.S);  // K splits of this tile
    const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_byte *)lds;

    // ---- copy sources.  Rows past the expert's segment read its first row and
    // columns past N read column 0: they only feed accumulator rows and
    // columns that are never stored, and every copy stays in bounds.
    // The tile's ceil(rows / 32) subtiles are split evenly over the WM wave rows:
    // wave row wm owns tile rows [wm * per * 32, +live_sm * 32) (per <= SM since
    // rows <= BM).  In LDS, wave row wm's rows always start at wm * WTM, so the
    // operand reads have fixed offsets; the copies place the rows accordingly.
    const int nsub = (rows + 31) / 32;
    const int per = (nsub + WM - 1) / WM;
    const int live_sm = min(per, max(0, nsub - wm * per));
    const int wrow = wm * per * 32;  // first tile row of this wave
    // With two stages every wait in the loop drains all of a wave's copies, so
    // copies whose RPD rows all lie past the tile's live rows are skipped (live
    // rows are a prefix of each wave row region, so the first row decides).
    constexpr bool SKIP_DEAD = (STAGES == 2);
    uint32_t a_live = 0;  // wave-uniform: bit q = A copy q carries live rows
    const uint16_t *a_src[A_PW];
#pragma unroll
    for (int q = 0; q < A_PW; ++q) {
        const int m0 = (w + NW * q) * RPD;  // first LDS row of copy q
        const int reg0 = m0 / WTM, off0 = m0 % WTM;
        if (!SKIP_DEAD || (off0 < per * 32 && reg0 * per * 32 + off0 < rows)) a_live |= 1u << q;
        const int m = (w + NW * q) * RPD + lane / CPR;  // LDS row of this lane's chunk
        const int c = (lane % CPR) ^ swz<BK>(m);        // logical chunk held by physical slot lane % CPR
        const int reg = m / WTM, off = m % WTM;         // wave row region and row inside it
        const int r = reg * per * 32 + off;             // tile row
        long src = row0 + ((off < per * 32 && r < rows) ? r : 0);
        if (GATHER) {
            const int a = sorted_assign[src];
            src = (a >= 0 && (a >> 1) < T) ? (a >> 1) : 0;
        }
        a_src[q] = A + (size_t)src * K + c * 8;
    }
    // B copy cw + CW q (cw: this wave's index among the CW copying waves): band
    // kq = (cw + CW q) / HPB, columns [(cw % HPB) 128, +128) of the LDS tile;
    // lane: 16-column block lane / 8, k row 4 kq + (lane % 8) / 2, 8 columns at 8 (lane % 2)
    const int cw = SPEC ? max(w - NW, 0) : w;
    const int ncol = (cw % HPB) * 128 + (lane >> 3) * 16 + (lane & 1) * 8;
    const int mat = DUAL ? (cw % HPB) * 128 / BNC : 0;  // uniform: one matrix per copy
    int gcol = n0 + ncol - mat * BNC;
    if (gcol >= N) gcol = 0;
    const uint32_t b_voff = (uint32_t)((((lane & 7) >> 1) * N + gcol) * 2);
    const uint16_t *b_base = (mat ? B1 : B0) + (size_t)e * K * N + (size_t)(cw / HPB) * 4 * N;
    size_t b_row[B_PW];  // first weight row of B copy q, relative to the k-tile's first row, times N
#pragma unroll
    for (int q = 0; q < B_PW; ++q) b_row[q] = (size_t)4 * (NW / HPB) * q * N;

    // copy m (m < A_PW: A copy m; else B copy m - A_PW) of k-tile kt into stage s
    auto copy_one = [&](int m, int s, int k0, const uint16_t *bk) {
        const uint32_t sa = lds0 + s * STAGE_BYTES;
        if (m < A_PW) {
            if ((a_live >> m) & 1) dma16(a_src[m] + k0, sa + (w + NW * m) * 1024);
        } else {
            const int q = m - A_PW;
            dma16_s(b_voff, bk + b_row[q], sa + A_BYTES + (w + NW * q) * 1024);
        }
    };
    auto issue = [&](int s, int kt) {
        const int k0 = kt * BK;
        const uint16_t *bk = b_base + (size_t)k0 * N;
#pragma unroll
        for (int m = 0; m < A_PW + B_PW; ++m) copy_one(m, s, k0, bk);
    };
    // SPEC copies: A of k-tile kt into A stage s (compute waves), B of k-tile kt into B stage t (loader waves)
    auto issue_a = [&](int s, int kt) {
        const int k0 = kt * BK;
        const uint32_t sa = lds0 + s * A_BYTES;
#pragma unroll
        for (int q = 0; q < A_PW; ++q)
            if ((a_live >> q) & 1) dma16(a_src[q] + k0, sa + (w + NW * q) * 1024);
    };
    auto issue_b = [&](int t, int kt) {
        const int k0 = kt * BK;
        const uint32_t sb = lds0 + 2 * A_BYTES + t * B_BYTES;
#pragma unroll
        for (int q = 0; q < B_PW; ++q)
            dma16_s(b_voff, b_base + (size_t)(k0 + 4 * (CW / HPB) * q) * N, sb + (cw + CW * q) * 1024);
    };

    f32x16 acc[NB][SM][SJ];
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int i = 0; i < SM; ++i)
#pragma unroll
            for (int j = 0; j < SJ; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][i][j][r] = 0.0f;


    // per-lane LDS read offsets.  A operand (32 rows x 16 k): row lane % 32, chunk 2 ks + lane / 32.
    int a_row[SM], a_swz[SM];
#pragma unroll
    for (int i = 0; i < SM; ++i) {
        const int m = wm * WTM + i * 32 + (lane & 31);
        a_row[i] = m * BK * 2;
        a_swz[i] = swz<BK>(m);
    }
    // B operand (16 k x 32 columns): 16-lane group g holds columns 16 (g % 2) + [0, 16) at k 8 (g / 2) + [0, 8),
    // read as two transposing 4-k-row reads of blocks (kq, n16)
    const int g = lane >> 4;
    const int b_lane = (g >> 1) * 2 * KQ_ROW + (g & 1) * 128 + (lane & 15) * 8;

    // MFMA operands of one 16-k step: SM A fragments, NB x SJ B fragments
    struct Frags {
        bf16x8 a[SM];
        bf16x8 b[NB][SJ];
    };
    // lv: compile-time count of live subtiles (LV >= 0) or LV = -1 for the runtime live_sm
    // ao, bo: byte offsets of the A and B stages in LDS
    auto read_frags = [&](int ao, int bo, int ks, Frags &f, auto lv) {
        constexpr int LV = decltype(lv)::value;
        const int nl = LV >= 0 ? LV : live_sm;
        if (nl == 0) return;  // this wave's rows are all padding
        const lds_byte *L = (const lds_byte *)lds + ao;
        const lds_byte *LB = (const lds_byte *)lds + bo;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int j = 0; j < SJ; ++j) {
                const int cb = b * BNC + wn * WNC + j * 32;  // LDS tile column of the subtile
                const lds_byte *p = LB + b_lane + ks * 4 * KQ_ROW + (cb >> 4) * 128;
                const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)p);
                const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16 *)(p + KQ_ROW));
                f.b[b][j] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            if (i >= nl) break;  // uniform per wave
            f.a[i] = *(const lds_bf16x8 *)(L + a_row[i] + (((2 * ks + (lane >> 5)) ^ a_swz[i]) << 4));
        }
    };
    // MFMAs of one k-step; copies [c0, c1) of k-tile ck into stage cs, if any,
    // are placed after them one by one (copy c0 + m after MFMA m)
    auto mma = [&](const Frags &f, auto lv, int c0 = 0, int c1 = 0, int cs = 0, int ck = 0) {
        constexpr int LV = decltype(lv)::value;
        const int nl = LV >= 0 ? LV : live_sm;
        const int ck0 = ck * BK;
        const uint16_t *cbk = b_base + (size_t)ck0 * N;
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            if (i >= nl) break;  // uniform per wave
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < SJ; ++j) {
                    acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[b][j], acc[b][i][j], 0, 0, 0);
                    if (LV >= 0 && c0 + (i * NB + b) * SJ + j < c1) copy_one(c0 + (i * NB + b) * SJ + j, cs, ck0, cbk);
                }
        }
        if (LV >= 0) {
            for (int m = c0 + (LV > 0 ? LV : 0) * NB * SJ; m < c1; ++m) copy_one(m, cs, ck0, cbk);
        } else {
            for (int m = c0; m < c1; ++m) copy_one(m, cs, ck0, cbk);
        }
        // Schedule the k-step as one MFMA, then one LDS read (of the next k-step's
        // operands, read before this step in the source), alternating for as long
        // as both last: left to itself the compiler bunches the reads and the two
        // waves of a SIMD then wait for LDS at the same time (measured on the
        // Mixtral-shaped prefill: first layer 1747 -> 1696 us, second 904 -> 841).
        if constexpr (LV > 0) {
            constexpr int NM = LV * NB * SJ, NR = LV + 2 * NB * SJ;
#pragma unroll
            for (int q = 0; q < (NM < NR ? NM : NR); ++q) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
            }
            if constexpr (NM > NR) __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
            if constexpr (NR > NM) __builtin_amdgcn_sched_group_barrier(0x100, NR - NM, 0);
        }
    };

    // The tile's last k-step with the copies [M0, M1) of k-tile kt into stage s
    // placed between its MFMAs (copy M0 + m after MFMA m): right after the barrier
    // both waves of a SIMD issue their copies at the same time, and issued in one
    // run they would leave the matrix unit idle meanwhile.
    auto mma_issue = [&](const Frags &f, auto lv, int s, int kt, auto m0, auto m1) {
        constexpr int LV = decltype(lv)::value;
        static_assert(LV >= 0, "compile-time live count");
        constexpr int M0 = decltype(m0)::value, DPW_ = decltype(m1)::value;
        const int k0 = kt * BK;
        const uint16_t *bk = b_base + (size_t)k0 * N;
#pragma unroll
        for (int i = 0; i < LV; ++i)
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int j = 0; j < SJ; ++j) {
                    acc[b][i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[b][j], acc[b][i][j], 0, 0, 0);
                    const int m = M0 + (i * NB + b) * SJ + j;  // a constant once the loops are unrolled
                    if (m < DPW_) copy_one(m, s, k0, bk);
                }
#pragma unroll
        for (int m = M0 + LV * NB * SJ; m < DPW_; ++m) copy_one(m, s, k0, bk);
    };

    // ---- main loop over a ring of two LDS stages.  The operands of k-step ks+1 are
    // read while k-step ks is multiplied; the workgroup barrier sits before the last
    // k-step of a tile, so the next tile's first reads overlap that step's MFMAs.
    // After the barrier every wave has finished reading tile kt (the barrier waits for
    // outstanding LDS reads), so tile kt + 2 is copied into its stage in two groups:
    // its weight (B) copies between the MFMAs of tile kt's last k-step, its A copies
    // between those of the first k-step of tile kt + 1.  Issued in one run, all
    // copies of a wave queue behind each other in the memory pipeline while both
    // waves of a SIMD wait to issue their next MFMA; in two runs the B copies, whose
    // weights come from HBM, keep the longest lead (measured on the Mixtral-shaped
    // prefill, A/B in one process: second layer 845 / 841 -> 807 / 806 us, first
    // layer 1659 / 1645 -> 1661 / 1630 us; the Zipf-skewed layer 567 / 552 -> 551 /
    // 547 and 311 / 305 -> 300 / 301 us).  Copies past the last k-tile re-read it.
    static_assert(SPEC || STAGES == 2, "the split copy groups assume a ring of two stages");
    constexpr int KS = BK / 16;
    constexpr int DPW = A_PW + B_PW;
    // this block's K range: k-tiles [kt0, kt0 + KT) of the K / BK
    const int kt0 = split * (K / BK) / SK;
    const int KT = (split + 1) * (K / BK) / SK - kt0;
    auto ktile = [&](int t) { return kt0 + (t < KT ? t : KT - 1); };
    auto main_loop = [&](auto lv) {
        Frags f[2];
#pragma unroll
        for (int s = 0; s < STAGES; ++s) issue(s, ktile(s));
        // this wave's copies of k-tile 0 have landed: at most one stage's copies remain
        if constexpr (SKIP_DEAD) {
            wait_live_stage<A_PW, B_PW>(__popc(a_live));
        } else {
            wait_vmcnt<(STAGES - 1) * DPW>();
        }
        __syncthreads();                    // ... everyone's
        read_frags(0, A_BYTES, 0, f[0], lv);
        for (int kt = 0; kt < KT; ++kt) {
            const int s = kt & 1;
            const int so = s * STAGE_BYTES;
#pragma unroll
            for (int ks = 0; ks + 1 < KS; ++ks) {
                read_frags(so, so + A_BYTES, ks + 1, f[(ks + 1) & 1], lv);
                if (ks == 0 && kt > 0)
                    mma(f[0], lv, 0, A_PW, s ^ 1, ktile(kt + 1));  // A copies of k-tile kt+1
                else
                    mma(f[ks & 1], lv);
            }
            wait_vmcnt<0>();  // k-tile kt+1 has landed (this wave's copies)
            __syncthreads();  // ... everyone's; and k-tile kt is fully read
            const int sn = (s ^ 1) * STAGE_BYTES;
            if (kt + 1 < KT) read_frags(sn, sn + A_BYTES, 0, f[0], lv);
            // B copies of k-tile kt+2 into stage s
            mma_issue(f[(KS - 1) & 1], lv, s, ktile(kt + 2), std::integral_constant<int, A_PW>{},
                      std::integral_constant<int, DPW>{});
        }
    };
    // ---- SPEC: compute waves.  A stage kt & 1, B stage kt % BST.  Barrier P publishes
    // k-tile 0, barrier kt publishes k-tile kt+1 (the loader waves wait for their copies
    // of it before that barrier) and frees the stages of k-tile kt.
    auto main_loop_spec = [&](auto lv) {
        Frags f[2];
        issue_a(0, kt0);
        issue_a(1, ktile(1));
        wait_live_stage<A_PW, 0>(__popc(a_live));  // A of k-tile 0 has landed
        __syncthreads();                            // barrier P
        read_frags(0, 2 * A_BYTES, 0, f[0], lv);
        for (int kt = 0; kt < KT; ++kt) {
            const int ao = (kt & 1) * A_BYTES, bo = 2 * A_BYTES + (kt % BST) * B_BYTES;
#pragma unroll
            for (int ks = 0; ks + 1 < KS; ++ks) {
                read_frags(ao, bo, ks + 1, f[(ks + 1) & 1], lv);
                mma(f[ks & 1], lv);
            }
            wait_vmcnt<0>();  // A of k-tile kt+1 has landed (this wave's copies)
            __syncthreads();  // barrier kt
            if (kt + 2 < KT) issue_a(kt & 1, kt0 + kt + 2);
            if (kt + 1 < KT)
                read_frags(((kt + 1) & 1) * A_BYTES, 2 * A_BYTES + ((kt + 1) % BST) * B_BYTES, 0, f[0], lv);
            mma(f[(KS - 1) & 1], lv);
        }
    };
    // ---- SPEC: loader waves.  B of k-tile t goes to stage t % BST, BST - 1 tiles ahead.
    auto loader_loop = [&]() {
#pragma unroll
        for (int t = 0; t < BST; ++t)
            if (t < KT) issue_b(t, kt0 + t);
        wait_groups<B_PW, BST - 1>(min(BST, KT) - 1);  // k-tile 0 has landed
        __syncthreads();                                 // barrier P
        for (int kt = 0; kt < KT; ++kt) {
            // k-tile kt+1 has landed: later tiles issued so far are kt+2 .. min(kt+BST-1, KT-1)
            wait_groups<B_PW, BST - 2>(max(0, min(BST - 2, KT - 2 - kt)));
            __syncthreads();  // barrier kt: k-tile kt is fully read, its stage is free
            if (kt + BST < KT) issue_b(kt % BST, kt0 + kt + BST);
        }
    };
    // every live count 0 .. SM gets its own copy of the loop, free of per-subtile
    // tests and with its MFMAs and LDS reads interleaved (a wave row of a tile
    // whose subtile count is odd has one subtile fewer than the other)
    if constexpr (SPEC) {
        if (w >= NW) {  // loader wave: the main loop's barriers, the one below, the epilogue's
            loader_loop();
            wait_vmcnt<0>();
            __syncthreads();
            if (SK == 1) __syncthreads();
            if (folded) fold_combine<NW + BLD, BNC>(fold, C, part, T, E, N, NT, n0, row0, rows, SK, lds);
            return;
        }
        with_live_count<SM>(live_sm, [&](auto lv) { main_loop_spec(lv); });
    } else {
        with_live_count<SM>(live_sm, [&](auto lv) { main_loop(lv); });
    }
    wait_vmcnt<0>();
    __syncthreads();

    // ---- K split: the fp32 partial sums go to part[split][row][col] (SwiGLU: the
    // W3 products at col + N), a tail tile's to part[part][tail tile][tile row][tile
    // column] (SwiGLU: W3 at + BNC); a later kernel adds them and applies the epilogue
    // 32x32 accumulator layout: register r of lane l holds row 8(r/4) + 4(l/32) + r%4, column l%32
    if (SK > 1) {
        constexpr int NC = DUAL ? 2 : 1;
        const int tpos = __builtin_amdgcn_readfirstlane(tl.tpos);
        const int RW = tpos >= 0 ? NC * BNC : NC * N;  // floats per partial row
        const int WO = tpos >= 0 ? BNC : N;            // SwiGLU: offset of the W3 products
        const int c0 = tpos >= 0 ? n0 : 0;             // first column of a partial row
        float *pb = tpos >= 0 ? part + ((size_t)split * tl.ntail + tpos) * BM * (size_t)RW
                              : part + ((size_t)split * 2 * T + row0) * (size_t)RW;
#pragma unroll
        for (int i = 0; i < SM; ++i) {
            if (i >= live_sm) break;
#pragma unroll
            for (int j = 0; j < SJ; ++j) {
                const int n = n0 + wn * WNC + j * 32 + (lane & 31);
                if (n >= N) continue;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int rl = wrow + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                    if (rl >= rows) continue;
                    float *dst = pb + (size_t)rl * RW + (n - c0);
                    dst[0] = acc[0][i][j][r];
                    if (DUAL) dst[WO] = acc[NB - 1][i][j][r];
                }
            }
        }
        if (folded) fold_combine<NW + BLD, BNC>(fold, C, part, T, E, N, NT, n0, row0, rows, SK, lds);
        return;
    }

    // ---- epilogue: values -> bf16 tile in LDS -> 16-byte row stores
    uint16_t *Cs = reinterpret_cast<uint16_t *>(lds);
    const uint16_t *bias_e = bias ? bias + (size_t)e * N : nullptr;
#pragma unroll
    for (int i = 0; i < SM; ++i) {
        if (i >= live_sm) break;  // padding subtiles may alias the next wave row's tile rows
#pragma unroll
        for (int j = 0; j < SJ; ++j) {
            const int cl = wn * WNC + j * 32 + (lane & 31);  // tile column
            const int n = n0 + cl;
            float bv = 0.0f;
            if (EPI != EPI_SWIGLU && bias_e != nullptr && n < N) bv = bf16_to_f32(bias_e[n]);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = wrow + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                float v;
                if (EPI == EPI_SWIGLU) v = silu_bf16out(acc[0][i][j][r]) * acc[NB - 1][i][j][r];
                else if (EPI == EPI_ACT_RELU) v = apply_act_bf16out<ACT_RELU>(acc[0][i][j][r] + bv);
                else if (EPI == EPI_ACT_GELU) v = apply_act_bf16out<ACT_GELU>(acc[0][i][j][r] + bv);
                else v = acc[0][i][j][r] + bv;
                Cs[rl * BNC + cl] = (uint16_t)f32_to_bf16_bits(v);
            }
        }
    }
    __syncthreads();
    constexpr int VPR = BNC / 8;  // 16-byte vectors per output row
    for (int idx = tid; idx < BM * VPR; idx += NW * kWave) {
        const int rl = idx / VPR, cv = idx % VPR;
        const int n = n0 + cv * 8;
        if (rl < rows && n < N)
            *reinterpret_cast<u32x4 *>(C + (size_t)(row0 + rl) * N + n) =
                *reinterpret_cast<const u32x4 *>(Cs + rl * BNC + cv * 8);
    }
    if (folded) fold_combine<NW + BLD, BNC>(fold, C, part, T, E, N, NT, n0, row0, rows, SK, lds);
}

// Tail split, second half: the tail tiles (see tail_plan) ran as f K parts
// into part[part][tail tile][tile row][tile column] (SwiGLU: W3 products at
// + BNC); the parts are added in order (0 + part 0 + part 1 + ..., as the
// split reduce does), the epilogue applied and the bf16 tile stored.  Block
// b: tail tile b / RB, tile rows [(b % RB) RPB PR, +RPB PR); a thread takes 4
// columns of PR rows RPB apart, with the PR rows' loads of a part in flight
// together.  The grid covers the largest possible tail; without a tail every
// block leaves at once, so few blocks keep that case cheap.
template <int BMB, int BM, int BNC>
struct TailReduceGrid {
    static constexpr int Q = BNC / 4;                       // 4-column groups per tile row
    static constexpr int RPB = 256 / Q;                     // tile rows per pass of a block
    static constexpr int PR = 4;                            // passes (rows per thread)
    static constexpr int RB = (BM + RPB * PR - 1) / (RPB * PR);  // blocks per tile
    static constexpr int blocks = kCus * RB;                // fewer than kCus tail tiles
};
template <int BMB, int BM, int BNC, int EPI>
__global__ __launch_bounds__(256) void tail_reduce_kernel(const float *__restrict__ part, int T,
                                                          const int32_t *__restrict__ offsets, int E, int NT, int kts,
                                                          const uint16_t *__restrict__ bias, uint16_t *__restrict__ C,
                                                          int N) {
    using G = TailReduceGrid<BMB, BM, BNC>;
    static_assert(256 % G::Q == 0, "whole rows per pass");
    constexpr bool DUAL = (EPI == EPI_SWIGLU);
    constexpr int RW = (DUAL ? 2 : 1) * BNC;  // floats per partial row
    constexpr int PR = G::PR;
    const int tile = blockIdx.x / G::RB, rb = blockIdx.x % G::RB;
    const TileTable tt = tile_table<BMB, BM>(offsets, E, 2 * T, NT);
    const TailPlan tp = tail_plan(tt.total, kts, true);
    const int ntail = tt.total - tp.F;
    if (tp.f == 1 || tile >= ntail) return;  // uniform per block
    Tile tl;
    tile_at<BNC>(tt, E, NT, tp.F + tile, tl);
    const int r0 = rb * G::RPB * PR + (int)threadIdx.x / G::Q, cq = ((int)threadIdx.x % G::Q) * 4;
    const int n = tl.n0 + cq;
    if (r0 >= tl.rows || n >= N) return;
    const size_t pstride = (size_t)ntail * BM * RW;
    const float *src = part + ((size_t)tile * BM + r0) * RW + cq;
    float u[PR][4], v[PR][4];
#pragma unroll
    for (int k = 0; k < PR; ++k)
#pragma unroll
        for (int c = 0; c < 4; ++c) u[k][c] = v[k][c] = 0.0f;
    for (int p = 0; p < tp.f; ++p) {
        f32x4 a[PR], b2[PR];
#pragma unroll
        for (int k = 0; k < PR; ++k) {  // rows past the tile read its row r0 (in bounds) and are not stored
            const float *q = src + p * pstride + (r0 + k * G::RPB < tl.rows ? (size_t)k * G::RPB * RW : 0);
            a[k] = *reinterpret_cast<const f32x4 *>(q);
            b2[k] = DUAL ? *reinterpret_cast<const f32x4 *>(q + BNC) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int k = 0; k < PR; ++k)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                u[k][c] += a[k][c];
                v[k][c] += b2[k][c];
            }
    }
#pragma unroll
    for (int k = 0; k < PR; ++k) {
        const int rl = r0 + k * G::RPB;
        if (rl < tl.rows) store_epilogue<EPI, 4>(C + (size_t)(tl.row0 + rl) * N + n, u[k], v[k], bias, tl.e, N, n);
    }
}

// Tile shapes, BK = 64, one workgroup per CU:
//   big: row tiles of 256 rows (up to 320 when a small tail is spread over
//        them) x 256 weight columns (SwiGLU: 128 outputs of both W1 and W3);
//        8 waves copy both operands through two (A, B) stages, 144 KB of LDS;
//   mid: no SwiGLU, at most 160 expected rows per expert, where the layer
//        streams its weights: row tiles of 128 rows (up to 192) x 128 or 256
//        columns; 8 compute waves copy A through two stages and 2 loader waves
//        keep the weights 5 (128 columns) or 2 (256 columns) k-tiles ahead,
//        144 KB of LDS.  Measured on the 8-expert layer at T = 512 (cold
//        weights): first layer 60.1 -> 54.8 us with 256 columns; second layer
//        with K split in 2 instead of 4, the same time and half the partials.
constexpr int kBK = 64;

}  // namespace

GemmPlan gemm_plan(const colibri_moe_shape_t &s, bool up) {
    const bool dual = up && s.act == COLIBRI_ACT_SWIGLU;
    const bool mid = !dual && 2L * s.T <= 160L * s.E;  // <= 160 expected rows per expert
    const long K = up ? s.d : s.h, N = up ? s.h : s.d;
    const long A = 2L * s.T;
    const long KT = K / kBK;
    const int BMB = mid ? 128 : 256;
    GemmPlan best{mid, BMB, 0, 1, false};
    double best_cost = 1e300;
    // Expected row tiles: one per expert while experts hold at most a tile's
    // rows, else one per base tile height.  Estimated time: (rounds of 256
    // resident workgroups) x (k-tiles per block + 2, a per-block start-up cost)
    // x the k-tile time (measured: ~0.85 us per 128 weight columns for the
    // weight-streaming mid shapes, whose weight stream sets the pace; ~1.9 us
    // for a big tile), plus, when K is split, the fp32 partials written and
    // read once (~5 TB/s) and a ~4 us reduce launch.  Splits keep at least 4
    // k-tiles per block.  Ties keep the wider tile and the smaller S.
    const int widths[2] = {256, 128};
    for (int wi = 0; wi < (mid ? 2 : 1); ++wi) {
        const long BNC = mid ? widths[wi] : (dual ? 128 : 256);
        const long NT = (N + BNC - 1) / BNC;
        const long rt = std::max<long>(std::min<long>(s.E, A), (A + BMB - 1) / BMB);
        const long tiles = rt * NT;
        const double t_kt = mid ? 0.85 * (double)BNC / 128 : 1.9;
        for (long S = 1; S <= KT / 4 || S == 1; ++S) {
            const double part_bytes = (double)S * A * N * (dual ? 2 : 1) * 4;
            double us = (double)((tiles * S + 255) / 256) * ((double)KT / S + 2.0) * t_kt;
            if (S > 1) us += 2.0 * part_bytes / 5.0e6 + 4.0;
            if (us < best_cost - 1e-9) best_cost = us, best = {mid, BMB, (int)BNC, (int)S, false};
        }
    }
    // No K split: when the expected tiles fill whole rounds of one workgroup per
    // CU plus a last round of at most half the CUs, that round's tiles run as
    // K parts (tail_plan; the kernel decides from the actual tile count, the
    // parts' sums go through the partials and a small reduce).
    // A first layer of a prefill-sized batch (at least 4096 rows) always allows
    // the split: a skewed routing cuts the experts into other row tiles than
    // the even spread the estimate assumes (a Zipf-skewed 16-expert layer at
    // T = 8192: 1140 tiles, where 1280 were expected), and the kernel finds
    // the actual tail itself.
    if (best.S == 1) {
        const long NT = (N + best.BNC - 1) / best.BNC;
        const long tiles = std::max<long>(std::min<long>(s.E, A), (A + BMB - 1) / BMB) * NT;
        best.tail = tiles <= (1L << 30) &&
                    (tail_plan((int)tiles, (int)KT, true).f > 1 || (up && !mid && A >= 4096 && KT >= 8));
    }
    return best;
}

namespace {

template <int BMB, int BM, int BN, int WPE, int BLD, int BST, int EPI>
hipError_t launch_shape(bool gather, const colibri_moe_shape_t &s, const void *Am, const int32_t *sa,
                        const int32_t *offsets, const void *B0, const void *B1, const void *bias, void *C, int K, int N,
                        int S, bool tail, float *part, const CombineFold *fold, hipStream_t st) {
    constexpr int BNC = EPI == EPI_SWIGLU ? BN / 2 : BN;
    const int A = 2 * s.T;
    const int NT = (N + BNC - 1) / BNC;
    // bound on the row tiles of all experts: sum over live experts of ceil(rows / H),
    // H = BM for the pair tiling (BMB = 256), else BMB
    constexpr int H = BMB == 256 ? BM : BMB;
    const int mtiles = (int)std::min<long>(A, ((long)A + (long)(H - 1) * std::min(s.E, A)) / H);
    // a tail split adds fewer than kCus blocks (f * tail <= kCus)
    const dim3 grid(S > 1 ? mtiles * NT * S : mtiles * NT + (tail ? kCus : 0));
    constexpr int threads = (2 * 4 + BLD) * kWave;
    const CombineFold cf = fold ? *fold : CombineFold{};
    if (gather)
        ffn_gemm_kernel<BMB, BM, BN, kBK, 2, 4, 2, EPI, true, WPE, BLD, BST><<<grid, threads, 0, st>>>(
            (const uint16_t *)Am, sa, s.T, offsets, s.E, (const uint16_t *)B0, (const uint16_t *)B1,
            (const uint16_t *)bias, (uint16_t *)C, K, N, NT, S, tail ? 1 : 0, part, cf);
    else
        ffn_gemm_kernel<BMB, BM, BN, kBK, 2, 4, 2, EPI, false, WPE, BLD, BST><<<grid, threads, 0, st>>>(
            (const uint16_t *)Am, sa, s.T, offsets, s.E, (const uint16_t *)B0, (const uint16_t *)B1,
            (const uint16_t *)bias, (uint16_t *)C, K, N, NT, S, tail ? 1 : 0, part, cf);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess && tail) {
        constexpr int blocks = TailReduceGrid<BMB, BM, BNC>::blocks;
        tail_reduce_kernel<BMB, BM, BNC, EPI><<<blocks, 256, 0, st>>>(part, s.T, offsets, s.E, NT, K / kBK,
                                                                      (const uint16_t *)bias, (uint16_t *)C, N);
        e = hipGetLastError();
    }
    return e;
}

template <int EPI>
hipError_t launch_gemm(const GemmPlan &p, bool gather, const colibri_moe_shape_t &s, const void *Am, const int32_t *sa,
                       const int32_t *offsets, const void *B0, const void *B1, const void *bias, void *C, int K, int N,
                       float *part, hipStream_t st, const CombineFold *fold = nullptr) {
    if constexpr (EPI != EPI_SWIGLU) {
        if (p.mid && p.BNC == 256)
            return launch_shape<128, 192, 256, 2, 2, 3, EPI>(gather, s, Am, sa, offsets, B0, B1, bias, C, K, N, p.S,
                                                             p.tail, part, fold, st);
        if (p.mid)
            return launch_shape<128, 192, 128, 2, 2, 6, EPI>(gather, s, Am, sa, offsets, B0, B1, bias, C, K, N, p.S,
                                                             p.tail, part, fold, st);
    }
    return launch_shape<256, 320, 256, 2, 0, 2, EPI>(gather, s, Am, sa, offsets, B0, B1, bias, C, K, N, p.S, p.tail,
                                                     part, fold, st);
}

}  // namespace

bool gemm_fold_ok(const colibri_moe_shape_t &s) {
    if (s.dtype != COLIBRI_BF16 || s.T <= 0) return false;
    const GemmPlan p = gemm_plan(s, false);
    return !p.tail && p.S <= kFoldMaxSplits;
}

int gemm_splits(const colibri_moe_shape_t &s, bool up) {
    if (s.dtype != COLIBRI_BF16 || s.T <= 0) return 1;
    return gemm_plan(s, up).S;
}

size_t gemm_scratch_bytes(const colibri_moe_shape_t &s, bool up) {
    if (s.dtype != COLIBRI_BF16 || s.T <= 0) return 0;
    const GemmPlan p = gemm_plan(s, up);
    const bool dual = up && s.act == COLIBRI_ACT_SWIGLU;
    if (p.tail)  // fewer than kCus tail tiles' parts: [part][tail tile][BM][(dual ? 2 : 1) BNC]
        return align256((size_t)kCus * (p.mid ? 192 : 320) * (size_t)p.BNC * (dual ? 2 : 1) * 4);
    if (p.S <= 1) return 0;
    return align256((size_t)p.S * 2 * s.T * (size_t)(up ? s.h : s.d) * (dual ? 2 : 1) * 4);
}

hipError_t launch_gemm_up(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                          const int32_t *offsets, const colibri_moe_experts_t &w, void *H, void *scratch,
                          hipStream_t st) {
    const bool gather = sorted_assign != nullptr;
    const GemmPlan p = gemm_plan(s, true);
    float *part = static_cast<float *>(scratch);
    hipError_t e;
    switch (s.act) {
        case COLIBRI_ACT_RELU:
            e = launch_gemm<EPI_ACT_RELU>(p, gather, s, x_rows, sorted_assign, offsets, w.w1, nullptr, w.b1, H, s.d,
                                          s.h, part, st);
            break;
        case COLIBRI_ACT_GELU:
            e = launch_gemm<EPI_ACT_GELU>(p, gather, s, x_rows, sorted_assign, offsets, w.w1, nullptr, w.b1, H, s.d,
                                          s.h, part, st);
            break;
        default:
            e = launch_gemm<EPI_SWIGLU>(p, gather, s, x_rows, sorted_assign, offsets, w.w1, w.w3, nullptr, H, s.d, s.h,
                                        part, st);
    }
    if (e == hipSuccess && p.S > 1) e = launch_split_reduce(s, true, p.S, offsets, w, H, part, st);
    return e;
}

hipError_t launch_gemm_down(const colibri_moe_shape_t &s, const void *H, const int32_t *offsets,
                            const colibri_moe_experts_t &w, void *y, void *scratch, bool reduce, hipStream_t st,
                            const CombineFold *fold) {
    const void *b2 = s.act == COLIBRI_ACT_SWIGLU ? nullptr : w.b2;
    const GemmPlan p = gemm_plan(s, false);
    if (fold && p.tail) return hipErrorInvalidValue;  // the second layer never runs a tail split
    float *part = static_cast<float *>(scratch);
    hipError_t e = launch_gemm<EPI_BIAS_ONLY>(p, false, s, H, nullptr, offsets, w.w2, nullptr, b2, y, s.h, s.d, part,
                                              st, fold);
    if (e == hipSuccess && p.S > 1 && reduce && !fold) e = launch_split_reduce(s, false, p.S, offsets, w, y, part, st);
    return e;
}

}  // namespace colibri
