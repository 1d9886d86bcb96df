// Internal interface between the C-ABI layer (abi.cpp) and the kernel files.
// Every launcher enqueues on `st` and returns the launch status; arguments
// have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "colibri_moe.h"

namespace colibri {

// gate_mode: a colibri_gate_t
hipError_t launch_route(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r,
                        int32_t *topk_idx, float *topk_gate, float *logits, hipStream_t st,
                        int gate_mode = COLIBRI_GATE_PAIR);

// route + dispatch in one launch for small batches (T <= 32; fp32 with E <= 2:
// T <= 64); the results equal launch_route followed by launch_dispatch bit for bit
bool route_dispatch_fusable(const colibri_moe_shape_t &s);
hipError_t launch_route_dispatch(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r,
                                 int32_t *topk_idx, float *topk_gate, int32_t *counts, int32_t *offsets,
                                 int32_t *sorted_assign, int32_t *assign_pos, hipStream_t st,
                                 int gate_mode = COLIBRI_GATE_PAIR);

// scratch: dispatch_scratch_bytes(s) bytes (256-aligned) or nullptr; with it,
// large batches run the multi-workgroup path (same result)
size_t dispatch_scratch_bytes(const colibri_moe_shape_t &s);
// zero [nzero] (or nullptr): int32 words the dispatch kernels set to 0 on the
// way (the arrival counts of a folded combine, see CombineFold)
hipError_t launch_dispatch(const colibri_moe_shape_t &s, const int32_t *topk_idx, int32_t *counts,
                           int32_t *offsets, int32_t *sorted_assign, int32_t *assign_pos, hipStream_t st,
                           void *scratch = nullptr, int32_t *zero = nullptr, size_t nzero = 0);

hipError_t launch_gather_rows(const colibri_moe_shape_t &s, const void *x, const int32_t *sorted_assign,
                              void *x_sorted, hipStream_t st);

// Scratch the two FFN layers need besides their inputs and outputs (256-byte multiples).
size_t ffn_up_scratch_bytes(const colibri_moe_shape_t &s);
size_t ffn_down_scratch_bytes(const colibri_moe_shape_t &s);
// Workspace of the whole FFN: H [2T, h] plus the larger of the two scratches.
size_t ffn_workspace_bytes(const colibri_moe_shape_t &s);

hipError_t launch_ffn_up(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                         const int32_t *offsets, const colibri_moe_experts_t &w, void *h_rows, void *scratch,
                         hipStream_t st);
// reduce = false (when ffn_down_splits(s) > 1) leaves the split partials in
// scratch; fold: the combine folded into the second layer (see CombineFold)
struct CombineFold;
hipError_t launch_ffn_down(const colibri_moe_shape_t &s, const void *h_rows, const int32_t *offsets,
                           const colibri_moe_experts_t &w, void *y_sorted, void *scratch, hipStream_t st,
                           bool reduce = true, const CombineFold *fold = nullptr);
// Decode-sized batches (bf16, T <= 64) use the weight-streaming kernel.
struct DecodePlan {
    int NCB;            // column blocks per expert
    int slots;          // live-expert slots in the grid (min(E, 2T))
    int W;              // waves per workgroup (split of each workgroup's K range)
    int S;              // K splits across workgroups (partials reduced by the next kernel)
    int MB;             // 16-row subtiles per row chunk
    size_t part_bytes;  // fp32 partial-sum scratch when S > 1
};
bool ffn_decode_eligible(const colibri_moe_shape_t &s);
// q8: int8 weights (half the bytes per k-step)
DecodePlan decode_plan(const colibri_moe_shape_t &s, bool up, bool q8 = false);
// scratch for any decode layout of this shape (bf16 or int8 weights, fused or not)
size_t ffn_decode_scratch_bytes(const colibri_moe_shape_t &s);
// The weights of the decode kernels: bf16 (q8 = false, scales null) or int8
// codes with one fp32 scale per output column.
struct DecodeWeights {
    const void *w1, *w3, *w2;
    const float *s1, *s3, *s2;
    const void *b1, *b2;
    bool q8;
};
inline DecodeWeights decode_weights(const colibri_moe_experts_t &w) {
    return {w.w1, w.w3, w.w2, nullptr, nullptr, nullptr, w.b1, w.b2, false};
}
inline DecodeWeights decode_weights(const colibri_moe_experts_q8_t &w) {
    return {w.q1, w.q3, w.q2, w.s1, w.s3, w.s2, w.b1, w.b2, true};
}
// reduce = false leaves the first layer's split partials in scratch (for decode_fuse_h)
hipError_t launch_decode_up(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                            const int32_t *offsets, const DecodeWeights &w, void *H, void *scratch,
                            hipStream_t st, bool reduce = true);
// reduce = false leaves the split partials in scratch for launch_combine_partials.
// h_partials != nullptr: H is not read; each workgroup rebuilds its slice from
// the first layer's split partials (decode_fuse_h).
hipError_t launch_decode_down(const colibri_moe_shape_t &s, const void *H, const int32_t *offsets,
                              const DecodeWeights &w, void *y, void *scratch, bool reduce, hipStream_t st,
                              const float *h_partials = nullptr);
// Decode sizes whose second layer rebuilds H from the first layer's partials;
// the scratch then holds the first layer's partials, then (256-aligned) the second's.
bool decode_fuse_h(const colibri_moe_shape_t &s, bool q8 = false);
// A shared expert's second layer left as S split partials [S][rows][d] fp32
// (row t = token t, `stride` = rows * d floats per split) with its bias b2 [d]
// (bf16) or nullptr: the combine forms the shared row from them as the reduce
// would.  part == nullptr: none.
struct SharedPartials {
    const float *part = nullptr;
    int S = 0;
    size_t stride = 0;
    const uint16_t *b2 = nullptr;
};
// The combine folded into the epilogue of the second layer's grouped GEMM
// (bf16, T > 64).  Every tile stores its Y rows (or its split partials) as
// usual, then counts itself in at arrive[t * NT + column tile] for each token t
// of its rows (NT = the layer's column tiles); the tile whose count completes
// token t's 2 S arrivals (two slots, S K splits each) forms out[t] over its
// columns with the combine's own arithmetic (combine_common.h), so the output
// does not depend on which tile finishes last and equals the separate
// combine's bit for bit.  arrive must be zero on entry (the layer's dispatch
// zeroes it).  Both slots of every token must hold a valid expert, which the
// layer's routing guarantees.  A shared expert enters as finished rows only
// (its split partials go to the separate combine, which has the registers).
struct CombineFold {
    int32_t *arrive = nullptr;        // [T][NT] counts
    const int32_t *sorted = nullptr;  // sorted row -> assignment 2 t + slot
    const int32_t *pos = nullptr;     // assignment -> sorted row
    const int32_t *idx = nullptr;     // expert of each assignment (split partials)
    const float *gate = nullptr;
    uint16_t *out = nullptr;
    const uint16_t *shared = nullptr;    // [T, d] or nullptr
    const uint16_t *residual = nullptr;  // [T, d] or nullptr
    const uint16_t *b2 = nullptr;  // second-layer bias [E][d] or nullptr (split partials)
};
// Arrival counts a folded combine needs for shape s (0: the combine cannot be
// folded at this shape).
size_t combine_fold_counts(const colibri_moe_shape_t &s);
// COLIBRI_COMBINE_AUTO: fold at this shape (measured faster than the kernel).
bool combine_fold_preferred(const colibri_moe_shape_t &s);
// combine straight from the second layer's S split partials (adds them, b2,
// rounds Y, then gates).  shared, residual: optional [T, d] dtype addends (as
// in launch_combine); sp: the shared row from partials instead of `shared`
hipError_t launch_combine_partials(const colibri_moe_shape_t &s, const float *part, int S, const int32_t *assign_pos,
                                   const int32_t *topk_idx, const float *topk_gate, const void *b2, void *out,
                                   hipStream_t st, const void *shared = nullptr, const void *residual = nullptr,
                                   SharedPartials sp = SharedPartials{});
// bf16 grouped MFMA GEMMs for T > 64 (ffn_gemm.hip).  A layer whose K is split
// (gemm_splits > 1) writes fp32 partials [S][2T][cols] to scratch and then
// reduces them (the second layer only when `reduce`; otherwise
// launch_combine_partials adds them).
struct GemmPlan {
    bool mid;  // weight-streaming tile shapes (no SwiGLU, <= 160 expected rows per expert)
    int BMB;   // base row-tile height
    int BNC;   // output columns per tile
    int S;     // K splits
    bool tail; // first layer, S == 1: the last, partial round of tiles runs as two K halves
};
GemmPlan gemm_plan(const colibri_moe_shape_t &s, bool up);
int gemm_splits(const colibri_moe_shape_t &s, bool up);
// The second layer's plan admits the folded combine (no tail split, few K splits).
bool gemm_fold_ok(const colibri_moe_shape_t &s);
size_t gemm_scratch_bytes(const colibri_moe_shape_t &s, bool up);
hipError_t launch_gemm_up(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                          const int32_t *offsets, const colibri_moe_experts_t &w, void *H, void *scratch,
                          hipStream_t st);
hipError_t launch_gemm_down(const colibri_moe_shape_t &s, const void *H, const int32_t *offsets,
                            const colibri_moe_experts_t &w, void *y, void *scratch, bool reduce, hipStream_t st,
                            const CombineFold *fold = nullptr);
// Adds the S split partials of one layer and applies that layer's epilogue
// (bias + activation, SwiGLU, or bias only), storing the dtype result.
hipError_t launch_split_reduce(const colibri_moe_shape_t &s, bool up, int S, const int32_t *offsets,
                               const colibri_moe_experts_t &w, void *C, const float *part, hipStream_t st);
// K splits of the second layer as launch_ffn_down runs it (1: no partials);
// q8: as the int8-weight decode layers run it.
int ffn_down_splits(const colibri_moe_shape_t &s, bool q8 = false);
// Both layers with H and the scratch carved from ws (H first, then the scratch).
// reduce = false (when ffn_down_splits(s) > 1) leaves the second layer's split
// partials in the scratch, at *down_partials.
// fold (combine_fold_counts(s) > 0 only): the combine folded into the second
// layer, which then writes out instead of leaving Y or partials to a combine.
hipError_t launch_ffn_layers(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                             const int32_t *offsets, const colibri_moe_experts_t &w, void *y_sorted, void *ws,
                             bool reduce, hipStream_t st, const float **down_partials,
                             const CombineFold *fold = nullptr);
// launch_ffn_layers with int8 expert weights: decode sizes only (bf16, T <= 64).
hipError_t launch_ffn_layers_q8(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                                const int32_t *offsets, const colibri_moe_experts_q8_t &w, void *y_sorted, void *ws,
                                bool reduce, hipStream_t st, const float **down_partials);
// Per-column int8 quantization of a weight tensor [E][K][N] (colibri_moe_quantize_q8).
hipError_t launch_quantize_q8(const void *w, colibri_dtype_t dtype, int E, int K, int N, int8_t *q, float *scale,
                              hipStream_t st);
// 4-bit expert weights (ffn_decode_q4.hip): decode sizes with d, h multiples of 128.
bool ffn_q4_eligible(const colibri_moe_shape_t &s);
size_t ffn_decode_q4_scratch_bytes(const colibri_moe_shape_t &s);
int ffn_down_splits_q4(const colibri_moe_shape_t &s);
hipError_t launch_ffn_layers_q4(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                                const int32_t *offsets, const colibri_moe_experts_q4_t &w, void *y_sorted, void *ws,
                                bool reduce, hipStream_t st, const float **down_partials);
// 4-bit codes with zero points in groups of 128 k (colibri_moe_quantize_q4).
hipError_t launch_quantize_q4(const void *w, colibri_dtype_t dtype, int E, int K, int N, uint32_t *q, float *scale,
                              uint8_t *zero, hipStream_t st);
// H then Y (launch_ffn_layers with the second layer reduced).
hipError_t launch_expert_ffn(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                             const int32_t *offsets, const colibri_moe_experts_t &w, void *y_sorted, void *ws,
                             hipStream_t st);

// shared, residual: optional [T, d] dtype rows added after the gated pair
hipError_t launch_combine(const colibri_moe_shape_t &s, const void *y_sorted, const int32_t *assign_pos,
                          const float *topk_gate, void *out, hipStream_t st, const void *shared = nullptr,
                          const void *residual = nullptr, SharedPartials sp = SharedPartials{});
// offsets[0] = 0, offsets[1] = n (a one-expert group of n rows) by a kernel,
// so the step can sit in a captured graph
hipError_t launch_pair_offsets(int32_t *offsets, int n, hipStream_t st);

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace colibri
