// Internal interface between the C-ABI layer (abi.cpp) and the kernel files.
// Every launcher enqueues on `st` and returns the launch status; arguments
// have already been validated by the caller.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "colibri_moe.h"

namespace colibri {

hipError_t launch_route(const colibri_moe_shape_t &s, const void *x, const void *w_r, const float *b_r,
                        int32_t *topk_idx, float *topk_gate, float *logits, hipStream_t st);

hipError_t launch_dispatch(const colibri_moe_shape_t &s, const int32_t *topk_idx, int32_t *counts,
                           int32_t *offsets, int32_t *sorted_assign, int32_t *assign_pos, hipStream_t st);

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
hipError_t launch_ffn_down(const colibri_moe_shape_t &s, const void *h_rows, const int32_t *offsets,
                           const colibri_moe_experts_t &w, void *y_sorted, void *scratch, hipStream_t st);
// H then Y, with H and the scratch carved from ws.
hipError_t launch_expert_ffn(const colibri_moe_shape_t &s, const void *x_rows, const int32_t *sorted_assign,
                             const int32_t *offsets, const colibri_moe_experts_t &w, void *y_sorted, void *ws,
                             hipStream_t st);

hipError_t launch_combine(const colibri_moe_shape_t &s, const void *y_sorted, const int32_t *assign_pos,
                          const float *topk_gate, void *out, hipStream_t st);

inline size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace colibri
