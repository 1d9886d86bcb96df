/*
 * colibri_moe.h -- C ABI of the MI355X (gfx950) forward pass of one
 * Mixture-of-Experts layer, as described by the Colibri write-ups:
 *
 *   [zskr]   http://www.zskr.cn/news/2272131  "Colibri: a lightweight C MoE
 *            inference engine for edge devices"
 *   [rkmt]   http://news.rkmt.cn/news/2271114
 *   [hnwysp] https://www.hnwysp.cn/news/30485
 *   [nxbn]   http://m.nxbn.cn/news/48047
 *
 * The layer maps tokens X [T, d] to out [T, d]:
 *   1. router logits   l = X W_r + b_r                       ([zskr] section 3.2, step 1)
 *   2. top-2 experts per token, ties to the lower index, and gates
 *      g = softmax over all experts renormalised over the chosen two
 *                                                             ([zskr] 3.2; [hnwysp] 3.1, 4.3)
 *   3. dispatch: per-expert counts, offsets and a stable expert-sorted
 *      permutation of the 2T assignments                      ([zskr] 3.2, 3.3)
 *   4. per expert, a two-layer FFN on its rows                ([zskr] 1; [nxbn] 3.1; [hnwysp] 3.2)
 *        ReLU / GELU : y = act(x W1 + b1) W2 + b2
 *        SwiGLU      : y = (silu(x W1) * (x W3)) W2
 *   5. combine: out[t] = g0 y(t, slot 0) + g1 y(t, slot 1)   ([nxbn] 3.3, output aggregation)
 *
 * Conventions for every entry point
 *   - Tensor arguments are HIP device pointers, row-major, owned by the
 *     caller; nothing is allocated, freed or synchronised inside a call
 *     (colibri_moe_graph_create / _destroy, which make and free a HIP graph,
 *     aside).
 *     Work is enqueued on `stream` (0 = the null stream) and the call returns
 *     without waiting for it.
 *   - Arguments are validated on the host before anything is launched; an
 *     invalid call launches nothing and returns a negative status.
 *   - Tensors marked "16-byte aligned" must start on a 16-byte boundary.
 *   - Assignment a = 2t + s is token t's slot s (slot 0 = the larger logit).
 *   - topk_idx entries must lie in [0, E) (the router never produces
 *     anything else).  Entries outside that range are skipped by dispatch:
 *     they are not counted, their assign_pos is -1, and the unused tail of
 *     sorted_assign is -1; the FFN and combine skip such rows.
 *   - Calls are reentrant: there is no global state.  Concurrent calls need
 *     separate workspaces (the pages' one-context-per-thread rule, [nxbn] 3.3).
 *   - Status codes: 0 = success, negative = error ([nxbn] 3.3 and 5.1 use the
 *     same convention).
 */
#ifndef COLIBRI_MOE_H
#define COLIBRI_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    COLIBRI_OK = 0,
    COLIBRI_ERR_INVALID_ARG = -1,  /* null required pointer, T < 0, misaligned pointer */
    COLIBRI_ERR_WORKSPACE = -2,    /* ws_bytes smaller than the call needs */
    COLIBRI_ERR_UNSUPPORTED = -3,  /* k != 2, E outside [2, 64], d or h not a multiple of 64,
                                      unknown dtype / activation, act/weights mismatch */
    COLIBRI_ERR_HIP = -4           /* a HIP launch failed */
} colibri_status_t;

/* Storage type of X, W_r, W1, W3, W2, b1, b2, Y and out.  Router bias,
 * logits and gates are always fp32; arithmetic accumulates in fp32. */
typedef enum { COLIBRI_F32 = 0, COLIBRI_BF16 = 1 } colibri_dtype_t;

typedef enum {
    COLIBRI_ACT_RELU = 0,   /* H = max(x W1 + b1, 0) */
    COLIBRI_ACT_GELU = 1,   /* H = z * Phi(z), exact erf form, z = x W1 + b1 */
    COLIBRI_ACT_SWIGLU = 2  /* H = silu(x W1) * (x W3); no biases */
} colibri_act_t;

/* Problem shape.  k must be 2; 2 <= E <= 64; d and h multiples of 64; T >= 0. */
typedef struct {
    int32_t T, d, h, E, k;
    colibri_dtype_t dtype;
    colibri_act_t act;
} colibri_moe_shape_t;

/* Expert parameters, all experts packed contiguously ([zskr] 2.2: one
 * contiguous block per expert set; [nxbn] 3.1: W1 | b1 | W2 | b2 per expert).
 *   w1 [E][d][h]  16-byte aligned
 *   w3 [E][d][h]  16-byte aligned, SwiGLU only (NULL otherwise)
 *   w2 [E][h][d]  16-byte aligned
 *   b1 [E][h], b2 [E][d]  ReLU/GELU only; NULL means zero.  Must be NULL for SwiGLU. */
typedef struct {
    const void *w1, *w3, *w2;
    const void *b1, *b2;
} colibri_moe_experts_t;

/* Bytes of device workspace that colibri_moe_layer_forward needs for this
 * shape (every other entry point needs no more).  Returns 0 for an invalid
 * shape or T = 0. */
size_t colibri_moe_workspace_size(const colibri_moe_shape_t *s);

/* Steps 1-2: router logits, deterministic top-2 and gates
 * ([zskr] 3.2 routing chain; [hnwysp] 3.1 colibri_route_topk).
 *   x         [T, d] dtype, 16-byte aligned
 *   w_r       [d, E] dtype, 16-byte aligned
 *   b_r       [E] fp32, or NULL (zero)
 *   topk_idx  [T, 2] int32 out: slot 0 = best expert, slot 1 = second best under
 *             (logit descending, index ascending); NaN ranks below -inf
 *   topk_gate [T, 2] fp32 out: g0 = 1 / (1 + exp(l1 - l0)), g1 = 1 - g0
 *   logits    [T, E] fp32 out, or NULL: the fp32 logits the selection used */
int colibri_moe_route(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                      int32_t *topk_idx, float *topk_gate, float *logits, hipStream_t stream);

/* Step 3: dispatch ([zskr] 3.2: count per expert, then build offsets;
 * [zskr] 3.3: one contiguous region per expert; [hnwysp] 2.2: pass row
 * offsets instead of copying rows).
 *   topk_idx       [T, 2] int32 in
 *   expert_counts  [E] int32 out
 *   expert_offsets [E + 1] int32 out, offsets[0] = 0, offsets[E] = 2T
 *   sorted_assign  [2T] int32 out: assignments grouped by expert, ascending a
 *                  inside a group
 *   assign_pos     [2T] int32 out: inverse permutation
 *   x, x_sorted    optional pair: when both are non-NULL, x_sorted[p] =
 *                  x[sorted_assign[p] / 2] ([T, d] -> [2T, d], dtype, 16-byte aligned)
 *   ws, ws_bytes   optional scratch (may be NULL / 0): with at least
 *                  colibri_moe_dispatch_workspace_size(s) bytes, 256-byte aligned,
 *                  large batches (2T >= 4096) spread the dispatch over the chip
 *                  (count, scan and scatter kernels); the result is the same */
/* Scratch that lets colibri_moe_dispatch use its multi-workgroup path (0 for
 * batches that do not need it, and for an invalid shape). */
size_t colibri_moe_dispatch_workspace_size(const colibri_moe_shape_t *s);

int colibri_moe_dispatch(const colibri_moe_shape_t *s, const int32_t *topk_idx, int32_t *expert_counts,
                         int32_t *expert_offsets, int32_t *sorted_assign, int32_t *assign_pos,
                         const void *x, void *x_sorted, void *ws, size_t ws_bytes, hipStream_t stream);

/* Step 4: the grouped expert FFN over the expert-sorted rows
 * ([zskr] 2.1 grouped GEMM; [nxbn] 2.1 fused matmul + activation kernel).
 *   x_rows         if sorted_assign != NULL: X [T, d] and row p reads token
 *                  sorted_assign[p] / 2; else already sorted rows [2T, d]
 *   expert_offsets [E + 1] int32: rows [offsets[e], offsets[e+1]) use expert e
 *   w              expert weights (layout above)
 *   y_sorted       [2T, d] dtype out, 16-byte aligned
 *   ws, ws_bytes   device workspace for the hidden activations H [2T, h]
 *                  (stored in dtype, i.e. bf16 for bf16 layers) */
int colibri_moe_expert_ffn(const colibri_moe_shape_t *s, const void *x_rows, const int32_t *sorted_assign,
                           const int32_t *expert_offsets, const colibri_moe_experts_t *w, void *y_sorted,
                           void *ws, size_t ws_bytes, hipStream_t stream);

/* Step 4, first layer alone: H = act(x W1[e] + b1[e]), or silu(x W1[e]) * (x W3[e])
 * for SwiGLU, for every expert-sorted row ([zskr] section 1: the expert's
 * first FFN layer).  Arguments as for colibri_moe_expert_ffn; h_rows [2T, h]
 * dtype out, 16-byte aligned.  ws holds split-K scratch (see
 * colibri_moe_workspace_size; the layer workspace is always enough). */
int colibri_moe_expert_ffn_up(const colibri_moe_shape_t *s, const void *x_rows, const int32_t *sorted_assign,
                              const int32_t *expert_offsets, const colibri_moe_experts_t *w, void *h_rows,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/* Step 4, second layer alone: Y[p] = H[p] W2[e] + b2[e] over the expert-sorted
 * rows.  h_rows [2T, h] dtype in (16-byte aligned), y_sorted [2T, d] out. */
int colibri_moe_expert_ffn_down(const colibri_moe_shape_t *s, const void *h_rows, const int32_t *expert_offsets,
                                const colibri_moe_experts_t *w, void *y_sorted, void *ws, size_t ws_bytes,
                                hipStream_t stream);

/* Step 5: gate-weighted combine fused with the un-permute ([nxbn] 3.3).
 *   out[t] = g[t,0] * y_sorted[assign_pos[2t]] + g[t,1] * y_sorted[assign_pos[2t+1]],
 *   summed in fp32 and stored in dtype.  out [T, d], 16-byte aligned. */
int colibri_moe_combine(const colibri_moe_shape_t *s, const void *y_sorted, const int32_t *assign_pos,
                        const float *topk_gate, void *out, hipStream_t stream);

/* Steps 1-5 in one call ([nxbn] 3.3: one call is one complete MoE forward).
 * topk_idx_out [T, 2], topk_gate_out [T, 2] and expert_counts_out [E] are
 * optional copies of the routing results (NULL = not wanted).  ws must hold
 * colibri_moe_workspace_size(s) bytes, 256-byte aligned. */
int colibri_moe_layer_forward(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                              const colibri_moe_experts_t *w, void *out, int32_t *topk_idx_out,
                              float *topk_gate_out, int32_t *expert_counts_out, void *ws, size_t ws_bytes,
                              hipStream_t stream);

/* Where colibri_moe_layer_forward (and _ex, _q8, _q4, whatever their
 * options) leaves its routing and dispatch results inside the caller's
 * workspace: byte offsets from the workspace start.  Once the call's work on
 * its stream has completed, the workspace holds
 *   expert_offsets [E + 1], sorted_assign [2T], assign_pos [2T]   int32 (always),
 *   topk_idx [T, 2] int32, topk_gate [T, 2] fp32, expert_counts [E] int32
 *       (each only when the call's own output pointer for it was NULL),
 * with the meaning of colibri_moe_dispatch's outputs ([zskr] section 3.2:
 * counts per expert, then offsets; 3.3: one contiguous row range per expert).
 * The next call that uses the workspace overwrites them.  Returns
 * COLIBRI_ERR_INVALID_ARG for a NULL layout, the shape's status otherwise
 * (the offsets are those of colibri_moe_workspace_size's workspace; T >= 1). */
typedef struct {
    size_t topk_idx, topk_gate, expert_counts, expert_offsets, sorted_assign, assign_pos;
} colibri_moe_workspace_layout_t;
int colibri_moe_workspace_layout(const colibri_moe_shape_t *s, colibri_moe_workspace_layout_t *layout);

/* ------------------------------------------------------------------ allocation-free layer
 * For callers that cannot allocate device memory or pass a workspace (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): colibri_moe_layer_forward with its workspace taken from a
 * device array inside the library instead of from the caller.
 *   - The array holds COLIBRI_MOE_NOALLOC_SCRATCH_BYTES (32 MiB); every GPU
 *     the library runs on holds its own copy until the process ends.  Shapes
 *     whose colibri_moe_workspace_size exceeds it are rejected with
 *     COLIBRI_ERR_WORKSPACE before anything is launched (every decode batch of
 *     the 8-expert and Mixtral-shaped layers fits, and the 8-expert layer up
 *     to T = 512; the prefill batches do not).
 *   - The call allocates and frees nothing; its first call on a device looks
 *     up that device's copy of the array (hipGetSymbolAddress) and caches it.
 *   - Every call on one GPU uses that GPU's one array, and the array keeps
 *     whatever the last call left in it (nothing in it needs to start at
 *     zero): calls that overlap on one GPU -- on different streams, or from
 *     different threads without ordering -- race and give wrong results.
 *     Order them on one stream, or use colibri_moe_layer_forward with
 *     separate workspaces.
 * Arguments, results and every other status as for colibri_moe_layer_forward
 * (with the same inputs it returns bit-identical outputs). */
#define COLIBRI_MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int colibri_moe_layer_forward_noalloc(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                                      const colibri_moe_experts_t *w, void *out, int32_t *topk_idx_out,
                                      float *topk_gate_out, int32_t *expert_counts_out, hipStream_t stream);

/* ------------------------------------------------------------------ layer variants
 * Gating of the chosen pair (the selection itself always ranks the logits
 * under (logit descending, index ascending)):
 *   COLIBRI_GATE_PAIR     g0 = 1 / (1 + exp(l1 - l0)), g1 = 1 - g0: softmax over
 *                         the two chosen logits, i.e. softmax over all experts
 *                         renormalised over the pair (Mixtral's top-2; the default)
 *   COLIBRI_GATE_SOFTMAX  g_s = exp(l_s - l0) / sum_e exp(l_e - l0): softmax over
 *                         all E experts, the chosen two taken unnormalised
 *                         (DeepSeek-MoE's "softmax top-2", [rkmt] section 5.2)
 *   COLIBRI_GATE_LINEAR   g_s = l_s: no softmax, the logits weight the outputs
 *                         (LINEAR_SCORE, [zskr] section 2.3) */
typedef enum { COLIBRI_GATE_PAIR = 0, COLIBRI_GATE_SOFTMAX = 1, COLIBRI_GATE_LINEAR = 2 } colibri_gate_t;

/* Where the combine (step 5) runs in a layer call:
 *   COLIBRI_COMBINE_AUTO      the library's choice for the shape (the faster of
 *                             the two below as measured on MI355X)
 *   COLIBRI_COMBINE_SEPARATE  a kernel of its own after the FFN
 *   COLIBRI_COMBINE_FOLD      folded into the epilogue of the second FFN layer
 *                             where that layer is a grouped GEMM (bf16, T > 64,
 *                             no shared expert left as split partials): the
 *                             tile that completes a token's two expert rows
 *                             writes its output ([nxbn] section 2.1 fuses the
 *                             stages after the matmul into its kernel); else
 *                             as SEPARATE
 * The output is the same bit for bit whichever runs. */
typedef enum {
    COLIBRI_COMBINE_AUTO = 0,
    COLIBRI_COMBINE_SEPARATE = 1,
    COLIBRI_COMBINE_FOLD = 2
} colibri_combine_t;

/* Options of colibri_moe_layer_forward_ex:
 *   gate      gating of the routed pair (above)
 *   shared    an always-on shared expert applied to every token with weight 1
 *             ([rkmt] section 5.2: Qwen2-MoE's shared expert beside the routed
 *             ones), one expert in the layout of colibri_moe_experts_t
 *             (w1 [1][d][shared_h] ...), same activation; or NULL
 *   residual  [T, d] dtype, 16-byte aligned, added to the output ([nxbn]
 *             section 2.1: residual add fused with the expert computation); or
 *             NULL.  It may be the same buffer as out (an in-place update).
 *   combine   where the combine runs (above; a zeroed struct gives AUTO)
 * out[t] = g0 y(t, slot 0) + g1 y(t, slot 1) + y_shared(t) + residual[t], summed
 * in fp32 and rounded once; y_shared is stored in dtype like the routed rows. */
typedef struct {
    colibri_gate_t gate;
    const colibri_moe_experts_t *shared;
    int32_t shared_h; /* hidden width of the shared expert (0: h); a multiple of 64 */
    const void *residual;
    int32_t combine; /* colibri_combine_t */
} colibri_moe_layer_opts_t;

/* Workspace of colibri_moe_layer_forward_ex for these options (NULL opts =
 * the plain layer: equal to colibri_moe_workspace_size). */
size_t colibri_moe_workspace_size_ex(const colibri_moe_shape_t *s, const colibri_moe_layer_opts_t *opts);

/* Steps 1-2 with a choice of gating; colibri_moe_route is gate = COLIBRI_GATE_PAIR. */
int colibri_moe_route_ex(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                         colibri_gate_t gate, int32_t *topk_idx, float *topk_gate, float *logits, hipStream_t stream);

/* Step 5 with the optional addends: out[t] = g0 y0 + g1 y1 + shared_y[t] +
 * residual[t].  shared_y [T, d] and residual [T, d] are dtype, 16-byte aligned,
 * or NULL. */
int colibri_moe_combine_ex(const colibri_moe_shape_t *s, const void *y_sorted, const int32_t *assign_pos,
                           const float *topk_gate, const void *shared_y, const void *residual, void *out,
                           hipStream_t stream);

/* Steps 1-5 with the options above (NULL opts = colibri_moe_layer_forward).
 * ws must hold colibri_moe_workspace_size_ex(s, opts) bytes, 256-byte aligned. */
int colibri_moe_layer_forward_ex(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                                 const colibri_moe_experts_t *w, const colibri_moe_layer_opts_t *opts, void *out,
                                 int32_t *topk_idx_out, float *topk_gate_out, int32_t *expert_counts_out, void *ws,
                                 size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ multi-layer step, graph replay
 * A decode step through L MoE layers in sequence, each with its own weights,
 * in place on x [T, d]:
 *   for l = 0 .. L-1:  x <- layer_l(x) + x   (residual != 0)   or   x <- layer_l(x)
 * where layer_l is colibri_moe_layer_forward_ex with that layer's parameters
 * (the residual add is the fused one of [nxbn] section 2.1).  The pages keep
 * the launches of a step few and run routing and the GEMMs on two streams so
 * that they overlap ([zskr] section 5.3); here a step is captured once into a
 * HIP graph and replayed as one launch, and (T > 8) each layer's shared expert
 * (which reads only x) sits on a parallel branch of the graph beside routing
 * and the routed FFN. */
typedef struct {
    const void *w_r;                     /* [d, E] dtype */
    const float *b_r;                    /* [E] fp32 or NULL */
    colibri_moe_experts_t experts;       /* the layer's routed experts */
    colibri_gate_t gate;                 /* gating of the chosen pair */
    const colibri_moe_experts_t *shared; /* shared expert or NULL (as colibri_moe_layer_opts_t) */
    int32_t shared_h;                    /* its hidden width (0: h) */
} colibri_moe_layer_params_t;

/* Workspace of a step (the layers run one after another and share it):
 * the largest colibri_moe_workspace_size_ex over the layers; 0 for an invalid
 * shape, L or layer. */
size_t colibri_moe_step_workspace_size(const colibri_moe_shape_t *s, int32_t L,
                                       const colibri_moe_layer_params_t *layers);

/* Runs the step on `stream`, eagerly (one layer after another, shared experts
 * on the same stream).  1 <= L <= 4096; x 16-byte aligned; ws as for the
 * layer.  T = 0 is a no-op. */
int colibri_moe_step_forward(const colibri_moe_shape_t *s, int32_t L, const colibri_moe_layer_params_t *layers,
                             int32_t residual, void *x, void *ws, size_t ws_bytes, hipStream_t stream);

/* Captures the same step into an executable HIP graph on the current device
 * (T >= 1).  The graph holds x, ws and every weight pointer: they must stay
 * valid, and launches of one graph must not overlap (they share x and ws).
 * Creating a graph creates and destroys two streams and two events and
 * launches nothing; the graph lives until colibri_moe_graph_destroy.  Each
 * replay computes exactly what colibri_moe_step_forward computes (the same
 * kernels in the same order on each branch). */
typedef struct colibri_moe_graph colibri_moe_graph_t;
int colibri_moe_graph_create(const colibri_moe_shape_t *s, int32_t L, const colibri_moe_layer_params_t *layers,
                             int32_t residual, void *x, void *ws, size_t ws_bytes, colibri_moe_graph_t **graph);
/* Replays the step on `stream` (same device as at creation). */
int colibri_moe_graph_launch(colibri_moe_graph_t *graph, hipStream_t stream);
/* Frees the graph (NULL: no-op).  No launch of it may still be pending. */
int colibri_moe_graph_destroy(colibri_moe_graph_t *graph);

/* ------------------------------------------------------------------ int8 expert weights
 * Expert weights stored as int8 codes with one fp32 scale per output column
 * ([zskr] section 5.3: per-channel INT8 quantization of the expert weights,
 * scales kept beside them, halving the weight bytes):
 *   W[e][k][n] = s[e][n] * q[e][k][n],  q in [-127, 127].
 *   q1 [E][d][h], q3 [E][d][h] (SwiGLU only, else NULL), q2 [E][h][d]   int8, 16-byte aligned
 *   s1 [E][h], s3 [E][h] (SwiGLU only, else NULL), s2 [E][d]             fp32, 4-byte aligned
 *   b1 [E][h], b2 [E][d]   as in colibri_moe_experts_t (NULL = zero; NULL for SwiGLU)
 * The layer computes exactly what it computes with the dequantized weights
 * s * q stored in full precision (each column's sum is formed from the
 * codes and multiplied by its scale).  These entry points stream weights at
 * decode sizes: they take bf16 layers with T <= 64 and return
 * COLIBRI_ERR_UNSUPPORTED for other shapes. */
typedef struct {
    const int8_t *q1, *q3, *q2;
    const float *s1, *s3, *s2;
    const void *b1, *b2;
} colibri_moe_experts_q8_t;

/* Per-column int8 quantization of one weight tensor (producing q1, q3 or q2
 * and its scales).  For every expert e and column n, in fp32:
 *   amax = max over k of |w[e][k][n]|,  s[e][n] = amax / 127  (1 when amax = 0),
 *   q[e][k][n] = w[e][k][n] / s[e][n] rounded to nearest (ties to even),
 *   clamped to [-127, 127].
 *   w [E][K][N] dtype, 16-byte aligned; q [E][K][N] int8 out; s [E][N] fp32 out.
 * E, K, N >= 1; N a multiple of 4. */
int colibri_moe_quantize_q8(const void *w, colibri_dtype_t dtype, int32_t E, int32_t K, int32_t N, int8_t *q,
                            float *s, hipStream_t stream);

/* Step 4 with int8 expert weights; arguments as for colibri_moe_expert_ffn.
 * ws must hold colibri_moe_workspace_size(s) bytes, 256-byte aligned. */
int colibri_moe_expert_ffn_q8(const colibri_moe_shape_t *s, const void *x_rows, const int32_t *sorted_assign,
                              const int32_t *expert_offsets, const colibri_moe_experts_q8_t *w, void *y_sorted,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/* Steps 1-5 with int8 expert weights; arguments as for colibri_moe_layer_forward. */
int colibri_moe_layer_forward_q8(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                                 const colibri_moe_experts_q8_t *w, void *out, int32_t *topk_idx_out,
                                 float *topk_gate_out, int32_t *expert_counts_out, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/* ------------------------------------------------------------------ 4-bit expert weights
 * Expert weights stored as 4-bit codes with a zero point, in groups of 128
 * input channels ([rkmt] section 4.2: 4-bit AWQ weights, quantization group
 * 128, zero point; a quarter of the bf16 weight bytes plus the group scales):
 *   W[e][k][n] = s[e][k/128][n] * (q[e][k][n] - z[e][k/128][n]),  q, z in [0, 15].
 *   q1 [E][d/8][h], q3 [E][d/8][h] (SwiGLU only, else NULL), q2 [E][h/8][d]
 *       uint32 words, 16-byte aligned; word (e, j, n) packs the codes of
 *       k = 8j .. 8j+7 of column n: the code of k = 8j + 2m in bits 4m .. 4m+3
 *       and of k = 8j + 2m + 1 in bits 16 + 4m .. 16 + 4m + 3 (m = 0..3)
 *   s1, s3 [E][d/128][h], s2 [E][h/128][d]   fp32 group scales, 16-byte aligned
 *   z1, z3 [E][d/128][h], z2 [E][h/128][d]   uint8 zero points, 4-byte aligned
 *   b1 [E][h], b2 [E][d]   as in colibri_moe_experts_t (NULL = zero; NULL for SwiGLU)
 * The layer computes what it computes with the dequantized weights in full
 * precision: each group's sum is formed from the codes and scaled once.
 * These entry points stream weights at decode sizes: they take bf16 layers
 * with T <= 64 and d, h multiples of 128, and return COLIBRI_ERR_UNSUPPORTED
 * for other shapes. */
typedef struct {
    const uint32_t *q1, *q3, *q2;
    const float *s1, *s3, *s2;
    const uint8_t *z1, *z3, *z2;
    const void *b1, *b2;
} colibri_moe_experts_q4_t;

/* 4-bit quantization of one weight tensor (producing q1, q3 or q2 with its
 * scales and zero points), AWQ's min-max rounding with zero point.  For every
 * expert e, group g (k = 128 g .. 128 g + 127) and column n, in fp32:
 *   mx, mn = the largest and smallest w[e][k][n] of the group,
 *   s = max(mx - mn, 1e-5) / 15,   z = -rint(mn / s) clamped to [0, 15],
 *   q[e][k][n] = rint(w[e][k][n] / s) + z clamped to [0, 15]
 * (rint: nearest, ties to even).  AWQ's activation-aware choice of scales
 * needs calibration activations and is not done here.
 *   w [E][K][N] dtype, 16-byte aligned;  q [E][K/8][N] uint32 out (packed as
 *   above, 16-byte aligned);  s [E][K/128][N] fp32 out, 16-byte aligned;
 *   z [E][K/128][N] uint8 out, 4-byte aligned.
 * E, N >= 1; K >= 128 a multiple of 128; N a multiple of 4. */
int colibri_moe_quantize_q4(const void *w, colibri_dtype_t dtype, int32_t E, int32_t K, int32_t N, uint32_t *q,
                            float *s, uint8_t *z, hipStream_t stream);

/* Step 4 with 4-bit expert weights; arguments as for colibri_moe_expert_ffn.
 * ws must hold colibri_moe_workspace_size(s) bytes, 256-byte aligned. */
int colibri_moe_expert_ffn_q4(const colibri_moe_shape_t *s, const void *x_rows, const int32_t *sorted_assign,
                              const int32_t *expert_offsets, const colibri_moe_experts_q4_t *w, void *y_sorted,
                              void *ws, size_t ws_bytes, hipStream_t stream);

/* Steps 1-5 with 4-bit expert weights; arguments as for colibri_moe_layer_forward. */
int colibri_moe_layer_forward_q4(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                                 const colibri_moe_experts_q4_t *w, void *out, int32_t *topk_idx_out,
                                 float *topk_gate_out, int32_t *expert_counts_out, void *ws, size_t ws_bytes,
                                 hipStream_t stream);

/* Human-readable name of a status code (static storage). */
const char *colibri_moe_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* COLIBRI_MOE_H */
