// C ABI of the MoE layer: host-side validation, workspace carving and the
// launch sequence.  Every argument is checked before anything is launched;
// nothing here allocates, frees or waits on the device, except that
// colibri_moe_graph_create / _destroy make and free a HIP graph.
//
// Error convention follows the Colibri write-up [nxbn] http://m.nxbn.cn/news/48047
// sections 3.3 and 5.1 (0 = success, negative codes for errors), failing
// loudly instead of the silent zero output that [zskr]
// http://www.zskr.cn/news/2272131 section 5.2 reports for a wrong pointer.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <mutex>
#include <new>

#include "colibri_moe.h"
#include "launchers.h"
#include "validate.h"

using namespace colibri;

namespace {

constexpr int32_t kMaxTokens = 1 << 28;  // keeps assignment ids 2t+s and row counts in int32

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int check_shape(const colibri_moe_shape_t *s) {
    if (!s) return COLIBRI_ERR_INVALID_ARG;
    if (s->k != 2) return COLIBRI_ERR_UNSUPPORTED;
    if (s->E < 2 || s->E > 64) return COLIBRI_ERR_UNSUPPORTED;
    if (s->d <= 0 || s->h <= 0 || s->d % 64 || s->h % 64) return COLIBRI_ERR_UNSUPPORTED;
    if (s->d > (1 << 20) || s->h > (1 << 20)) return COLIBRI_ERR_UNSUPPORTED;
    if (s->dtype != COLIBRI_F32 && s->dtype != COLIBRI_BF16) return COLIBRI_ERR_UNSUPPORTED;
    if (s->act != COLIBRI_ACT_RELU && s->act != COLIBRI_ACT_GELU && s->act != COLIBRI_ACT_SWIGLU)
        return COLIBRI_ERR_UNSUPPORTED;
    if (s->T < 0) return COLIBRI_ERR_INVALID_ARG;
    if (s->T > kMaxTokens) return COLIBRI_ERR_UNSUPPORTED;
    return COLIBRI_OK;
}

size_t elem_size(const colibri_moe_shape_t *s) { return s->dtype == COLIBRI_F32 ? 4 : 2; }

// Checks the expert parameters a call reads: the first layer (W1, W3, b1),
// the second layer (W2, b2), or both.
int check_experts(const colibri_moe_shape_t *s, const colibri_moe_experts_t *w, bool up = true, bool down = true) {
    if (!w) return COLIBRI_ERR_INVALID_ARG;
    if ((up && !w->w1) || (down && !w->w2)) return COLIBRI_ERR_INVALID_ARG;
    if ((w->w1 && !aligned(w->w1, 16)) || (w->w2 && !aligned(w->w2, 16))) return COLIBRI_ERR_INVALID_ARG;
    if (s->act == COLIBRI_ACT_SWIGLU) {
        if (up && !w->w3) return COLIBRI_ERR_INVALID_ARG;
        if (w->w3 && !aligned(w->w3, 16)) return COLIBRI_ERR_INVALID_ARG;
        if (w->b1 || w->b2) return COLIBRI_ERR_UNSUPPORTED;
    } else {
        if (w->w3) return COLIBRI_ERR_UNSUPPORTED;
        const size_t es = elem_size(s);
        if ((w->b1 && !aligned(w->b1, es)) || (w->b2 && !aligned(w->b2, es))) return COLIBRI_ERR_INVALID_ARG;
    }
    return COLIBRI_OK;
}

// int8 expert weights: decode-size bf16 layers only, codes and scales present
// for the layers the call reads, no W3 outside SwiGLU and no biases inside it.
int check_experts_q8(const colibri_moe_shape_t *s, const colibri_moe_experts_q8_t *w) {
    if (!w) return COLIBRI_ERR_INVALID_ARG;
    if (s->dtype != COLIBRI_BF16 || s->T > 64) return COLIBRI_ERR_UNSUPPORTED;
    if (!w->q1 || !w->q2 || !w->s1 || !w->s2) return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(w->q1, 16) || !aligned(w->q2, 16) || !aligned(w->s1, 4) || !aligned(w->s2, 4))
        return COLIBRI_ERR_INVALID_ARG;
    if (s->act == COLIBRI_ACT_SWIGLU) {
        if (!w->q3 || !w->s3) return COLIBRI_ERR_INVALID_ARG;
        if (!aligned(w->q3, 16) || !aligned(w->s3, 4)) return COLIBRI_ERR_INVALID_ARG;
        if (w->b1 || w->b2) return COLIBRI_ERR_UNSUPPORTED;
    } else {
        if (w->q3 || w->s3) return COLIBRI_ERR_UNSUPPORTED;
        if ((w->b1 && !aligned(w->b1, 2)) || (w->b2 && !aligned(w->b2, 2))) return COLIBRI_ERR_INVALID_ARG;
    }
    return COLIBRI_OK;
}

// 4-bit expert weights: decode-size bf16 layers with d, h multiples of 128;
// codes, scales and zero points present for the layers the call reads.
int check_experts_q4(const colibri_moe_shape_t *s, const colibri_moe_experts_q4_t *w) {
    if (!w) return COLIBRI_ERR_INVALID_ARG;
    if (!ffn_q4_eligible(*s)) return COLIBRI_ERR_UNSUPPORTED;
    auto ok = [](const uint32_t *q, const float *sc, const uint8_t *z) {
        return q && sc && z && aligned(q, 16) && aligned(sc, 16) && aligned(z, 4);
    };
    if (!ok(w->q1, w->s1, w->z1) || !ok(w->q2, w->s2, w->z2)) return COLIBRI_ERR_INVALID_ARG;
    if (s->act == COLIBRI_ACT_SWIGLU) {
        if (!ok(w->q3, w->s3, w->z3)) return COLIBRI_ERR_INVALID_ARG;
        if (w->b1 || w->b2) return COLIBRI_ERR_UNSUPPORTED;
    } else {
        if (w->q3 || w->s3 || w->z3) return COLIBRI_ERR_UNSUPPORTED;
        if ((w->b1 && !aligned(w->b1, 2)) || (w->b2 && !aligned(w->b2, 2))) return COLIBRI_ERR_INVALID_ARG;
    }
    return COLIBRI_OK;
}

// The shared expert runs as a one-expert group over the T token rows of x:
// shape {ceil(T / 2), d, shared_h, E = 1} (the FFN kernels work on 2T rows
// of a shape; its one expert gets rows [0, T), so x is read in place and its
// outputs land in token order).
colibri_moe_shape_t shared_shape(const colibri_moe_shape_t *s, const colibri_moe_layer_opts_t *o) {
    colibri_moe_shape_t sh = *s;
    sh.T = (s->T + 1) / 2;
    sh.h = o->shared_h ? o->shared_h : s->h;
    sh.E = 1;
    return sh;
}

bool has_shared(const colibri_moe_layer_opts_t *o) { return o && o->shared; }

int check_opts(const colibri_moe_shape_t *s, const colibri_moe_layer_opts_t *o) {
    if (!o) return COLIBRI_OK;
    if (o->gate != COLIBRI_GATE_PAIR && o->gate != COLIBRI_GATE_SOFTMAX && o->gate != COLIBRI_GATE_LINEAR)
        return COLIBRI_ERR_UNSUPPORTED;
    if (o->residual && !aligned(o->residual, 16)) return COLIBRI_ERR_INVALID_ARG;
    if (o->combine != COLIBRI_COMBINE_AUTO && o->combine != COLIBRI_COMBINE_SEPARATE &&
        o->combine != COLIBRI_COMBINE_FOLD)
        return COLIBRI_ERR_UNSUPPORTED;
    if (o->shared_h < 0 || o->shared_h % 64 || o->shared_h > (1 << 20)) return COLIBRI_ERR_UNSUPPORTED;
    if (o->shared) {
        const colibri_moe_shape_t sh = shared_shape(s, o);
        return check_experts(&sh, o->shared);
    }
    return COLIBRI_OK;
}

struct LayerWorkspace {
    size_t idx, gate, counts, offsets, sorted, pos, disp, arrive, y, sh_offsets, sh_y, sh_ffn, ffn, total;
};

// The plain layer's regions, then (with a shared expert) its offsets, output
// rows and FFN scratch of its own, so that it may run beside the routed FFN;
// the routed FFN region last.
LayerWorkspace layer_workspace(const colibri_moe_shape_t *s, const colibri_moe_layer_opts_t *o = nullptr) {
    LayerWorkspace L{};
    const size_t A = 2 * (size_t)s->T;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        size_t at = off;
        off += align256(bytes);
        return at;
    };
    L.idx = take(A * 4);
    L.gate = take(A * 4);
    L.counts = take((size_t)s->E * 4);
    L.offsets = take((size_t)(s->E + 1) * 4);
    L.sorted = take(A * 4);
    L.pos = take(A * 4);
    L.disp = take(dispatch_scratch_bytes(*s));
    L.arrive = take(combine_fold_counts(*s) * 4);
    L.y = take(A * s->d * elem_size(s));
    if (has_shared(o)) {
        const colibri_moe_shape_t sh = shared_shape(s, o);
        L.sh_offsets = take(2 * 4);
        L.sh_y = take(2 * (size_t)sh.T * s->d * elem_size(s));
        L.sh_ffn = take(ffn_workspace_bytes(sh));
    }
    L.ffn = take(ffn_workspace_bytes(*s));
    L.total = off;
    return L;
}

int hip_status(hipError_t e) { return e == hipSuccess ? COLIBRI_OK : COLIBRI_ERR_HIP; }

// ------------------------------------------------------------------ COLIBRI_MOE_VALIDATE=1
// The argument groups the entry points share; each adds its checks to v.
void v_router(Validator &v, const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r) {
    v.finite(x, (size_t)s->T * s->d, s->dtype).finite(w_r, (size_t)s->d * s->E, s->dtype);
    v.finite(b_r, (size_t)s->E, COLIBRI_F32);
}

void v_experts(Validator &v, const colibri_moe_shape_t *s, const colibri_moe_experts_t *w, bool up = true,
               bool down = true) {
    const size_t E = s->E, d = s->d, h = s->h;
    if (up) v.finite(w->w1, E * d * h, s->dtype).finite(w->w3, E * d * h, s->dtype).finite(w->b1, E * h, s->dtype);
    if (down) v.finite(w->w2, E * h * d, s->dtype).finite(w->b2, E * d, s->dtype);
}

void v_experts_q8(Validator &v, const colibri_moe_shape_t *s, const colibri_moe_experts_q8_t *w) {
    const size_t E = s->E, d = s->d, h = s->h;
    v.range(w->q1, E * d * h).range(w->q3, E * d * h).range(w->q2, E * h * d);
    v.finite(w->s1, E * h, COLIBRI_F32).finite(w->s3, E * h, COLIBRI_F32).finite(w->s2, E * d, COLIBRI_F32);
    v.finite(w->b1, E * h, s->dtype).finite(w->b2, E * d, s->dtype);
}

void v_experts_q4(Validator &v, const colibri_moe_shape_t *s, const colibri_moe_experts_q4_t *w) {
    const size_t E = s->E, d = s->d, h = s->h;
    v.range(w->q1, E * d / 8 * h * 4).range(w->q3, E * d / 8 * h * 4).range(w->q2, E * h / 8 * d * 4);
    v.finite(w->s1, E * d / 128 * h, COLIBRI_F32).finite(w->s3, E * d / 128 * h, COLIBRI_F32);
    v.finite(w->s2, E * h / 128 * d, COLIBRI_F32);
    v.range(w->z1, E * d / 128 * h).range(w->z3, E * d / 128 * h).range(w->z2, E * h / 128 * d);
    v.finite(w->b1, E * h, s->dtype).finite(w->b2, E * d, s->dtype);
}

// the layer's outputs and workspace
void v_layer_out(Validator &v, const colibri_moe_shape_t *s, const void *out, const int32_t *idx, const float *gate,
                 const int32_t *counts) {
    const size_t T = s->T;
    v.range(out, T * s->d * elem_size(s)).range(idx, 2 * T * 4).range(gate, 2 * T * 4).range(counts, s->E * 4);
}

// a stream under graph capture cannot be waited on; a captured step is
// validated once, before its capture starts
bool capturing(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone;
}

void v_opts(Validator &v, const colibri_moe_shape_t *s, const colibri_moe_layer_opts_t *o) {
    if (!o) return;
    v.finite(o->residual, (size_t)s->T * s->d, s->dtype);
    if (o->shared) {
        const colibri_moe_shape_t sh = shared_shape(s, o);
        v_experts(v, &sh, o->shared);
    }
}

// the rows the FFN reads: X [T, d] through sorted_assign, or sorted rows [2T, d];
// offsets [E + 1] and sorted_assign [2T] as dispatch writes them
void v_ffn_rows(Validator &v, const colibri_moe_shape_t *s, const void *x_rows, const int32_t *sorted_assign,
                const int32_t *offsets, int K) {
    const size_t A = 2 * (size_t)s->T;
    v.finite(x_rows, (sorted_assign ? (size_t)s->T : A) * K, s->dtype);
    v.indices(sorted_assign, A, -1, (int32_t)A - 1).offsets(offsets, s->E + 1, (int32_t)A);
}


// A second stream for the shared expert: forked from the main stream before
// routing (it reads only x), joined before the combine.  aux == nullptr: the
// shared expert runs on the main stream.
struct Branch {
    hipStream_t aux = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};

// Steps 1-5 after the shape and expert checks.  ffn(sorted, offsets, y, ffn_ws,
// reduce, &partials) runs both FFN layers; with Sd > 1 second-layer K splits
// the combine adds the splits' partials (with b2) instead of a separate reduce.
// The layer's own tensor arguments (not the experts, not the workspace).
int check_layer_io(const void *x, const void *w_r, const float *b_r, const void *out, const int32_t *topk_idx_out,
                   const float *topk_gate_out, const int32_t *expert_counts_out) {
    if (!x || !w_r || !out) return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w_r, 16) || !aligned(out, 16) || (b_r && !aligned(b_r, 4)) ||
        (topk_idx_out && !aligned(topk_idx_out, 4)) || (topk_gate_out && !aligned(topk_gate_out, 4)) ||
        (expert_counts_out && !aligned(expert_counts_out, 4)))
        return COLIBRI_ERR_INVALID_ARG;
    return COLIBRI_OK;
}

// vexp(v) adds the checks of the weights (and of a caller workspace) under
// COLIBRI_MOE_VALIDATE=1.
template <class Ffn, class VExp>
int layer_forward_impl(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r, void *out,
                       int32_t *topk_idx_out, float *topk_gate_out, int32_t *expert_counts_out, void *ws,
                       size_t ws_bytes, hipStream_t stream, const void *b2, int Sd, Ffn ffn, VExp vexp,
                       const colibri_moe_layer_opts_t *opts = nullptr, const Branch &br = Branch{}) {
    const int io = check_layer_io(x, w_r, b_r, out, topk_idx_out, topk_gate_out, expert_counts_out);
    if (io != COLIBRI_OK) return io;
    const LayerWorkspace L = layer_workspace(s, opts);
    if (ws_bytes < L.total) return COLIBRI_ERR_WORKSPACE;
    if (!ws || !aligned(ws, 256)) return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled() && !capturing(stream)) {
        Validator v(stream);
        v_router(v, s, x, w_r, b_r);
        v_layer_out(v, s, out, topk_idx_out, topk_gate_out, expert_counts_out);
        v_opts(v, s, opts);
        vexp(v);
        if (v.status() != COLIBRI_OK) return v.status();
    }

    char *base = static_cast<char *>(ws);
    int32_t *idx = topk_idx_out ? topk_idx_out : reinterpret_cast<int32_t *>(base + L.idx);
    float *gate = topk_gate_out ? topk_gate_out : reinterpret_cast<float *>(base + L.gate);
    int32_t *counts = expert_counts_out ? expert_counts_out : reinterpret_cast<int32_t *>(base + L.counts);
    int32_t *offsets = reinterpret_cast<int32_t *>(base + L.offsets);
    int32_t *sorted = reinterpret_cast<int32_t *>(base + L.sorted);
    int32_t *pos = reinterpret_cast<int32_t *>(base + L.pos);
    void *y = base + L.y;
    void *ffn_ws = base + L.ffn;

    const int gate_mode = opts ? opts->gate : COLIBRI_GATE_PAIR;
    const void *residual = opts ? opts->residual : nullptr;
    void *sh_y = has_shared(opts) ? base + L.sh_y : nullptr;

    hipError_t e = hipSuccess;
    const bool branch = sh_y && br.aux;
    // a split second layer of the shared expert is left as partials for the
    // combine, which forms the shared row from them as the reduce would
    SharedPartials shp;
    if (sh_y) {
        // the shared expert over all T rows of x (a one-expert group, no gather)
        hipStream_t ss = stream;
        if (branch) {
            e = hipEventRecord(br.fork, stream);
            if (e == hipSuccess) e = hipStreamWaitEvent(br.aux, br.fork, 0);
            ss = br.aux;
        }
        const colibri_moe_shape_t sh = shared_shape(s, opts);
        int32_t *sh_off = reinterpret_cast<int32_t *>(base + L.sh_offsets);
        if (e == hipSuccess) e = launch_pair_offsets(sh_off, s->T, ss);
        const int sh_S = ffn_down_splits(sh);
        if (e == hipSuccess && sh_S > 1) {
            shp.S = sh_S;
            shp.stride = 2 * (size_t)sh.T * sh.d;
            shp.b2 = sh.act == COLIBRI_ACT_SWIGLU ? nullptr : static_cast<const uint16_t *>(opts->shared->b2);
            e = launch_ffn_layers(sh, x, nullptr, sh_off, *opts->shared, nullptr, base + L.sh_ffn, false, ss,
                                  &shp.part);
            sh_y = nullptr;
        } else if (e == hipSuccess) {
            e = launch_ffn_layers(sh, x, nullptr, sh_off, *opts->shared, sh_y, base + L.sh_ffn, true, ss, nullptr);
        }
        if (e == hipSuccess && branch) e = hipEventRecord(br.join, ss);
    }
    // the combine folded into the second layer's epilogue where that layer is a
    // grouped GEMM and the caller (or, by default, the library) picks it; a
    // shared expert on a parallel branch is joined before the second layer then
    const size_t narrive = combine_fold_counts(*s);
    // (its counts are zeroed by the dispatch kernels; a shared expert left as
    // split partials goes to the separate combine)
    const int mode = opts ? opts->combine : COLIBRI_COMBINE_AUTO;
    const bool fold = narrive > 0 && !route_dispatch_fusable(*s) && shp.part == nullptr &&
                      (mode == COLIBRI_COMBINE_FOLD || (mode == COLIBRI_COMBINE_AUTO && combine_fold_preferred(*s)));
    int32_t *arrive = fold ? reinterpret_cast<int32_t *>(base + L.arrive) : nullptr;
    if (e == hipSuccess) {
        if (route_dispatch_fusable(*s)) {
            e = launch_route_dispatch(*s, x, w_r, b_r, idx, gate, counts, offsets, sorted, pos, stream, gate_mode);
        } else {
            e = launch_route(*s, x, w_r, b_r, idx, gate, nullptr, stream, gate_mode);
            if (e == hipSuccess)
                e = launch_dispatch(*s, idx, counts, offsets, sorted, pos, stream,
                                    dispatch_scratch_bytes(*s) ? base + L.disp : nullptr, arrive,
                                    fold ? narrive : 0);
        }
    }
    if (e != hipSuccess) return hip_status(e);
    const float *part = nullptr;
    if (fold) {
        if (branch) e = hipStreamWaitEvent(stream, br.join, 0);
        CombineFold cf;
        cf.arrive = arrive;
        cf.sorted = sorted;
        cf.pos = pos;
        cf.idx = idx;
        cf.gate = gate;
        cf.out = static_cast<uint16_t *>(out);
        cf.shared = static_cast<const uint16_t *>(sh_y);
        cf.residual = static_cast<const uint16_t *>(residual);
        cf.b2 = s->act == COLIBRI_ACT_SWIGLU ? nullptr : static_cast<const uint16_t *>(b2);
        if (e == hipSuccess) e = ffn(sorted, offsets, y, ffn_ws, false, &part, &cf);
        return hip_status(e);
    }
    e = Sd > 1 ? ffn(sorted, offsets, nullptr, ffn_ws, false, &part, nullptr)
               : ffn(sorted, offsets, y, ffn_ws, true, nullptr, nullptr);
    if (e == hipSuccess && branch) e = hipStreamWaitEvent(stream, br.join, 0);
    if (e != hipSuccess) return hip_status(e);
    if (Sd > 1)
        e = launch_combine_partials(*s, part, Sd, pos, idx, gate, s->act == COLIBRI_ACT_SWIGLU ? nullptr : b2, out,
                                    stream, sh_y, residual, shp);
    else
        e = launch_combine(*s, y, pos, gate, out, stream, sh_y, residual, shp);
    return hip_status(e);
}

constexpr int32_t kMaxLayers = 4096;

colibri_moe_layer_opts_t step_opts(const colibri_moe_layer_params_t &p, const void *residual) {
    colibri_moe_layer_opts_t o{};
    o.gate = p.gate;
    o.shared = p.shared;
    o.shared_h = p.shared_h;
    o.residual = residual;
    return o;
}

int check_step(const colibri_moe_shape_t *s, int32_t L, const colibri_moe_layer_params_t *layers) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (L < 1 || L > kMaxLayers) return COLIBRI_ERR_UNSUPPORTED;
    if (!layers) return COLIBRI_ERR_INVALID_ARG;
    for (int32_t l = 0; l < L; ++l) {
        const colibri_moe_layer_params_t &p = layers[l];
        if (!p.w_r || !aligned(p.w_r, 16) || (p.b_r && !aligned(p.b_r, 4))) return COLIBRI_ERR_INVALID_ARG;
        const colibri_moe_layer_opts_t o = step_opts(p, nullptr);
        st = check_opts(s, &o);
        if (st == COLIBRI_OK) st = check_experts(s, &p.experts);
        if (st != COLIBRI_OK) return st;
    }
    return COLIBRI_OK;
}

size_t step_workspace(const colibri_moe_shape_t *s, int32_t L, const colibri_moe_layer_params_t *layers) {
    size_t need = 0;
    for (int32_t l = 0; l < L; ++l) {
        const colibri_moe_layer_opts_t o = step_opts(layers[l], nullptr);
        need = std::max(need, layer_workspace(s, &o).total);
    }
    return need;
}

// One layer of a step, in place on x.
int step_layer(const colibri_moe_shape_t *s, const colibri_moe_layer_params_t &p, bool residual, void *x, void *ws,
               size_t ws_bytes, hipStream_t stream, const Branch &br) {
    const colibri_moe_layer_opts_t o = step_opts(p, residual ? x : nullptr);
    return layer_forward_impl(
        s, x, p.w_r, p.b_r, x, nullptr, nullptr, nullptr, ws, ws_bytes, stream, p.experts.b2, ffn_down_splits(*s),
        [&](const int32_t *sorted, const int32_t *offsets, void *y, void *ffn_ws, bool reduce, const float **part,
            const CombineFold *fold) {
            return launch_ffn_layers(*s, x, sorted, offsets, p.experts, y, ffn_ws, reduce, stream, part, fold);
        },
        [&](Validator &v) {
            v_experts(v, s, &p.experts);
            v.range(ws, ws_bytes);
        },
        &o, br);
}

int check_step_buffers(const colibri_moe_shape_t *s, int32_t L, const colibri_moe_layer_params_t *layers, void *x,
                       void *ws, size_t ws_bytes) {
    if (!x || !aligned(x, 16)) return COLIBRI_ERR_INVALID_ARG;
    if (ws_bytes < step_workspace(s, L, layers)) return COLIBRI_ERR_WORKSPACE;
    if (!ws || !aligned(ws, 256)) return COLIBRI_ERR_INVALID_ARG;
    return COLIBRI_OK;
}

// ------------------------------------------------------------------ allocation-free layer
// Workspace of colibri_moe_layer_forward_noalloc: a file-scope device array,
// one copy on every GPU the library runs on, kept until the process ends.  In
// host code `scratch` only names the symbol; its device address on the
// current GPU comes from hipGetSymbolAddress, looked up once per device and
// cached below, and only that address is ever handed to a kernel.
static __device__ __align__(256) uint8_t scratch[COLIBRI_MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of the current GPU's copy of `scratch`.
int noalloc_scratch(void **ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return COLIBRI_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return COLIBRI_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr || !aligned(p, 256)) return COLIBRI_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return COLIBRI_OK;
}

}  // namespace

struct colibri_moe_graph {
    hipGraphExec_t exec;
    int device;
};

extern "C" {

size_t colibri_moe_workspace_size(const colibri_moe_shape_t *s) {
    if (check_shape(s) != COLIBRI_OK || s->T == 0) return 0;
    return layer_workspace(s).total;
}

int colibri_moe_workspace_layout(const colibri_moe_shape_t *s, colibri_moe_workspace_layout_t *layout) {
    if (!layout) return COLIBRI_ERR_INVALID_ARG;
    const int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_ERR_INVALID_ARG;
    // the routing and dispatch regions lead every layer workspace, whatever the options
    const LayerWorkspace L = layer_workspace(s);
    *layout = {L.idx, L.gate, L.counts, L.offsets, L.sorted, L.pos};
    return COLIBRI_OK;
}

int colibri_moe_route(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                      int32_t *topk_idx, float *topk_gate, float *logits, hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    if (!x || !w_r || !topk_idx || !topk_gate) return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w_r, 16) || !aligned(topk_idx, 4) || !aligned(topk_gate, 4) ||
        (b_r && !aligned(b_r, 4)) || (logits && !aligned(logits, 4)))
        return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled()) {
        Validator v(stream);
        v_router(v, s, x, w_r, b_r);
        v.range(topk_idx, 2 * (size_t)s->T * 4).range(topk_gate, 2 * (size_t)s->T * 4);
        v.range(logits, (size_t)s->T * s->E * 4);
        if (v.status() != COLIBRI_OK) return v.status();
    }
    return hip_status(launch_route(*s, x, w_r, b_r, topk_idx, topk_gate, logits, stream));
}

size_t colibri_moe_dispatch_workspace_size(const colibri_moe_shape_t *s) {
    if (check_shape(s) != COLIBRI_OK || s->T == 0) return 0;
    return dispatch_scratch_bytes(*s);
}

int colibri_moe_dispatch(const colibri_moe_shape_t *s, const int32_t *topk_idx, int32_t *expert_counts,
                         int32_t *expert_offsets, int32_t *sorted_assign, int32_t *assign_pos, const void *x,
                         void *x_sorted, void *ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    if (!topk_idx || !expert_counts || !expert_offsets || !sorted_assign || !assign_pos)
        return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(topk_idx, 4) || !aligned(expert_counts, 4) || !aligned(expert_offsets, 4) ||
        !aligned(sorted_assign, 4) || !aligned(assign_pos, 4))
        return COLIBRI_ERR_INVALID_ARG;
    if ((x == nullptr) != (x_sorted == nullptr)) return COLIBRI_ERR_INVALID_ARG;
    if (x && (!aligned(x, 16) || !aligned(x_sorted, 16))) return COLIBRI_ERR_INVALID_ARG;
    const size_t dneed = dispatch_scratch_bytes(*s);
    void *dws = (dneed && ws && ws_bytes >= dneed && aligned(ws, 256)) ? ws : nullptr;
    if (validate_enabled()) {
        Validator v(stream);
        const size_t A = 2 * (size_t)s->T;
        v.indices(topk_idx, A, 0, s->E - 1);  // the input contract: every index in [0, E)
        v.range(expert_counts, (size_t)s->E * 4).range(expert_offsets, (size_t)(s->E + 1) * 4);
        v.range(sorted_assign, A * 4).range(assign_pos, A * 4).range(dws, dneed);
        v.range(x, (size_t)s->T * s->d * elem_size(s)).range(x_sorted, A * s->d * elem_size(s));
        if (v.status() != COLIBRI_OK) return v.status();
    }
    hipError_t e =
        launch_dispatch(*s, topk_idx, expert_counts, expert_offsets, sorted_assign, assign_pos, stream, dws);
    if (e == hipSuccess && x) e = launch_gather_rows(*s, x, sorted_assign, x_sorted, stream);
    return hip_status(e);
}

int colibri_moe_expert_ffn(const colibri_moe_shape_t *s, const void *x_rows, const int32_t *sorted_assign,
                           const int32_t *expert_offsets, const colibri_moe_experts_t *w, void *y_sorted, void *ws,
                           size_t ws_bytes, hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    st = check_experts(s, w);
    if (st != COLIBRI_OK) return st;
    if (!x_rows || !expert_offsets || !y_sorted) return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(x_rows, 16) || !aligned(y_sorted, 16) || !aligned(expert_offsets, 4) ||
        (sorted_assign && !aligned(sorted_assign, 4)))
        return COLIBRI_ERR_INVALID_ARG;
    const size_t need = ffn_workspace_bytes(*s);
    if (ws_bytes < need) return COLIBRI_ERR_WORKSPACE;
    if (!ws || !aligned(ws, 256)) return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled()) {
        Validator v(stream);
        v_ffn_rows(v, s, x_rows, sorted_assign, expert_offsets, s->d);
        v_experts(v, s, w);
        v.range(y_sorted, 2 * (size_t)s->T * s->d * elem_size(s)).range(ws, ws_bytes);
        if (v.status() != COLIBRI_OK) return v.status();
    }
    return hip_status(launch_expert_ffn(*s, x_rows, sorted_assign, expert_offsets, *w, y_sorted, ws, stream));
}

int colibri_moe_expert_ffn_up(const colibri_moe_shape_t *s, const void *x_rows, const int32_t *sorted_assign,
                              const int32_t *expert_offsets, const colibri_moe_experts_t *w, void *h_rows, void *ws,
                              size_t ws_bytes, hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    st = check_experts(s, w, true, false);
    if (st != COLIBRI_OK) return st;
    if (!x_rows || !expert_offsets || !h_rows) return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(x_rows, 16) || !aligned(h_rows, 16) || !aligned(expert_offsets, 4) ||
        (sorted_assign && !aligned(sorted_assign, 4)))
        return COLIBRI_ERR_INVALID_ARG;
    const size_t need = ffn_up_scratch_bytes(*s);
    if (ws_bytes < need) return COLIBRI_ERR_WORKSPACE;
    if (need && (!ws || !aligned(ws, 256))) return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled()) {
        Validator v(stream);
        v_ffn_rows(v, s, x_rows, sorted_assign, expert_offsets, s->d);
        v_experts(v, s, w, true, false);
        v.range(h_rows, 2 * (size_t)s->T * s->h * elem_size(s)).range(need ? ws : nullptr, ws_bytes);
        if (v.status() != COLIBRI_OK) return v.status();
    }
    return hip_status(launch_ffn_up(*s, x_rows, sorted_assign, expert_offsets, *w, h_rows, ws, stream));
}

int colibri_moe_expert_ffn_down(const colibri_moe_shape_t *s, const void *h_rows, const int32_t *expert_offsets,
                                const colibri_moe_experts_t *w, void *y_sorted, void *ws, size_t ws_bytes,
                                hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    st = check_experts(s, w, false, true);
    if (st != COLIBRI_OK) return st;
    if (!h_rows || !expert_offsets || !y_sorted) return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(h_rows, 16) || !aligned(y_sorted, 16) || !aligned(expert_offsets, 4)) return COLIBRI_ERR_INVALID_ARG;
    const size_t need = ffn_down_scratch_bytes(*s);
    if (ws_bytes < need) return COLIBRI_ERR_WORKSPACE;
    if (need && (!ws || !aligned(ws, 256))) return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled()) {
        Validator v(stream);
        v_ffn_rows(v, s, h_rows, nullptr, expert_offsets, s->h);
        v_experts(v, s, w, false, true);
        v.range(y_sorted, 2 * (size_t)s->T * s->d * elem_size(s)).range(need ? ws : nullptr, ws_bytes);
        if (v.status() != COLIBRI_OK) return v.status();
    }
    return hip_status(launch_ffn_down(*s, h_rows, expert_offsets, *w, y_sorted, ws, stream));
}

int colibri_moe_combine(const colibri_moe_shape_t *s, const void *y_sorted, const int32_t *assign_pos,
                        const float *topk_gate, void *out, hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    if (!y_sorted || !assign_pos || !topk_gate || !out) return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(y_sorted, 16) || !aligned(out, 16) || !aligned(assign_pos, 4) || !aligned(topk_gate, 4))
        return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled()) {
        Validator v(stream);
        const size_t A = 2 * (size_t)s->T;
        v.finite(y_sorted, A * s->d, s->dtype).indices(assign_pos, A, -1, (int32_t)A - 1);
        v.finite(topk_gate, A, COLIBRI_F32).range(out, (size_t)s->T * s->d * elem_size(s));
        if (v.status() != COLIBRI_OK) return v.status();
    }
    return hip_status(launch_combine(*s, y_sorted, assign_pos, topk_gate, out, stream));
}

int colibri_moe_layer_forward(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                              const colibri_moe_experts_t *w, void *out, int32_t *topk_idx_out, float *topk_gate_out,
                              int32_t *expert_counts_out, void *ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    st = check_experts(s, w);
    if (st != COLIBRI_OK) return st;
    return layer_forward_impl(s, x, w_r, b_r, out, topk_idx_out, topk_gate_out, expert_counts_out, ws, ws_bytes,
                              stream, w->b2, ffn_down_splits(*s),
                              [&](const int32_t *sorted, const int32_t *offsets, void *y, void *ffn_ws, bool reduce,
                                  const float **part, const CombineFold *fold) {
                                  return launch_ffn_layers(*s, x, sorted, offsets, *w, y, ffn_ws, reduce, stream,
                                                           part, fold);
                              },
                              [&](Validator &v) {
                                  v_experts(v, s, w);
                                  v.range(ws, ws_bytes);
                              });
}

int colibri_moe_layer_forward_noalloc(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                                      const colibri_moe_experts_t *w, void *out, int32_t *topk_idx_out,
                                      float *topk_gate_out, int32_t *expert_counts_out, hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    st = check_experts(s, w);
    if (st != COLIBRI_OK) return st;
    st = check_layer_io(x, w_r, b_r, out, topk_idx_out, topk_gate_out, expert_counts_out);
    if (st != COLIBRI_OK) return st;
    if (layer_workspace(s).total > (size_t)COLIBRI_MOE_NOALLOC_SCRATCH_BYTES) return COLIBRI_ERR_WORKSPACE;
    void *ws = nullptr;
    st = noalloc_scratch(&ws);
    if (st != COLIBRI_OK) return st;
    // the same launch sequence as colibri_moe_layer_forward, on the device array
    return layer_forward_impl(s, x, w_r, b_r, out, topk_idx_out, topk_gate_out, expert_counts_out, ws,
                              (size_t)COLIBRI_MOE_NOALLOC_SCRATCH_BYTES, stream, w->b2, ffn_down_splits(*s),
                              [&](const int32_t *sorted, const int32_t *offsets, void *y, void *ffn_ws, bool reduce,
                                  const float **part, const CombineFold *fold) {
                                  return launch_ffn_layers(*s, x, sorted, offsets, *w, y, ffn_ws, reduce, stream,
                                                           part, fold);
                              },
                              [&](Validator &v) { v_experts(v, s, w); });
}

int colibri_moe_layer_forward_q8(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                                 const colibri_moe_experts_q8_t *w, void *out, int32_t *topk_idx_out,
                                 float *topk_gate_out, int32_t *expert_counts_out, void *ws, size_t ws_bytes,
                                 hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    st = check_experts_q8(s, w);
    if (st != COLIBRI_OK) return st;
    return layer_forward_impl(s, x, w_r, b_r, out, topk_idx_out, topk_gate_out, expert_counts_out, ws, ws_bytes,
                              stream, w->b2, ffn_down_splits(*s, true),
                              [&](const int32_t *sorted, const int32_t *offsets, void *y, void *ffn_ws, bool reduce,
                                  const float **part, const CombineFold *fold) {
                                  if (fold) return hipErrorInvalidValue;  // decode sizes only: never folded
                                  return launch_ffn_layers_q8(*s, x, sorted, offsets, *w, y, ffn_ws, reduce, stream,
                                                              part);
                              },
                              [&](Validator &v) {
                                  v_experts_q8(v, s, w);
                                  v.range(ws, ws_bytes);
                              });
}

int colibri_moe_expert_ffn_q8(const colibri_moe_shape_t *s, const void *x_rows, const int32_t *sorted_assign,
                              const int32_t *expert_offsets, const colibri_moe_experts_q8_t *w, void *y_sorted,
                              void *ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    st = check_experts_q8(s, w);
    if (st != COLIBRI_OK) return st;
    if (!x_rows || !expert_offsets || !y_sorted) return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(x_rows, 16) || !aligned(y_sorted, 16) || !aligned(expert_offsets, 4) ||
        (sorted_assign && !aligned(sorted_assign, 4)))
        return COLIBRI_ERR_INVALID_ARG;
    const size_t need = ffn_workspace_bytes(*s);
    if (ws_bytes < need) return COLIBRI_ERR_WORKSPACE;
    if (!ws || !aligned(ws, 256)) return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled()) {
        Validator v(stream);
        v_ffn_rows(v, s, x_rows, sorted_assign, expert_offsets, s->d);
        v_experts_q8(v, s, w);
        v.range(y_sorted, 2 * (size_t)s->T * s->d * elem_size(s)).range(ws, ws_bytes);
        if (v.status() != COLIBRI_OK) return v.status();
    }
    return hip_status(
        launch_ffn_layers_q8(*s, x_rows, sorted_assign, expert_offsets, *w, y_sorted, ws, true, stream, nullptr));
}

int colibri_moe_quantize_q8(const void *w, colibri_dtype_t dtype, int32_t E, int32_t K, int32_t N, int8_t *q,
                            float *scale, hipStream_t stream) {
    if (!w || !q || !scale) return COLIBRI_ERR_INVALID_ARG;
    if (dtype != COLIBRI_F32 && dtype != COLIBRI_BF16) return COLIBRI_ERR_UNSUPPORTED;
    if (E < 1 || K < 1 || N < 1 || N % 4) return COLIBRI_ERR_UNSUPPORTED;
    if ((int64_t)E * K * N > ((int64_t)1 << 40)) return COLIBRI_ERR_UNSUPPORTED;
    if (!aligned(w, 16) || !aligned(q, 4) || !aligned(scale, 4)) return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled()) {
        Validator v(stream);
        const size_t n = (size_t)E * K * N;
        v.finite(w, n, dtype).range(q, n).range(scale, (size_t)E * N * 4);
        if (v.status() != COLIBRI_OK) return v.status();
    }
    return hip_status(launch_quantize_q8(w, dtype, E, K, N, q, scale, stream));
}

int colibri_moe_quantize_q4(const void *w, colibri_dtype_t dtype, int32_t E, int32_t K, int32_t N, uint32_t *q,
                            float *scale, uint8_t *zero, hipStream_t stream) {
    if (!w || !q || !scale || !zero) return COLIBRI_ERR_INVALID_ARG;
    if (dtype != COLIBRI_F32 && dtype != COLIBRI_BF16) return COLIBRI_ERR_UNSUPPORTED;
    if (E < 1 || K < 128 || K % 128 || N < 1 || N % 4) return COLIBRI_ERR_UNSUPPORTED;
    if ((int64_t)E * K * N > ((int64_t)1 << 40)) return COLIBRI_ERR_UNSUPPORTED;
    if (!aligned(w, 16) || !aligned(q, 16) || !aligned(scale, 16) || !aligned(zero, 4))
        return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled()) {
        Validator v(stream);
        const size_t n = (size_t)E * K * N;
        v.finite(w, n, dtype).range(q, n / 2).range(scale, n / 128 * 4).range(zero, n / 128);
        if (v.status() != COLIBRI_OK) return v.status();
    }
    return hip_status(launch_quantize_q4(w, dtype, E, K, N, q, scale, zero, stream));
}

int colibri_moe_layer_forward_q4(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                                 const colibri_moe_experts_q4_t *w, void *out, int32_t *topk_idx_out,
                                 float *topk_gate_out, int32_t *expert_counts_out, void *ws, size_t ws_bytes,
                                 hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    st = check_experts_q4(s, w);
    if (st != COLIBRI_OK) return st;
    return layer_forward_impl(s, x, w_r, b_r, out, topk_idx_out, topk_gate_out, expert_counts_out, ws, ws_bytes,
                              stream, w->b2, ffn_down_splits_q4(*s),
                              [&](const int32_t *sorted, const int32_t *offsets, void *y, void *ffn_ws, bool reduce,
                                  const float **part, const CombineFold *fold) {
                                  if (fold) return hipErrorInvalidValue;  // decode sizes only: never folded
                                  return launch_ffn_layers_q4(*s, x, sorted, offsets, *w, y, ffn_ws, reduce, stream,
                                                              part);
                              },
                              [&](Validator &v) {
                                  v_experts_q4(v, s, w);
                                  v.range(ws, ws_bytes);
                              });
}

int colibri_moe_expert_ffn_q4(const colibri_moe_shape_t *s, const void *x_rows, const int32_t *sorted_assign,
                              const int32_t *expert_offsets, const colibri_moe_experts_q4_t *w, void *y_sorted,
                              void *ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    st = check_experts_q4(s, w);
    if (st != COLIBRI_OK) return st;
    if (!x_rows || !expert_offsets || !y_sorted) return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(x_rows, 16) || !aligned(y_sorted, 16) || !aligned(expert_offsets, 4) ||
        (sorted_assign && !aligned(sorted_assign, 4)))
        return COLIBRI_ERR_INVALID_ARG;
    const size_t need = ffn_workspace_bytes(*s);
    if (ws_bytes < need) return COLIBRI_ERR_WORKSPACE;
    if (!ws || !aligned(ws, 256)) return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled()) {
        Validator v(stream);
        v_ffn_rows(v, s, x_rows, sorted_assign, expert_offsets, s->d);
        v_experts_q4(v, s, w);
        v.range(y_sorted, 2 * (size_t)s->T * s->d * elem_size(s)).range(ws, ws_bytes);
        if (v.status() != COLIBRI_OK) return v.status();
    }
    return hip_status(
        launch_ffn_layers_q4(*s, x_rows, sorted_assign, expert_offsets, *w, y_sorted, ws, true, stream, nullptr));
}

size_t colibri_moe_workspace_size_ex(const colibri_moe_shape_t *s, const colibri_moe_layer_opts_t *opts) {
    if (check_shape(s) != COLIBRI_OK || s->T == 0 || check_opts(s, opts) != COLIBRI_OK) return 0;
    return layer_workspace(s, opts).total;
}

int colibri_moe_route_ex(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                         colibri_gate_t gate, int32_t *topk_idx, float *topk_gate, float *logits, hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (gate != COLIBRI_GATE_PAIR && gate != COLIBRI_GATE_SOFTMAX && gate != COLIBRI_GATE_LINEAR)
        return COLIBRI_ERR_UNSUPPORTED;
    if (s->T == 0) return COLIBRI_OK;
    if (!x || !w_r || !topk_idx || !topk_gate) return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(w_r, 16) || !aligned(topk_idx, 4) || !aligned(topk_gate, 4) ||
        (b_r && !aligned(b_r, 4)) || (logits && !aligned(logits, 4)))
        return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled()) {
        Validator v(stream);
        v_router(v, s, x, w_r, b_r);
        v.range(topk_idx, 2 * (size_t)s->T * 4).range(topk_gate, 2 * (size_t)s->T * 4);
        v.range(logits, (size_t)s->T * s->E * 4);
        if (v.status() != COLIBRI_OK) return v.status();
    }
    return hip_status(launch_route(*s, x, w_r, b_r, topk_idx, topk_gate, logits, stream, gate));
}

int colibri_moe_combine_ex(const colibri_moe_shape_t *s, const void *y_sorted, const int32_t *assign_pos,
                           const float *topk_gate, const void *shared_y, const void *residual, void *out,
                           hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    if (!y_sorted || !assign_pos || !topk_gate || !out) return COLIBRI_ERR_INVALID_ARG;
    if (!aligned(y_sorted, 16) || !aligned(out, 16) || !aligned(assign_pos, 4) || !aligned(topk_gate, 4) ||
        (shared_y && !aligned(shared_y, 16)) || (residual && !aligned(residual, 16)))
        return COLIBRI_ERR_INVALID_ARG;
    if (validate_enabled()) {
        Validator v(stream);
        const size_t A = 2 * (size_t)s->T;
        v.finite(y_sorted, A * s->d, s->dtype).indices(assign_pos, A, -1, (int32_t)A - 1);
        v.finite(topk_gate, A, COLIBRI_F32).range(out, (size_t)s->T * s->d * elem_size(s));
        v.finite(shared_y, (size_t)s->T * s->d, s->dtype).finite(residual, (size_t)s->T * s->d, s->dtype);
        if (v.status() != COLIBRI_OK) return v.status();
    }
    return hip_status(launch_combine(*s, y_sorted, assign_pos, topk_gate, out, stream, shared_y, residual));
}

int colibri_moe_layer_forward_ex(const colibri_moe_shape_t *s, const void *x, const void *w_r, const float *b_r,
                                 const colibri_moe_experts_t *w, const colibri_moe_layer_opts_t *opts, void *out,
                                 int32_t *topk_idx_out, float *topk_gate_out, int32_t *expert_counts_out, void *ws,
                                 size_t ws_bytes, hipStream_t stream) {
    int st = check_shape(s);
    if (st != COLIBRI_OK) return st;
    st = check_opts(s, opts);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    st = check_experts(s, w);
    if (st != COLIBRI_OK) return st;
    return layer_forward_impl(
        s, x, w_r, b_r, out, topk_idx_out, topk_gate_out, expert_counts_out, ws, ws_bytes, stream, w->b2,
        ffn_down_splits(*s),
        [&](const int32_t *sorted, const int32_t *offsets, void *y, void *ffn_ws, bool reduce, const float **part,
            const CombineFold *fold) {
            return launch_ffn_layers(*s, x, sorted, offsets, *w, y, ffn_ws, reduce, stream, part, fold);
        },
        [&](Validator &v) {
            v_experts(v, s, w);
            v.range(ws, ws_bytes);
        },
        opts);
}

size_t colibri_moe_step_workspace_size(const colibri_moe_shape_t *s, int32_t L,
                                       const colibri_moe_layer_params_t *layers) {
    if (check_step(s, L, layers) != COLIBRI_OK || s->T == 0) return 0;
    return step_workspace(s, L, layers);
}

int colibri_moe_step_forward(const colibri_moe_shape_t *s, int32_t L, const colibri_moe_layer_params_t *layers,
                             int32_t residual, void *x, void *ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_step(s, L, layers);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_OK;
    st = check_step_buffers(s, L, layers, x, ws, ws_bytes);
    for (int32_t l = 0; l < L && st == COLIBRI_OK; ++l)
        st = step_layer(s, layers[l], residual != 0, x, ws, ws_bytes, stream, Branch{});
    return st;
}

int colibri_moe_graph_create(const colibri_moe_shape_t *s, int32_t L, const colibri_moe_layer_params_t *layers,
                             int32_t residual, void *x, void *ws, size_t ws_bytes, colibri_moe_graph_t **graph) {
    if (!graph) return COLIBRI_ERR_INVALID_ARG;
    *graph = nullptr;
    int st = check_step(s, L, layers);
    if (st != COLIBRI_OK) return st;
    if (s->T == 0) return COLIBRI_ERR_UNSUPPORTED;
    st = check_step_buffers(s, L, layers, x, ws, ws_bytes);
    if (st != COLIBRI_OK) return st;
    if (validate_enabled()) {  // once here: a stream under capture cannot be waited on
        Validator v(nullptr);
        v.finite(x, (size_t)s->T * s->d, s->dtype).range(ws, ws_bytes);
        for (int32_t l = 0; l < L; ++l) {
            const colibri_moe_layer_params_t &p = layers[l];
            v.finite(p.w_r, (size_t)s->d * s->E, s->dtype).finite(p.b_r, (size_t)s->E, COLIBRI_F32);
            v_experts(v, s, &p.experts);
            const colibri_moe_layer_opts_t o = step_opts(p, nullptr);
            v_opts(v, s, &o);
        }
        if (v.status() != COLIBRI_OK) return v.status();
    }

    int device = 0;
    if (hipGetDevice(&device) != hipSuccess) return COLIBRI_ERR_HIP;
    // a capture stream of our own (the caller's may be the null stream, which
    // cannot be captured) and the shared experts' branch
    hipStream_t cs = nullptr, aux = nullptr;
    Branch br;
    hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&aux, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&br.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&br.join, hipEventDisableTiming);
    br.aux = aux;
    hipGraph_t g = nullptr;
    hipGraphExec_t exec = nullptr;
    // A few tokens (T <= 8): both the shared and the routed FFN split K until
    // each alone fills the chip, and side by side they only contend (measured
    // on the 15 + 1 shared layer at T = 1: 458 us for 8 layers with the branch,
    // 432 without); from there on the branch pays (T = 64: 977 against 1180).
    const Branch use = s->T > 8 ? br : Branch{};
    if (e == hipSuccess) e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e == hipSuccess) {
        for (int32_t l = 0; l < L && st == COLIBRI_OK; ++l)
            st = step_layer(s, layers[l], residual != 0, x, ws, ws_bytes, cs, use);
        const hipError_t ce = hipStreamEndCapture(cs, &g);  // always ends the capture
        if (st == COLIBRI_OK && ce != hipSuccess) e = ce;
        if (st == COLIBRI_OK && e == hipSuccess) e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    }
    if (g) (void)hipGraphDestroy(g);
    if (br.join) (void)hipEventDestroy(br.join);
    if (br.fork) (void)hipEventDestroy(br.fork);
    if (aux) (void)hipStreamDestroy(aux);
    if (cs) (void)hipStreamDestroy(cs);
    if (st == COLIBRI_OK && e != hipSuccess) st = COLIBRI_ERR_HIP;
    if (st != COLIBRI_OK) {
        if (exec) (void)hipGraphExecDestroy(exec);
        return st;
    }
    colibri_moe_graph_t *gr = new (std::nothrow) colibri_moe_graph_t{exec, device};
    if (!gr) {
        (void)hipGraphExecDestroy(exec);
        return COLIBRI_ERR_HIP;
    }
    *graph = gr;
    return COLIBRI_OK;
}

int colibri_moe_graph_launch(colibri_moe_graph_t *graph, hipStream_t stream) {
    if (!graph || !graph->exec) return COLIBRI_ERR_INVALID_ARG;
    int device = -1;
    if (hipGetDevice(&device) != hipSuccess) return COLIBRI_ERR_HIP;
    if (device != graph->device) return COLIBRI_ERR_INVALID_ARG;
    return hip_status(hipGraphLaunch(graph->exec, stream));
}

int colibri_moe_graph_destroy(colibri_moe_graph_t *graph) {
    if (!graph) return COLIBRI_OK;
    const hipError_t e = graph->exec ? hipGraphExecDestroy(graph->exec) : hipSuccess;
    delete graph;
    return hip_status(e);
}

const char *colibri_moe_status_string(int status) {
    switch (status) {
        case COLIBRI_OK: return "ok";
        case COLIBRI_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, negative T)";
        case COLIBRI_ERR_WORKSPACE: return "workspace too small";
        case COLIBRI_ERR_UNSUPPORTED: return "unsupported shape or configuration";
        case COLIBRI_ERR_HIP: return "HIP launch error";
        default: return "unknown status";
    }
}

}  // extern "C"
