// Plain fp64 CPU oracle of the Colibri MoE layer forward pass.
//
// TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
// reference that the GPU path is checked against.  Only the test suite, the
// smoke check and the benchmark's CPU-baseline leg may load it; the product
// library never links or calls it, and it shares no code, header or table
// with the HIP path.
//
// Pages cited (Colibri write-ups; each page is named by its address):
//   [zskr]  http://www.zskr.cn/news/2272131   "Colibri: a lightweight C MoE inference engine for edge devices"
//   [rkmt]  http://news.rkmt.cn/news/2271114
//   [hnwysp] https://www.hnwysp.cn/news/30485
//   [nxbn]  http://m.nxbn.cn/news/48047
//
// Every value is widened exactly to double (fp32 and bf16 are subsets of
// fp64) and every sum is taken in double, in the order stated at each step.
// Conversions to fp32/bf16 round to nearest, ties to even.
//
// Readings of points the pages leave open (listed in full in the design notes):
//  * gate weights are the softmax over all E renormalised over the chosen two
//    ([hnwysp] section 3.1 takes softmax then the top-k; the verbose log in
//    [hnwysp] section 4.3 prints gate pairs that sum to one);
//  * selection ranks the raw logits (softmax is monotone; [zskr] section 2.3
//    LINEAR_SCORE mode ranks logits) under the total order
//    (logit descending, expert index ascending); NaN ranks below -inf;
//  * tokens inside an expert's segment keep ascending assignment order
//    a = 2t + s, the order of the counting loop in [zskr] section 3.2;
//  * expert = two-layer FFN (ReLU / exact-erf GELU, or SwiGLU with W1, W3, W2);
//  * the other gatings: DeepSeek-MoE's softmax top-2 ([rkmt] section 5.2)
//    keeps the two softmax probabilities as they are; LINEAR_SCORE ([zskr]
//    section 2.3) weights the outputs by the raw logits;
//  * a shared expert ([rkmt] section 5.2) sees every token and adds its
//    output with weight one; a residual row ([nxbn] section 2.1) is added last;
//  * 4-bit weights ([rkmt] section 4.2, AWQ with zero point, group 128): the
//    groups run along the input channels, and the codes come from AWQ's
//    closing min-max rounding (its activation-aware scale search needs
//    calibration data and is not part of the stored format).
//
// Parity is pinned by the CPU tests (brute-force top-2, exhaustive tie
// patterns, the page's printed gate pairs, a hand-worked dispatch, library
// matmuls, and whole-layer invariants).

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>
#ifdef _OPENMP
#include <omp.h>
#endif

namespace {

enum { DT_F32 = 0, DT_BF16 = 1 };
enum { ACT_RELU = 0, ACT_GELU = 1, ACT_SWIGLU = 2 };

inline double widen_bf16(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return (double)f;
}

inline double load(const void *p, int dt, size_t i) {
    if (dt == DT_F32) return (double)((const float *)p)[i];
    return widen_bf16(((const uint16_t *)p)[i]);
}

// Round a double to the nearest value with `mant` explicit mantissa bits and
// the fp32 exponent range (fp32: 23, bf16: 7), ties to even.  Subnormals keep
// a fixed quantum of 2^(-126-mant).  Overflow goes to +-inf.
double round_to_format(double v, int mant) {
    if (!std::isfinite(v) || v == 0.0) return v;
    int e = std::ilogb(v);
    if (e < -126) e = -126;
    double q = std::ldexp(1.0, e - mant);
    double r = std::nearbyint(v / q) * q;  // default rounding mode: nearest-even
    if (std::fabs(r) >= std::ldexp(1.0, 128)) r = std::copysign(INFINITY, v);
    return r;
}

double round_to_dtype(double v, int dt) { return round_to_format(v, dt == DT_F32 ? 23 : 7); }

// Total order used for expert selection: a beats b when its logit is larger,
// or equal with a smaller index.  NaN ranks below every number.
bool beats(double la, int a, double lb, int b) {
    bool na = std::isnan(la), nb = std::isnan(lb);
    if (na != nb) return nb;          // the non-NaN one wins
    if (!na && la != lb) return la > lb;
    return a < b;
}

double act_relu(double z) { return z > 0.0 ? z : 0.0; }
double act_gelu(double z) { return 0.5 * z * (1.0 + std::erf(z / std::sqrt(2.0))); }
double act_silu(double z) { return z / (1.0 + std::exp(-z)); }

// Step 5, shared by the bf16/fp32 and the int8-weight FFN: the hidden row
// from the first layer's sums u (and v for SwiGLU), and the output row from H
// and the second layer's weights w2at(j, c).
void hidden_row(int h, int act, int mirror, int dt, int e, const std::vector<double> &u,
                const std::vector<double> &v, const void *b1, std::vector<double> &H) {
    for (int j = 0; j < h; ++j) {
        double hv;
        if (act == ACT_SWIGLU) {
            hv = act_silu(u[j]) * v[j];
        } else {
            double z = u[j] + (b1 ? load(b1, dt, (size_t)e * h + j) : 0.0);
            hv = (act == ACT_RELU) ? act_relu(z) : act_gelu(z);
        }
        H[j] = mirror ? round_to_dtype(hv, dt) : hv;
    }
}

template <class W2At>
void output_row(int h, int d, int act, int mirror, int dt, int e, const std::vector<double> &H, W2At w2at,
                const void *b2, std::vector<double> &y, double *yo) {
    std::fill(y.begin(), y.end(), 0.0);
    for (int j = 0; j < h; ++j) {
        const double hj = H[j];
        for (int c = 0; c < d; ++c) y[c] += hj * w2at(j, c);
    }
    for (int c = 0; c < d; ++c) {
        double yv = y[c] + ((act != ACT_SWIGLU && b2) ? load(b2, dt, (size_t)e * d + c) : 0.0);
        yo[c] = mirror ? round_to_dtype(yv, dt) : yv;
    }
}

}  // namespace

extern "C" {

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

// Step 1, router logits ([zskr] section 3.2, first step of the routing chain:
// logits = input x routing weights, no softmax yet; [rkmt] section 3.1 stores a
// router bias [E] beside the router weight):
//   logits[t,e] = (sum_{j ascending} x[t,j] * w_r[j,e]) + b_r[e]
// x [T,d], w_r [d,E] row-major in dtype `dt`; b_r [E] fp32 or NULL (= 0).
void oracle_logits(int T, int d, int E, int dt, const void *x, const void *w_r, const float *b_r,
                   double *logits) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) {
            double s = 0.0;
            for (int j = 0; j < d; ++j)
                s += load(x, dt, (size_t)t * d + j) * load(w_r, dt, (size_t)j * E + e);
            logits[(size_t)t * E + e] = s + (b_r ? (double)b_r[e] : 0.0);
        }
    }
}

// Step 2, deterministic top-2 ([zskr] section 3.2: a fixed comparison network,
// so the selected sequence is deterministic; [hnwysp] section 3.1: the top-k
// indices come out strictly descending by score).  Slot 0 holds the winner of
// the total order, slot 1 the winner among the rest.
void oracle_top2(int T, int E, const double *logits, int32_t *idx) {
    for (int t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        int i0 = 0;
        for (int e = 1; e < E; ++e)
            if (beats(l[e], e, l[i0], i0)) i0 = e;
        int i1 = -1;
        for (int e = 0; e < E; ++e) {
            if (e == i0) continue;
            if (i1 < 0 || beats(l[e], e, l[i1], i1)) i1 = e;
        }
        idx[2 * t] = i0;
        idx[2 * t + 1] = i1;
    }
}

// Step 3, gate weights: softmax over all E experts ([hnwysp] section 3.1),
// then the two chosen probabilities renormalised to sum to one (the gate pairs
// printed in [hnwysp] section 4.3 sum to one).
void oracle_gates(int T, int E, const double *logits, const int32_t *idx, double *gate) {
    std::vector<double> p(E);
    for (int t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        double m = -INFINITY;
        for (int e = 0; e < E; ++e) m = std::max(m, l[e]);
        double z = 0.0;
        for (int e = 0; e < E; ++e) {
            p[e] = std::exp(l[e] - m);
            z += p[e];
        }
        for (int e = 0; e < E; ++e) p[e] /= z;
        double p0 = p[idx[2 * t]], p1 = p[idx[2 * t + 1]];
        gate[2 * t] = p0 / (p0 + p1);
        gate[2 * t + 1] = p1 / (p0 + p1);
    }
}

// Step 3 with a choice of gating (the selection of step 2 is the same in
// every mode):
//   mode 0: the pair softmax above;
//   mode 1: softmax over all E experts, the chosen two taken as they are, not
//           renormalised (the DeepSeek-MoE softmax top-2 router of [rkmt]
//           section 5.2: softmax over every expert, then the top two):
//           gate[s] = exp(l[idx_s]) / sum_e exp(l[e]);
//   mode 2: no softmax, each chosen logit weights its expert's output
//           (the LINEAR_SCORE mode of [zskr] section 2.3): gate[s] = l[idx_s].
void oracle_gates_mode(int T, int E, int mode, const double *logits, const int32_t *idx, double *gate) {
    if (mode == 0) {
        oracle_gates(T, E, logits, idx, gate);
        return;
    }
    for (int t = 0; t < T; ++t) {
        const double *l = logits + (size_t)t * E;
        if (mode == 2) {
            gate[2 * t] = l[idx[2 * t]];
            gate[2 * t + 1] = l[idx[2 * t + 1]];
            continue;
        }
        double m = -INFINITY;
        for (int e = 0; e < E; ++e) m = std::max(m, l[e]);
        double z = 0.0;
        for (int e = 0; e < E; ++e) z += std::exp(l[e] - m);
        gate[2 * t] = std::exp(l[idx[2 * t]] - m) / z;
        gate[2 * t + 1] = std::exp(l[idx[2 * t + 1]] - m) / z;
    }
}

// Step 4, dispatch ([zskr] section 3.2: count assignments per expert over
// i = t*k + s, then build dispatch offsets; [zskr] section 3.3: one contiguous
// region per expert).  Assignment a = 2t + s.
//   counts[e]   = #{a : idx[a] = e}
//   offsets[0]  = 0, offsets[e+1] = offsets[e] + counts[e]
//   sorted_assign lists the assignments of expert 0, then expert 1, ..., each
//   group in ascending a;  assign_pos[sorted_assign[p]] = p.
void oracle_dispatch(int T, int E, const int32_t *idx, int32_t *counts, int32_t *offsets,
                     int32_t *sorted_assign, int32_t *assign_pos) {
    const int A = 2 * T;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int a = 0; a < A; ++a) counts[idx[a]] += 1;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
    int p = 0;
    for (int e = 0; e < E; ++e)
        for (int a = 0; a < A; ++a)
            if (idx[a] == e) sorted_assign[p++] = a;
    for (int q = 0; q < A; ++q) assign_pos[sorted_assign[q]] = q;
}

// Step 5, one expert applied to one token row ([zskr] section 1 and [nxbn]
// section 3.1: each expert is a two-layer FFN stored W1 | b1 | W2 | b2;
// [hnwysp] section 3.2: each layer is an affine map):
//   relu/gelu: u = x W1[e] + b1[e];  H = act(u);        y = H W2[e] + b2[e]
//   swiglu:    u = x W1[e];  v = x W3[e];  H = silu(u) * v;  y = H W2[e]
// W1, W3 [E][d][h], W2 [E][h][d], b1 [E][h], b2 [E][d] (NULL = zero).
// Each sum runs over the contraction index in ascending order, then adds the
// bias.  mirror != 0: H is rounded to `dt` before the second product and y is
// rounded to `dt` (the GPU stores both in that type); mirror == 0: no rounding.
// Rows: for r in [0, nrows): token row_token[r] of x [*, d], expert row_expert[r].
// y_out [nrows, d] in double.
void oracle_ffn_rows(int d, int h, int dt, int act, int mirror, const void *x, int nrows,
                     const int32_t *row_token, const int32_t *row_expert, const void *w1,
                     const void *w3, const void *w2, const void *b1, const void *b2, double *y_out) {
#pragma omp parallel
    {
        std::vector<double> xr(d), u(h), v(h), H(h), y(d);
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < nrows; ++r) {
            const int t = row_token[r], e = row_expert[r];
            const size_t wdh = (size_t)e * d * h;
            for (int k = 0; k < d; ++k) xr[k] = load(x, dt, (size_t)t * d + k);
            std::fill(u.begin(), u.end(), 0.0);
            std::fill(v.begin(), v.end(), 0.0);
            for (int k = 0; k < d; ++k) {
                const double xk = xr[k];
                for (int j = 0; j < h; ++j) u[j] += xk * load(w1, dt, wdh + (size_t)k * h + j);
                if (act == ACT_SWIGLU)
                    for (int j = 0; j < h; ++j) v[j] += xk * load(w3, dt, wdh + (size_t)k * h + j);
            }
            hidden_row(h, act, mirror, dt, e, u, v, b1, H);
            const size_t whd = (size_t)e * h * d;
            output_row(h, d, act, mirror, dt, e, H, [&](int j, int c) { return load(w2, dt, whd + (size_t)j * d + c); },
                       b2, y, y_out + (size_t)r * d);
        }
    }
}

// Step 6, combine ([nxbn] section 3.3: the expert outputs are summed weighted by
// their gating scores):  out[t] = g[2t] * y[assign_pos[2t]] + g[2t+1] * y[assign_pos[2t+1]],
// in double, then rounded to `dt`.  y_sorted [2T, d] double, out [T, d] double.
// (oracle_combine_ex below with neither addend.)
void oracle_combine_ex(int T, int d, int dt, const double *y_sorted, const int32_t *assign_pos, const double *gate,
                       const double *shared_y, const void *residual, double *out);
void oracle_combine(int T, int d, int dt, const double *y_sorted, const int32_t *assign_pos,
                    const double *gate, double *out) {
    oracle_combine_ex(T, d, dt, y_sorted, assign_pos, gate, nullptr, nullptr, out);
}

// Step 6 with two optional addends: the output of a shared expert applied to
// every token with weight one ([rkmt] section 5.2: Qwen2-MoE runs one shared
// expert beside its routed ones) and a residual row ([nxbn] section 2.1: the
// residual add belongs to the expert computation):
//   out[t] = g[2t] y[assign_pos[2t]] + g[2t+1] y[assign_pos[2t+1]] + shared_y[t] + residual[t]
// in double, then rounded to `dt`.  shared_y [T, d] double or NULL;
// residual [T, d] in `dt` or NULL.
void oracle_combine_ex(int T, int d, int dt, const double *y_sorted, const int32_t *assign_pos, const double *gate,
                       const double *shared_y, const void *residual, double *out) {
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; ++t) {
        const double *y0 = y_sorted + (size_t)assign_pos[2 * t] * d;
        const double *y1 = y_sorted + (size_t)assign_pos[2 * t + 1] * d;
        for (int c = 0; c < d; ++c) {
            const size_t i = (size_t)t * d + c;
            double v = gate[2 * t] * y0[c] + gate[2 * t + 1] * y1[c];
            if (shared_y) v += shared_y[i];
            if (residual) v += load(residual, dt, i);
            out[i] = round_to_dtype(v, dt);
        }
    }
}

// The whole layer, steps 1-6 in order.  Every output array is required.
void oracle_layer(int T, int d, int h, int E, int dt, int act, int mirror, const void *x,
                  const void *w_r, const float *b_r, const void *w1, const void *w3, const void *w2,
                  const void *b1, const void *b2, double *logits, int32_t *idx, double *gate,
                  int32_t *counts, int32_t *offsets, int32_t *sorted_assign, int32_t *assign_pos,
                  double *y_sorted, double *out) {
    oracle_logits(T, d, E, dt, x, w_r, b_r, logits);
    oracle_top2(T, E, logits, idx);
    oracle_gates(T, E, logits, idx, gate);
    oracle_dispatch(T, E, idx, counts, offsets, sorted_assign, assign_pos);
    std::vector<int32_t> rt(2 * (size_t)T), re(2 * (size_t)T);
    for (int p = 0; p < 2 * T; ++p) {
        rt[p] = sorted_assign[p] / 2;
        re[p] = idx[sorted_assign[p]];
    }
    oracle_ffn_rows(d, h, dt, act, mirror, x, 2 * T, rt.data(), re.data(), w1, w3, w2, b1, b2, y_sorted);
    oracle_combine(T, d, dt, y_sorted, assign_pos, gate, out);
}

// ---- int8 expert weights ([zskr] section 5.3: the expert weights are quantized
// to INT8 per channel, with their scales stored beside them).  A channel is an
// output column n of one expert; the scale is symmetric.

// Quantization of w [E][K][N] (dt), in fp32 as defined:
//   amax = max_k |w[e][k][n]|;  s[e][n] = amax / 127, or 1 when amax = 0;
//   q[e][k][n] = w / s rounded to nearest, ties to even, clamped to [-127, 127].
void oracle_quantize_q8(const void *w, int dt, int E, int K, int N, int8_t *q, float *scale) {
    // Work is split over (expert, block of 256 columns); inside a block the
    // rows are walked in order so that every read is contiguous.
    constexpr int NB = 256;
    const int nblk = (N + NB - 1) / NB;
#pragma omp parallel for schedule(dynamic, 1)
    for (long eb = 0; eb < (long)E * nblk; ++eb) {
        const int e = (int)(eb / nblk), n0 = (int)(eb % nblk) * NB, n1 = std::min(N, n0 + NB);
        const size_t base = (size_t)e * K * N;
        float amax[NB], sc[NB];
        for (int n = n0; n < n1; ++n) amax[n - n0] = 0.0f;
        for (int k = 0; k < K; ++k)
            for (int n = n0; n < n1; ++n) {
                const float a = std::fabs((float)load(w, dt, base + (size_t)k * N + n));
                if (a > amax[n - n0]) amax[n - n0] = a;
            }
        for (int n = n0; n < n1; ++n) {
            sc[n - n0] = amax[n - n0] > 0.0f ? amax[n - n0] / 127.0f : 1.0f;
            scale[(size_t)e * N + n] = sc[n - n0];
        }
        for (int k = 0; k < K; ++k)
            for (int n = n0; n < n1; ++n) {
                const size_t i = base + (size_t)k * N + n;
                float r = std::nearbyint((float)load(w, dt, i) / sc[n - n0]);  // default mode: ties to even
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                q[i] = (int8_t)r;
            }
    }
}

// Step 5 with int8 expert weights: the same two-layer FFN on the dequantized
// weights W[k][n] = s[n] * q[k][n], each formed exactly in double.
//   q1, q3 [E][d][h] with s1, s3 [E][h];  q2 [E][h][d] with s2 [E][d];
//   x, b1, b2 and the rounding of H and y in the storage type dt.
void oracle_ffn_rows_q8(int d, int h, int dt, int act, int mirror, const void *x, int nrows,
                        const int32_t *row_token, const int32_t *row_expert, const int8_t *q1, const float *s1,
                        const int8_t *q3, const float *s3, const int8_t *q2, const float *s2, const void *b1,
                        const void *b2, double *y_out) {
#pragma omp parallel
    {
        std::vector<double> xr(d), u(h), v(h), H(h), y(d);
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < nrows; ++r) {
            const int t = row_token[r], e = row_expert[r];
            const size_t wdh = (size_t)e * d * h;
            for (int k = 0; k < d; ++k) xr[k] = load(x, dt, (size_t)t * d + k);
            std::fill(u.begin(), u.end(), 0.0);
            std::fill(v.begin(), v.end(), 0.0);
            for (int k = 0; k < d; ++k) {
                const double xk = xr[k];
                for (int j = 0; j < h; ++j)
                    u[j] += xk * ((double)s1[(size_t)e * h + j] * (double)q1[wdh + (size_t)k * h + j]);
                if (act == ACT_SWIGLU)
                    for (int j = 0; j < h; ++j)
                        v[j] += xk * ((double)s3[(size_t)e * h + j] * (double)q3[wdh + (size_t)k * h + j]);
            }
            hidden_row(h, act, mirror, dt, e, u, v, b1, H);
            const size_t whd = (size_t)e * h * d;
            output_row(h, d, act, mirror, dt, e, H,
                       [&](int j, int c) { return (double)s2[(size_t)e * d + c] * (double)q2[whd + (size_t)j * d + c]; },
                       b2, y, y_out + (size_t)r * d);
        }
    }
}

// ---- 4-bit expert weights ([rkmt] section 4.2: 4-bit AWQ weights with a zero
// point and a quantization group of 128).  A group is 128 consecutive input
// channels k of one output column n of one expert; it has one fp32 scale and
// one integer zero point.  AWQ's search for activation-aware scales needs
// calibration activations; what is defined here is the storage format and the
// min-max rounding that search ends with, in fp32, ties to even:
//   mx, mn = the group's largest and smallest weight
//   s = max(mx - mn, 1e-5) / 15
//   z = -rint(mn / s) clamped to [0, 15]
//   q = rint(w / s) + z clamped to [0, 15]
// and the weight a code stands for is W = s * (q - z).
constexpr int kQ4Group = 128;

// q [E][K][N] codes (one per byte), scale and zero [E][K/128][N]; K % 128 == 0.
void oracle_quantize_q4(const void *w, int dt, int E, int K, int N, uint8_t *q, float *scale, uint8_t *zero) {
    const int G = K / kQ4Group;
#pragma omp parallel for schedule(dynamic, 1)
    for (long eg = 0; eg < (long)E * G; ++eg) {
        const int e = (int)(eg / G), g = (int)(eg % G);
        const size_t base = (size_t)e * K * N + (size_t)g * kQ4Group * N;  // row k0 = 128 g of expert e
        const size_t sz = ((size_t)e * G + g) * N;
        std::vector<float> mx(N), mn(N), sc(N), zf(N);
        for (int n = 0; n < N; ++n) mx[n] = mn[n] = (float)load(w, dt, base + n);
        for (int k = 1; k < kQ4Group; ++k)
            for (int n = 0; n < N; ++n) {
                const float v = (float)load(w, dt, base + (size_t)k * N + n);
                if (v > mx[n]) mx[n] = v;
                if (v < mn[n]) mn[n] = v;
            }
        for (int n = 0; n < N; ++n) {
            const float range = mx[n] - mn[n];
            sc[n] = (range > 1e-5f ? range : 1e-5f) / 15.0f;
            float z = -std::nearbyint(mn[n] / sc[n]);  // default mode: ties to even
            if (z < 0.0f) z = 0.0f;
            if (z > 15.0f) z = 15.0f;
            zf[n] = z;
            scale[sz + n] = sc[n];
            zero[sz + n] = (uint8_t)z;
        }
        for (int k = 0; k < kQ4Group; ++k)
            for (int n = 0; n < N; ++n) {
                const size_t i = base + (size_t)k * N + n;
                float r = std::nearbyint((float)load(w, dt, i) / sc[n]) + zf[n];
                if (r < 0.0f) r = 0.0f;
                if (r > 15.0f) r = 15.0f;
                q[i] = (uint8_t)r;
            }
    }
}

// Step 5 with 4-bit expert weights: the two-layer FFN on the dequantized
// weights W[k][n] = s[k / 128][n] * (q[k][n] - z[k / 128][n]), each formed
// exactly in double.  q1, q3 [E][d][h] with s1, z1, s3, z3 [E][d/128][h];
// q2 [E][h][d] with s2, z2 [E][h/128][d].
void oracle_ffn_rows_q4(int d, int h, int dt, int act, int mirror, const void *x, int nrows,
                        const int32_t *row_token, const int32_t *row_expert, const uint8_t *q1, const float *s1,
                        const uint8_t *z1, const uint8_t *q3, const float *s3, const uint8_t *z3, const uint8_t *q2,
                        const float *s2, const uint8_t *z2, const void *b1, const void *b2, double *y_out) {
    const int G1 = d / kQ4Group, G2 = h / kQ4Group;
#pragma omp parallel
    {
        std::vector<double> xr(d), u(h), v(h), H(h), y(d);
#pragma omp for schedule(dynamic, 1)
        for (int r = 0; r < nrows; ++r) {
            const int t = row_token[r], e = row_expert[r];
            const size_t wdh = (size_t)e * d * h;
            for (int k = 0; k < d; ++k) xr[k] = load(x, dt, (size_t)t * d + k);
            std::fill(u.begin(), u.end(), 0.0);
            std::fill(v.begin(), v.end(), 0.0);
            for (int k = 0; k < d; ++k) {
                const double xk = xr[k];
                const size_t gz = ((size_t)e * G1 + k / kQ4Group) * h;
                for (int j = 0; j < h; ++j)
                    u[j] += xk * ((double)s1[gz + j] * ((double)q1[wdh + (size_t)k * h + j] - (double)z1[gz + j]));
                if (act == ACT_SWIGLU)
                    for (int j = 0; j < h; ++j)
                        v[j] += xk * ((double)s3[gz + j] * ((double)q3[wdh + (size_t)k * h + j] - (double)z3[gz + j]));
            }
            hidden_row(h, act, mirror, dt, e, u, v, b1, H);
            const size_t whd = (size_t)e * h * d;
            output_row(h, d, act, mirror, dt, e, H,
                       [&](int j, int c) {
                           const size_t gz = ((size_t)e * G2 + j / kQ4Group) * d + c;
                           return (double)s2[gz] * ((double)q2[whd + (size_t)j * d + c] - (double)z2[gz]);
                       },
                       b2, y, y_out + (size_t)r * d);
        }
    }
}

// Round doubles to a storage type (for comparing against stored GPU values).
void oracle_round(const double *in, double *out, size_t n, int dt) {
    for (size_t i = 0; i < n; ++i) out[i] = round_to_dtype(in[i], dt);
}

}  // extern "C"
