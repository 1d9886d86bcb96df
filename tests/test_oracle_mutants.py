"""Mutation check of the pins: each planted mistake in a copy of the oracle
must make at least one pin fail.  The mistakes are planted in the oracle's
source text (CPU only); the real oracle is untouched."""
import os
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle
from tests import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "colibri_oracle.cpp")

# name -> (text in the oracle, planted replacement)
MUTANTS = {
    "tie_break_reversed": ("return a < b;", "return a > b;"),
    "nan_ranks_high": ("if (na != nb) return nb;", "if (na != nb) return na;"),
    "slot_order_swapped": ("idx[2 * t] = i0;\n        idx[2 * t + 1] = i1;",
                           "idx[2 * t] = i1;\n        idx[2 * t + 1] = i0;"),
    "gates_not_renormalised": ("gate[2 * t] = p0 / (p0 + p1);", "gate[2 * t] = p0;"),
    "dispatch_unstable": ("for (int a = 0; a < A; ++a)\n            if (idx[a] == e)",
                          "for (int a = A - 1; a >= 0; --a)\n            if (idx[a] == e)"),
    "router_bias_dropped": ("s + (b_r ? (double)b_r[e] : 0.0)", "s"),
    "router_weight_transposed": ("load(w_r, dt, (size_t)j * E + e)", "load(w_r, dt, (size_t)e * d + j)"),
    "b1_dropped": ("double z = u[j] + (b1 ? load(b1, dt, (size_t)e * h + j) : 0.0);", "double z = u[j];"),
    "gelu_tanh_approx": ("0.5 * z * (1.0 + std::erf(z / std::sqrt(2.0)))",
                         "0.5 * z * (1.0 + std::tanh(0.7978845608028654 * (z + 0.044715 * z * z * z)))"),
    "swiglu_operands_swapped": ("hv = act_silu(u[j]) * v[j];", "hv = u[j] * act_silu(v[j]);"),
    "w2_transposed": ("load(w2, dt, whd + (size_t)j * d + c)", "load(w2, dt, whd + (size_t)c * h + j)"),
    "h_not_rounded": ("H[j] = mirror ? round_to_dtype(hv, dt) : hv;", "H[j] = hv;"),
    "y_not_rounded": ("yo[c] = mirror ? round_to_dtype(yv, dt) : yv;", "yo[c] = yv;"),
    "combine_gates_swapped": ("gate[2 * t] * y0[c] + gate[2 * t + 1] * y1[c]",
                              "gate[2 * t + 1] * y0[c] + gate[2 * t] * y1[c]"),
    "b2_dropped": ("yv = y[c] + ((act != ACT_SWIGLU && b2) ? load(b2, dt, (size_t)e * d + c) : 0.0);",
                   "yv = y[c];"),
    "q8_scale_along_k": ("u[j] += xk * ((double)s1[(size_t)e * h + j] * (double)q1[wdh + (size_t)k * h + j]);",
                         "u[j] += xk * ((double)s1[(size_t)e * h + (k % h)] * (double)q1[wdh + (size_t)k * h + j]);"),
    "q8_w3_takes_w1_scale": ("v[j] += xk * ((double)s3[(size_t)e * h + j]",
                             "v[j] += xk * ((double)s1[(size_t)e * h + j]"),
    "q8_second_scale_dropped": ("return (double)s2[(size_t)e * d + c] * (double)q2[whd + (size_t)j * d + c];",
                                "return (double)q2[whd + (size_t)j * d + c];"),
    "q8_ties_away_from_zero": ("float r = std::nearbyint((float)load(w, dt, i) / sc[n - n0]);",
                               "float r = std::round((float)load(w, dt, i) / sc[n - n0]);"),
    "q8_zero_column_unguarded": ("sc[n - n0] = amax[n - n0] > 0.0f ? amax[n - n0] / 127.0f : 1.0f;",
                                 "sc[n - n0] = amax[n - n0] / 127.0f;"),
    "q8_scale_over_128": ("sc[n - n0] = amax[n - n0] > 0.0f ? amax[n - n0] / 127.0f : 1.0f;",
                          "sc[n - n0] = amax[n - n0] > 0.0f ? amax[n - n0] / 128.0f : 1.0f;"),
    "q4_zero_sign_flipped": ("float z = -std::nearbyint(mn[n] / sc[n]);", "float z = std::nearbyint(mn[n] / sc[n]);"),
    "q4_ties_away_from_zero": ("float r = std::nearbyint((float)load(w, dt, i) / sc[n]) + zf[n];",
                               "float r = std::round((float)load(w, dt, i) / sc[n]) + zf[n];"),
    "q4_scale_over_16": ("sc[n] = (range > 1e-5f ? range : 1e-5f) / 15.0f;",
                         "sc[n] = (range > 1e-5f ? range : 1e-5f) / 16.0f;"),
    "q4_zero_point_dropped": ("((double)q1[wdh + (size_t)k * h + j] - (double)z1[gz + j])",
                              "(double)q1[wdh + (size_t)k * h + j]"),
    "q4_w3_takes_w1_zero": ("((double)q3[wdh + (size_t)k * h + j] - (double)z3[gz + j])",
                            "((double)q3[wdh + (size_t)k * h + j] - (double)z1[gz + j])"),
    "q4_second_layer_unscaled": ("return (double)s2[gz] * ((double)q2[whd + (size_t)j * d + c] - (double)z2[gz]);",
                                 "return ((double)q2[whd + (size_t)j * d + c] - (double)z2[gz]);"),
    "softmax_gates_renormalised": ("gate[2 * t] = std::exp(l[idx[2 * t]] - m) / z;",
                                   "gate[2 * t] = std::exp(l[idx[2 * t]] - m) / (std::exp(l[idx[2 * t]] - m) + "
                                   "std::exp(l[idx[2 * t + 1]] - m));"),
    "softmax_gates_unscaled": ("gate[2 * t + 1] = std::exp(l[idx[2 * t + 1]] - m) / z;",
                               "gate[2 * t + 1] = std::exp(l[idx[2 * t + 1]] - m);"),
    "linear_gates_slots_swapped": ("gate[2 * t] = l[idx[2 * t]];", "gate[2 * t] = l[idx[2 * t + 1]];"),
    "shared_expert_dropped": ("if (shared_y) v += shared_y[i];", "(void)shared_y;"),
    "shared_expert_row_offset": ("if (shared_y) v += shared_y[i];", "if (shared_y) v += shared_y[c];"),
    "residual_dropped": ("if (residual) v += load(residual, dt, i);", "(void)residual;"),
    "residual_subtracted": ("if (residual) v += load(residual, dt, i);", "if (residual) v -= load(residual, dt, i);"),
    "rounding_via_fp32": ("double round_to_dtype(double v, int dt) { return round_to_format(v, dt == DT_F32 ? 23 : 7); }",
                          "double round_to_dtype(double v, int dt) { return round_to_format(dt == DT_F32 ? v : (double)(float)v, dt == DT_F32 ? 23 : 7); }"),
}


@pytest.fixture(scope="module")
def mutant_libs():
    src = open(SRC).read()
    tmp = tempfile.mkdtemp(prefix="oracle_mutants_")

    def build(item):
        name, (old, new) = item
        assert src.count(old) == 1, f"mutant {name}: target text not found exactly once"
        path = os.path.join(tmp, f"{name}.cpp")
        with open(path, "w") as f:
            f.write(src.replace(old, new))
        so = os.path.join(tmp, f"lib{name}.so")
        flags = [f for f in oracle.CFLAGS if f != "-O3"] + ["-O1"]
        subprocess.check_call(["g++", *flags, path, "-o", so])
        return name, so

    with ThreadPoolExecutor(max_workers=4) as ex:
        built = dict(ex.map(build, MUTANTS.items()))
    return built


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_libs):
    lib = oracle.load_library(mutant_libs[name])
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake '{name}'"
