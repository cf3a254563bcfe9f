"""Plant one plausible mistake at a time in a copy of the oracle (on the CPU)
and require that at least one pin fails, so the pins are known to be able to
catch: a swapped nibble order, a wrong exponent bias, a dropped term, a wrong
tie-break, a missing normalisation, a sign error, swapped or transposed
operands, an unstable sort, a lost permutation, a dropped shared term."""
import os

import pytest

import oracle
import oracle_pins
from oracle import build as obuild

SRC = obuild.SRC

MUTANTS = {
    "nibble_order_swapped": ("int code = (i % 2 == 0) ? (byte & 0xF) : (byte >> 4);",
                             "int code = (i % 2 == 0) ? (byte >> 4) : (byte & 0xF);"),
    "e2m1_subnormal_wrong": ("(e == 0) ? 0.5 * m", "(e == 0) ? 1.0 * m"),
    "e2m1_bias_wrong": ("ldexp(1.0 + 0.5 * m, e - 1)", "ldexp(1.0 + 0.5 * m, e)"),
    "e8m0_bias_wrong": ("return ldexp(1.0, s - 127);", "return ldexp(1.0, s - 128);"),
    "scale_block_shifted": ("s[r * (cols / 32) + i / 32]", "s[r * (cols / 32) + (i / 32 + 1) % (cols / 32)]"),
    "router_drops_last_term": ("for (int i = 0; i < d; ++i) acc += x[t * d + i]",
                               "for (int i = 0; i < d - 1; ++i) acc += x[t * d + i]"),
    "tie_break_reversed": ("(la == lb && a < b)", "(la == lb && a > b)"),
    "topk_picks_smallest": ("return la > lb ||", "return la < lb ||"),
    "softmax_not_normalised": ("w[t * k + r] = exp(l[idx[t * k + r]] - m) / z;",
                               "w[t * k + r] = exp(l[idx[t * k + r]] - m);"),
    "weights_in_selection_order": ("w[t * k + r] = exp(l[idx[t * k + r]] - m) / z;",
                                   "w[t * k + r] = exp(l[sel[r]] - m) / z;"),
    "silu_sign": ("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    "gate_up_swapped": ("if (j < f) g[r * f + j] = acc;\n        else u[r * f + (j - f)] = acc;",
                        "if (j < f) u[r * f + j] = acc;\n        else g[r * f + (j - f)] = acc;"),
    "down_h_reversed": ("acc += row[j] * h[r * f + j];", "acc += row[j] * h[r * f + (f - 1 - j)];"),
    "permute_unstable": ("for (int64_t p = 0; p < P; ++p) {\n    int e = idx[p];",
                         "for (int64_t p = P - 1; p >= 0; --p) {\n    int e = idx[p];"),
    "combine_ignores_permutation": ("y_perm[(int64_t)pair_pos[t * k + s] * d + o]",
                                    "y_perm[(int64_t)(t * k + s) * d + o]"),
    "combine_drops_shared": ("double acc = shared ? shared[t * d + o] : 0.0;",
                             "double acc = 0.0;"),
    "combine_keeps_zero_weights": ("if (ws != 0.0) acc += ws", "if (1) acc += ws"),
    "shared_down_transposed": ("bf16_value(w2[(int64_t)o * f + j])", "bf16_value(w2[(int64_t)j * d + o])"),
    "sigmoid_bias_ignored": ("sel[e] = sigmoid_score(l[e]) + (bias ? (double)bias[e] : 0.0);",
                             "sel[e] = sigmoid_score(l[e]);"),
    "sigmoid_selects_on_logit": ("sel[e] = sigmoid_score(l[e]) + (bias ? (double)bias[e] : 0.0);",
                                 "sel[e] = l[e] + (bias ? (double)bias[e] : 0.0);"),
    "sigmoid_weights_biased": ("double s = sigmoid_score(l[idx[t * k + r]]);",
                               "double s = sigmoid_score(l[idx[t * k + r]]) + (bias ? bias[idx[t * k + r]] : 0.0);"),
    "sigmoid_norm_inverted": ("w[t * k + r] = norm ? s / z : s;", "w[t * k + r] = norm ? s : s / z;"),
    "sigmoid_sign": ("return 1.0 / (1.0 + exp(-l));", "return 1.0 / (1.0 + exp(l));"),
    "mx_quant_emax_wrong": ("int E = (int)floor(log2(X)) - 2;", "int E = (int)floor(log2(X)) - 1;"),
    "mx_quant_ceil_scale": ("int E = (int)floor(log2(X)) - 2;", "int E = (int)ceil(log2(X)) - 2;"),
    "mx_quant_ties_odd": ("(dc == db && (c & 1) == 0)", "(dc == db && (c & 1) == 1)"),
    "mx_quant_ties_away": ("(dc == db && (c & 1) == 0)", "(dc == db)"),
    "mx_quant_sign_dropped": ("int code = best | (signbit(vb[i]) ? 8 : 0);", "int code = best;"),
    "qact_h_not_quantised": ("  quantize_rows(n, f, h);\n", "\n"),
    "qact_x_not_quantised": ("  quantize_rows(n, d, xq);\n", "\n"),
    "rvq_two_stages": ("for (int s = 0; s < 3; ++s) {\n    uint8_t i = idx[", "for (int s = 0; s < 2; ++s) {\n    uint8_t i = idx["),
    "rvq_slice_group_swapped": ("int g = c / 8, j = c % 8, sl = g / 16, gi = g % 16;",
                                "int g = c / 8, j = c % 8, sl = g % 16 % (cols / 128), gi = g / 16 % 16;"),
    "rvq_codeword_offset": ("w += (double)cb[((int64_t)s * 256 + i) * 8 + j];",
                            "w += (double)cb[((int64_t)s * 256 + i) * 8 + (j + 1) % 8];"),
    "bf16_decode_wrong": ("uint32_t u = (uint32_t)b << 16;", "uint32_t u = (uint32_t)(b & 0xFF7F) << 16;"),
}


def _build_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site of {name} not found"
    src = src.replace(old, new, 1)
    path = os.path.join(tmp_path, f"oracle_{name}.c")
    with open(path, "w") as fh:
        fh.write(src)
    return obuild.build(path, os.path.join(tmp_path, f"liboracle_{name}.so"))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    lib = _build_mutant(name, str(tmp_path))
    o = oracle.Oracle(lib)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except Exception as exc:  # any failure of a pin counts as caught
            caught.append(f"{pin.__name__}: {type(exc).__name__}")
    assert caught, f"no pin catches mutant {name}"


# Mistakes planted in the oracle's per-token path (Python), which the
# full-size GPU tests use as their expected values.
PY_MUTANTS = {
    "token_outputs_slot_swap": ("y[rows, slots] = ffn(", "y[rows, (slots + 1) % k] = ffn("),
    "token_outputs_rows_of_first_token": ("ffn(get_expert(int(e)), x64[rows])",
                                          "ffn(get_expert(int(e)), x64[rows * 0])"),
    "token_outputs_no_shared": ("shared_y)\n    return out", "None)\n    return out"),
}


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_token_outputs_mutant_is_caught(name):
    import inspect
    import textwrap
    import numpy as np
    old, new = PY_MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(oracle.Oracle.token_outputs))
    assert src.count(old) == 1, f"mutation site of {name} not found"
    ns = {"np": np, "to_f64": oracle.to_f64}
    exec(src.replace(old, new), ns)
    o = oracle.Oracle()
    o.token_outputs = ns["token_outputs"].__get__(o)
    with pytest.raises(AssertionError):
        oracle_pins.pin_token_outputs_equal_layer(o)
