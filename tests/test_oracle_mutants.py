"""Planted mistakes in the oracle are caught by its pins.

Each mutant is a copy of ``oracle/pa_oracle.c`` with one plausible mistake
(a dropped term, a flipped sign, a wrong index, a transposed operand, an
off-by-one in the causal window...), compiled on the CPU into a temporary
library.  The pins must reject every mutant; a surviving mutant means the pins
leave that part of the oracle unchecked.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

# (name, [(original text, replacement, occurrence index or None for "the only one")])
MUTANTS = [
    ("gqa_modulo_decode", [("int32_t kh = h / group;", "int32_t kh = h % Hkv;", 0)]),
    ("gqa_modulo_prefill", [("int32_t kh = h / group;", "int32_t kh = h % Hkv;", 1)]),
    ("scale_dropped", [("s[j] = scale * dot;", "s[j] = dot;", None)]),
    ("exp_sign_flipped", [("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);", None)]),
    ("first_weight_dropped_from_z", [("z += s[j];", "if (j) z += s[j];", None)]),
    ("shift_by_min", [("if (s[j] > m)", "if (s[j] < m)", None)]),
    ("k_read_from_v_pool", [("const uint16_t *k_row = k_pool", "const uint16_t *k_row = v_pool", None)]),
    ("values_paired_reversed", [("const uint16_t *v_row = v_pool + (int64_t)slots[j]",
                                 "const uint16_t *v_row = v_pool + (int64_t)slots[n - 1 - j]", None)]),
    ("k_head_and_dim_transposed", [
        ("const uint16_t *k_row = k_pool + (int64_t)slots[j] * slot_stride + (int64_t)kh * D;",
         "const uint16_t *k_row = k_pool + (int64_t)slots[j] * slot_stride + (int64_t)kh;", None),
        ("widen_bf16(k_row[d])", "widen_bf16(k_row[(int64_t)d * (slot_stride / D)])", None)]),
    ("normalised_by_count", [("out[d] /= z;", "out[d] /= (double)n;", None)]),
    ("lse_without_max", [("*lse = m + log(z);", "*lse = log(z);", None)]),
    ("lse_without_log", [("*lse = m + log(z);", "*lse = m + z;", None)]),
    ("empty_lse_zero", [("*lse = -INFINITY;\n        return;", "*lse = 0.0;\n        return;", 0)]),
    ("empty_out_garbage", [("out[d] = 0.0;\n        *lse = -INFINITY;", "out[d] = 1.0;\n        *lse = -INFINITY;", 0)]),
    ("fp8_empty_lse_zero", [("*lse = -INFINITY;\n        return;", "*lse = 0.0;\n        return;", 1)]),
    ("fp8_empty_out_garbage", [("out[d] = 0.0;\n        *lse = -INFINITY;", "out[d] = 1.0;\n        *lse = -INFINITY;", 1)]),
    ("query_head_zero_decode", [("attend_one_row(D, q + row * D,", "attend_one_row(D, q + (row / Hq) * Hq * D,", 0)]),
    ("query_head_zero_prefill", [("attend_one_row(D, q + row * D,", "attend_one_row(D, q + (row / Hq) * Hq * D,", 1)]),
    ("decode_list_one_short", [("(int64_t)kv_indptr[b + 1] - kv_indptr[b],\n                           (double)sm_scale",
                                "(int64_t)kv_indptr[b + 1] - kv_indptr[b] - 1,\n                           (double)sm_scale", None)]),
    ("causal_window_one_short", [("prefix + i + 1,", "prefix + i,", None)]),
    ("causal_top_left", [("int64_t prefix = L - chunk;", "int64_t prefix = 0;", None)]),
    ("causal_ignored", [("prefix + i + 1,", "L,", None)]),
    ("prefill_row_in_chunk_wrong", [("int64_t i = t - qo_indptr[b];", "int64_t i = t - qo_indptr[b] - (b > 0);", None)]),
    ("merge_weight_sign", [("double w = exp(lse_parts[i] - M);", "double w = exp(M - lse_parts[i]);", None)]),
    ("merge_lse_without_log", [("*lse = M + log(wsum);", "*lse = M;", None)]),
    ("merge_first_part_dropped", [("for (int32_t i = 0; i < n; i++) {\n        double w",
                                   "for (int32_t i = 1; i < n; i++) {\n        double w", None)]),
    ("merge_unnormalised", [("out[d] /= wsum;", "out[d] /= (double)n;", None)]),
    ("rope_adjacent_pairs", [("widen_bf16(x[i]), x2 = widen_bf16(x[i + half]);",
                              "widen_bf16(x[(2 * i) % D]), x2 = widen_bf16(x[(2 * i + 1) % D]);", None)]),
    ("rope_sign_flipped", [("out[i] = x1 * c - x2 * sn;", "out[i] = x1 * c + x2 * sn;", None)]),
    ("rope_frequency_exponent", [("pow(theta, -2.0 * (double)i / (double)D)", "pow(theta, -(double)i / (double)D)", None)]),
    ("rope_second_half_unrotated", [("out[i + half] = x2 * c + x1 * sn;", "out[i + half] = x2;", None)]),
    ("e4m3_bias_8", [("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)", None)]),
    ("e4m3_subnormal_scale", [("ldexp((double)m / 8.0, -6)", "ldexp((double)m / 8.0, -7)", None)]),
    ("e4m3_mantissa_width", [("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 16.0, e - 7)", None)]),
    ("e4m3_sign_ignored", [("return sign ? -mag : mag;", "return mag;", None)]),
    ("e4m3_no_nan", [("if (e == 0xF && m == 0x7)\n        return NAN;", "if (0)\n        return NAN;", None)]),
    ("fp8_k_scale_dropped", [("acc += widen_bf16(q_row[d]) * (k_scale * e4m3_value(kc[d]));",
                              "acc += widen_bf16(q_row[d]) * e4m3_value(kc[d]);", None)]),
    ("fp8_v_scale_dropped", [("out[d] += w[j] * (v_scale * e4m3_value(vc[d]));",
                              "out[d] += w[j] * e4m3_value(vc[d]);", None)]),
    ("fp8_values_from_k_codes", [("const uint8_t *vc = v_codes", "const uint8_t *vc = k_codes", None)]),
    ("fp8_scales_as_float_product", [("(double)sm_scale, (double)k_scale, (double)v_scale,",
                                      "(double)(float)(sm_scale * k_scale), 1.0, (double)v_scale,", None)]),
    ("fp8_lse_without_max", [("*lse = top + log(total);", "*lse = log(total);", None)]),
    ("fp8_exp_unshifted", [("w[j] = exp(w[j] - top);", "w[j] = exp(w[j]);", None)]),
    ("fp8_gqa_modulo", [("head / per_kv_head, kv_indices", "head % Hkv, kv_indices", None)]),
    ("e4m3_encode_ties_up", [("(err == best_err && (c & 1) == 0)", "(err == best_err)", None)]),
    ("e4m3_encode_truncates", [("if (err < best_err || (err == best_err && (c & 1) == 0))",
                                "if (e4m3_value((uint8_t)c) <= a)", None)]),
    ("e4m3_encode_saturates_to_nan", [("return sign | 0x7E;", "return 0x7F;", None)]),
    ("e4m3_encode_sign_dropped", [("return (uint8_t)(sign | best);", "return (uint8_t)best;", None)]),
    ("e4m3_encode_nan_to_zero", [("if (isnan(x))\n        return 0x7F;", "if (isnan(x))\n        return 0x00;", None)]),
    ("e4m3_encode_scale_multiplies", [("e4m3_encode(x[i] / (double)scale)", "e4m3_encode(x[i] * (double)scale)", None)]),
    ("e4m3_encode_float_quotient", [("e4m3_encode(x[i] / (double)scale)",
                                     "e4m3_encode((double)(float)(x[i] / (double)scale))", None)]),
    ("fp8_prefill_window_one_short", [("- c_len + pos_in_chunk + 1;", "- c_len + pos_in_chunk;", None)]),
    ("fp8_prefill_top_left", [("((int64_t)kv_indptr[b + 1] - kv_indptr[b]) - c_len + pos_in_chunk + 1;",
                               "pos_in_chunk + 1;", None)]),
    ("fp8_prefill_gqa_modulo", [("head / (Hq / Hkv),", "head % Hkv,", None)]),
    ("fp8_prefill_scales_swapped", [("(double)k_scale, (double)v_scale, w, out + row * D",
                                     "(double)v_scale, (double)k_scale, w, out + row * D", None)]),
    ("rope_position_off_by_one", [("(double)positions[t] * inv_freq", "(double)(positions[t] + 1) * inv_freq", None)]),
]


def _mutate(src: str, edits):
    for old, new, occurrence in edits:
        count = src.count(old)
        if occurrence is None:
            assert count == 1, f"mutation anchor must be unique: {old!r} ({count})"
            src = src.replace(old, new)
        else:
            assert count > occurrence, f"mutation anchor occurrence missing: {old!r}"
            pos = -1
            for _ in range(occurrence + 1):
                pos = src.index(old, pos + 1)
            src = src[:pos] + new + src[pos + len(old):]
    return src


@pytest.mark.parametrize("name,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, edits):
    with open(oracle.SOURCE) as f:
        src = f.read()
    mutated = _mutate(src, edits)
    assert mutated != src
    c_path = os.path.join(tmp_path, f"{name}.c")
    so_path = os.path.join(tmp_path, f"lib{name}.so")
    with open(c_path, "w") as f:
        f.write(mutated)
    oracle.build(c_path, so_path)
    mutant = oracle.Oracle(so_path)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, oracle.OracleError) as e:
            caught.append(f"{pin.__name__}: {str(e)[:60]}")
    assert caught, f"mutant {name} survived every pin"
