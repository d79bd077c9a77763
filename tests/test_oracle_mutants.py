"""Mutation test of the oracle's pins (CPU only).

Each case plants one plausible mistake (a dropped term, a wrong sign, a
transposed operand, an off-by-one, a wrong rounding) in a copy of
``oracle/adam_oracle.c``, builds the copy into a temporary directory, and
requires at least one quick pin from tests/pins.py to fail on it.  The real
oracle must pass all of them.  Nothing here touches the GPU path.
"""
import os

import pytest

import pins
from oracle import Oracle
from oracle import build as oracle_build

SOURCE = oracle_build.SOURCE

MUTANTS = {
    "l2_decay_dropped": [("scaled_grad = grad_part + decay_part;", "scaled_grad = grad_part;")],
    "l2_decay_sign": [("scaled_grad = grad_part + decay_part;", "scaled_grad = grad_part - decay_part;")],
    "update_sign": [("return P - step;", "return P + step;")],
    "adamw_decay_dropped": [("update = update + decay_part;", "update = update;")],
    "adamw_decay_sign": [("update = update + decay_part;", "update = update - decay_part;")],
    "eps_inside_root": [("sqrtf(v_unbiased) + s->eps", "sqrtf(v_unbiased + s->eps)")],
    "root_missing": [("sqrtf(v_unbiased) + s->eps", "v_unbiased + s->eps")],
    "moment_average_transposed": [("float keep = beta * m;", "float keep = beta * x;"),
                                  ("float take = one_minus_beta * x;", "float take = one_minus_beta * m;")],
    "second_moment_uses_beta1": [("moment_average(s->beta2, grad_sq, *V)",
                                  "moment_average(s->beta1, grad_sq, *V)")],
    "corrections_swapped": [("next_m / s->bc1", "next_m / s->bc2")],
    "correction_off_by_one": [("oracle_pow_int((double)beta1, t)", "oracle_pow_int((double)beta1, t - 1)")],
    "power_rounded_to_float": [("oracle_pow_int((double)beta2, t))", "(float)oracle_pow_int((double)beta2, t))")],
    "correction_flag_ignored": [("if (bias_correction == 1) {", "if (1) {")],
    "grad_scale_dropped_adamw": [("scaled_grad = G * s->grad_scale;", "scaled_grad = G;")],
    "grad_scale_dropped_l2": [("float grad_part = G * s->grad_scale;", "float grad_part = G;")],
    "square_of_raw_grad": [("float grad_sq = scaled_grad * scaled_grad;", "float grad_sq = scaled_grad * G;")],
    "moments_stored_swapped": [("*M = next_m;\n    *V = next_v;", "*M = next_v;\n    *V = next_m;")],
    "rne_ties_away": [("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)")],
    "rne_truncates": [("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u)))", "if (0)")],
    "nan_not_quieted": [("return (uint16_t)((b >> 16) | 0x0040u);", "return (uint16_t)(b >> 16);")],
    "decode_sign_fix_dropped": [("(uint16_t)(bf16 - (rem < 0 ? 1u : 0u))", "(uint16_t)(bf16)")],
    "encode_carry_dropped": [("(uint16_t)(high + (r < 0 ? 1u : 0u))", "(uint16_t)(high)")],
    "decode_halves_swapped": [("((uint32_t)high << 16) | (uint32_t)low", "((uint32_t)low << 16) | (uint32_t)high")],
    "param_out_truncated": [("return out_type == ORACLE_F16 ? oracle_f16_rne(x) : oracle_bf16_rne(x);",
                             "return out_type == ORACLE_F16 ? oracle_f16_rne(x) : (uint16_t)(bits_from_f32(x) >> 16);")],
    "remainder_param_out_rne": [("p_out[i] = p[i];", "p_out[i] = oracle_bf16_rne(P_new);")],
    "bf16_grad_index_shift": [("((const uint16_t *)g)[i]", "((const uint16_t *)g)[i ? i - 1 : 0]")],
    "one_minus_beta_wrong": [("float one_minus_beta = 1.0f - beta;", "float one_minus_beta = beta - 1.0f;")],
    "sumsq_carry_dropped": [("    uint64_t carry = s < lo;\n", "    uint64_t carry = 0;\n")],
    "sumsq_round_truncates": [("round_up = sticky || (m & 1u);", "round_up = 0;")],
    "sumsq_ties_away": [("round_up = sticky || (m & 1u);", "round_up = 1;")],
    "sumsq_square_in_float": [("acc_add_double(a, x * x);", "acc_add_double(a, (double)((float)x * (float)x));")],
    "sumsq_merge_drops_flags": [("    into->has_inf |= from->has_inf;\n", "")],
    "sumsq_bit_position_off_by_one": [("int shift = (e - 53) - ACC_LSB_EXP;", "int shift = (e - 52) - ACC_LSB_EXP;")],
    "f16_ties_away": [("double r = rint(a / spacing) * spacing;", "double r = round(a / spacing) * spacing;")],
    "f16_truncates": [("double r = rint(a / spacing) * spacing;", "double r = trunc(a / spacing) * spacing;")],
    "f16_subnormal_spacing": [("int low = e - 1 < -14 ? -14 : e - 1;", "int low = e - 1 < -15 ? -15 : e - 1;")],
    "f16_overflow_early": [("if (r >= 65536.0)", "if (r >= 65504.0)")],
    "f16_decode_bias": [("mag = ldexp(1024.0 + f, e - 25);", "mag = ldexp(1024.0 + f, e - 24);")],
    "f16_decode_subnormal": [("mag = ldexp((double)f, -24);", "mag = ldexp((double)f, -25);")],
    "f16_grad_read_as_bf16": [("return g_type == ORACLE_F16 ? oracle_f16_to_f32(h) : oracle_bf16_to_f32(h);",
                               "return oracle_bf16_to_f32(h);")],
    "f16_out_cast_as_bf16": [("return out_type == ORACLE_F16 ? oracle_f16_rne(x) : oracle_bf16_rne(x);",
                              "return oracle_bf16_rne(x);")],
    "scaled_bf16_limit_not_halved": [("return ldexpf(2.0f - ldexpf(1.0f, -7), 126);",
                                      "return ldexpf(2.0f - ldexpf(1.0f, -7), 127);")],
    "scaled_f16_limit_not_halved": [("return ldexpf(2.0f - ldexpf(1.0f, -10), 14);",
                                     "return ldexpf(2.0f - ldexpf(1.0f, -10), 15);")],
    "scaled_rscale_not_reciprocal": [("float rscale = scale > 0.0f ? 1.0f / scale : 0.0f;",
                                      "float rscale = scale > 0.0f ? scale : 0.0f;")],
    "scaled_absmax_ignores_negatives": [("return neg_lo > hi ? neg_lo : hi;", "return hi;")],
    "scaled_absmax_drops_nan": [("        if (isnan(x[i]))\n            return NAN;\n", "")],
    "scaled_unscale_dropped": [("P[i] = state_to_f32(p[i], state_type) * scales[0];",
                                "P[i] = state_to_f32(p[i], state_type);")],
    "scaled_moment_scales_swapped": [("M[i] = state_to_f32(m[i], state_type) * scales[1];",
                                      "M[i] = state_to_f32(m[i], state_type) * scales[2];")],
    "scaled_param_sync_from_stored": [("p_out[i] = cast_out(P[i], out_type);", "p_out[i] = p[i];")],
    "state16_moment_rounded_as_bf16": [("m[i] = f32_to_state(M, state_type);",
                                        "m[i] = f32_to_state(M, ORACLE_BF16);")],
    "state16_second_moment_from_first": [("float V = state_to_f32(v[i], state_type);",
                                          "float V = state_to_f32(m[i], state_type);")],
    "state16_param_not_rounded": [("p[i] = f32_to_state(P_new, state_type);",
                                   "p[i] = f32_to_state(P, state_type);")],
    "state16_param_out_from_float": [("store_out(p_out, i, state_to_f32(p[i], state_type), out_type);",
                                      "store_out(p_out, i, P_new, out_type);")],
    "f32_param_out_dropped": [("((float *)p_out)[i] = x;", "((float *)p_out)[i] = 0.0f;")],
    "scaled_scale_not_returned": [("    scales[1] = oracle_rescale_store(M, m, n, state_type);\n", "")],
}


def _mutant_library(tmp_path, name):
    src = open(SOURCE).read()
    for old, new in MUTANTS[name]:
        assert src.count(old) == 1, (name, old)
        src = src.replace(old, new)
    path = os.path.join(str(tmp_path), f"{name}.c")
    with open(path, "w") as f:
        f.write(src)
    return Oracle(oracle_build.build(source=path, output=os.path.join(str(tmp_path), f"lib{name}.so"),
                                     werror=False))


def test_real_oracle_passes_quick_pins(oracle_default):
    assert pins.run_quick(oracle_default) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    failures = pins.run_quick(_mutant_library(tmp_path, name), stop_at_first=True)
    assert failures, f"no pin caught the planted mistake {name!r}"
