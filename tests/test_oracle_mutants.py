"""Planted mistakes in copies of the oracle must each fail at least one pin.

Each mutant is oracle.c with one textual change (a dropped term, a wrong
coefficient, sign or index, a skipped rounding rule), built with the same
flags into a temporary library.  This shows the pins in oracle_pins.py are
strong enough that a plausible slip anywhere in the oracle is caught.
"""
import os

import pytest

import oracle
from oracle import build as oracle_build
from oracle_pins import ALL_PINS

MUTANTS = {
    "m_uses_beta2": ("float m_old = s->beta1 * *m;", "float m_old = s->beta2 * *m;"),
    "v_uses_g_not_g2": ("float v_in = s->one_m_b2 * g2;", "float v_in = s->one_m_b2 * g;"),
    "no_bias_correction_2": ("float root_hat = root / s->bc2_sqrt;", "float root_hat = root;"),
    "no_eps": ("float den = root_hat + s->eps;", "float den = root_hat;"),
    "no_weight_decay": ("float w_decayed = *w * s->decay;", "float w_decayed = *w;"),
    "update_sign": ("float w_new = w_decayed - delta;", "float w_new = w_decayed + delta;"),
    "clip_ignored": ("float g = g_raw * c;", "float g = g_raw;"),
    "norm_sums_values": ("acc = acc + x * x;\n    }\n    return acc;\n}\n\n/* Same for a bf16",
                         "acc = acc + x;\n    }\n    return acc;\n}\n\n/* Same for a bf16"),
    "clip_no_clamp": ("if (c > 1.0) c = 1.0;", ""),
    "clip_no_epsilon": ("double c = max_norm / (norm + 1e-6);", "double c = max_norm / norm;"),
    "step_size_no_correction": ("s->step_size = (float)(lr / (1.0 - p1));",
                                "s->step_size = (float)lr;"),
    "decay_ignores_lr": ("s->decay = (float)(1.0 - lr * wd);", "s->decay = (float)(1.0 - wd);"),
    "power_off_by_one": ("while (t > 0) {", "t += 1;\n    while (t > 0) {"),
    "bf16_truncates": ("kept += 1u;", "kept += 0u;"),
    "bf16_ties_away": ("(dropped == 0x8000u && (kept & 1u))", "(dropped == 0x8000u)"),
    "bf16_grad_decode": ("uint32_t u = (uint32_t)h << 16;", "uint32_t u = (uint32_t)h << 15;"),
    "copy_of_old_master": (
        "oracle_update_one(&master[i], &exp_avg[i], &exp_avg_sq[i], g, clip, &s);\n"
        "        if (param_bf16) param_bf16[i] = oracle_f32_to_bf16(master[i]);",
        "if (param_bf16) param_bf16[i] = oracle_f32_to_bf16(master[i]);\n"
        "        oracle_update_one(&master[i], &exp_avg[i], &exp_avg_sq[i], g, clip, &s);"),
    "moment_order_swapped": ("*m = m_new;\n    *v = v_new;", "*m = v_new;\n    *v = m_new;"),
    "scale_not_applied": ("return (float)(grad_scale * clip);", "return (float)clip;"),
    "scale_squared_in_norm": ("double norm = grad_scale * sqrt(sumsq);",
                              "double norm = grad_scale * grad_scale * sqrt(sumsq);"),
    # 8-bit moment state
    "q8_subnormal_exponent": ("mag = ldexp((double)M, 1 - bias - mbits);",
                              "mag = ldexp((double)M, -bias - mbits);"),
    "q8_ties_away": ("(d == best_d && (c & 1) == 0)", "(d == best_d)"),
    "q8_saturates": ("if (a >= next) return (uint8_t)(sign | (top + 1));",
                     "if (a >= next) return (uint8_t)(sign | top);"),
    "q8_no_overflow_candidate": ("for (int c = 1; c <= top + 1; ++c) {", "for (int c = 1; c <= top; ++c) {"),
    "q8_largest_e4m3": ("const double largest = format == ORACLE_E4M3 ? 448.0 : 57344.0;",
                        "const double largest = format == ORACLE_E4M3 ? 480.0 : 57344.0;"),
    "q8_exponent_floor": ("int e = -127;\n    while", "int e = -126;\n    while"),
    "q8_exponent_inclusive": ("while (ldexp(largest, e) < absmax) ++e;",
                              "while (ldexp(largest, e) <= absmax) ++e;"),
    "q8_scale_bias": ("(float)ldexp(oracle_fp8_value(codes[i], format), s - 127);",
                      "(float)ldexp(oracle_fp8_value(codes[i], format), s - 126);"),
    "q8_scale_index": ("const int s = scales[i / ORACLE_QBLOCK];",
                       "const int s = scales[i / (2 * ORACLE_QBLOCK)];"),
    "q8_step_one_scale": ("const int64_t blk = b0 / ORACLE_QBLOCK;", "const int64_t blk = 0;"),
    "q8_m_decoded_as_e5m2": ("oracle_dequantize(m_codes + b0, m_scales + blk, len, ORACLE_E4M3, m);",
                             "oracle_dequantize(m_codes + b0, m_scales + blk, len, ORACLE_E5M2, m);"),
    "q8_nan_block_codes": ("memset(codes + b0, 255, (size_t)len);", "memset(codes + b0, 0, (size_t)len);"),
    "q8_nan_block_ignored": ("if (!isfinite(a)) finite = 0;", "if (!isfinite(a)) finite = 1;"),
}


@pytest.fixture(scope="module")
def source():
    with open(oracle_build.SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, source, tmp_path):
    old, new = MUTANTS[name]
    assert source.count(old) == 1, f"mutation anchor for {name} not unique in oracle.c"
    src = tmp_path / "oracle_mutant.c"
    src.write_text(source.replace(old, new))
    lib = oracle_build.build(str(src), str(tmp_path / "liboracle_mutant.so"))
    o = oracle.Oracle(lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(o)
        except (AssertionError, ValueError, OverflowError, ZeroDivisionError):
            caught.append(pin.__name__)
    assert caught, f"mutant {name} passed every pin"
    os.remove(lib)
