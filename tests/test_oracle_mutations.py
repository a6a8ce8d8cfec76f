"""Planted mistakes in copies of the oracle must each fail a pin (CPU only).

Each mutation rewrites one plausible error into a temporary copy of
oracle/fp8_oracle.c (a wrong tie rule, a lost sign, a dropped term, a wrong
index or bias, a reciprocal instead of a division, an extra rounding, ...),
compiles it with the oracle's own gcc flags, points the oracle wrapper at it and
runs the pin tests.  At least one pin must fail for every mutation; the real
oracle must pass all of them.  The committed oracle is never modified.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "fp8_oracle.c")

MUTATIONS = {
    "ties_round_up": ("return (unsigned char)(sign | (unsigned)((lo & 1) ? lo + 1 : lo));",
                      "return (unsigned char)(sign | (unsigned)(lo + 1));"),
    "negative_zero_lost": ("unsigned sign = signbit(t) ? 0x80u : 0u;",
                           "unsigned sign = (t < 0.0f) ? 0x80u : 0u;"),
    "saturate_to_nan": ("if (a >= ORACLE_E4M3_MAX) return (unsigned char)(sign | 0x7Eu);",
                        "if (a >= ORACLE_E4M3_MAX) return (unsigned char)(sign | 0x7Fu);"),
    "subnormal_scale": ("if (e == 0u) mag = ldexp((double)m, -9);",
                        "if (e == 0u) mag = ldexp((double)m, -10);"),
    "fnuz_bias": ("else mag = ldexp(1.0 + (double)m / 8.0, (int)e - 7);",
                  "else mag = ldexp(1.0 + (double)m / 8.0, (int)e - 8);"),
    "reciprocal_not_division": ("float t = isnan(v) ? v : v / s_act;", "float t = isnan(v) ? v : v * (1.0f / s_act);"),
    "transposed_operand": ("const unsigned char* b = wq + n * K;", "const unsigned char* b = wq + m * K;"),
    "dropped_weight_scale": ("val = (acc * (double)s_act) * (double)s_w[n];", "val = acc * (double)s_act;"),
    "epilogue_through_fp32": ("out[m * ldo + n] = oracle_f64_to_bf16(val);",
                              "out[m * ldo + n] = oracle_f64_to_bf16((double)(float)val);"),
    "rms_missing_mean": ("return (float)(1.0 / sqrt(ss / (double)K + (double)eps));",
                         "return (float)(1.0 / sqrt(ss + (double)eps));"),
    "rms_missing_eps": ("return (float)(1.0 / sqrt(ss / (double)K + (double)eps));",
                        "return (float)(1.0 / sqrt(ss / (double)K));"),
    "fused_skips_bf16": ("float yb = oracle_bf16_to_f32(oracle_f32_to_bf16(yf));", "float yb = yf;"),
    "weight_scale_fnuz_max": ("s = (amax == 0.0f) ? 1.0f : amax / 448.0f;", "s = (amax == 0.0f) ? 1.0f : amax / 240.0f;"),
    "bf16_truncates": ("r = nearbyint(q);\n        res = ldexp(r, ex - 8);", "r = floor(q);\n        res = ldexp(r, ex - 8);"),
    "gamma_ignored": ("float yk = xn * oracle_bf16_to_f32(gamma[k]);", "float yk = xn;"),
    "silu_sigmoid_sign": ("return (float)(d / (1.0 + exp(-d)));", "return (float)(d / (1.0 + exp(d)));"),
    "silu_mul_skips_bf16": ("float hb = oracle_bf16_to_f32(oracle_f32_to_bf16(sig_g * u));", "float hb = sig_g * u;"),
    "silu_in_fp32": ("return (float)(d / (1.0 + exp(-d)));", "return (float)g / (1.0f + expf(-g));"),
    "silu_mul_swapped": ("float hf = s * oracle_bf16_to_f32(up[m * ldu + i]);",
                         "float hf = silu_f32(oracle_bf16_to_f32(up[m * ldu + i])) * oracle_bf16_to_f32(gate[m * ldg + i]);"),
    "per_token_tensor_amax": ("const float s = oracle_act_scale(row, ldx, gamma, eps, 1, K);",
                              "const float s = oracle_act_scale(x, ldx, gamma, eps, M, K);"),
    "requant_to_min_scale": ("if (scales[i] > s_max) s_max = scales[i];", "if (scales[i] < s_max) s_max = scales[i];"),
    "requant_drops_shard_scale": ("w = (float)d * scales[i];", "w = (float)d;"),
    "requant_shard_offset": ("r0 += rows[i];", "r0 += rows[0];"),
    "requant_reciprocal": ("out[e] = oracle_e4m3_encode(w / s_max);", "out[e] = oracle_e4m3_encode(w * (1.0f / s_max));"),
    "per_tensor_amax_first_row": ("for (int64_t i = 0; i < N * K; ++i) {\n        float a = fabsf(W[i]);",
                                  "for (int64_t i = 0; i < K; ++i) {\n        float a = fabsf(W[i]);"),
    "rows_scale_first_row": ("oracle_scaled_mm(xq + m * K, wq, s_rows[m], s_w,",
                             "oracle_scaled_mm(xq + m * K, wq, s_rows[0], s_w,"),
}

PIN_TESTS = [
    pins.test_e4m3_table_structure,
    pins.test_e4m3_table_matches_exact_enumeration,
    pins.test_e4m3_roundtrip_all_finite_codes,
    pins.test_e4m3_hand_values,
    lambda: [pins.test_quant_encoder_exhaustive_bf16(s) for s in (1.0, 0.5, 3.0, 1.0 / 7.0, 0.2)],
    pins.test_encoder_random_fp32_vs_brute_force,
    pins.test_bf16_rounding_against_exact_and_torch,
    pins.test_tiny_product_hand_worked,
    pins.test_double_rounding_trap,
    pins.test_brute_force_2x3x4_against_exact_rationals,
    pins.test_invariants_scale_zero_identity_sign_merge,
    pins.test_rmsnorm_closed_forms,
    pins.test_rmsnorm_against_numpy_formula,
    lambda: pins.test_fused_quant_is_byte_exact_against_unfused(3, 32),
    pins.test_act_scale_and_weight_quant_definitions,
    pins.test_silu_against_scipy_expit_all_bf16,
    pins.test_silu_closed_forms_and_identities,
    pins.test_silu_mul_product_and_power_of_two_scaling,
    lambda: pins.test_silu_mul_quant_is_byte_exact_against_unfused(1),
    pins.test_per_token_brute_force_against_exact_rationals,
    pins.test_per_token_rows_are_independent_and_scale_covariant,
    pins.test_per_token_rmsnorm_row_is_the_static_quant_of_that_row,
    pins.test_rows_gemm_with_equal_scales_is_the_per_tensor_gemm,
    pins.test_requant_brute_force_against_exact_rationals,
    pins.test_requant_matches_ieee_steps_and_nearest_search,
    pins.test_requant_equal_scales_is_the_identity,
    pins.test_requant_power_of_two_ratio_closed_form,
    pins.test_requant_sign_symmetry_and_monotone_in_the_ratio,
    pins.test_weight_per_tensor_definition,
    pins.test_max_scale_layer_with_equal_scales_is_the_exact_merge,
]


def _failing_pins(stop_at_first=False):
    failed = 0
    for t in PIN_TESTS:
        try:
            with np.errstate(all="ignore"):
                t()
        except (AssertionError, ValueError, IndexError):
            failed += 1
            if stop_at_first:
                break
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "mut.c")
        so = os.path.join(d, "libmut.so")
        with open(c, "w") as f:
            f.write(src.replace(old, new))
        subprocess.check_call(["gcc", *oracle.GCC_FLAGS, "-Wno-unused", c, "-o", so, "-lm"])
        saved = oracle._lib
        oracle._lib = oracle.load(so)
        try:
            n_failed = _failing_pins(stop_at_first=True)
        finally:
            oracle._lib = saved
    assert n_failed >= 1, f"planted mistake '{name}' passed every pin"


def test_real_oracle_passes_every_pin():
    assert _failing_pins() == 0
