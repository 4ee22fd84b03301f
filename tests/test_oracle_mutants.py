"""Mutation tests of the oracle's pins (CPU only).

Each mutant is a copy of ``oracle/oracle.c`` with one plausible mistake
planted by text substitution, built into a temporary library.  The pins must
fail on every mutant.  s01-s15 are the mistakes listed in the Pitfalls table
(section 5) of "Elementwise kernels in C: RMSNorm, RoPE, SiLU-mul, embedding,
add, argmax", each with the test the page says catches it; x01-x45 are further
slips (a wrong sign, index, dropped term or rounding) in the same code, x11-x16
in the softmax, x17-x20 in LayerNorm, x21-x25 in the GELU-gated multiply, x26-x29
in the RoPE cache, x30-x34 in multi-axis RoPE, x35-x40 in the f16 storage,
x41-x44 in the f32 range of the normalisation statistics, x45 in GELU's
infinite limit.
"""
import os
import tempfile

import pytest

import oracle
from pins import PINS

SRC = open(oracle.SRC).read()

# name -> (pin the page names as the catcher or None, [(old, new), ...])
MUTANTS = {
    "s01_eps_outside_root": ("rmsnorm_eps_is_inside_the_root",
                             [("1.0 / sqrt(ms + (double)eps)", "1.0 / (sqrt(ms) + (double)eps)")]),
    "s02_no_division_by_d": ("rmsnorm_eps_is_inside_the_root",
                             [("const double ms = ss / (double)d;", "const double ms = ss;")]),
    "s03_no_gain": ("hand_example",
                    [("v[i] = v[i] * inv * ld(dt, w, i);", "v[i] = v[i] * inv;")]),
    "s15_accumulator_per_call": ("rmsnorm_rows_are_independent_and_in_place",
                                 [("    double ss = 0.0;\n    for (int64_t i = 0; i < d; ++i) ss += v[i] * v[i];",
                                   "    static double ss = 0.0;\n    for (int64_t i = 0; i < d; ++i) ss += v[i] * v[i];")]),
    "s04_layouts_swapped": ("rope_interleaved_layout_and_position_zero",
                            [("if (layout == 0) {", "if (layout == 1) {")]),
    "s05_minus_theta": ("hand_example",
                        [("const double s = sin(ang);", "const double s = -sin(ang);")]),
    "s06_b_from_new_a": ("rope_is_a_rotation",
                         [("mu * (a * s + b * c)", "mu * (an * s + b * c)")]),
    "s07_rotate_all_D": ("rope_partial_rotary_and_scaling",
                         [("const int64_t rr = r;", "const int64_t rr = D;")]),
    "s08_ignore_mu": ("rope_partial_rotary_and_scaling",
                      [("const int64_t rr = r;\n    const double mu = (double)mu_f;",
                        "const int64_t rr = r;\n    const double mu = 1.0;")]),
    "s09_silu_as_sigmoid": ("silu_mul_saturates_without_nan",
                            [("const double s = gv / (1.0 + e);", "const double s = 1.0 / (1.0 + e);")]),
    "s10_exp_plus_g": ("silu_mul_saturates_without_nan",
                       [("double e = exp(-gv);", "double e = exp(gv);")]),
    "s11_row_at_id_not_id_times_d": ("embedding_gathers_rows",
                                     [("const size_t off = (size_t)ids[t] * (size_t)d;",
                                       "const size_t off = (size_t)ids[t];")]),
    "s12_argmax_ge": ("argmax_ties_nan_and_empty",
                      [("if (best < 0 || v > bv) {", "if (best < 0 || v >= bv) {")]),
    "s13_argmax_no_nan_check": ("argmax_ties_nan_and_empty",
                                [("if (isnan(v)) continue;", "")]),
    "s14_argmax_zero_for_none": ("argmax_ties_nan_and_empty",
                                 [("out[r] = best;", "out[r] = best < 0 ? 0 : best;")]),
    "x01_bf16_truncates": (None, [("nearbyint(v / q) * q", "trunc(v / q) * q")]),
    "x02_bf16_wrong_precision": (None, [("ldexp(1.0, binade - 7)", "ldexp(1.0, binade - 8)")]),
    "x03_angle_not_rounded_to_f32": (None, [("const double ang = (double)orc_rope_angle(p, inv_freq[i]);",
                                            "const double ang = (double)p * (double)inv_freq[i];")]),
    "x04_fused_norm_of_unrounded_sum": (None, [("for (int64_t i = 0; i < d; ++i) v[i] = ld(dt, h, r * d + i);",
                                                "for (int64_t i = 0; i < d; ++i) v[i] = ld(dt, x, r * d + i)"
                                                " + ld(dt, res, r * d + i);")]),
    "x05_cos_sin_swapped": (None, [("const double c = cos(ang);", "const double c = sin(ang);")]),
    "x06_silu_no_overflow_limit": (None, [("double e = exp(-gv);\n        if (e > FLT_MAX) e = INFINITY;",
                                           "double e = exp(-gv);\n")]),
    "x07_gain_reversed": (None, [("v[i] = v[i] * inv * ld(dt, w, i);", "v[i] = v[i] * inv * ld(dt, w, d - 1 - i);")]),
    "x08_add_subtracts": (None, [("st(dt, y, i, ld(dt, a, i) + ld(dt, b, i));",
                                  "st(dt, y, i, ld(dt, a, i) - ld(dt, b, i));")]),
    "x09_half_pairs_reversed": (None, [("*ib = i + r / 2;", "*ib = r - 1 - i;")]),
    "x10_rotation_sign": (None, [("mu * (a * c - b * s)", "mu * (a * c + b * s)")]),
    "x11_softmax_no_max_subtraction": ("softmax_max_is_subtracted",
                                       [("z[i] = exp(z[i] - m);", "z[i] = exp(z[i]);")]),
    "x12_softmax_min_subtracted": ("softmax_max_is_subtracted",
                                   [("else if (v > m) m = v;", "else if (v < m || m == -INFINITY) m = v;")]),
    "x13_temperature_multiplies": ("softmax_temperature",
                                   [("ld(dt, x, r * n + i) / (double)t;", "ld(dt, x, r * n + i) * (double)t;")]),
    "x14_softmax_divides_by_n": ("softmax_closed_forms",
                                 [("const double v = z[i] / sum;", "const double v = z[i] / (double)n;")]),
    "x15_softmax_no_f32_quotient_limit": ("softmax_special_values",
                                          [("if (v > FLT_MAX) v = INFINITY;\n            if (v < -FLT_MAX) v = -INFINITY;\n", "")]),
    "x16_softmax_exp_sign": ("softmax_temperature",
                             [("z[i] = exp(z[i] - m);", "z[i] = exp(m - z[i]);")]),
    "x17_layernorm_not_centred": ("layernorm_closed_forms",
                                  [("double v = f32_range(ld(dt, x, r * d + i) - mu) * inv * ld(dt, g, i);",
                                    "double v = f32_range(ld(dt, x, r * d + i)) * inv * ld(dt, g, i);")]),
    "x18_layernorm_eps_outside_root": ("layernorm_closed_forms",
                                       [("1.0 / sqrt(var + (double)eps);", "1.0 / (sqrt(var) + (double)eps);")]),
    "x19_layernorm_bias_dropped": ("layernorm_closed_forms", [("if (b) v += ld(dt, b, i);", "")]),
    "x20_variance_over_d_minus_1": ("layernorm_invariants",
                                    [("const double var = f32_range(ss) / (double)d;",
                                      "const double var = f32_range(ss) / (double)(d - 1);")]),
    "x21_gelu_no_sqrt2": ("gelu_brute", [("erfc(-x / sqrt(2.0))", "erfc(-x)")]),
    "x22_gelu_tanh_cubic_coefficient": ("gelu_brute", [("0.044715 * x * x * x", "0.44715 * x * x * x")]),
    "x23_geglu_up_ignored": ("gelu_symmetry_and_limits",
                             [("        double v = gl * u;\n", "        double v = gl;\n")]),
    "x24_gelu_forms_swapped": ("gelu_brute", [("if (form == 0) {", "if (form == 1) {")]),
    "x26_cache_transposed": ("rope_cached_rotation",
                             [("? (double)cos_c[(int64_t)p * half + i] : NAN;", "? (double)cos_c[i * max_pos + p] : NAN;")]),
    "x27_cached_rotation_sign": ("rope_cached_rotation",
                                 [("w[ia] = mu * (a * c - b * sn);", "w[ia] = mu * (a * c + b * sn);")]),
    "x28_cache_bad_position_zero": ("rope_cached_rotation",
                                    [("? (double)sin_c[(int64_t)p * half + i] : NAN;",
                                      "? (double)sin_c[(int64_t)p * half + i] : 0.0;"),
                                     ("? (double)cos_c[(int64_t)p * half + i] : NAN;",
                                      "? (double)cos_c[(int64_t)p * half + i] : 1.0;")]),
    "x29_cache_uses_cos_for_sin": ("rope_cache_values",
                                   [("sin_c[p * half + i] = (float)sin(ang);", "sin_c[p * half + i] = (float)cos(ang);")]),
    "x30_multi_axis_offset_stuck": ("rope_multi_brute_force",
                                    [("            off += da;\n            foff += da / 2;",
                                      "            foff += da / 2;")]),
    "x31_multi_freq_offset_stuck": ("rope_multi_brute_force",
                                    [("            foff += da / 2;", "            foff += 0;")]),
    "x32_multi_axis0_position": ("rope_multi_brute_force",
                                 [("const int32_t p = pos[t * A + a];", "const int32_t p = pos[t * A];")]),
    "x33_multi_half_of_first_axis": ("rope_multi_brute_force",
                                     [("rope_pair(layout, da, j, &ia, &ib);",
                                       "rope_pair(layout, dims[0], j, &ia, &ib);")]),
    "x34_multi_rotation_sign": ("rope_multi_axes_decompose",
                                [("w[ib] = mu * (x1 * sa + x2 * ca);", "w[ib] = mu * (x2 * ca - x1 * sa);")]),
    "x35_f16_truncates": ("f16_rounding_exhaustive",
                          [("const double r = nearbyint(a / q) * q;", "const double r = floor(a / q) * q;")]),
    "x36_f16_subnormal_spacing": ("f16_rounding_exhaustive",
                                  [("if (binade < -14) binade = -14;", "if (binade < -15) binade = -15;")]),
    "x37_f16_read_without_subnormals": ("f16_storage_through_ops",
                                        [("v = ldexp((double)fr, -24);", "v = ldexp((double)(1024 + fr), -25);")]),
    "x38_f16_read_bias": ("f16_storage_through_ops",
                          [("v = ldexp((double)(1024 + fr), ex - 25);", "v = ldexp((double)(1024 + fr), ex - 24);")]),
    "x39_f16_nan_read_as_inf": ("f16_storage_through_ops",
                                [("v = fr ? NAN : INFINITY;", "v = INFINITY;")]),
    "x40_f16_stored_as_bf16": ("f16_rounding_exhaustive",
                               [("((uint16_t*)p)[i] = orc_f16_from_f64(v);", "((uint16_t*)p)[i] = orc_bf16_from_f64(v);")]),
    "x25_gelu_tanh_no_f32_limit": ("gelu_symmetry_and_limits",
                                   [("if (e > FLT_MAX) e = INFINITY;  /* the f32", "/* the f32")]),
    "x41_rms_sum_of_squares_in_f64_range": ("norm_statistics_beyond_f32",
                                            [("    ss = f32_range(ss);\n", "")]),
    "x42_layernorm_variance_in_f64_range": ("norm_statistics_beyond_f32",
                                            [("const double var = f32_range(ss) / (double)d;",
                                              "const double var = ss / (double)d;")]),
    "x43_layernorm_sum_in_f64_range": ("norm_statistics_beyond_f32",
                                       [("const double mu = f32_range(sum) / (double)d;",
                                         "const double mu = sum / (double)d;")]),
    "x45_gelu_infinite_up_as_zero_times_inf": ("gelu_symmetry_and_limits",
                                               [("        if (form == 0 && isinf(u) && isfinite(x) && x != 0.0)\n"
                                                 "            v = ((x > 0.0) == (u > 0.0)) ? INFINITY : -INFINITY;\n", "")]),
    "x44_f32_range_threshold_at_flt_max_squared": ("norm_statistics_beyond_f32",
                                                   [("if (v >= 0x1.ffffffp127) return INFINITY;",
                                                     "if (v >= 0x1.ffffffp254) return INFINITY;")]),
}


def _build_mutant(name, subs, tmp):
    src = SRC
    for old, new in subs:
        assert src.count(old) == 1, f"{name}: pattern must occur once: {old!r}"
        src = src.replace(old, new)
    path = os.path.join(tmp, f"{name}.c")
    with open(path, "w") as f:
        f.write(src)
    lib = os.path.join(tmp, f"lib{name}.so")
    oracle.build(src=path, out=lib)
    return oracle.Oracle(lib)


@pytest.fixture(scope="module")
def tmpdir_mut():
    with tempfile.TemporaryDirectory() as d:
        yield d


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmpdir_mut):
    named, subs = MUTANTS[name]
    m = _build_mutant(name, subs, tmpdir_mut)
    m.set_threads(1)              # s15's shared accumulator must not race
    failed = []
    # the page's catcher runs first: a mutant with state (s15's accumulator
    # shared across calls) must meet it before other pins have moved that state
    order = ([named] if named is not None else []) + [p for p in PINS if p != named]
    for pin_name in order:
        try:
            PINS[pin_name](m)
        except AssertionError:
            failed.append(pin_name)
    assert failed, f"mutant {name} survived every pin"
    if named is not None:
        assert named in failed, f"{name}: the page's catcher {named} did not fail (failed: {failed})"


def test_unmutated_source_passes_every_pin(tmpdir_mut):
    """Control: the same build route with no substitution passes."""
    m = _build_mutant("control", [], tmpdir_mut)
    m.set_threads(1)
    for pin in PINS.values():
        pin(m)
