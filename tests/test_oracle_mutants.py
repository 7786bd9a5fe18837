"""Planted mistakes in the oracle must fail a pin.

Each case copies oracle/adaln_oracle.c, applies one plausible mistake (a
sign, a dropped term, a swapped operand, a missing rounding), compiles the
copy, points the oracle module at it and runs the fast pins.  At least one
pin must fail for every mutant -- otherwise the pins would not notice that
mistake in the real oracle.  CPU only.
"""

from __future__ import annotations

import os

import pytest

import test_oracle_pins as P

MUTANTS = {
    "welford_delta_sign": ("float delta = x - s->mean;", "float delta = s->mean - x;"),
    "welford_m2_uses_delta_squared": ("s->m2 = fmaf(delta, x - s->mean, s->m2);", "s->m2 = fmaf(delta, delta, s->m2);"),
    "welford_count_not_incremented": ("s->n = s->n + 1.0f;", "s->n = s->n + 0.5f;"),
    "combine_drops_cross_term": ("c.m2 = (a.m2 + b.m2) + (delta * delta) * (a.n * f);", "c.m2 = (a.m2 + b.m2);"),
    "combine_wrong_weight": ("float f = b.n / c.n;", "float f = a.n / c.n;"),
    "combine_wrong_guard": ("if (b.n == 0.0f) return a;", "if (b.n == 0.0f) return b;"),
    "unbiased_variance_fp32": ("float var = lane[0].m2 / (float)D;", "float var = lane[0].m2 / (float)(D - 1);"),
    "eps_dropped_fp32": ("float t = var + eps;", "float t = var;"),
    "fp64_no_mean_subtraction": ("double c = (double)orc_f32_from_bf16(x[j]) - mean;", "double c = (double)orc_f32_from_bf16(x[j]);"),
    "xhat_not_rounded": ("float xhat = rb(n);", "float xhat = n;"),
    "one_plus_scale_not_rounded": ("float one_plus = rb(1.0f + orc_f32_from_bf16(sc));", "float one_plus = 1.0f + orc_f32_from_bf16(sc);"),
    "shift_and_scale_swapped": ("const uint16_t* sc = scale + (r / S) * D;", "const uint16_t* sc = shift + (r / S) * D;"),
    "gate_product_not_rounded": ("float t = rb(orc_f32_from_bf16(g[j]) * orc_f32_from_bf16(upd[i]));", "float t = orc_f32_from_bf16(g[j]) * orc_f32_from_bf16(upd[i]);"),
    "qk_affine_swapped": ("float y = w ? fmaf(orc_f32_from_bf16(w[j]), xn, orc_f32_from_bf16(b[j])) : xn;", "float y = w ? fmaf(orc_f32_from_bf16(b[j]), xn, orc_f32_from_bf16(w[j])) : xn;"),
    "gelu_cubic_coeff": ("const double k1 = 0.044715;", "const double k1 = 0.0447;"),
    "gelu_sign": ("return z / (1.0 + exp(-2.0 * u));", "return z / (1.0 + exp(2.0 * u));"),
    "rne_ties_away": ("if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;", "if (dropped >= 0x8000u) kept += 1u;"),
    "fused_norms_old_residual": ("return orc_ln_modulate(res_out, B, S, D, scale, shift", "return orc_ln_modulate(res, B, S, D, scale, shift"),
    "fused_skips_residual_update": ("int rc = orc_residual_gate_add(res, gate, upd, B, S, D, mode, res_out);", "int rc = orc_residual_gate_add(res, gate, upd, B, S, D, mode, res_out); memcpy(res_out, res, (size_t)(B * S * D) * 2);"),
    "rms_eps_dropped": ("  float t = ms + eps;\n  float s = sqrtf(t);\n  return 1.0f / s;", "  float t = ms;\n  float s = sqrtf(t);\n  return 1.0f / s;"),
    "rms_sum_not_divided": ("return 1.0 / sqrt(ss / (double)D + (double)eps);", "return 1.0 / sqrt(ss + (double)eps);"),
    "rms_lane_sum_drops_partner": ("lane[l] = lane[l] + lane[l + off];", "lane[l] = lane[l];"),
    "fp64_tail_product_not_rounded": ("double y = rb64(xhat * one_plus);", "double y = xhat * one_plus;"),
    "qk_rms_rounds_before_weight": ("float y = w ? xn * orc_f32_from_bf16(w[j]) : xn;", "float y = w ? rb(xn) * orc_f32_from_bf16(w[j]) : xn;"),
    "modulate_scale_row_per_sample": ("const uint16_t* sc = scale + b * ssc_b + s * ssc_s;", "const uint16_t* sc = scale + b * ssc_b;"),
    "temb_slice_order_swapped": ("out[(m * R + r) * D + d] = table[m * D + d] + t;", "out[(r * nmod + m) * D + d] = table[m * D + d] + t;"),
    "temb_table_row_wrong": ("out[(m * R + r) * D + d] = table[m * D + d] + t;", "out[(m * R + r) * D + d] = table[d] + t;"),
    "fp8_ties_away": ("if (a > mid || (a == mid && ((lo + 1) & 1) == 0)) code = lo + 1;", "if (a >= mid) code = lo + 1;"),
    "fp8_subnormal_step": ("double v = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);", "double v = e == 0 ? ldexp((double)m, -10) : ldexp(1.0 + m / 8.0, e - 7);"),
    "fp8_no_clamp": ("        if (v > 448.0f) v = 448.0f;\n", ""),
    "fp8_scale_not_inverted": ("        float v = orc_f32_from_bf16(y[i]) * inv;", "        float v = orc_f32_from_bf16(y[i]) * qscale;"),
    "fold_rounds_xhat": ("o[j] = orc_bf16_from_f32(fmaf(w, n, orc_f32_from_bf16(sh[j])));", "o[j] = orc_bf16_from_f32(fmaf(w, rb(n), orc_f32_from_bf16(sh[j])));"),
    "fold_weight_not_rounded": ("float w = rb(1.0f + orc_f32_from_bf16(sc[j]));", "float w = 1.0f + orc_f32_from_bf16(sc[j]);"),
    "bias_not_rounded": ("double z = rb64((double)orc_f32_from_bf16(x[i]) + (double)orc_f32_from_bf16(bias[j]));", "double z = (double)orc_f32_from_bf16(x[i]) + (double)orc_f32_from_bf16(bias[j]);"),
}

ANCHOR_COUNT = {"shift_and_scale_swapped": 3}

FAST_PINS = [
    lambda o: P.test_worked_d4(o, P.FP32),
    lambda o: P.test_worked_d4(o, P.FP64),
    lambda o: [P.test_constant_rows(o, m, D, c) for m in (P.FP32, P.FP64) for D in (12, 4096) for c in (1.0, -3.5)],
    lambda o: P.test_moments_of_xhat(o, P.FP32),
    lambda o: P.test_moments_of_xhat(o, P.FP64),
    lambda o: P.test_shift_invariance_fp64_bitwise(o),
    lambda o: P.test_welford_small_exact_cases(o),
    lambda o: P.test_combine_identities(o),
    lambda o: P.test_combine_vs_fractions(o),
    lambda o: P.test_fp32_stats_vs_fractions(o, 64),
    lambda o: P.test_fp64_stats_vs_fractions(o),
    lambda o: P.test_bf16_from_f64_matches_f32_path_on_floats(o),
    lambda o: P.test_elementwise_tail_equals_torch_eager(o),
    lambda o: P.test_residual_gate_add_equals_torch_eager(o, P.FP32),
    lambda o: P.test_qk_fp64_equals_torch_affine_layer_norm(o),
    lambda o: P.test_qk_fp32_within_one_ulp_of_fp64(o),
    lambda o: P.test_fused_residual_worked_d4(o, P.FP32),
    lambda o: P.test_fused_residual_equals_torch_eager_chain(o),
    lambda o: P.test_rms_worked_d4(o, P.FP32),
    lambda o: P.test_rms_fp64_mode_equals_torch_rms_norm(o),
    lambda o: P.test_rms_constant_rows(o, P.FP32, 2240),
    lambda o: P.test_rms_tail_equals_torch_eager(o),
    lambda o: P.test_qk_rms_fp64_equals_torch_rms_norm(o),
    lambda o: P.test_qk_rms_fp32_equals_torch_fp32_tail(o),
    lambda o: P.test_elementwise_tail_fp64_mode_equals_torch_eager(o, "layer"),
    lambda o: P.test_elementwise_tail_fp64_mode_equals_torch_eager(o, "rms"),
    lambda o: P.test_modulate_worked(o, P.FP32),
    lambda o: P.test_modulate_equals_torch_eager(o, P.FP32, True),
    lambda o: P.test_temb_slices_equal_torch_chunks(o, False),
    lambda o: P.test_fp8_decode_table_vs_torch(o),
    lambda o: P.test_fp8_encode_vs_torch(o),
    lambda o: P.test_ln_modulate_fp8_worked(o, P.FP32),
    lambda o: P.test_ln_modulate_fp8_tail_vs_torch(o, 0.0123),
    lambda o: P.test_fold_worked(o, P.FP32),
    lambda o: P.test_fold_fp32_tail_exact(o),
    lambda o: P.test_gelu_f64_vs_torch(o),
    lambda o: P.test_bias_gelu_rounds_after_bias(o),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(orc, tmp_path, name):
    src = open(os.path.join(os.path.dirname(orc.__file__), "adaln_oracle.c")).read()
    old, new = MUTANTS[name]
    # the mistake is planted at every occurrence of its anchor (the LayerNorm and RMSNorm
    # chains share some source lines); the anchor must exist
    want = ANCHOR_COUNT.get(name, 1)
    assert src.count(old) == want, "mutation anchor found %d times, expected %d: %r" % (src.count(old), want, old)
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = orc.compile_source(str(path), str(tmp_path / "libmutant.so"))
    saved = orc._lib
    orc._lib = orc.load_library(lib)
    try:
        caught = []
        for i, pin in enumerate(FAST_PINS):
            try:
                pin(orc)
            except (AssertionError, ValueError, FloatingPointError):
                caught.append(i)
                break
        assert caught, "mutant %s passed every pin" % name
    finally:
        orc._lib = saved


def test_unmutated_oracle_passes_fast_pins(orc):
    for pin in FAST_PINS:
        pin(orc)
