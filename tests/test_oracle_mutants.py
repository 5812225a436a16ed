"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that the pins catch every one of them: a dropped term, a wrong sign or index,
a transposed operand, a lost parameter, a rounding slip in a codec.

Each mutant is one textual change of ``oracle/dcn4_oracle.c``, compiled into
a temporary library; the pins run in a child process so that a mutant that
reads out of bounds cannot crash the test runner."""
import os
import subprocess
import sys

import pytest

import oracle

SRC = open(oracle._SRC).read()
HERE = os.path.dirname(os.path.abspath(__file__))


def sub(old, new):
    return lambda s: s.replace(old, new)


def subs(*pairs):
    """several replacements applied one after another"""
    def f(s):
        for old, new in pairs:
            s = s.replace(old, new)
        return s
    return f


MUTANTS = {
    # offsets: x and y exchanged
    "dxdy_swapped_f32": subs(("float dx = load_f32(dtype, om, row + 2 * k);",
                              "float dx = load_f32(dtype, om, row + 2 * k + 1);"),
                             ("float dy = load_f32(dtype, om, row + 2 * k + 1);",
                              "float dy = load_f32(dtype, om, row + 2 * k);")),
    "dxdy_swapped_f64": subs(("double dx = load_f32(dtype, om, row + 2 * k);",
                              "double dx = load_f32(dtype, om, row + 2 * k + 1);"),
                             ("double dy = load_f32(dtype, om, row + 2 * k + 1);",
                              "double dy = load_f32(dtype, om, row + 2 * k);")),
    # taps enumerated column-major
    "tap_order_f64": sub("int k = i * s->kw + j; /* R3 */", "int k = j * s->kh + i;"),
    "tap_order_f32": sub("            int k = i * s->kw + j;\n            float dx",
                         "            int k = j * s->kh + i;\n            float dx"),
    # a bilinear corner dropped
    "corner_dropped_f32": sub("for (int r = 0; r < 4; ++r)", "for (int r = 0; r < 3; ++r)"),
    "corner_dropped_f64": sub("if (yy >= 0.0 && yy < s->H && xx >= 0.0 && xx < s->W) {\n        int64_t idx",
                              "if (!(a && b) && yy >= 0.0 && yy < s->H && xx >= 0.0 && xx < s->W) {\n        int64_t idx"),
    # fraction measured from the wrong side
    "row_fraction_flipped_f32": sub("r.lh = ty - fy;", "r.lh = 1.0f - (ty - fy);"),
    "col_fraction_flipped_f64": sub("double lh = py - y0, lw = px - x0;",
                                    "double lh = py - y0, lw = 1.0 - (px - x0);"),
    # corner weights transposed
    "weights_transposed_f32": sub("{hh * hw, hh * q.lw, q.lh * hw, q.lh * q.lw}",
                                  "{hh * hw, q.lh * hw, hh * q.lw, q.lh * q.lw}"),
    "weights_transposed_f64": sub("double w = (a ? lh : 1.0 - lh) * (b ? lw : 1.0 - lw);",
                                  "double w = (a ? lw : 1.0 - lw) * (b ? lh : 1.0 - lh);"),
    # convolution parameters lost or misapplied
    "dilation_ignored_f32": sub("by = (float)(yo * s->sh - s->ph + i * s->dh);",
                                "by = (float)(yo * s->sh - s->ph + i);"),
    "dilation_ignored_f64": sub("*py = (double)(yo * s->sh - s->ph + i * s->dh)",
                                "*py = (double)(yo * s->sh - s->ph + i)"),
    "stride_ignored_f32": sub("bx = (float)(xo * s->sw - s->pw + j * s->dw);",
                              "bx = (float)(xo - s->pw + j * s->dw);"),
    "pad_sign_f64": sub("*px = (double)(xo * s->sw - s->pw + j * s->dw)",
                        "*px = (double)(xo * s->sw + s->pw + j * s->dw)"),
    "offset_scale_ignored_f32": sub("ty = s->offset_scale * dy;", "ty = dy;"),
    "offset_scale_ignored_f64": sub("(double)s->offset_scale * dx", "dx"),
    # multi-scale: scale on the grid only, or centre lost
    "ms_scale_grid_only_f32": sub("ty = sg * uy;", "ty = sg * (float)(i - hy) + dy;"),
    "ms_centre_lost_f64": sub("*px = (double)(xo * s->sw - s->pw + hx) + sg",
                              "*px = (double)(xo * s->sw - s->pw) + sg"),
    # predicted per-pixel scale (R13): ignored, indexed transposed, clamped
    # the other way, or clamped with fmin (which turns a NaN into Smax)
    "pixel_scale_ignored_f32": sub("  if (s->pixel_scales) S = S * pscales[p * s->G + g];\n  if (s->max_scale > 0.0f && S > s->max_scale)",
                                   "  if (s->max_scale > 0.0f && S > s->max_scale)"),
    "pixel_scale_group_dropped_f64": sub("S = S * (double)pscales[p * s->G + g];",
                                         "S = S * (double)pscales[p * s->G];"),
    "pixel_scale_stride_f32": sub("S = S * pscales[p * s->G + g];", "S = S * pscales[p + g];"),
    "clamp_as_floor_f32": sub("if (s->max_scale > 0.0f && S > s->max_scale) S = s->max_scale;",
                              "if (s->max_scale > 0.0f && S < s->max_scale) S = s->max_scale;"),
    "clamp_fmin_f32": sub("if (s->max_scale > 0.0f && S > s->max_scale) S = s->max_scale;",
                          "if (s->max_scale > 0.0f) S = fminf(S, s->max_scale);"),
    # backward (R14): a factor lost, axes or corners exchanged, a sign flipped
    "bwd_weight_lost_in_gx": sub("const double t = m * w[r] * gyc;", "const double t = w[r] * gyc;"),
    "bwd_corner_weights_reversed_gx": sub("const double t = m * w[r] * gyc;",
                                          "const double t = m * w[3 - r] * gyc;"),
    "bwd_axes_swapped": subs(("gom[row + 2 * k] = m * f * gdc;", "gom[row + 2 * k] = m * f * GDR_;"),
                             ("gom[row + 2 * k + 1] = m * f * gdr;", "gom[row + 2 * k + 1] = m * f * gdc;"),
                             ("m * f * GDR_;", "m * f * gdr;")),
    "bwd_scale_factor_lost": sub("const double f = s->multiscale ? (double)sg : (double)s->offset_scale;",
                                 "const double f = 1.0;"),
    "bwd_row_derivative_sign": sub("const double dBr = hw * (v[2] - v[0]) + lw * (v[3] - v[1]);",
                                   "const double dBr = hw * (v[0] - v[2]) + lw * (v[3] - v[1]);"),
    "bwd_col_derivative_weights": sub("const double dBc = hh * (v[1] - v[0]) + lh * (v[3] - v[2]);",
                                      "const double dBc = lh * (v[1] - v[0]) + hh * (v[3] - v[2]);"),
    "bwd_sample_unweighted": sub("gm += gyc * B;", "gm += gyc * (v[0] + v[1] + v[2] + v[3]);"),
    # gradients of the scales (R17): the clamp, an axis, the direction or a
    # chain-rule factor lost
    "scale_grad_clamp_ignored": sub("if (clamped) dS = aS = 0.0;", "if (0) dS = aS = 0.0;"),
    "scale_grad_axes_swapped": sub("dS += m * (uy * gdr + ux * gdc);",
                                   "dS += m * (ux * gdr + uy * gdc);"),
    "scale_grad_direction_dropped": sub("const double uy = (float)(i - hy) + dy;",
                                        "const double uy = (float)(i - hy);"),
    "scale_grad_sigma_factor_lost": sub("if (gs) gs[g] += sig * dS;", "if (gs) gs[g] += dS;"),
    "scale_grad_prior_factor_lost": sub("if (gp) gp[p * G + g] = (double)scales[g] * dS;",
                                        "if (gp) gp[p * G + g] = dS;"),
    # DCNv3's softmax weights (R18): no max shift, the sum over the offsets,
    # a term of the sum lost, the offsets not passed through, the maximum
    # taken without the first weight
    "softmax_no_max_shift": subs(
        ("sum += exp((double)load_f32(dtype, om, base + 2 * K + k) - M);",
         "sum += exp((double)load_f32(dtype, om, base + 2 * K + k));"),
        ("exp((double)load_f32(dtype, om, base + 2 * K + k) - M) / sum;",
         "exp((double)load_f32(dtype, om, base + 2 * K + k)) / sum;")),
    "softmax_sum_over_offsets": sub("sum += exp((double)load_f32(dtype, om, base + 2 * K + k) - M);",
                                    "sum += exp((double)load_f32(dtype, om, base + k) - M);"),
    "softmax_last_term_lost": sub("for (int k = 0; k < K; ++k) sum +=", "for (int k = 0; k < K - 1; ++k) sum +="),
    "softmax_offsets_half_copied": sub("for (int i = 0; i < 2 * K; ++i) out[base + i]",
                                       "for (int i = 0; i < K; ++i) out[base + i]"),
    "softmax_max_skips_first": sub("for (int k = 0; k < K; ++k) {\n      const double m = load_f32(dtype, om, base + 2 * K + k);",
                                   "for (int k = 1; k < K; ++k) {\n      const double m = load_f32(dtype, om, base + 2 * K + k);"),
    # merged offset/weight layer: weight transposed, bias lost, a term lost
    "linear_weight_transposed": sub("(double)load_f32(dtype, weight, (int64_t)j * Cin + k);",
                                    "(double)load_f32(dtype, weight, (int64_t)k * Nout + j);"),
    "linear_bias_lost": sub("out[r * Nout + j] = acc + b;", "out[r * Nout + j] = acc;"),
    "linear_last_feature_lost": sub("for (int32_t k = 0; k < Cin; ++k) {\n        const double t",
                                    "for (int32_t k = 0; k < Cin - 1; ++k) {\n        const double t"),
    # the depthwise 3x3 convolution
    "dwconv_taps_flipped": sub("const int32_t yy = y + i - 1, xs = xx + j - 1;",
                               "const int32_t yy = y + 1 - i, xs = xx + 1 - j;"),
    "dwconv_taps_transposed": sub("const float wv = load_f32(dtype, w, (int64_t)(i * 3 + j) * C + c);",
                                  "const float wv = load_f32(dtype, w, (int64_t)(j * 3 + i) * C + c);"),
    "dwconv_bias_lost": sub("s64 += (double)bias[c];\n            acc = acc + bias[c];",
                            "acc = acc + bias[c];"),
    "dwconv_border_wrapped": sub("if (yy < 0 || yy >= H || xs < 0 || xs >= W) continue;  /* zero padding */",
                                 "if (yy < 0 || yy >= H) continue;"),
    # group bookkeeping
    "group_channels_interleaved": sub("int c = g * D + d;", "int c = d * s->G + g;"),
    "group_row_shared": sub("const int64_t row = (p * G + g) * 3 * K;",
                            "const int64_t row = (p * G) * 3 * K;"),
    "weight_index_fixed_f32": sub("float m = load_f32(dtype, om, row + 2 * K + k);",
                                  "float m = load_f32(dtype, om, row + 2 * K);"),
    "weight_dropped_f32": sub("float coef = m * w[r];", "float coef = w[r];"),
    "weight_dropped_f64": sub("acc += m * bilinear_zero_pad(", "acc += bilinear_zero_pad("),
    # borders
    "inside_test_low_f32": sub("if (!(yf >= -1.0f && yf <= (float)(s->H - 1)",
                               "if (!(yf >= 0.0f && yf <= (float)(s->H - 1)"),
    "inside_test_high_f32": sub("xf <= (float)(s->W - 1)))", "xf <= (float)(s->W - 2)))"),
    # the integer part taken from the offset alone, or the fraction's sign lost
    "base_dropped_f32": sub("float yf = by + fy, xf = bx + fx;", "float yf = fy, xf = bx + fx;"),
    "fraction_abs_f32": sub("r.lw = tx - fx;", "r.lw = fabsf(tx) - floorf(fabsf(tx));"),
    "corner_bound_off_by_one_f64": sub("xx < s->W) {", "xx <= s->W) {"),
    # codecs
    "bf16_round_half_up": sub("u += 0x7fffu + lsb;", "u += 0x8000u;"),
    "f16_subnormal_truncated": sub("double q = nearbyint(a * ldexp(1.0, 24));",
                                   "double q = floor(a * ldexp(1.0, 24));"),
    "f16_decode_bias": sub("v = ldexp((double)(1024 + f), e - 25);",
                           "v = ldexp((double)(1024 + f), e - 24);"),
    # counters and cost model
    "term_count_per_group": sub("terms += D;", "terms += 1;"),
    "ideal_bytes_om_2k": sub("int64_t om = (int64_t)s->N * Ho * Wo * s->G * 3 * K;",
                             "int64_t om = (int64_t)s->N * Ho * Wo * s->G * 2 * K;"),
    "output_size_off_by_one": sub("ho = ho / s->sh + 1;", "ho = ho / s->sh;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, tmp_path):
    src = MUTANTS[name](SRC)
    assert src != SRC, f"mutant {name} does not change the oracle source"
    csrc = tmp_path / "dcn4_oracle.c"
    csrc.write_text(src)
    (tmp_path / "dcn4_oracle.h").write_text(open(os.path.join(os.path.dirname(oracle._SRC), "dcn4_oracle.h")).read())
    lib = str(tmp_path / "libmutant.so")
    oracle.build(str(csrc), lib)
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_pins.py"), lib],
                       capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(HERE),
                       env={**os.environ, "PYTHONPATH": os.pathsep.join(
                           [os.path.dirname(HERE), HERE])})
    caught = r.returncode < 0 or "CAUGHT" in r.stdout
    assert caught, f"mutant {name} passed every pin:\n{r.stdout}\n{r.stderr[-2000:]}"
