"""Planted mistakes in the oracle must each fail at least one pin.

Each case copies ``oracle/mn_oracle.c``, applies one textual change that
models a plausible slip (a dropped term, a wrong sign, divisor or index, a
swapped operand), builds it with the oracle's own gcc recipe into a
temporary directory and runs the pin battery on it. The mutant must fail.
The real oracle source is never modified.
"""
import os

import pytest

import oracle
import oracle_pins

MUTANTS = {
    "rms_eps_dropped": ("return 1.0 / sqrt(ss / (double)D + eps);",
                        "return 1.0 / sqrt(ss / (double)D + 0.0 * eps);"),
    "rms_eps_outside_sqrt": ("return 1.0 / sqrt(ss / (double)D + eps);",
                             "return 1.0 / (sqrt(ss / (double)D) + eps);"),
    "ln_sample_variance": ("*rstd = 1.0 / sqrt(v / (double)D + eps);",
                           "*rstd = 1.0 / sqrt(v / (double)(D > 1 ? D - 1 : 1) + eps);"),
    "ln_uncentred_variance": ("v += (x[j] - mu) * (x[j] - mu);", "v += x[j] * x[j];"),
    "ln_mean_divisor": ("double mu = s / (double)D;", "double mu = s / (double)(D + 1);"),
    "rms_c1_divisor": ("c1 /= (double)D;\n        if (dX) {",
                       "c1 /= (double)(D + 1);\n        if (dX) {"),
    "ln_c2_sign": ("- c2 -", "+ c2 -"),
    "ln_c2_dropped": ("c2 += w.dy[j] * w.g[j];", "c2 += 0.0;"),
    "ln_dx_rstd_dropped": ("dX[i * D + j] = r * (w.dy[j] * w.g[j] - c2 - w.xh[j] * c1);",
                           "dX[i * D + j] = (w.dy[j] * w.g[j] - c2 - w.xh[j] * c1);"),
    "rms_dgamma_uses_x": ("dgamma[j] += w.dy[j] * w.xh[j];", "dgamma[j] += w.dy[j] * w.x[j];"),
    "ln_dbeta_weighted": ("dbeta[j] += w.dy[j];", "dbeta[j] += w.dy[j] * w.g[j];"),
    "fused_dh_dropped": ("dX[i * D + j] = present(DH) ? w.dh[j] + d : d;",
                         "dX[i * D + j] = d;"),
    "fused_residual_ignored": ("w->x[j] = w->x[j] + w->r[j];", "w->x[j] = w->x[j];"),
    "rms_gamma_reversed": ("Y[i * D + j] = w.x[j] * r * w.g[j];",
                           "Y[i * D + j] = w.x[j] * r * w.g[D - 1 - j];"),
    "ln_beta_sign": ("* w.g[j] + w.b[j];", "* w.g[j] - w.b[j];"),
    "rms_dy_wrong_row": ("get_row(DY, i, D, w.dy);\n        double r = rms_rstd",
                         "get_row(DY, (i + 1) % N, D, w.dy);\n        double r = rms_rstd"),
    "codec_exponent_off_by_one": ("ldexp((double)(1024 + f), e - 25)",
                                  "ldexp((double)(1024 + f), e - 24)"),
    "codec_ties_away": ("return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;", "return fl + 1.0;"),
    "codec_subnormal_scale": ("v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);"),
    "bf16_decode_exponent": ("v = ldexp((double)(128 + f), e - 134);",
                             "v = ldexp((double)(128 + f), e - 133);"),
    "bf16_encode_mantissa": ("return (uint16_t)encode_binary(v, 7, -126, 127);",
                             "return (uint16_t)encode_binary(v, 7, -125, 127);"),
    "f32_operand_stride": ("const float* f = (const float*)a.p + o;",
                           "const float* f = (const float*)a.p + o / 2;"),
    "bf16_reads_f16_table": ("for (int64_t j = 0; j < D; ++j) dst[j] = bf16_table[b[j]];",
                             "for (int64_t j = 0; j < D; ++j) dst[j] = f16_table[b[j]];"),
    "dyt_derivative_linear": ("double s = 1.0 - t * t;", "double s = 1.0 - t;"),
    "dyt_dx_alpha_dropped": ("dX[i * D + j] = w.dy[j] * w.g[j] * alpha * s;",
                             "dX[i * D + j] = w.dy[j] * w.g[j] * s;"),
    "dyt_dalpha_gamma_dropped": ("da += w.dy[j] * w.g[j] * w.x[j] * s;",
                                 "da += w.dy[j] * w.x[j] * s;"),
    "poly_power_factor_dropped": ("dX[i * D + j] += (double)p * pow(w.x[j], (double)(p - 1)) * du;",
                                  "dX[i * D + j] += pow(w.x[j], (double)(p - 1)) * du;"),
    "poly_weights_reversed": ("y += wp[p - 1] * (pow(w.x[j], (double)p) * r[p - 1]);",
                              "y += wp[3 - p] * (pow(w.x[j], (double)p) * r[p - 1]);"),
    "modrms_scale_not_offset": ("Y[i * D + j] = w.g[j] * (w.x[j] * r) * (1.0 + w.r[j]) + w.b[j];",
                                "Y[i * D + j] = w.g[j] * (w.x[j] * r) * w.r[j] + w.b[j];"),
    "modrms_sample_interleaved": ("const int64_t b = i / S;\n        get_row(X, i, D, w.x);\n"
                                  "        get_row(SC, b, D, w.r);\n        get_row(SH",
                                  "const int64_t b = i % B;\n        get_row(X, i, D, w.x);\n"
                                  "        get_row(SC, b, D, w.r);\n        get_row(SH"),
    "modrms_dscale_unweighted": ("dscale[b * D + j] += w.dy[j] * w.xh[j] * w.g[j];",
                                 "dscale[b * D + j] += w.dy[j] * w.xh[j];"),
    "gn_gamma_by_group": ("Y[slice * M + k] = (w.x[k] - mu) * r * gam[c] + bet[c];",
                          "Y[slice * M + k] = (w.x[k] - mu) * r * gam[g] + bet[c];"),
    "gemv_layernorm_as_rms": ("int rc = ln ? ln_forward(X, G, B, M, K, eps, xn, mean, rstd)",
                              "int rc = 0 ? ln_forward(X, G, B, M, K, eps, xn, mean, rstd)"),
    "gemv_w_row_off_by_one": ("get_row(W, k, N, wrow);", "get_row(W, (k + 1) % K, N, wrow);"),
    "gn_channel_stride": ("const int64_t c = g * (C / groups) + k / L;\n                if (dX)",
                          "const int64_t c = g * (C / groups) + k % (C / groups);\n"
                          "                if (dX)"),
}


def _build_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    with open(oracle.SRC_PATH) as f:
        src = f.read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    src = src.replace(old, new, 1)
    path = os.path.join(tmp_path, f"{name}.c")
    with open(path, "w") as f:
        f.write(src)
    return oracle.Oracle(oracle.compile_library(path, os.path.join(tmp_path, f"lib{name}.so")))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    o = _build_mutant(str(tmp_path), name)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(o)
        except AssertionError as e:
            caught.append(f"{pin.__name__}: {str(e)[:120]}")
            break
    assert caught, f"no pin catches the planted mistake {name}"
