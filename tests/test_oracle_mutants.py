"""Planted mistakes in the oracle must be caught by its pins.

Each case copies oracle.c, applies one textual mutation (a dropped term, a wrong sign,
a wrong index, a transposed operand, a wrong count), compiles the copy with gcc into a
temporary library, and runs every pin in oracle_pins.py against it.  The test passes
when at least one pin fails on the mutant.  The real oracle source is never modified.
"""
import os
import shutil

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTATIONS = [
    ("rms_count", "double mean_sq = sum_sq / (double)N;",
     "double mean_sq = sum_sq / (double)(N + 1);"),
    ("rms_eps_outside_sqrt", "return 1.0 / sqrt(mean_sq + eps);",
     "return 1.0 / (sqrt(mean_sq) + eps);"),
    ("rms_drop_eps", "return 1.0 / sqrt(mean_sq + eps);", "return 1.0 / sqrt(mean_sq);"),
    ("ln_unbiased_var", "double var = sum_dev_sq / (double)N;",
     "double var = sum_dev_sq / (double)(N - 1);"),
    ("ln_drop_eps", "*rstd_out = 1.0 / sqrt(var + eps);", "*rstd_out = 1.0 / sqrt(var);"),
    ("ln_var_about_zero", "double d = elem(x, dtype, base + j) - mu;",
     "double d = elem(x, dtype, base + j);"),
    ("ln_beta_sign", "y[k * N + j] = xhat * elem(gamma, gdtype, j) + elem(beta, gdtype, j);",
     "y[k * N + j] = xhat * elem(gamma, gdtype, j) - elem(beta, gdtype, j);"),
    ("rms_gamma_reversed",
     "y[k * N + j] = elem(x, dtype, row * N + j) * r * elem(gamma, gdtype, j);",
     "y[k * N + j] = elem(x, dtype, row * N + j) * r * elem(gamma, gdtype, N - 1 - j);"),
    ("rms_gamma_read_as_x_type",
     "y[k * N + j] = elem(x, dtype, row * N + j) * r * elem(gamma, gdtype, j);",
     "y[k * N + j] = elem(x, dtype, row * N + j) * r * elem(gamma, dtype, j);"),
    ("ln_beta_read_as_x_type", "xhat * elem(gamma, gdtype, j) + elem(beta, gdtype, j);",
     "xhat * elem(gamma, gdtype, j) + elem(beta, dtype, j);"),
    ("f16_exponent_bias", "v = ldexp((double)(frac + 1024), e - 25);",
     "v = ldexp((double)(frac + 1024), e - 24);"),
    ("f16_no_implicit_bit", "v = ldexp((double)(frac + 1024), e - 25);",
     "v = ldexp((double)frac, e - 25);"),
    ("f16_subnormal_scale", "v = ldexp((double)frac, -24);", "v = ldexp((double)frac, -25);"),
    ("f16_sign_dropped", "return (h & 0x8000) ? -v : v;", "return v;"),
    ("round_exponent_off", "int e = k - 1;", "int e = k;"),
    ("round_bf16_precision", "p = 8, emin = -126, emax = 127;", "p = 9, emin = -126, emax = 127;"),
    ("round_f16_range", "p = 11, emin = -14, emax = 15;", "p = 11, emin = -14, emax = 14;"),
    ("round_ties_away", "const double n = nearbyint(a / q);", "const double n = round(a / q);"),
    ("round_no_overflow", "if (a >= ldexp(2.0 - ldexp(1.0, -p), emax)) return v > 0 ? INFINITY : -INFINITY;",
     "if (a >= ldexp(4.0, emax)) return v > 0 ? INFINITY : -INFINITY;"),
    ("residual_dropped", "elem(x, dtype, row * N + j) + elem(res, dtype, row * N + j)",
     "elem(x, dtype, row * N + j)"),
    ("rms_dx_sign", "dx[k * N + j] = r * (g - xhat * c1);", "dx[k * N + j] = r * (g + xhat * c1);"),
    ("ln_dx_drop_c2", "dx[k * N + j] = r * (g - c2 - xhat * c1);",
     "dx[k * N + j] = r * (g - xhat * c1);"),
    ("ln_c2_from_dy", "sum_g += g;", "sum_g += elem(dy, dtype, base + j);"),
    ("rms_c1_from_dy", "double xhat = elem(x, dtype, base + j) * r;\n      sum_g_xhat += g * xhat;",
     "double xhat = elem(x, dtype, base + j) * r;\n      sum_g_xhat += elem(dy, dtype, base + j) * xhat;"),
    ("rms_c1_count", "const double c1 = sum_g_xhat / (double)N;\n    for",
     "const double c1 = sum_g_xhat / (double)(N + 1);\n    for"),
    ("dgamma_drop_dy", "double term = d * xhat;", "double term = xhat;"),
    ("dbeta_times_xhat", "sb[j - c0] += d;", "sb[j - c0] += d * xhat;"),
    ("dgamma_transposed_dy", "double d = elem(dy, dtype, i * N + j);",
     "double d = elem(dy, dtype, j * M + i);"),
    ("dgamma_wrong_row_stats", "double xhat = (elem(x, dtype, i * N + j) - m) * r[i];",
     "double xhat = (elem(x, dtype, i * N + j) - m) * r[M - 1 - i];"),
    ("dgamma_no_centering", "const double m = mu ? mu[i] : 0.0;", "const double m = 0.0;"),
    ("bf16_decode_shift", "<< 16;", "<< 15;"),
    # the magnitudes that size the dgamma/dbeta parity bound
    ("dgamma_scale_no_sqrt", "if (dgamma_scale) dgamma_scale[j] = sqrt(sg2[j - c0]);",
     "if (dgamma_scale) dgamma_scale[j] = sg2[j - c0];"),
    ("dbeta_scale_no_sqrt", "if (dbeta_scale) dbeta_scale[j] = sqrt(sb2[j - c0]);",
     "if (dbeta_scale) dbeta_scale[j] = sb2[j - c0];"),
    ("dgamma_scale_times_100", "if (dgamma_scale) dgamma_scale[j] = sqrt(sg2[j - c0]);",
     "if (dgamma_scale) dgamma_scale[j] = 100.0 * sqrt(sg2[j - c0]);"),
    ("dbeta_scale_times_100", "if (dbeta_scale) dbeta_scale[j] = sqrt(sb2[j - c0]);",
     "if (dbeta_scale) dbeta_scale[j] = 100.0 * sqrt(sb2[j - c0]);"),
    ("dgamma_scale_from_dy", "sg2[j - c0] += term * term;", "sg2[j - c0] += d * d;"),
    ("dbeta_scale_not_squared", "sb2[j - c0] += d * d;", "sb2[j - c0] += d;"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_mutant(tmp_path, name, old, new):
    src = open(oracle.SRC_PATH).read()
    assert src.count(old) == 1, f"mutation {name}: target text must occur exactly once"
    mutant_src = tmp_path / "oracle_mutant.c"
    mutant_src.write_text(src.replace(old, new))
    shutil.copy(os.path.join(os.path.dirname(oracle.SRC_PATH), "oracle.h"), tmp_path / "oracle.h")
    lib = oracle.build(src=str(mutant_src), out=str(tmp_path / f"liboracle_{name}.so"))
    mutant = oracle.Oracle(lib)
    failures = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except AssertionError as e:
            failures.append(f"{pin.__name__}: {e}")
    assert failures, f"no pin caught the planted mistake {name!r}"
