"""Mutation check of the oracle's pins (CPU only).

Each mutant is a copy of ``oracle/gn_oracle.c`` with one plausible mistake planted
(a dropped term, a wrong sign, a wrong index or divisor, swapped outputs, a wrong
rounding step), compiled into a temporary library. Every pin in test_oracle.py is
then run against the mutant; at least one must fail, or the pins could not have
told that mistake apart from the definition.
"""
import ctypes
import os
import subprocess

import pytest
import torch

import tests.test_oracle as pins
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "gn_oracle.c")

MUTANTS = {
    "mean_divisor": ("const double mu = sum / (double)M;", "const double mu = sum / (double)(M + 1);"),
    "unbiased_var": ("const double v = ss / (double)M;", "const double v = ss / (double)(M - 1);"),
    "eps_outside_sqrt": ("1.0 / sqrt(v + (double)eps)", "1.0 / (sqrt(v) + (double)eps)"),
    "beta_sign": ("const double pre = gm * xhat + bt;\n                y[base + s]",
                  "const double pre = gm * xhat - bt;\n                y[base + s]"),
    "relu_eats_nan_and_negzero": ("static double gno_relu(double v) { return v < 0.0 ? 0.0 : v; }",
                                  "static double gno_relu(double v) { return v > 0.0 ? v : 0.0; }"),
    "gate_blocks_nan": ("static double gno_gate(double r, double g) { return r <= 0.0 ? 0.0 : g; }",
                        "static double gno_gate(double r, double g) { return r > 0.0 ? g : 0.0; }"),
    "gate_on_wrong_side": ("static double gno_gate(double r, double g) { return r <= 0.0 ? 0.0 : g; }",
                           "static double gno_gate(double r, double g) { return r <= 0.0 ? g : 0.0; }"),
    "forward_group_index": ("const int64_t ng = n * G + c / Cg;\n            const double gm",
                            "const int64_t ng = n * G + c % G;\n            const double gm"),
    "dx_c2_sign": ("dx[base + s] = rs[ng] * (gm * g_ - c1[ng] - xhat * c2[ng]);",
                   "dx[base + s] = rs[ng] * (gm * g_ - c1[ng] + xhat * c2[ng]);"),
    "dx_drop_c1": ("dx[base + s] = rs[ng] * (gm * g_ - c1[ng] - xhat", "dx[base + s] = rs[ng] * (gm * g_ - xhat"),
    "dx_drop_gamma": ("dx[base + s] = rs[ng] * (gm * g_", "dx[base + s] = rs[ng] * (g_"),
    "swap_dgamma_dbeta": ("if (dgamma) dgamma[c] = a;", "if (dgamma) dgamma[c] = b;"),
    "c2_from_s1": ("b += gno_gamma(gamma, c) * s2[n * C + c];", "b += gno_gamma(gamma, c) * s1[n * C + c];"),
    "c1_no_mean": ("c1[n * G + g] = a / (double)M;", "c1[n * G + g] = a;"),
    "s2_without_xhat": ("b += g_ * xhat;", "b += g_;"),
    "bf16_truncate": ("\n    double k = nearbyint(ldexp(a, -q));", "\n    double k = floor(ldexp(a, -q));"),
    "f16_truncate": ("const double k = nearbyint(ldexp(a, -q));", "const double k = floor(ldexp(a, -q));"),
    "bf16_precision": ("int q = (e - 1) - 7;", "int q = (e - 1) - 8;"),
    "bf16_nan_payload": ("return signbit(v) ? 0xFFC0 : 0x7FC0;", "return 0x7F80;"),
    "f16_exponent_bias": ("else v = ldexp((double)(f + 1024), e - 25);", "else v = ldexp((double)(f + 1024), e - 24);"),
    "f16_no_subnormals": ("if (e == 0) v = ldexp((double)f, -24);", "if (e == 0) v = 0.0;"),
    "f16_precision": ("int q = (e - 1) - 10;    /* quantum", "int q = (e - 1) - 9;    /* quantum"),
    "f16_overflow_edge": ("if (r >= 65536.0) return", "if (r >= 65504.0) return"),
    # the per-channel magnitudes behind every dgamma/dbeta bar (gno_channel_abs_sums)
    "abs_sums_times_2": ("a += fabs(g_);", "a += 2.0 * fabs(g_);"),
    "abs_sums_times_100": ("abs_dy[c] += a;\n            abs_dyxhat[c] += b;",
                           "abs_dy[c] += 100.0 * a;\n            abs_dyxhat[c] += 100.0 * b;"),
    "abs_sums_gate_dropped": ("if (act) g_ = gno_gate(gno_relu(gno_gamma(gamma, c) * xhat + gno_beta(beta, c)), g_);\n"
                              "                a +=", "a +="),
    "abs_sums_no_rstd": ("(gno_load(x, x_dt, base + s) - mean[ng]) * rstd[ng];",
                         "(gno_load(x, x_dt, base + s) - mean[ng]);"),
    "abs_sums_channel_index": ("const int64_t ng = n * G + c / Cg;\n            const int64_t base = (n * C + c) * S;\n"
                               "            double a = 0.0, b = 0.0;",
                               "const int64_t ng = n * G + c / Cg;\n            const int64_t base = (n * C + (c + 1) % C) * S;\n"
                               "            double a = 0.0, b = 0.0;"),
    "abs_sums_group_index": ("const int64_t ng = n * G + c / Cg;\n            const int64_t base = (n * C + c) * S;\n"
                             "            double a = 0.0, b = 0.0;",
                             "const int64_t ng = n * G + c % G;\n            const int64_t base = (n * C + c) * S;\n"
                             "            double a = 0.0, b = 0.0;"),
}

PINS = [
    pins.test_closed_form_mean_zero_and_variance_ratio,
    lambda: pins.test_constant_input_maps_to_beta_exactly(0.3),
    pins.test_single_element_groups_match_printed_rstd,
    pins.test_nan_and_inf_stay_in_their_group,
    lambda: pins.test_against_torch_float64_group_norm("tiny"),
    lambda: pins.test_against_torch_float64_group_norm("ragged"),
    pins.test_special_cases_instance_norm_and_layer_norm,
    pins.test_exact_rational_brute_force_on_eight_elements,
    pins.test_backward_against_central_differences_all_elements,
    pins.test_backward_closed_forms,
    pins.test_round_bf16_matches_torch_on_fp32_values,
    pins.test_round_bf16_ties_double_rounding_and_specials,
    pins.test_f16_decode_exhaustive_against_numpy,
    pins.test_round_f16_against_numpy_ties_and_specials,
    lambda: pins.test_against_torch_float64_group_norm("f16"),
    pins.test_relu_option_against_torch_autograd,
    pins.test_relu_keeps_negative_zero_and_nan_group_gradient,
    lambda: pins.test_channel_abs_sums_against_torch_autograd(torch.bfloat16, False),
    lambda: pins.test_channel_abs_sums_against_torch_autograd(torch.float16, True),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} must be unique"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / f"lib_{name}.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-o",
                    str(lib), str(path), "-lm"], check=True)
    return str(lib)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_kill_mutant(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    lib_path = _build_mutant(tmp_path, name, old, new)
    real = O._load()
    mutant = ctypes.CDLL(lib_path)
    for fn in ("gno_group_stats", "gno_forward", "gno_forward_at", "gno_backward", "gno_backward_at",
               "gno_round_bf16", "gno_round_bf16_array", "gno_round_f32_array", "gno_channel_abs_sums",
               "gno_relu_value", "gno_gate_value", "gno_round_f16", "gno_round_f16_array",
               "gno_f16_decode_array"):
        getattr(mutant, fn).argtypes = getattr(real, fn).argtypes
        getattr(mutant, fn).restype = getattr(real, fn).restype
    monkeypatch.setattr(O, "_lib", mutant)
    killed_by = []
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError):
            killed_by.append(getattr(pin, "__name__", "lambda"))
    assert killed_by, f"mutant {name} survived every pin"
