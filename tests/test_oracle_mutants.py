"""Planted mistakes: every plausible slip in the oracle must trip a pin.

Each case edits one line of a temporary copy of oracle/ga_oracle.c (a dropped
term, a wrong sign or index, a swapped operand, a wrong rounding rule), builds
it with gcc, and runs the pins against that copy.  At least one pin must fail;
the real oracle passes all of them (test_oracle_pins.py).  Every edit keeps
all memory accesses inside the caller's buffers.
"""
import os
import subprocess

import pytest

import oracle
import oracle_pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "ga_oracle.c")

MUTANTS = {
    "gelu_cubic_coefficient": ("0.044715 * s * s * s", "0.04715 * s * s * s"),
    "gelu_scale_constant": ("sqrt(2.0 / M_PI)", "sqrt(1.0 / M_PI)"),
    "gelu_half_dropped": ("return 0.5 * s * (1.0 + tanh", "return s * (1.0 + tanh"),
    "gelu_tanh_argument_sign": ("tanh(k * (s", "tanh(-k * (s"),
    "sample_std": ("*std = sqrt(q / (double)d);", "*std = sqrt(q / (double)(d > 1 ? d - 1 : 1));"),
    "variance_not_std": ("*std = sqrt(q / (double)d);", "*std = q / (double)d;"),
    "mean_drops_first_term": ("for (int64_t i = 0; i < d; ++i) s += g[i];",
                              "for (int64_t i = 1; i < d; ++i) s += g[i];"),
    "variance_about_zero": ("q += (g[i] - mu) * (g[i] - mu);", "q += g[i] * g[i];"),
    "cutoff_sign": ("mean + (double)z * std", "mean - (double)z * std"),
    "cutoff_ignores_z": ("mean + (double)z * std", "mean + 1.6448536 * std"),
    "up_from_gate_half": ("load_elem(in, row + d + i, dtype)", "load_elem(in, row + i, dtype)"),
    "gate_from_up_half": ("g[i] = load_elem(in, row + i, dtype)", "g[i] = load_elem(in, row + d + i, dtype)"),
    "relu_dropped": ("if (!(s > 0.0)) s = 0.0;", ";"),
    "threshold_reversed": ("double s = g[i] - cut;", "double s = cut - g[i];"),
    "gelu_output_transposed": ("store_elem(out, r * d + i, dtype, y);",
                               "store_elem(out, i * T + r, dtype, y);"),
    "gelu_ignores_live": ("const int64_t n = clamp_live(live, T);", "const int64_t n = T;"),
    "round_ties_away": ("double r = rint(", "double r = round("),
    "round_truncates": ("double r = rint(", "double r = trunc("),
    "round_via_float": ("double r = rint(ldexp(x, mbits - E));",
                        "double r = rint((double)(float)ldexp(x, mbits - E));"),
    "decode_exponent_off_by_one": ("(int)expf - bias - mbits)", "(int)expf - bias - mbits + 1)"),
    "subnormals_not_clamped": ("if (E < emin) E = emin;", ";"),
    "bf16_field_widths": ("case GAO_BF16: *ebits = 8; *mbits = 7;",
                          "case GAO_BF16: *ebits = 7; *mbits = 8;"),
    "silu_sign": ("x / (1.0 + exp(-x))", "x / (1.0 + exp(x))"),
    "silu_operands_swapped": ("gao_silu(gate) * up", "gao_silu(up) * gate"),
    "silu_ignores_live": ("const int64_t n = clamp_live(live, M);", "const int64_t n = M;"),
    "roundtrip_z_not_rounded": ("const double z_t = round_to((double)z, dtype);",
                                "const double z_t = (double)z;"),
    "roundtrip_shift_not_rounded": ("double s = round_to(g[i] - cut, dtype);", "double s = g[i] - cut;"),
    "roundtrip_gelu_not_rounded": ("const double h = round_to(gao_gelu_tanh(s), dtype);",
                                   "const double h = gao_gelu_tanh(s);"),
    "roundtrip_mean_not_rounded": ("const double mean_t = round_to(mean, dtype);", "const double mean_t = mean;"),
    "roundtrip_sample_std": ("const double std_t = round_to(std, dtype);",
                             "const double std_t = round_to(std * sqrt((double)d / (double)(d > 1 ? d - 1 : 1)), dtype);"),
    "erf_argument_unscaled": ("erf(x / sqrt(2.0))", "erf(x / 2.0)"),
    "erf_gelu_half_dropped": ("return 0.5 * x * (1.0 + erf", "return x * (1.0 + erf"),
    "squared_relu_not_squared": ("return r * r;", "return r;"),
    "squared_relu_leaks_negatives": ("const double r = x > 0.0 ? x : 0.0;", "const double r = x;"),
    "gelu_and_mul_modes_swapped": ("approximate ? gao_gelu_tanh(gate) : gao_gelu_erf(gate)",
                                   "approximate ? gao_gelu_erf(gate) : gao_gelu_tanh(gate)"),
    "gelu_and_mul_up_from_gate": ("const double up = load_elem(in, r * 2 * d + d + i, dtype);\n"
                                  "            const double act",
                                  "const double up = load_elem(in, r * 2 * d + i, dtype);\n"
                                  "            const double act"),
    "down_weight_transposed": ("wrow[k] = load_elem(w, h * d + k, dtype);",
                               "wrow[k] = load_elem(w, k * H + h, dtype);"),
    "down_output_transposed": ("store_elem(y, r * H + h, dtype, s);", "store_elem(y, h * T + r, dtype, s);"),
    "down_ignores_live": ("const int64_t n = clamp_live(live, T);\n    if (n == 0) return 0;",
                          "const int64_t n = T;\n    if (n == 0) return 0;"),
    "down_drops_first_term": ("for (int64_t k = 0; k < d; ++k) {\n                s += ",
                              "for (int64_t k = 1; k < d; ++k) {\n                s += "),
    "down_activation_unrounded": ("NULL, NULL, NULL, NULL)) goto done;\n"
                                  "    for (int64_t i = 0; i < n * d; ++i) a[i] = load_elem(a_bits, i, dtype);",
                                  "a, NULL, NULL, NULL)) goto done;"),
    "down_abs_signed": ("m += fabs(a[r * d + k] * wrow[k]);", "m += a[r * d + k] * wrow[k];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor vanished: {old!r}"
    mutated = src.replace(old, new, 1)
    path = tmp_path / "mutant.c"
    path.write_text(mutated)
    lib = tmp_path / f"libmutant_{name}.so"
    subprocess.run(["gcc", "-std=gnu11", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                    str(path), "-o", str(lib), "-lm"], check=True)
    mutant = oracle.Oracle(str(lib))
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(mutant)
        except Exception as exc:  # noqa: BLE001 - any failure counts as caught
            caught.append((pin.__name__, type(exc).__name__))
            break
    assert caught, f"planted mistake {name!r} passed every pin"
