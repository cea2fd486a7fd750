"""Plausible mistakes planted in the CPU oracle must each fail a pin.

Every mutant is a copy of oracle/oracle.c with one textual change, built with
gcc into a temporary directory; the pin checks of _pins.py then run against it
until one fails.  A mutant that passes every pin means the pins have a hole.
"""
import os

import pytest

import oracle
import oracle.build as obuild
import _pins

MUTANTS = {
    "fma_like_no_product_rounding": (
        "out[j] = rnd(rnd(x[j] * c[j]) + rnd(partner * s[j]));",
        "out[j] = rnd(x[j] * c[j] + partner * s[j]);"),
    "partner_sign_flipped": (
        "double partner = (j < h) ? -x[j + h] : x[j - h];",
        "double partner = (j < h) ? x[j + h] : -x[j - h];"),
    "second_half_uses_first_half_angle": (
        "out[j] = rnd(rnd(x[j] * c[j]) + rnd(partner * s[j]));",
        "out[j] = rnd(rnd(x[j] * c[j % h]) + rnd(partner * s[j % h]));"),
    "partner_not_rotated": (
        "double partner = (j < h) ? -x[j + h] : x[j - h];",
        "double partner = (j < h) ? -x[j] : x[j];"),
    "tail_dropped": (
        "out_row[j] = x_row[j]; /* tail: the bits themselves */",
        "out_row[j] = 0;"),
    "table_row_s_major": (
        "            int64_t row = b * S + s;\n            for (int64_t j = 0; j < R; ++j) {",
        "            int64_t row = s * B + b;\n            for (int64_t j = 0; j < R; ++j) {"),
    "cos_and_sin_swapped": (
        "cos_out[row * R + j] = oracle_double_to_bf16(cos(f), 0);",
        "cos_out[row * R + j] = oracle_double_to_bf16(sin(f), 0);"),
    "cos_in_float": (
        "double f = (double)freqs[s * stride_s + b * stride_b + j];",
        "double f = (double)(float)(freqs[s * stride_s + b * stride_b + j] * 1.0001f);"),
    "grid_frequency_over_all_columns": (
        "const double omega = pow(theta, -2.0 * i / dims[k]);",
        "const double omega = pow(theta, -2.0 * i / (dims[0] + dims[1] + dims[2]));"),
    "grid_axes_reversed": (
        "const double pos[3] = {(double)(t + (t_offset ? t_offset[b] : 0)), (double)h,\n"
        "                                   (double)w};",
        "const double pos[3] = {(double)w, (double)h,\n"
        "                                   (double)(t + (t_offset ? t_offset[b] : 0))};"),
    "grid_second_half_not_repeated": (
        "row[j + half] = row[j];",
        "row[j + half] = -row[j];"),
    "grid_offset_ignored": (
        "(double)(t + (t_offset ? t_offset[b] : 0))",
        "(double)t"),
    "gemm_uncompensated_sum": (
        "                c += e;",
        "                c += 0.0 * e;"),
    "gemm_sticky_ignored": (
        "out[m * out_stride + n] = oracle_double_to_bf16(hi, (lo > 0) - (lo < 0));",
        "out[m * out_stride + n] = oracle_double_to_bf16(hi, 0);"),
    "gemm_last_term_dropped": (
        "for (int64_t k = 0; k < K; ++k) {\n                double prod",
        "for (int64_t k = 0; k < K - 1; ++k) {\n                double prod"),
    "gelu_without_sqrt2": (
        "return 0.5 * x * erfc(-x / sqrt(2.0));",
        "return 0.5 * x * erfc(-x);"),
    "gelu_tanh_approximation": (
        "return 0.5 * x * erfc(-x / sqrt(2.0));",
        "return 0.5 * x * (1.0 + tanh(0.7978845608028654 * (x + 0.044715 * x * x * x)));"),
    "gelu_small_branch_ignores_lost_part": (
        "return oracle_double_to_bf16(sum, (lost > 0) - (lost < 0));",
        "return oracle_double_to_bf16(sum, 0);"),
    "gate_and_up_swapped": (
        "const uint16_t *gate = input + r * in_stride;\n        const uint16_t *up = gate + hidden;",
        "const uint16_t *up = input + r * in_stride;\n        const uint16_t *gate = up + hidden;"),
    "gelu_not_rounded_before_mul": (
        "double gl = oracle_bf16_to_double(oracle_gelu_bf16(gate[j]));",
        "double gl = oracle_gelu_exact(oracle_bf16_to_double(gate[j]));"),
    "ties_away_from_zero": (
        "up = fmod(whole, 2.0) != 0.0; /* tie: to even */",
        "up = 1;"),
    "sticky_ignored": (
        "else if (mag_sticky > 0)\n        up = 1;",
        "else if (0)\n        up = 1;"),
    "no_subnormal_step": (
        "if (q < -133)\n        q = -133;",
        "if (q < -126)\n        q = -126;"),
}


def _source():
    with open(obuild.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = _source()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = os.path.join(tmp_path, "mutant.c")
    with open(path, "w") as f:
        f.write(src.replace(old, new))
    lib = obuild.build(source=path, out=os.path.join(tmp_path, "libmutant.so"), werror=False)
    mutant = oracle.Oracle(lib)
    for check in _pins.ALL_CHECKS:
        try:
            check(mutant)
        except (AssertionError, ValueError):
            return
    pytest.fail(f"mutant {name} passed every pin")
