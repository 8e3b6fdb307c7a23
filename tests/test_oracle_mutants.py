"""Plausible mistakes planted in copies of the oracle must each fail at least one pin.

Each mutant is a textual edit of lrar_oracle.cpp, compiled to a temporary library on the
CPU; the real oracle is untouched. This shows the pins are strong enough to catch a dropped
term, a wrong sign or index, or a misplaced constant anywhere in the oracle.
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "rms_without_sqrt": ("return std::sqrt(sum_sq / r + eps);", "return (sum_sq / r + eps);"),
    "eps_outside_sqrt": ("return std::sqrt(sum_sq / r + eps);",
                         "return std::sqrt(sum_sq / r) + eps;"),
    "rms_sum_not_mean": ("return std::sqrt(sum_sq / r + eps);",
                         "return std::sqrt(sum_sq + eps);"),
    "eps_dropped": ("return std::sqrt(sum_sq / r + eps);", "return std::sqrt(sum_sq / r);"),
    "first_r_coordinates": ("z += q[j] * (o_row[d - r + j] / rho);",
                            "z += q[j] * (o_row[j] / rho);"),
    "norm_over_head": ("for (int j = d - r; j < d; ++j) sum_sq += o_row[j] * o_row[j];",
                       "for (int j = 0; j < r; ++j) sum_sq += o_row[j] * o_row[j];"),
    "score_temperature": ("z += q[j] * (o_row[d - r + j] / rho);",
                          "z += q[j] * (o_row[d - r + j] / rho) / std::sqrt((double)r);"),
    "softmax_sign": ("alpha[i] = std::exp(z[i] - m);", "alpha[i] = std::exp(m - z[i]);"),
    "softmax_no_normalise": ("for (size_t i = 0; i < n; ++i) alpha[i] /= l;", ""),
    "mix_first_source_only": (
        "for (int i = 0; i < n; ++i) s += a[i] * row_of(src[i], ld[i], t)[j];\n      h[j] = s;",
        "for (int i = 0; i < n; ++i) s += a[i] * row_of(src[0], ld[0], t)[j];\n      h[j] = s;"),
    "stats_unshifted_acc": ("for (int i = 0; i < n; ++i) v += e[i] * row_of(src[i], ld[i], t)[j];",
                            "for (int i = 0; i < n; ++i) v += std::exp(z[i]) * row_of(src[i], ld[i], t)[j];"),
    "merge_no_rescale_l": ("double l_new = l[t] * scale_old;", "double l_new = l[t];"),
    "merge_no_rescale_acc": ("double v = acc[t * d + j] * scale_old;", "double v = acc[t * d + j];"),
    "bwd_drop_norm_term": ("gi[d - r + j] += dz * (q[j] / rho[i] - q_dot_k * k / (r * rho3));",
                           "gi[d - r + j] += dz * (q[j] / rho[i]);"),
    "bwd_norm_term_sign": ("gi[d - r + j] += dz * (q[j] / rho[i] - q_dot_k * k / (r * rho3));",
                           "gi[d - r + j] += dz * (q[j] / rho[i] + q_dot_k * k / (r * rho3));"),
    "bwd_missing_r": ("gi[d - r + j] += dz * (q[j] / rho[i] - q_dot_k * k / (r * rho3));",
                      "gi[d - r + j] += dz * (q[j] / rho[i] - q_dot_k * k / (rho3));"),
    "bwd_direct_only": ("const double dz = a[i] * g_dot_diff;  // dL/dz_i (Lemma 2)",
                        "const double dz = 0.0 * g_dot_diff;"),
    "bwd_no_h_subtract": ("for (int j = 0; j < d; ++j) g_dot_diff += g[j] * (o[j] - h[j]);\n      const double dz = a[i]",
                          "for (int j = 0; j < d; ++j) g_dot_diff += g[j] * (o[j]);\n      const double dz = a[i]"),
    "bwd_dq_unnormalised": ("dq[j] += dz * (k / rho[i]);", "dq[j] += dz * k;"),
    "bwd_dq_transposed_slot": ("gi[d - r + j] += dz", "gi[d - 1 - j] += dz"),
    "fullrms_mean_over_r": ("const double rho_d = std::sqrt(sum_sq / d + eps);",
                            "const double rho_d = std::sqrt(sum_sq / r + eps);"),
    "fullrms_eps_outside": ("const double rho_d = std::sqrt(sum_sq / d + eps);",
                            "const double rho_d = std::sqrt(sum_sq / d) + eps;"),
    "keys_from_value_tail": ("const double* k = row_of(key[i], key_ld[i], t);",
                             "const double* k = row_of(src[i], ld[i], t) + d - r;"),
    "keys_first_row_only": ("const double* k = row_of(key[i], key_ld[i], t);",
                            "const double* k = row_of(key[i], key_ld[i], 0);"),
    "round_truncates": ("return std::nearbyint(x / spacing) * spacing;",
                        "return std::trunc(x / spacing) * spacing;"),
    "round_no_subnormal_floor": ("if (lead < -126) lead = -126;", ""),
    "mergeacc_drops_prev": ("const double prev = b ? row_of(b, b_ld, t)[j] : 0.0;",
                            "const double prev = 0.0;"),
    "mergeacc_routes_old_sum": ("const double* srcs[1] = {b_out};",
                                "const double* srcs[1] = {b ? b : o};"),
    "mergeacc_unrounded": ("b_out[t * d + j] = round_to_format(prev + row_of(o, o_ld, t)[j], p);",
                           "b_out[t * d + j] = prev + row_of(o, o_ld, t)[j];"),
    "keys_rms_over_d": ("const double rho = std::sqrt(sum_sq / r + eps);\n      double zi",
                        "const double rho = std::sqrt(sum_sq / d + eps);\n      double zi"),
}


@pytest.fixture(scope="module")
def source_text():
    with open(oracle.SOURCE) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, source_text, tmp_path):
    old, new = MUTANTS[name]
    assert source_text.count(old) >= 1, f"mutation site for {name} not found"
    text = source_text.replace(old, new)
    src = tmp_path / f"{name}.cpp"
    src.write_text(text)
    lib = oracle.compile_oracle(str(src), str(tmp_path / f"lib{name}.so"), opt="-O1")
    mut = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(mut)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
    os.remove(lib)
