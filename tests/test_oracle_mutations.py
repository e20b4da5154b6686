"""Planted mistakes in a COPY of the oracle source must be caught by the pins.

Each mutation is a plausible slip (a flipped sign, a wrong index, a dropped factor)
applied to the text of oracle/ne_oracle.c, compiled into a temporary library on the
CPU, and run through a battery of the pins in test_oracle.py.  The real oracle is
never modified.
"""
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "ne_oracle.c")

MUTATIONS = {
    "rope_rotation_sign": ("yr[i1] = a * s + b * c;", "yr[i1] = a * s - b * c;"),
    "rope_half_split_partner": ("i1 = half ? i + D / 2 : 2 * i + 1;", "i1 = half ? D - 1 - i : 2 * i + 1;"),
    "rope_half_split_ignored_in_backward": ("dq + IDX4(b, 0, h, 0, T, Hq, D), (size_t)Hq * D, T, D, base, -1, half);",
                                            "dq + IDX4(b, 0, h, 0, T, Hq, D), (size_t)Hq * D, T, D, base, -1, 0);"),
    "rope_frequency_exponent": ("pow(base, -2.0 * (double)i / (double)D)", "pow(base, -1.0 * (double)i / (double)D)"),
    "gqa_head_mapping": ("const int g = h / G;", "const int g = h % Hkv;"),
    "mask_includes_future": [
        ("for (int j = lo; j <= i; ++j) {\n            double s = 0.0;",
         "for (int j = lo; j < T; ++j) {\n            double s = 0.0;"),
        ("for (int j = lo; j <= i; ++j) {\n            Pi[j] = exp(Pi[j] - m);",
         "for (int j = lo; j < T; ++j) {\n            Pi[j] = exp(Pi[j] - m);"),
        ("for (int j = lo; j <= i; ++j) Pi[j] /= l;", "for (int j = lo; j < T; ++j) Pi[j] /= l;"),
        ("for (int j = i + 1; j < T; ++j) Pi[j] = 0.0;", ""),
    ],
    "window_off_by_one": ("return (window > 0 && i - window + 1 > 0) ? i - window + 1 : 0;",
                          "return (window > 0 && i - window > 0) ? i - window : 0;"),
    "window_column_short": ("return (window > 0 && j + window - 1 < T - 1) ? j + window - 1 : T - 1;",
                            "return (window > 0 && j + window - 2 < T - 1) ? j + window - 2 : T - 1;"),
    "softmax_scale_missing": ("            s *= scale;\n", "\n"),
    "dq_scale_missing": ("for (int d = 0; d < D; ++d) dqi[d] *= scale;", ""),
    "ds_sign": ("* (dp - di);", "* (di - dp);"),
    "dq_forward_rotation": ("dq + IDX4(b, 0, h, 0, T, Hq, D), (size_t)Hq * D, T, D, base, -1, half);",
                            "dq + IDX4(b, 0, h, 0, T, Hq, D), (size_t)Hq * D, T, D, base, 1, half);"),
    "dk_forward_rotation": ("dk + IDX4(b, 0, g, 0, T, Hkv, D), (size_t)Hkv * D, T, D, base, -1, half);",
                            "dk + IDX4(b, 0, g, 0, T, Hkv, D), (size_t)Hkv * D, T, D, base, 1, half);"),
    "dv_uses_ds": ("dvj[d] += p * dOi[d];", "dvj[d] += s * dOi[d];"),
    "dk_uses_rotated_k": ("dkj[d] += s * qi[d];", "dkj[d] += s * kr[(size_t)i * D + d];"),
    "lse_without_max": ("lse_row[i] = m + log(l);", "lse_row[i] = log(l);"),
    "delta_from_value": ("di += dOi[d] * od[d];", "di += dOi[d] * od[d] * 0.5;"),
    "qknorm_gain_once": ("y[r * D + d] = gain * xr[d] * rho;", "y[r * D + d] = xr[d] * rho;"),
    "qknorm_sum_not_mean": ("const double rho = 1.0 / sqrt(ss / (double)D + eps);\n        for (int d = 0; d < D; ++d) y",
                            "const double rho = 1.0 / sqrt(ss + eps);\n        for (int d = 0; d < D; ++d) y"),
    "qknorm_bwd_projection_dropped": ("g[d] = gain * rho * (g[d] - xr[d] * rho * rho * dot / (double)D);",
                                      "g[d] = gain * rho * g[d];"),
    "qknorm_bwd_wrong_rho_power": ("g[d] = gain * rho * (g[d] - xr[d] * rho * rho * dot / (double)D);",
                                   "g[d] = gain * rho * (g[d] - xr[d] * rho * dot / (double)D);"),
}


def battery():
    """Run a set of pins; return the names of those that failed."""
    failed = []
    checks = [
        ("autograd", lambda: pins.test_against_torch_float64_autograd((1, 19, 4, 2, 6), 10.0, 1.0)),
        ("autograd_norope", lambda: pins.test_against_torch_float64_autograd((1, 17, 4, 4, 8), 0.0, 1.0)),
        ("brute", lambda: pins.test_fwd_matches_brute_force((1, 4, 4, 2, 4), 3.0)),
        ("fd", pins.test_finite_differences_every_entry_tiny),
        ("d2", pins.test_d2_rotation_by_t_radians),
        ("zero_q", pins.test_zero_queries_give_uniform_weights),
        ("single", pins.test_single_token),
        ("window_autograd", lambda: pins.test_window_against_torch_float64_autograd((2, 37, 6, 2, 16), 10000.0, 8)),
        ("window_zero_q", pins.test_window_zero_queries_average_the_window),
        ("qknorm_autograd", lambda: pins.test_qk_norm_against_torch_float64_autograd((2, 37, 6, 2, 16), 10000.0, 0,
                                                                                    (1.2, 1e-6))),
        ("qknorm_self_score", pins.test_qk_norm_self_score_closed_form),
        ("qknorm_invariance", pins.test_qk_norm_rescaling_rows_changes_nothing),
        ("half_split_rope", pins.test_half_split_rope_is_the_interleaved_rotation_of_reordered_dimensions),
        ("half_split_relative", pins.test_half_split_scores_depend_only_on_relative_position),
        ("half_split_fd", pins.test_half_split_finite_differences_every_entry_tiny),
    ]
    for name, fn in checks:
        try:
            fn()
        except AssertionError:
            failed.append(name)
    return failed


def test_unmutated_copy_passes_battery(tmp_path):
    lib = tmp_path / "lib_copy.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", SRC, "-o", str(lib), "-lm"],
                   check=True)
    with oracle.use_library(str(lib)):
        assert battery() == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    edits = MUTATIONS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    text = open(SRC).read()
    for old, new in edits:
        assert text.count(old) == 1, f"mutation anchor for {name} not unique in the oracle source"
        text = text.replace(old, new)
    src = tmp_path / "mutant.c"
    src.write_text(text)
    lib = tmp_path / "mutant.so"
    subprocess.run(["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", str(src), "-o", str(lib), "-lm"],
                   check=True)
    with oracle.use_library(str(lib)):
        failed = battery()
    assert failed, f"planted mistake {name} was not caught by any pin"
