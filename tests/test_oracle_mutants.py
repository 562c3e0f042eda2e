"""The pins are strong enough to catch plausible mistakes in the oracle.

Each case copies rmsnorm_oracle.c, plants one mistake by text substitution,
builds the copy with gcc into a temporary directory and runs every pin check
on it.  The copy must fail at least one check.  Nothing here touches the GPU.
"""

import os
import tempfile

import pytest

import oracle
from tests.oracle_checks import ALL_CHECKS

SRC = os.path.join(os.path.dirname(oracle.__file__), "rmsnorm_oracle.c")

# (name, text in the source, replacement, occurrence to replace: 0 = first)
MUTANTS = [
    ("mean_over_H_minus_1", "double ms = ss / (double)H;", "double ms = ss / (double)(H > 1 ? H - 1 : 1);", 0),
    ("eps_outside_sqrt", "double r = 1.0 / sqrt(ms + eps);", "double r = 1.0 / (sqrt(ms) + eps);", 0),
    ("eps_dropped", "double r = 1.0 / sqrt(ms + eps);", "double r = 1.0 / sqrt(ms + 0.0 * eps);", 0),
    ("mean_subtracted", "ss += v * v;", "ss += (v - load_elem(x, x_dt, row)) * (v - load_elem(x, x_dt, row));", 0),
    ("weight_shifted_column", "double wj = w ? load_elem(w, w_dt, j) : 1.0;\n            y[i * H + j] = v * r * wj;",
     "double wj = w ? load_elem(w, w_dt, (j + 1) % H) : 1.0;\n            y[i * H + j] = v * r * wj;", 0),
    ("weight_indexed_by_row", "double wj = w ? load_elem(w, w_dt, j) : 1.0;\n            y[i * H + j] = v * r * wj;",
     "double wj = w ? load_elem(w, w_dt, (i + j) % H) : 1.0;\n            y[i * H + j] = v * r * wj;", 0),
    ("residual_subtracted", "load_elem(x, x_dt, i * x_stride + j) + load_elem(res, x_dt, i * r_stride + j)",
     "load_elem(x, x_dt, i * x_stride + j) - load_elem(res, x_dt, i * r_stride + j)", 0),
    ("residual_norm_of_x_only", "            h[i * H + j] = v;\n            ss += v * v;",
     "            h[i * H + j] = v;\n            { double xo = load_elem(x, x_dt, i * x_stride + j); ss += xo * xo; }", 0),
    ("bwd_second_term_dropped", "dx[i * H + j] = t1 - t2;", "dx[i * H + j] = t1;", 0),
    ("bwd_second_term_sign", "dx[i * H + j] = t1 - t2;", "dx[i * H + j] = t1 + t2;", 0),
    ("bwd_c_over_H_plus_1", "double t2 = xn * r * c / (double)H;", "double t2 = xn * r * c / (double)(H + 1);", 0),
    ("bwd_c_without_weight", "double g = load_elem(dy, x_dt, i * dy_stride + j) * (w ? load_elem(w, w_dt, j) : 1.0);",
     "double g = load_elem(dy, x_dt, i * dy_stride + j);", 0),
    ("bwd_dw_uses_x_not_xn", "if (dw) dw[j] += dyv * xn;", "if (dw) dw[j] += dyv * xv;", 0),
    ("bwd_dw_includes_weight", "if (dw) dw[j] += dyv * xn;", "if (dw) dw[j] += g * xn;", 0),
    ("bwd_extra_rrms", "double t1 = r * g;", "double t1 = r * r * g;", 0),
    ("adaln_scale_without_one", "double sc = load_elem(scale, c_dt, c * cond_stride + j);",
     "double sc = load_elem(scale, c_dt, c * cond_stride + j) - 1.0;", 0),
    ("adaln_scale_shift_swapped", "y[i * H + j] = v * r * wj * (1.0 + sc) + sh;",
     "y[i * H + j] = v * r * wj * (1.0 + sh) + sc;", 0),
    ("adaln_shift_inside", "y[i * H + j] = v * r * wj * (1.0 + sc) + sh;",
     "y[i * H + j] = v * r * (wj * (1.0 + sc) + sh);", 0),
    ("adaln_cond_row_per_row", "const int64_t c = i / rows_per_cond;", "const int64_t c = i % rows_per_cond;", 0),
    ("bwd_residual_grad_dropped", "                dh[i * H + j] += d;", "                dh[i * H + j] += 0.0 * d;", 0),
    ("bwd_residual_grad_subtracted", "                dh[i * H + j] += d;", "                dh[i * H + j] -= d;", 0),
    ("rope_pairs_neighbours", "double x1 = load_elem(x, x_dt, base + j + half);",
     "double x1 = load_elem(x, x_dt, base + (j + 1) % head_dim);", 0),
    ("rope_out0_sign", "o[j] = x0 * c - x1 * sn;", "o[j] = x0 * c + x1 * sn;", 0),
    ("rope_out1_terms_swapped", "o[j + half] = x0 * sn + x1 * c;", "o[j + half] = x0 * c + x1 * sn;", 0),
    ("rope_cos_from_sin_table", "double c = load_elem(cos_t, t_dt,", "double c = load_elem(cos_t ? sin_t : cos_t, t_dt,",
     0),
    ("rope_table_row_is_batch", "const int64_t srow = r % seq_len;", "const int64_t srow = r / seq_len;", 0),
    ("rope_table_row_clamped", "const int64_t srow = r % seq_len;",
     "const int64_t srow = r < seq_len ? r : seq_len - 1;", 0),
    ("rope_table_second_half", "double c = load_elem(cos_t, t_dt, srow * table_stride + j);",
     "double c = load_elem(cos_t, t_dt, srow * table_stride + j + half);", 0),
    ("rope_transpose_ignored", "if (transpose) sn = -sn;", "if (transpose > 1) sn = -sn;", 0),
    ("ln_no_mean_subtraction", "y[i * H + j] = (h[j] - mean) * rstd * wj + bj;",
     "y[i * H + j] = (h[j] - 0.0 * mean) * rstd * wj + bj;", 0),
    ("ln_unbiased_variance", "const double var = sq / (double)H;",
     "const double var = sq / (double)(H > 1 ? H - 1 : 1);", 0),
    ("ln_uncentred_variance", "for (int64_t j = 0; j < H; ++j) sq += (h[j] - mean) * (h[j] - mean);",
     "for (int64_t j = 0; j < H; ++j) sq += h[j] * h[j];", 0),
    ("ln_eps_outside_root", "const double rstd = 1.0 / sqrt(var + eps);",
     "const double rstd = 1.0 / (sqrt(var) + eps);", 0),
    ("ln_bias_before_weight", "y[i * H + j] = (h[j] - mean) * rstd * wj + bj;",
     "y[i * H + j] = ((h[j] - mean) * rstd + bj) * wj;", 0),
    ("ln_residual_ignored", "if (res) v += load_elem(res, x_dt, i * r_stride + j);",
     "if (res) v += 0.0 * load_elem(res, x_dt, i * r_stride + j);", 0),
    ("round_half_away", "double q = rint(a / quantum);", "double q = round(a / quantum);", 0),
    ("f16_subnormal_scale", "v = ldexp((double)f, -24);", "v = ldexp((double)f, -25);", 0),
    ("f16_no_subnormal_quantum", "if (lead < emin) lead = emin;", "if (lead < emin - 30) lead = emin - 30;", 0),
]


def _mutant_source(text, old, new, occurrence):
    start = -1
    for _ in range(occurrence + 1):
        start = text.find(old, start + 1)
        assert start >= 0, f"pattern not found: {old!r}"
    return text[:start] + new + text[start + len(old):]


@pytest.mark.parametrize("name,old,new,occ", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, occ, tmp_path):
    with open(SRC) as f:
        text = f.read()
    src = tmp_path / f"{name}.c"
    src.write_text(_mutant_source(text, old, new, occ))
    lib = oracle.build(force=True, src=str(src), out=str(tmp_path / f"{name}.so"))
    o = oracle.Oracle(lib)
    failed = []
    for check in ALL_CHECKS:
        try:
            check(o)
        except AssertionError:
            failed.append(check.__name__)
        except (ValueError, FloatingPointError, ZeroDivisionError):
            failed.append(check.__name__)
    assert failed, f"mutant {name} passed every pin"
