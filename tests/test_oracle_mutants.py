"""The pins catch plausible mistakes in the oracle.

Each mutant below is a copy of oracle/leapq_oracle.c with one plausible slip
(a dropped term, a wrong sign, index or axis, a transposed operand, another
rounding or tie rule).  It is compiled on the CPU into a temporary library,
and at least one pin of tests/pins.py must fail against it.  The mistakes are
planted in the oracle only; nothing here touches the GPU library.
"""
import os

import pytest

from oracle import build as obuild
from tests import pins

MUTANTS = [
    ("sum_pairs_i_i63", "s[i] = f[i] + f[i + 64];", "s[i] = f[i] + f[i + 63];"),
    ("sum_adjacent_tree", "for (int i = 0; i < h; ++i) s[i] = s[i] + s[i + h];\n    return s[0];\n}\n\n/* Dot",
     "for (int i = 0; i < h; ++i) s[i] = s[2 * i] + s[2 * i + 1];\n    return s[0];\n}\n\n/* Dot"),
    ("dot_fuse_upper", "fmaf(a[i], b[i], a[i + 64] * b[i + 64])", "fmaf(a[i + 64], b[i + 64], a[i] * b[i])"),
    ("residual_scale_axes", "((float)Q[r * D + c] * rho[r]) * sigma[c];\n}",
     "((float)Q[r * D + c] * rho[c]) * sigma[r];\n}"),
    ("read_transposed_codes", "col[r] = (float)Q[r * D + c];", "col[r] = (float)Q[c * D + r];"),
    ("read_no_sigma", "out[c] = sigma[c] * lqo_t128_dot(w, col);", "out[c] = lqo_t128_dot(w, col);"),
    ("read_row_token_wrong_coord", "out[c] = fmaf(xr, v[c], out[c]);", "out[c] = fmaf(x[c], v[c], out[c]);"),
    ("read_drop_column_token", "out[c] = out[c] + lqo_t128_dot(v, x);", "out[c] = out[c];"),
    ("append_sign", "u[c] = beta * (v[c] - r[c]);", "u[c] = beta * (v[c] + r[c]);"),
    ("append_coef_inverted", "float ci = gt / gam[i];", "float ci = gam[i] / gt;"),
    ("append_drop_current_token", "o[c] = fmaf(kq, u[c], o[c]);", "o[c] = o[c];"),
    ("append_read_undecayed", "r[c] = gt * bk[c];", "r[c] = gamma_of(n, gam) * bk[c];"),
    ("append_record_not_stored", "gam[n] = gt;", "gam[n] = 1.0f;"),
    ("current_lines_unscaled", "add_lines(out, C, idx, vec, gn);", "add_lines(out, C, idx, vec, 1.0f);"),
    ("current_coef_inverted", "float ci = gn / gam[i];", "float ci = gam[i] / gn;"),
    ("current_drop_gamma", "float a = gn * rho[r];", "float a = rho[r];"),
    ("pick_last_max", "score[cand] > best", "score[cand] >= best"),
    ("pick_row_not_zeroed", "v[c] = R[pick * D + c]; R[pick * D + c] = 0.0f;", "v[c] = R[pick * D + c];"),
    ("pick_col_energy_of_row", "score[D + c] = lqo_t128_dot(col, col);", "score[D + c] = lqo_t128_dot(R + c * D, R + c * D);"),
    ("smooth_axis", "col[r] = fabsf(R[r * D + c]);", "col[r] = fabsf(R[c * D + r]);"),
    ("smooth_mean_64", "* 0.0078125f", "* 0.015625f"),
    ("smooth_no_floor", "if (s < sigma_floor) s = sigma_floor;", ";"),
    ("smooth_no_sqrt", "s = sqrtf(m);", "s = m;"),
    ("quant_128", "rho[r] = M / lv;", "rho[r] = M / (lv + 1.0f);"),
    ("bits_levels_swapped", "return bits == 4 ? 7.0f : bits == 6 ? 31.0f : 127.0f;",
     "return bits == 4 ? 15.0f : bits == 6 ? 63.0f : 127.0f;"),
    ("quant_round_away", "rint((double)x[c] * (double)g)", "round((double)x[c] * (double)g)"),
    ("quant_truncate", "rint((double)x[c] * (double)g)", "trunc((double)x[c] * (double)g)"),
    ("quant_double_rounding", "(float)rint((double)x[c] * (double)g)", "rintf(x[c] * g)"),
    ("quant_no_tiny_guard", "if (!(M >= LQO_TINY)) {", "if (!(M > 0.0f)) {"),
    ("step_no_decay", "    for (int e = 0; e < D * D; ++e) S[e] = alpha * S[e];\n    float u[D];",
     "    float u[D];"),
    ("step_read_output_with_k", "oc = fmaf(S[r * D + c], q[r], oc);", "oc = fmaf(S[r * D + c], k[r], oc);"),
    ("bf16_truncate", "b += 0x7fffu + lsb;", "b += 0u * lsb;"),
    ("gate_softplus_sign", "log1p(exp(-fabs(x)))", "log1p(exp(fabs(x)))"),
    ("gate_rate_not_exponentiated", "exp(-exp((double)A_log) * sp)", "exp(-(double)A_log * sp)"),
    ("gate_drop_dt_bias", "double x = (double)a + (double)dt_bias;", "double x = (double)a;"),
    ("gate_beta_sign", "exp(-(double)b)", "exp((double)b)"),
    ("l2norm_no_sqrt", "1.0f / sqrtf(s + eps)", "1.0f / (s + eps)"),
    ("l2norm_eps_outside_root", "sqrtf(s + eps)", "(sqrtf(s) + eps)"),
    ("l2norm_scale_folded", "(x[r] * inv) * scale", "x[r] * (inv * scale)"),
    ("kda_ratio_inverted", "w[e] = (gt[e] / gi[e]) * ki[e];", "w[e] = (gi[e] / gt[e]) * ki[e];"),
    ("kda_read_undecayed", "x[e] = gt[e] * k[e];", "x[e] = k[e];"),
    ("kda_gamma_not_cumulative", "gt[e] = gp[e] * alpha[e];", "gt[e] = alpha[e];"),
    ("kda_rebuild_ratio_inverted", "w[r] = (gn[r] / gam[(size_t)i * D + r]) * rk[(size_t)i * D + r];",
     "w[r] = (gam[(size_t)i * D + r] / gn[r]) * rk[(size_t)i * D + r];"),
    ("kda_lines_unscaled", "M[r * D + c] = M[r * D + c] + g[r] * v[c];", "M[r * D + c] = M[r * D + c] + v[c];"),
    ("kda_rebuild_no_gamma", "float a = gn[r] * rho[r];", "float a = rho[r];"),
    ("bf16_records_not_rounded", "x[e] = bf16_to_f32(lqo_f32_to_bf16(x[e]));", "x[e] = x[e];"),
    ("r1_sweep_rows_for_columns", "                for (int r = 0; r < D; ++r) col[r] = R[r * D + c];\n                b[c] = lqo_t128_dot(col, a);",
     "                for (int r = 0; r < D; ++r) col[r] = R[c * D + r];\n                b[c] = lqo_t128_dot(col, a);"),
    ("r1_not_normalized", "for (int r = 0; r < D; ++r) a[r] = a[r] * inv;", ";"),
    ("r1_no_deflation", "        }\n        for (int r = 0; r < D; ++r)\n            for (int c = 0; c < D; ++c) R[r * D + c] = fmaf(-a[r], b[c], R[r * D + c]);",
     "        }\n"),
    ("r1_read_with_b", "float d = lqo_t128_dot(a, x);", "float d = lqo_t128_dot(b, x);"),
    ("r1_rebuild_unscaled", "float w = g * a[r];", "float w = a[r];"),
    ("r1_start_last_max", "if (e > best) { best = e; pick = r; }", "if (e >= best) { best = e; pick = r; }"),
    ("blk_no_projection", "for (int r = 0; r < D; ++r) A[j][r] = fmaf(-d, A[i][r], A[j][r]);", "(void)d;"),
    ("blk_not_normalized", "for (int r = 0; r < D; ++r) A[j][r] = A[j][r] * inv;", "(void)inv;"),
    ("blk_fold_cold", "lqo_quantize_block(R, C, smoothing, sigma_floor, 1, Q,", "lqo_quantize_block(R, C, smoothing, sigma_floor, 0, Q,"),
    ("blk_sweep_transposed", "for (int r = 0; r < D; ++r) A[j][r] = lqo_t128_dot(R + r * D, Z);", "cols_dot(R, Z, A[j]);"),
    ("blk_no_deflation", "*b = a + D;\n        for (int r = 0; r < D; ++r)\n            for (int c = 0; c < D; ++c) R[r * D + c] = fmaf(-a[r], b[c], R[r * D + c]);",
     "*b = a + D;\n        (void)a; (void)b;"),
    ("blk_start_last_max", "if (!used[r] && e[r] > best)", "if (!used[r] && e[r] >= best)"),
    ("blk_start_reused_row", "            used[pick] = 1;\n", ""),
    ("blk_unused_marked_live", "idx[j] = live[j] ? j : -1;", "idx[j] = j;"),
    ("keyrow_smooth_columns", "for (int c = 0; c < D; ++c) a[c] = fabsf(R[r * D + c]);",
     "for (int c = 0; c < D; ++c) a[c] = fabsf(R[c * D + r]);"),
    ("keyrow_no_sqrt", "sr = sqrtf(lqo_t128_sum(a) * (1.0f / 128.0f));", "sr = lqo_t128_sum(a) * (1.0f / 128.0f);"),
    ("keyrow_boundary_axes", "((float)Q[r * D + c] * rho_col[c]) * sigma_row[r];",
     "((float)Q[r * D + c] * rho_col[r]) * sigma_row[c];"),
    ("fp8_truncate", "(unsigned)rint((q - 1.0) * 8.0)", "(unsigned)floor((q - 1.0) * 8.0)"),
    ("fp8_subnormal_exponent", "ldexp((double)m, -9)", "ldexp((double)m, -10)"),
    ("fp8_no_scale", "float sf = (float)s, inv = 1.0f / sf;", "float sf = 1.0f, inv = 1.0f;"),
    ("fp8_contiguous_groups", "for (int c = j; c < D; c += 4)\n            if (fabsf(u[c]) > M)",
     "for (int c = 32 * j; c < 32 * j + 32; ++c)\n            if (fabsf(u[c]) > M)"),
    ("fp8_record_unrounded", "u[c] = lqo_e4m3_to_f32(lqo_f32_to_e4m3(u[c] * inv)) * sf;", "u[c] = u[c];"),
    ("kda_step_column_decay", "S[r * D + c] = alpha[r] * S[r * D + c];", "S[r * D + c] = alpha[c] * S[r * D + c];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path):
    import oracle
    src = open(obuild.SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not unique ({src.count(old)})"
    mpath = os.path.join(tmp_path, f"{name}.c")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    so = obuild.build(mpath, os.path.join(tmp_path, f"lib{name}.so"))
    L = oracle.lib(so)
    failed = []
    for pin in pins.ALL:
        try:
            pin(L)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            failed.append((pin.__name__, type(e).__name__))
            break
    assert failed, f"mutant {name} passes every pin"
