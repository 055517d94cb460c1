"""Plant plausible mistakes in a copy of the oracle and check that the pin
suite catches every one (CPU only; the planted copies live in a temp dir)."""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

# (name, original text, planted text): each original must occur exactly once
MUTANTS = [
    ("sum_not_mean", "double mean_sq = sum_sq / (double)hidden;", "double mean_sq = sum_sq;"),
    ("eps_outside_root", "sqrt(mean_sq + eps)", "(sqrt(mean_sq) + eps)"),
    ("no_gamma", "widen(gamma, i, dtype) * widen(x, base + i, dtype) / root",
     "widen(x, base + i, dtype) / root"),
    ("row_stride_ignored", "const int64_t base = t * x_stride;", "const int64_t base = t * hidden;"),
    ("residual_subtracted", "widen(x, at, dtype) + widen(residual, at, dtype)",
     "widen(x, at, dtype) - widen(residual, at, dtype)"),
    ("norm_sees_unrounded_sum", "oracle_rmsnorm(y, residual_out, gamma, rows, hidden, hidden, eps, dtype);",
     "for (int64_t t = 0; t < rows; ++t) { double ss = 0.0;"
     " for (int64_t i = 0; i < hidden; ++i) { double v = widen(x, t * hidden + i, dtype) + widen(residual, t * hidden + i, dtype); ss += v * v; }"
     " double root = sqrt(ss / (double)hidden + eps);"
     " for (int64_t i = 0; i < hidden; ++i) y[t * hidden + i] = widen(gamma, i, dtype) * (widen(x, t * hidden + i, dtype) + widen(residual, t * hidden + i, dtype)) / root; }"),
    ("rotation_sign", "out[h * head_dim + j] = a * c[j] - b * s[j];", "out[h * head_dim + j] = a * c[j] + b * s[j];"),
    ("interleaved_partner", "double b = widen(v, hb + j + half, dtype);", "double b = widen(v, hb + (j ^ 1), dtype);"),
    ("section_map", "if (j < sec_t + sec_h) {\n        return 1;", "if (j < sec_t + sec_h) {\n        return 2;"),
    ("frequency_exponent", "-2.0 * (double)j / (double)head_dim", "-1.0 * (double)j / (double)head_dim"),
    ("frequency_half_dim", "-2.0 * (double)j / (double)head_dim", "-2.0 * (double)j / (double)half"),
    ("q_token_stride_ignored", "q, t * q_token_stride,", "q, t * (int64_t)n_q_heads * head_dim,"),
    ("k_uses_q_positions_shifted", "pos[stream * pos_stride + t]", "pos[stream * pos_stride + (t > 0 ? t - 1 : t)]"),
    ("gate_up_swapped", "double g = widen(gate_up, t * gate_up_stride + i, dtype);\n            double u = widen(gate_up, t * gate_up_stride + inter + i, dtype);",
     "double u = widen(gate_up, t * gate_up_stride + i, dtype);\n            double g = widen(gate_up, t * gate_up_stride + inter + i, dtype);"),
    ("sigmoid_sign", "return 1.0 / (1.0 + exp(-g));", "return 1.0 / (1.0 + exp(g));"),
    ("naive_sigmoid_underflow", "double e = exp(g);\n    return e / (1.0 + e);", "return (float)(1.0 / (1.0 + exp(-(double)(float)g)));"),
    ("bf16_truncates", "nearbyint(a / quantum)", "floor(a / quantum)"),
    ("topk_ascending", "    if (x > y) {\n        return -1;\n    }\n    if (x < y) {\n        return 1;\n    }",
     "    if (x > y) {\n        return 1;\n    }\n    if (x < y) {\n        return -1;\n    }"),
    ("topk_ties_high_index_first", "return i < j ? -1 : (i > j ? 1 : 0);", "return i < j ? 1 : (i > j ? -1 : 0);"),
    ("topk_not_renormalised", "cum += exp(z[order[j]] / temperature - zt) / kept_sum;",
     "cum += exp(z[order[j]] / temperature - zt) / (kept_sum * 1.25);"),
    ("topk_sample_ge", "if (!found && cum > (double)u[r]) {", "if (!found && cum >= (double)u[r]) {"),
    ("topk_temperature_ignored", "const double zt = z[order[0]] / temperature;", "const double zt = z[order[0]]; temperature = 1.0;"),
    ("kv_seq_head_swapped", "const int64_t at = ((b * n_kv_heads + h) * max_seq + s) * head_dim;",
     "const int64_t at = ((h * n_seqs + b) * max_seq + s) * head_dim;"),
    ("kv_cache_gets_unrotated_k", "k_cache_out[at + d] = k_rot[h * head_dim + d];",
     "k_cache_out[at + d] = widen(k, t * k_token_stride + (int64_t)h * head_dim + d, dtype);"),
    ("kv_slot_ignored", "const int64_t b = seq_idx[t], s = slot[t];", "const int64_t b = seq_idx[t], s = slot[t] > 0 ? 0 : slot[t];"),
    ("ln_unbiased_variance", "double variance = sum_dev_sq / (double)hidden;",
     "double variance = sum_dev_sq / (double)(hidden - 1);"),
    ("ln_variance_not_centred", "double d = widen(x, row_at + i, dtype) - mean;",
     "double d = widen(x, row_at + i, dtype);"),
    ("ln_output_not_centred", "(widen(x, row_at + i, dtype) - mean) / root", "widen(x, row_at + i, dtype) / root"),
    ("ln_eps_outside_root", "double root = sqrt(variance + eps);", "double root = sqrt(variance) + eps;"),
    ("ln_beta_dropped", "v += widen(beta, i, dtype);", "v += 0.0;"),
    ("ln_beta_scaled_by_gamma", "v += widen(beta, i, dtype);", "v += widen(gamma, i, dtype) * widen(beta, i, dtype);"),
    ("ln_row_stride_ignored", "const int64_t row_at = t * x_stride;", "const int64_t row_at = t * hidden;"),
    ("ln_add_norms_x", "oracle_layernorm(y, residual_out, gamma, beta, rows, hidden, hidden, eps, dtype);",
     "oracle_layernorm(y, x, gamma, beta, rows, hidden, hidden, eps, dtype);"),
    ("lin_no_rms", "xn[n] = widen(x, xrow + n, dtype) / rms;", "xn[n] = widen(x, xrow + n, dtype);"),
    ("lin_rms_sum_not_mean", "double rms = sqrt(sum_sq / (double)n_in + eps);", "double rms = sqrt(sum_sq + eps);"),
    ("lin_eps_outside_root", "double rms = sqrt(sum_sq / (double)n_in + eps);", "double rms = sqrt(sum_sq / (double)n_in) + eps;"),
    ("lin_w_stride_ignored", "widen(w, k * w_stride + n, dtype)", "widen(w, k * n_in + n, dtype)"),
    ("lin_x_stride_ignored", "const int64_t xrow = m * x_stride;", "const int64_t xrow = m * n_in;"),
    ("lin_w_row_off_by_one", "widen(w, k * w_stride + n, dtype)", "widen(w, (k > 0 ? k - 1 : k) * w_stride + n, dtype)"),
    ("bf16_via_fp32", "int e = ilogb(a);", "a = (double)(float)a; int e = ilogb(a);"),
]


@pytest.mark.parametrize("name,orig,planted", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(name, orig, planted, tmp_path):
    src = open(SRC).read()
    assert src.count(orig) == 1, f"{name}: anchor text not found exactly once"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(orig, planted))
    lib = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-std=c99", "-O2", "-fPIC", "-shared", "-ffp-contract=off",
                    "-I", os.path.join(ROOT, "oracle"), str(mut), "-o", str(lib), "-lm"], check=True)
    env = dict(os.environ, NRS_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"planted mistake {name!r} passed every pin:\n{r.stdout[-2000:]}"
