"""The oracle's pins catch plausible mistakes (CPU only).

Each case below plants one mistake in a copy of ``oracle/sq_oracle.c`` (a
dropped term, a wrong sign, index or operand, another rounding rule, a wrong
constant), builds that copy with gcc into a temporary directory and runs
``tests/test_oracle_pins.py`` against it in a child process.  The pins must
fail for every one of them, and must pass for an unchanged copy built the same
way.  The oracle in the repository is never modified.
"""
import concurrent.futures as cf
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sq_oracle.c")

# (name, text in sq_oracle.c, replacement); each text occurs exactly once
MUTATIONS = [
    ("rounding_half_away", "float r = rintf(v);", "float r = roundf(v);"),
    ("token_scale_over_128", "float sc = a / 127.0f;\n        x_scale[m] = sc;",
     "float sc = a / 128.0f;\n        x_scale[m] = sc;"),
    ("token_multiply_form", "Xq[m * K + j] = quant_code(x / sc);", "Xq[m * K + j] = quant_code(x * (127.0f / a));"),
    ("token_smoothing_multiplies", "if (s) x = x / s[j];                        /* X' = X diag(s)^-1 */",
     "if (s) x = x * s[j];"),
    ("token_outliers_in_max", "if (skip && skip[j]) continue;", ""),
    ("weight_smoothing_divides", "Ws[n * K + j] = s ? w * s[j] : w;", "Ws[n * K + j] = s ? w / s[j] : w;"),
    ("tensor_max_first_row_only", "for (int64_t i = 0; i < N * K; ++i) {\n            float v = fabsf(Ws[i]);",
     "for (int64_t i = 0; i < K; ++i) {\n            float v = fabsf(Ws[i]);"),
    ("smooth_exponent", "pow((double)w, 1.0 - al)", "pow((double)w, al)"),
    ("smooth_floor", "act_max[j] > 1e-8f ? act_max[j] : 1e-8f", "act_max[j] > 1e-6f ? act_max[j] : 1e-6f"),
    ("absmax_not_running", "float a = amax[j];", "float a = 0.0f;"),
    ("gemm_transposed_operand", "t += (int64_t)A[m * K + k] * (int64_t)B[n * K + k];",
     "t += (int64_t)A[m * K + k] * (int64_t)B[k * N + n];"),
    ("gemm_no_overflow_count", "if (t > INT32_MAX || t < INT32_MIN) ++bad;\n            acc[m * N + n]",
     "acc[m * N + n]"),
    ("dequant_wrong_scale", "y = y * ws;", "y = y * xs;"),
    ("dequant_bias_dropped", "if (bias) y = y + bias[n];", ""),
    ("outlier_not_strict", "mask[j] = cmax[j] > threshold ? 1 : 0;", "mask[j] = cmax[j] >= threshold ? 1 : 0;"),
    ("side_wrong_column", "(double)orc_half_to_float(W16[cols[i] * K + j]);",
     "(double)orc_half_to_float(W16[cols[i] * K + c]);"),
    ("combine_sign", "(float)((double)y_int8[i] + side[i])", "(float)((double)y_int8[i] - side[i])"),
    ("half_subnormal_scale", "v = (float)mant * 0x1p-24f;", "v = (float)mant * 0x1p-25f;"),
    ("half_ties_up", "if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;",
     "if (rem >= 0x1000u) h += 1u;"),
    ("layernorm_eps_dropped", "double rstd = 1.0 / sqrt(var + (double)eps);", "double rstd = 1.0 / sqrt(var);"),
    ("layernorm_sample_variance", "double var = (double)v / (((double)K * (double)K) * 0x1p48);",
     "double var = (double)v / (((double)K * (double)(K - 1)) * 0x1p48);"),
    ("fold_beta_multiplies", "if (beta) beta_out[j] = beta[j] / s[j];", "if (beta) beta_out[j] = beta[j] * s[j];"),
    ("percentile_floor", "(int64_t)ceil(p * (double)n / 100.0)", "(int64_t)floor(p * (double)n / 100.0)"),
    ("kv_margin_dropped", "scale[h] = (margin * m) / 127.0f;", "scale[h] = m / 127.0f;"),
    ("dequantize_group_modulo", "scale[m * row_stride + j / group]", "scale[m * row_stride + j % group]"),
    ("fp8_ties_away", "double r = nearbyint((2.0 * f - 1.0) * 8.0);", "double r = floor((2.0 * f - 1.0) * 8.0 + 0.5);"),
    ("fp8_exponent_bias", "(((E + 7) << 3) | (int)r)", "(((E + 8) << 3) | (int)r)"),
    ("fp8_row_scale_127", "float sc = a / 448.0f;\n        scale[m] = sc;", "float sc = a / 127.0f;\n        scale[m] = sc;"),
    ("fp8_subnormal_units", "int64_t n = E == 0 ? m :", "int64_t n = E == 0 ? 8 + m :"),
    ("asym_scale_over_256", "float sc = (hi - lo) / 255.0f;", "float sc = (hi - lo) / 256.0f;"),
    ("asym_range_without_zero", "float lo = 0.0f, hi = 0.0f;", "float lo = 1e30f, hi = -1e30f;"),
    ("asym_zero_point_sign", "float zf = rintf(-lo / sc);", "float zf = rintf(lo / sc);"),
    ("asym_shift_before_rounding", "u = (int)rintf(x / sc) + z;", "u = (int)rintf(x / sc + (float)z);"),
    ("asym_correction_sign", "(int64_t)acc[m * N + n] - (int64_t)x_zero[m]", "(int64_t)acc[m * N + n] + (int64_t)x_zero[m]"),
    ("rowsum_dropped_row", "for (int64_t k = 0; k < K; ++k) t += Wq[n * K + k];", "for (int64_t k = 1; k < K; ++k) t += Wq[n * K + k];"),
]


def _build(src_text, out_dir):
    c = os.path.join(out_dir, "sq_oracle.c")
    with open(c, "w") as f:
        f.write(src_text)
    lib = os.path.join(out_dir, "liboracle.so")
    subprocess.run(["gcc", "-std=c99", "-O1", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-o", lib, c, "-lm"], check=True, capture_output=True)
    return lib


def _pins(lib):
    """pytest's exit status for the oracle pins run against `lib`."""
    env = dict(os.environ, SQ_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, (r.stdout + r.stderr)[-3000:]


def test_mutation_sites_are_unique():
    text = open(SRC).read()
    for name, old, _ in MUTATIONS:
        assert text.count(old) == 1, name


def test_every_planted_mistake_fails_a_pin(tmp_path):
    text = open(SRC).read()
    jobs = [("unchanged", text)] + [(name, text.replace(old, new)) for name, old, new in MUTATIONS]
    libs = {}
    for name, src in jobs:
        d = tmp_path / name
        d.mkdir()
        libs[name] = _build(src, str(d))
    with cf.ThreadPoolExecutor(max_workers=4) as ex:
        res = dict(zip(libs, ex.map(_pins, libs.values())))
    rc, out = res.pop("unchanged")
    assert rc == 0, out
    survivors = {name: rc for name, (rc, _) in res.items() if rc != 1}
    # exit status 1 = some pin failed; 0 would mean the mistake went unnoticed, and
    # anything else (collection error, crash) is not a pin catching it
    assert not survivors, {n: res[n][1] for n in survivors}
