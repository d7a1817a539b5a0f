"""Plant plausible mistakes in a copy of oracle.c (on the CPU) and check that
the pins catch every one of them: a dropped term, a wrong sign, a wrong or
transposed index, a swapped operand, a wrong constant, a wrong reading."""
import os

import pytest

import oracle
import oracle_checks as oc

# (name, original text, replacement).  Each original must occur exactly once.
MUTANTS = [
    ("sample_std", "double sd = sqrt(ss / (double)d);", "double sd = sqrt(ss / (double)(d - 1));"),
    ("hard_threshold_value", "if (m) m[count] = x[i] - theta;", "if (m) m[count] = x[i];"),
    ("non_strict_select", "if (x[i] > theta) {", "if (x[i] >= theta) {"),
    ("theta_sign", "double theta = mean + sd * z;", "double theta = mean - sd * z;"),
    ("k1_transposed", "s += ld(k1t, wdtype, i * r + j) * q[j];", "s += ld(k1t, wdtype, j * d_ff + i) * q[j];"),
    ("k2_reads_predictor_half", "g += ld(k2t, wdtype, i * rc + j) * q[r + j];",
     "g += ld(k2t, wdtype, i * rc + j) * q[j];"),
    ("v_column_index", "s += c[t] * ld(v, wdtype, (int64_t)S[t] * d_model + col);",
     "s += c[t] * ld(v, wdtype, (int64_t)col * d_ff + S[t]);"),
    ("gelu_dropped", "c[t] = oracle_gelu_tanh(m[t]) * g;", "c[t] = m[t] * g;"),
    ("gelu_constant", "(v + 0.044715 * v * v * v)", "(v + 0.04715 * v * v * v)"),
    ("quantile_coef", "4.5921953931549871457e4", "4.5921953931549871457e3"),
    ("quantile_tail_coef", "7.74545014278341407640e-4", "7.74545014278341407640e-3"),
    ("rms_sum_not_mean", "double inv = 1.0 / sqrt(ss / (double)d_model + eps);", "double inv = 1.0 / sqrt(ss + eps);"),
    ("gqa_modulo", "attn_query(dtype, q, h * hd, k1, k2, v, h / group,", "attn_query(dtype, q, h * hd, k1, k2, v, h % Hkv,"),
    ("softmax_unnormalised", "double w = exp(s[j] - smax) / den;", "double w = exp(s[j] - smax);"),
    ("softplus_as_relu", "return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));", "return (v > 0.0 ? v : 0.0);"),
    ("attn_compute_half_offset", "a += ld(q, dtype, qi + r + c) * ld(k2, dtype, (g * N + j) * rc + c);",
     "a += ld(q, dtype, qi + c) * ld(k2, dtype, (g * N + j) * rc + c);"),
    ("attn_prefix_short", "h / group, T, t + 1, hd, r, k_attn,", "h / group, T, t, hd, r, k_attn,"),
    ("attn_prefix_stride", "h / group, T, t + 1, hd, r, k_attn,", "h / group, t + 1, t + 1, hd, r, k_attn,"),
    ("bf16_widen_shift", "uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 16;",
     "uint32_t u = (uint32_t)((const uint16_t *)base)[i] << 15;"),
    ("mean_off_by_one", "double mean = s / (double)d;", "double mean = s / (double)(d + 1);"),
    ("huber_quadratic_scale", "if (u < delta) return u * u / (2.0 * delta);", "if (u < delta) return u * u / delta;"),
    ("huber_grad_slope", "if (u < delta) return u / delta;", "if (u < delta) return 1.0;"),
    ("huber_backward_no_std_term", "if (sd > 0.0) dth += z", "if (sd < 0.0) dth += z"),
    ("huber_backward_no_mean_term", "double dth = 1.0 / (double)d;", "double dth = 0.0;"),
    ("huber_backward_sign", "dx[r * d + j] -= A * dth;", "dx[r * d + j] += A * dth;"),
    ("huber_sample_std", "*sd = sqrt(ss / (double)d);", "*sd = sqrt(ss / (double)(d - 1));"),
]

# faster, smaller versions of the slow checks are enough to catch the mutants
FAST = [oc.check_quantile, oc.check_threshold_closed_form, oc.check_special_rows, oc.check_quantile_grid,
        oc.check_invariants, oc.check_ffn_dense_masked, oc.check_ffn_bf16_widening, oc.check_activations,
        oc.check_attention, oc.check_attention_prefill, oc.check_continuity, oc.check_decode_chain,
        oc.check_huber_function, oc.check_huber_limit, oc.check_huber_gradient_fd, oc.check_huber_autograd,
        oc.check_huber_invariances]


def _caught(path):
    failed = []
    with oracle.use_build(path):
        for chk in FAST:
            try:
                chk()
            except AssertionError:
                failed.append(chk.__name__)
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new, tmp_path, orc):
    src = oracle.source_text()
    assert src.count(old) == 1, f"mutation site for {name} not unique"
    path = oracle.compile_variant(src.replace(old, new), str(tmp_path / f"mut_{name}.so"))
    failed = _caught(path)
    assert failed, f"planted mistake {name} passed every pin"


def test_unmutated_copy_passes(tmp_path, orc):
    path = oracle.compile_variant(oracle.source_text(), str(tmp_path / "same.so"))
    assert _caught(path) == []
