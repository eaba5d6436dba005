"""Plants one plausible mistake at a time in a copy of the oracle's C source, builds
it with gcc, and checks that the pin suite catches every one. Runs on the CPU only;
the real oracle is never modified."""

import os

import pytest

import oracle_pins
from oracle import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "gdn_oracle.c")

# (name, text in gdn_oracle.c, replacement)
MUTANTS = [
    ("delta_sign", "m[j] = beta * (act[v_chan(s, h, j)] - alpha * m[j]);",
     "m[j] = beta * (act[v_chan(s, h, j)] + alpha * m[j]);"),
    ("delta_drops_beta", "m[j] = beta * (act[v_chan(s, h, j)]", "m[j] = (act[v_chan(s, h, j)]"),
    ("delta_drops_alpha", "- alpha * m[j]);", "- m[j]);"),
    ("update_drops_decay", "H[(long)i * dv + j] = alpha * H[(long)i * dv + j] + act",
     "H[(long)i * dv + j] = H[(long)i * dv + j] + act"),
    ("update_sign", "H[(long)i * dv + j] + act[k_chan(s, g, i)] * m[j];",
     "H[(long)i * dv + j] - act[k_chan(s, g, i)] * m[j];"),
    ("readout_uses_k", "o[(long)h * dv + j] += H[(long)i * dv + j] * act[q_chan(s, g, i)];",
     "o[(long)h * dv + j] += H[(long)i * dv + j] * act[k_chan(s, g, i)];"),
    ("transposed_state_read", "m[j] += H[(long)i * dv + j] * act[k_chan(s, g, i)];",
     "m[j] += H[(long)j * dk + i] * act[k_chan(s, g, i)];"),
    ("readout_unscaled", "const double scale = 1.0 / sqrt((double)dk);", "const double scale = 1.0;"),
    ("readout_scaled_by_dv", "const double scale = 1.0 / sqrt((double)dk);",
     "const double scale = 1.0 / sqrt((double)dv);"),
    ("conv_taps_reversed", "u += (double)conv_w[c * K + j] * x;", "u += (double)conv_w[c * K + (K - 1 - j)] * x;"),
    ("conv_roll_stuck", "conv_state[(long)j * C + c] = conv_state[(long)(j + 1) * C + c];",
     "conv_state[(long)j * C + c] = conv_state[(long)j * C + c];"),
    ("conv_no_silu", "return silu(u);", "return u;"),
    ("softplus_sign", "log1p(exp(-fabs(x)))", "log1p(exp(fabs(x)))"),
    ("gate_without_exp_of_A_log", "exp(-exp((double)A_log[h]) *", "exp(-((double)A_log[h]) *"),
    ("gate_without_dt_bias", "softplus((double)dt_raw[h] + (double)dt_bias[h])", "softplus((double)dt_raw[h])"),
    ("beta_sign", "static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }",
     "static double sigmoid(double x) { return 1.0 / (1.0 + exp(x)); }"),
    ("head_map_modulo", "const int g = h / (s->num_v_heads / s->num_k_heads);",
     "const int g = h % s->num_k_heads;"),
    ("l2_without_eps", "1.0 / sqrt(sq + s->l2_eps)", "1.0 / sqrt(sq)"),
    ("l2_k_uses_q_norm", "rk = 1.0 / sqrt(sk + s->l2_eps)", "rk = 1.0 / sqrt(sq + s->l2_eps)"),
    ("rms_sum_not_mean", "ms /= (double)dv;", ""),
    ("rms_without_eps", "1.0 / sqrt(ms + s->rms_eps)", "1.0 / sqrt(ms)"),
    ("no_z_gate", "out[e] = yn * silu((double)z[e]);", "out[e] = yn;"),
    ("z_gate_sigmoid", "out[e] = yn * silu((double)z[e]);", "out[e] = yn * sigmoid((double)z[e]);"),
    ("no_norm_weight", "const double yn = o[e] * r * (double)norm_w[j];", "const double yn = o[e] * r;"),
    ("k_reads_q_channels", "return (long)s->num_k_heads * s->head_k_dim + (long)g * s->head_k_dim + i;",
     "return (long)g * s->head_k_dim + i;"),
    ("v_offset_one_segment", "return 2L * s->num_k_heads * s->head_k_dim + (long)h * s->head_v_dim + j;",
     "return 1L * s->num_k_heads * s->head_k_dim + (long)h * s->head_v_dim + j;"),
    ("linear_transposed_weight", "(double)w[(long)n * K + k];", "(double)w[(long)k * N + n];"),
    ("linear_drops_last_term", "for (int k = 0; k < K; ++k) acc +=", "for (int k = 0; k < K - 1; ++k) acc +="),
    ("linear_float_accumulation", "      double acc = 0.0;\n      for (int k = 0; k < K; ++k) acc +=",
     "      float acc = 0.0f;\n      for (int k = 0; k < K; ++k) acc +="),
    ("linear_x_row_stride", "acc += (double)x[(long)m * K + k]", "acc += (double)x[(long)m * N + k]"),
]


def _first_failing_pin():
    for pin in oracle_pins.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError):
            return pin.__name__
    return None


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, "mutation site not found exactly once: %r" % old
    mutated = tmp_path / ("gdn_oracle_%s.c" % name)
    mutated.write_text(src.replace(old, new))
    lib = O.build(force=True, src=str(mutated), out=str(tmp_path / ("libgdn_oracle_%s.so" % name)))
    with O.use_library(lib):
        caught_by = _first_failing_pin()
    assert caught_by is not None, "planted mistake %s passed every pin" % name


def test_unmutated_copy_passes():
    assert _first_failing_pin() is None
