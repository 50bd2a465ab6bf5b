"""The pins must catch plausible mistakes.  Each case plants one mistake in a
copy of the oracle's C source (on the CPU), builds it, and runs the oracle's
pin and invariant tests against it in a subprocess: they must fail."""
import os
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "rnn_oracle.c")
sys.path.insert(0, os.path.join(ROOT, "oracle"))
from build import CFLAGS  # noqa: E402  (oracle/build.py)

MUTATIONS = {
    "lstm_drops_Rb": ("v = v + Rb[g * H + u];", ";"),
    "lstm_f_reads_o_gate": ("float pf_ = clipv(pre[2]", "float pf_ = clipv(pre[1]"),
    "peephole_o_uses_old_cell": ("Pd[H + u] * cnew", "Pd[H + u] * cp"),
    "peephole_f_uses_o_weights": ("Pd[2 * H + u] * cp", "Pd[H + u] * cp"),
    "reverse_starts_at_seq_end": ("t = reverse ? len - 1 - j : j", "t = reverse ? S - 1 - j : j"),
    "len0_keeps_initial_state": ("Yh[so + u] = len == 0 ? 0.0f : canon(h[u])", "Yh[so + u] = canon(h[u])"),
    "gru_lbr1_bias_swapped": ("                                ph = ph + Wb[2 * H + u];",
                              "                                ph = ph + Rb[2 * H + u];"),
    "gru_update_uses_z_not_1_minus_z": ("float omz = 1.0f - z;", "float omz = z;"),
    "gru_lbr0_forgets_reset": ("s[u] = r * h[u];", "s[u] = h[u];"),
    "clip_lower_bound_sign": ("(x < -c ? -c : x)", "(x < -c ? c : x)"),
    "single_cursor_for_beta": ("parsed[i].beta = beta[cb++];", "parsed[i].beta = beta[ca > 0 ? ca - 1 : 0];"),
    "hardsigmoid_default_beta": ("case ACT_HARDSIGMOID: return 0.5f;", "case ACT_HARDSIGMOID: return 0.0f;"),
    "gemm_k_descending": ("for (int64_t k = 0; k < K; k++) {", "for (int64_t k = K - 1; k >= 0; k--) {"),
    "y_not_zeroed_past_len": ("Y[i] = 0.0f;            /* positions", "(void)0;            /* positions"),
    "sigmoid_sign": ("1.0 / (1.0 + orc_exp(-(double)x))", "1.0 / (1.0 + orc_exp((double)x))"),
    "exp_poly_drops_constant_term": ("for (int i = 12; i >= 0; i--)", "for (int i = 12; i >= 1; i--)"),
    "exp_reduction_drops_ln2_tail": ("double r = (x - k * LN2_HI) - k * LN2_LO;",
                                     "double r = (x - k * LN2_HI);"),
    "tanh_wrong_denominator": ("copysign(m / (m + 2.0), x)", "copysign(m / (m + 1.0), x)"),
    "log1p_series_too_short": ("for (int n = 19; n >= 0; n--)", "for (int n = 2; n >= 0; n--)"),
    "layout1_state_index": ("(size_t)((b * D + d) * H)", "(size_t)((d * Bt + b) * H)"),
    "input_forget_uses_i": ("? 1.0f - ig", "? ig"),
    "no_nan_canonicalisation": ("if (v != v) {", "if (0) {"),
    "rnn_rec_added_last": ("""                        float pre = xw[u] + rec[u];
                        if (B) {
                            pre = pre + Wb[u];
                            pre = pre + Rb[u];
                        }""", """                        float pre = xw[u];
                        if (B) {
                            pre = pre + Wb[u];
                            pre = pre + Rb[u];
                        }
                        pre = pre + rec[u];"""),
    "lstm_fused_cell_update": ("float cnew = k1 + k2;", "float cnew = fmaf(fg, cp, k2);"),
    "bf16_truncates": ("u = u + 0x7FFFu + lsb;", "u = u + 0u * lsb;"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    mut = src.replace(old, new)
    cfile = tmp_path / "mut.c"
    cfile.write_text(mut)
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", *CFLAGS, "-o", str(lib), str(cfile), "-lm"], check=True)
    env = dict(os.environ, RNN_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py"),
                        os.path.join(ROOT, "tests", "test_oracle_invariants.py"),
                        os.path.join(ROOT, "tests", "test_oracle_elementary.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"planted mistake {name} was not caught:\n{r.stdout[-2000:]}"
