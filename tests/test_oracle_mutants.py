"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of ``oracle/oracle.c`` (on the CPU, in a
temporary directory), builds it, and runs the pin suites against the mutant:
the suite must fail.  A mutation that the pins let through would mean the
oracle is not pinned against that mistake.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "causal_range_off_by_one": ("for (int t = 0; t <= pos; ++t) {\n            const float* k", "for (int t = 0; t < pos; ++t) {\n            const float* k"),
    "attention_scale_dropped": ("att[t] = s / ACC_SQRT((acc_t)head_size);", "att[t] = s;"),
    "rmsnorm_eps_dropped": ("sum_sq / (acc_t)n + (acc_t)eps", "sum_sq / (acc_t)n"),
    "rmsnorm_sum_not_mean": ("sum_sq / (acc_t)n + (acc_t)eps", "sum_sq + (acc_t)eps"),
    "rope_sign_flipped": ("const acc_t R[2][2] = {{cos(a), -sin(a)}, {sin(a), cos(a)}};",
                          "const acc_t R[2][2] = {{cos(a), sin(a)}, {sin(a), cos(a)}};"),
    "rope_frequency_index": ("pow(theta, -(double)(2 * j) / (double)head_size)",
                             "pow(theta, -(double)j / (double)head_size)"),
    "swiglu_branches_swapped": ("const acc_t gate = (acc_t)h1[i] * logistic((acc_t)h1[i]);\n        hb[i] = (float)(gate * (acc_t)h3[i]);",
                                "const acc_t gate = (acc_t)h3[i] * logistic((acc_t)h3[i]);\n        hb[i] = (float)(gate * (acc_t)h1[i]);"),
    "attention_residual_overwrites": ("add_into(x, xb2, dim);", "memcpy(x, xb2, sizeof(float) * (size_t)dim);"),
    "ffn_residual_dropped": ("oracle_matvec(xb, w.w2 + lw * dim * hidden, hb, dim, hidden);\n        add_into(x, xb, dim);",
                             "oracle_matvec(xb, w.w2 + lw * dim * hidden, hb, dim, hidden);"),
    "kv_head_integer_kv_mul": ("return (int)(((int64_t)h * n_kv_heads) / n_heads);",
                               "return h / (n_heads / n_kv_heads) < n_kv_heads ? h / (n_heads / n_kv_heads) : n_kv_heads - 1;"),
    "matvec_transposed": ("for (int j = 0; j < n; ++j) s += (acc_t)row[j] * (acc_t)x[j];",
                          "for (int j = 0; j < n; ++j) s += (acc_t)w[(int64_t)j * d + i] * (acc_t)x[j];"),
    "argmax_last_maximum": ("for (int i = 0; i < n; ++i)\n        if (v[i] == top) return i;",
                            "for (int i = n - 1; i >= 0; --i)\n        if (v[i] == top) return i;"),
    "key_rope_skipped": ("oracle_rope(krow, KV, hs, pos, o->rope_theta);", ""),
    "ffn_norm_uses_attention_gain": ("oracle_rmsnorm(xb, x, w.rms_ffn + lw * dim, dim, o->norm_eps);",
                                     "oracle_rmsnorm(xb, x, w.rms_att + lw * dim, dim, o->norm_eps);"),
    "softmax_max_not_subtracted_wrongly": ("att[t] = ACC_EXP(att[t] - m);", "att[t] = ACC_EXP(att[t] + m);"),
    "sample_temperature_ignored": ("pi[i].p = (acc_t)logits[i] / (acc_t)temperature;", "pi[i].p = (acc_t)logits[i];"),
    "top_p_not_renormalised": ("const acc_t r = (acc_t)coin * mass;", "const acc_t r = (acc_t)coin;"),
    "top_p_ascending_order": ("if (x->p > y->p) return -1;\n    if (x->p < y->p) return 1;",
                              "if (x->p > y->p) return 1;\n    if (x->p < y->p) return -1;"),
    "top_p_ties_to_higher_index": ("return x->i - y->i;", "return y->i - x->i;"),
    "top_p_set_stops_below_p": ("while (k < n && mass < (acc_t)topp) mass += pi[k++].p;",
                                "while (k < n && mass + pi[k].p < (acc_t)topp) mass += pi[k++].p;\n        if (k == 0) mass += pi[k++].p;"),
    "multinomial_walks_sorted_order": ("if (topp <= 0 || topp >= 1) {", "if (0) {"),
    "stop_not_checked_on_forced_tokens": ("if (stop_token >= 0 && next == stop_token) break;",
                                          "if (stop_token >= 0 && i + 1 >= n_prompt && next == stop_token) break;"),
    "prompt_forcing_off_by_one": ("const int next = i + 1 < n_prompt ? prompt[i + 1]", "const int next = i + 2 < n_prompt ? prompt[i + 1]"),
}
PIN_FILES = ("test_oracle_sampling.py", "test_oracle_pins.py")


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    mut = tmp_path / "oracle_mut.c"
    mut.write_text(src.replace(old, new))
    so = tmp_path / "liboracle_mut.so"
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-std=c11", "-fPIC", "-shared", "-pthread",
                    "-I", os.path.join(ROOT, "oracle"), str(mut), "-o", str(so), "-lm"], check=True)
    env = dict(os.environ, ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider"] +
                       [os.path.join(ROOT, "tests", f) for f in PIN_FILES],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch mutant {name}:\n{r.stdout[-2000:]}"
