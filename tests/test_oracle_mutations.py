"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake into a temporary copy of the oracle's C source
(on the CPU only), builds it, and runs the pin suite against it: at least one
pin has to fail.  The real oracle is untouched.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "kda_oracle.c")

MUTATIONS = {
    "no_decay": ("*= exp(a[c]);", "*= 1.0;"),
    "decay_after_read": ("/* 2d. decay: S <- S Diag(e^a) */", "/* 2d. */ if (0)"),
    "write_sign": ("double d = bt * (vv[i] - r[i]);", "double d = bt * (vv[i] + r[i]);"),
    "no_read": ("r[i] = acc;", "r[i] = 0.0 * acc;"),
    "write_with_q": ("+= d * kn[c];", "+= d * qn[c];"),
    "output_with_k": ("acc += S[(size_t)i * K + c] * qn[c];", "acc += S[(size_t)i * K + c] * kn[c];"),
    "softplus_arg_sign": ("return -exp(A_log) * orc_softplus(x);", "return -exp(A_log) * orc_softplus(-x);"),
    "safe_missing_exp": ("lower_bound * orc_sigmoid(exp(A_log) * x)", "lower_bound * orc_sigmoid(A_log * x)"),
    "l2_eps": ("#define ORC_L2_EPS 1e-6", "#define ORC_L2_EPS 1e-2"),
    "no_beta_sigmoid": ("if (!(flags & ORC_FLAG_BETA_IS_PROB)) bt = orc_sigmoid(bt);", ""),
    "gva_head_map": ("hq = h / G;", "hq = h % Hqk;"),
    "ignore_h0": ("if (h0) memcpy", "if (0) memcpy"),
    "no_dt_bias": ("(dt_bias ? (double)dt_bias[(size_t)h * K + c] : 0.0)", "0.0"),
    "varlen_bos": ("bos = cu_seqlens[n]; eos", "bos = cu_seqlens[n] + (n > 0); eos"),
    "transposed_state_read": ("acc += S[(size_t)i * K + c] * kn[c];",
                              "acc += S[(size_t)(c % V) * K + (i % K)] * kn[c];"),
}


# mistakes planted in the gradient code, caught by tests/test_oracle_bwd.py
MUTATIONS_BWD = {
    "bwd_no_decay_carry": ("dS[(size_t)i * K + c] *= tk.ea[c];", "dS[(size_t)i * K + c] *= 1.0;"),
    "bwd_read_sign": ("const double dr = -tk.bt * du[i];", "const double dr = tk.bt * du[i];"),
    "bwd_no_read_key_term": ("dkn[c] += Sd[(size_t)i * K + c] * dr;", "dkn[c] += 0.0 * dr;"),
    "bwd_output_state_before_write": ("acc += St[(size_t)i * K + c] * dot[i];", "acc += Sp[(size_t)i * K + c] * dot[i];"),
    "bwd_decay_grad_no_exp": ("da[c] = tk.ea[c] * acc;", "da[c] = acc;"),
    "bwd_norm_no_projection": ("dqt[c] = tk.rq * (dqn[c] - tk.qn[c] * yq);", "dqt[c] = tk.rq * dqn[c];"),
    "bwd_beta_no_sigmoid_grad": ("dbt * tk.bt * (1.0 - tk.bt);", "dbt;"),
    "bwd_softplus_grad_sign": ("dadx = -Aexp * orc_sigmoid(x);", "dadx = Aexp * orc_sigmoid(x);"),
    "bwd_safe_grad_missing_exp": ("dadx = lower_bound * s * (1.0 - s) * Aexp;", "dadx = lower_bound * s * (1.0 - s);"),
    "bwd_gva_sum_one_head": ("for (int j = 0; j < G; ++j) {", "for (int j = 0; j < 1; ++j) {"),
    "bwd_dbeta_uses_v": ("dbt += acc * (tk.vv[i] - r[i]);", "dbt += acc * tk.vv[i];"),
    "bwd_checkpoint_off_by_one": ("memcpy(Sbuf, Sck + (size_t)blk * VK", "memcpy(Sbuf, Sck + (size_t)(blk > 0 ? blk - 1 : 0) * VK"),
}


def _run_pins(name, old, new, tmp_path, pin_file):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = tmp_path / "kda_oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libkda_oracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-w",
                           "-o", str(lib), str(mutated), "-lm"])
    env = dict(os.environ, KDA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pin_file)],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutation {name} survived every pin:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTATIONS_BWD))
def test_gradient_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS_BWD[name]
    _run_pins(name, old, new, tmp_path, "test_oracle_bwd.py")


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation anchor not found: {old}"
    mutated = tmp_path / "kda_oracle_mut.c"
    mutated.write_text(src.replace(old, new))
    lib = tmp_path / "libkda_oracle_mut.so"
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-w",
                           "-o", str(lib), str(mutated), "-lm"])
    env = dict(os.environ, KDA_ORACLE_LIB=str(lib))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"mutation {name} survived every pin:\n{r.stdout[-2000:]}"
