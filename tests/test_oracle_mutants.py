"""Planted mistakes: each plausible slip in the oracle must fail some pin.

Every case below edits one line of a copy of the oracle's C source (a dropped
term, a wrong sign, index or operand order), builds it, and runs the oracle
pin tests against that build in a child process.  The child must fail.  The
real oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")
PINS = ["tests/test_oracle_pre.py", "tests/test_oracle_scan.py",
        "tests/test_oracle_post_layer.py"]

MUTANTS = {
    "conv_taps_reversed": ("conv_w[(size_t)c * 4 + m]", "conv_w[(size_t)c * 4 + (3 - m)]"),
    "conv_history_row_off_by_one": ("(r < 3)", "(r < 2)"),
    "history_shifted": ("const int64_t src = T + r;", "const int64_t src = T + r - 1;"),
    "silu_drops_x": ("return x * sigmoid(x);", "return sigmoid(x);"),
    "l2_eps_outside_sqrt": ("const double inv = 1.0 / sqrt(ss + eps);",
                            "const double inv = 1.0 / (sqrt(ss) + eps);"),
    "split_k_reads_q_block": ("memcpy(kn + (size_t)t * hk * dk, row + hk * dk,",
                              "memcpy(kn + (size_t)t * hk * dk, row,"),
    "gate_drops_exp": ("g[i] = -exp(A_log[h])", "g[i] = -(A_log[h])"),
    "beta_sign": ("beta[i] = sigmoid(b[i]);", "beta[i] = sigmoid(-b[i]);"),
    "key_head_modulo": ("const int j = h / G;", "const int j = h % hk;"),
    "delta_sign": ("u[i] = bt * (v[i] - p);", "u[i] = bt * (p - v[i]);"),
    "decay_dropped": ("for (size_t e = 0; e < SS; ++e) S[e] *= alpha;", ";"),
    "state_transposed_in_output": ("acc += S[(size_t)i * dk + c] * q[c];",
                                   "acc += S[(size_t)c * dk + i] * q[c];"),
    "output_scale_dropped": ("ot[i] = acc * scale;", "ot[i] = acc;"),
    "rms_eps_dropped": ("const double inv = 1.0 / sqrt(ss / dv + eps);",
                        "const double inv = 1.0 / sqrt(ss / dv);"),
    "gamma_index": ("* gamma[i])", "* gamma[0])"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not unique: {old!r}"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new))
    lib = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(lib),
                    str(mut), "-lm"], check=True)
    env = dict(os.environ, GDN_ORACLE_LIB=str(lib), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        *PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode == 1, f"pins did not catch {name}:\n{r.stdout[-2000:]}"
