"""Each plausible slip, planted in a private copy of the oracle (on the CPU),
must make at least one pin in test_oracle_pins.py fail."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gdn_oracle.c")

# name -> list of (exact text in gdn_oracle.c, replacement)
MUTATIONS = {
    "drop_delta_correction": [("Ta[e] -= s * Gc[e];", "Ta[e] -= 0.0 * s * Gc[e];")],
    "flip_correction_sign": [("Ta[e] -= s * Gc[e];", "Ta[e] += s * Gc[e];")],
    "decay_also_on_write": [("S[x] = al * T[x] + U[x];", "S[x] = al * (T[x] + U[x]);")],
    "decay_not_on_correction": [("for (int e = 0; e < Dk; ++e) Ta[e] = Sa[e];",
                                 "for (int e = 0; e < Dk; ++e) Ta[e] = al * Sa[e];"),
                                ("S[x] = al * T[x] + U[x];", "S[x] = T[x] + U[x];")],
    "output_from_pre_update_state": [("const double *Sa = S + (size_t)a * Dk;\n                        double acc",
                                      "const double *Sa = T + (size_t)a * Dk;\n                        double acc")],
    "transposed_state_in_output": [("acc += qi[e] * Sa[e];", "acc += qi[e] * S[(size_t)e * Dk + a];")],
    "no_key_normalisation": [("kh[(size_t)i * Dk + c] = ki[c] / den;", "kh[(size_t)i * Dk + c] = ki[c];")],
    "beta_of_wrong_head": [("double bi = beta[tok0 + (size_t)i * sN + h];",
                            "double bi = beta[tok0 + (size_t)i * sN];")],
    "alpha_of_wrong_head": [("double al = alpha[((size_t)b * F + f) * H + h];",
                             "double al = alpha[((size_t)b * F + f) * H];")],
    "beta_logit_not_divided": [("sigmoid(bi) / (double)N", "sigmoid(bi)")],
    "eps_added_not_clamped": [("double den = nrm > eps ? nrm : eps;", "double den = nrm + eps;")],
    "gram_transposed_write": [("const double s = bt[i] * vi[a];\n                        for (int e = 0; e < Dk; ++e) Ua[e] += s * ki[e];",
                               "const double s = bt[i] * ki[a % Dk];\n                        for (int e = 0; e < Dk; ++e) Ua[e] += s * vi[e % Dv];")],
}


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    src = open(SRC).read()
    for old, new in MUTATIONS[name]:
        assert src.count(old) == 1, "mutation anchor not found: %r" % old
        src = src.replace(old, new)
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", str(c), "-o",
                    str(so), "-lm"], check=True)
    env = dict(os.environ, GDN_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       env=env, cwd=ROOT, capture_output=True, text=True)
    assert r.returncode != 0, "no pin caught mutation %s:\n%s" % (name, r.stdout[-2000:])
