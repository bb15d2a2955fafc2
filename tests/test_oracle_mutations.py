"""Each plausible slip, planted in a private copy of the oracle (on the CPU),
must make at least one pin fail: slips in the forward scan (gdn_oracle_scan)
against test_oracle_pins.py, slips in the backward pass (gdn_oracle_scan_bwd)
against test_oracle_bwd.py.  Each anchor must occur exactly once inside the
function it targets."""
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
    "reverse_flag_ignored": [("const int f = reverse ? F - 1 - step : step;", "const int f = step;")],
    "raw_keys_flag_ignored": [("if (!normalize_k) den = 1.0;", "if (!normalize_k) den = den;")],
    "eps_added_not_clamped": [("double den = nrm > eps ? nrm : eps;", "double den = nrm + eps;")],
    "gram_transposed_write": [("const double s = bt[i] * vi[a];\n                        for (int e = 0; e < Dk; ++e) Ua[e] += s * ki[e];",
                               "const double s = bt[i] * ki[a % Dk];\n                        for (int e = 0; e < Dk; ++e) Ua[e] += s * vi[e % Dv];")],
}


BWD_MUTATIONS = {
    "bwd_state_gradient_not_decayed": [("Dn[(size_t)a * Dk + c] = al * t;", "Dn[(size_t)a * Dk + c] = t;")],
    "bwd_state_gradient_no_correction": [
        ("for (int e = 0; e < Dk; ++e) t -= Dm[(size_t)a * Dk + e] * G[(size_t)c * Dk + e];", "")],
    "bwd_dG_sign": [("dG[(size_t)c * Dk + e] = -al * acc;", "dG[(size_t)c * Dk + e] = al * acc;")],
    "bwd_dG_not_symmetrised": [("(dG[(size_t)c * Dk + e] + dG[(size_t)e * Dk + c])", "2.0 * dG[(size_t)c * Dk + e]")],
    "bwd_no_normalisation_projection": [("dki[c] = (dkh[c] - khi[c] * proj) / nrm[i];", "dki[c] = dkh[c] / nrm[i];")],
    "bwd_dq_from_previous_state": [("acc += Sc[(size_t)a * Dk + e] * doi[a];", "acc += Sp[(size_t)a * Dk + e] * doi[a];")],
    "bwd_dalpha_without_correction": [
        ("for (int c = 0; c < Dk; ++c) t -= Sp[(size_t)a * Dk + c] * G[(size_t)c * Dk + e];\n"
         "                        T[(size_t)a * Dk + e] = t;",
         "T[(size_t)a * Dk + e] = t;")],
    "bwd_dbeta_missing_value_term": [("db += vi[a] * uk;", "db += 0.0 * uk;")],
    "bwd_dv_missing_beta": [("dv[ti * Dv + a] = bt[i] * uk;", "dv[ti * Dv + a] = uk;")],
    "bwd_logit_beta_not_divided": [("db = db * sg * (1.0 - sg) / (double)N;", "db = db * sg * (1.0 - sg);")],
}


def _function_span(src, name):
    start = src.index("int %s(" % name)
    nxt = src.find("\nint ", start + 1)
    return start, (len(src) if nxt < 0 else nxt)


def _plant(name, tmp_path, edits, scope, pins):
    src = open(SRC).read()
    lo, hi = _function_span(src, scope)
    body = src[lo:hi]
    for old, new in edits:
        assert body.count(old) == 1, "mutation anchor not found once in %s: %r" % (scope, old)
        body = body.replace(old, new)
    src = src[:lo] + body + src[hi:]
    c = tmp_path / "mut.c"
    so = tmp_path / "libmut.so"
    c.write_text(src)
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", str(c), "-o",
                    str(so), "-lm"], check=True)
    env = dict(os.environ, GDN_ORACLE_LIB=str(so), OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", pins)],
                       env=env, cwd=ROOT, capture_output=True, text=True)
    assert r.returncode != 0, "no pin caught mutation %s:\n%s" % (name, r.stdout[-2000:])


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    _plant(name, tmp_path, MUTATIONS[name], "gdn_oracle_scan", "test_oracle_pins.py")


@pytest.mark.slow
@pytest.mark.parametrize("name", sorted(BWD_MUTATIONS))
def test_backward_pins_catch_planted_mistake(name, tmp_path):
    _plant(name, tmp_path, BWD_MUTATIONS[name], "gdn_oracle_scan_bwd", "test_oracle_bwd.py")
