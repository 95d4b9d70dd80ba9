"""Planted mistakes in a copy of the oracle must fail the pins.

Each case copies oracle/oracle.c to a temporary directory, applies one textual
mutation (a dropped term, a wrong index, scale, factorial or multiplicity),
compiles it with gcc, points the oracle module at the mutant and runs the pin
that should catch it.  The pin must fail on the mutant and pass on the original.
CPU only.
"""
import os
import subprocess

import numpy as np
import pytest

import oracle

import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")


def _alpha_pins():
    pins.test_P2_is_linear_kernel()
    pins.test_P3_is_quadratic_kernel()
    pins.test_large_P_converges_to_softmax()


def _table_pins():
    pins.test_worked_example_d2_p2()
    for d in (2, 3, 4):
        for p in (2, 3):
            pins.test_table_counts_and_order(d, p)
            pins.test_symmetric_identity_exact(d, p)


def _feature_form_pins():
    pins.test_feature_form_equals_direct(8, 8, 4, 64, 1.0)
    pins.test_feature_form_equals_direct(3, 2, 3, 25, 1.0)
    pins.test_state_invariants()


def _causal_pins():
    pins.test_first_row_is_v0()
    pins.test_P1_is_cumulative_mean()


def _grad_pins():
    pins.test_grad_matches_finite_differences(4, 2)
    pins.test_grad_invariant_under_value_shift()


MUTANTS = {
    # alpha_p = 1/(p! c^p): factorial off by one
    "factorial": ("for (int s = 2; s <= p; ++s) fact *= s;",
                  "for (int s = 2; s <= p; ++s) fact *= s + 1;", _alpha_pins),
    # c = sqrt(dK) replaced by dK
    "scale": ("pow(sqrt((double)dK), p)", "pow((double)dK, p)", _alpha_pins),
    # Horner/power order: x^p paired with alpha_{p+1}
    "power_index": ("for (int p = 0; p < P; ++p) { w += a[p] * xp; xp *= x; }",
                    "for (int p = 0; p < P; ++p) { xp *= x; w += a[p] * xp; }", _alpha_pins),
    # causal sum excludes the diagonal
    "causal": ("den += w;\n        for (int j = 0; j < dV; ++j) yT[j] += w * vt[j];",
               "if (t == T) continue;\n        den += w;\n"
               "        for (int j = 0; j < dV; ++j) yT[j] += w * vt[j];",
               _causal_pins),
    # tables: a multiplicity of one for every monomial
    "multiplicity": ("count[key] += 1;", "count[key] = 1;", _table_pins),
    # tables: tuples sorted descending
    "sort_order": ("sorted[b - 1] > sorted[b]", "sorted[b - 1] < sorted[b]", _table_pins),
    # feature form: the C_p weight dropped from the query side
    "drop_C": ("a[fl.deg[f]] * (double)fl.cnt[f] * feat_value(&fl, f, qT)",
               "a[fl.deg[f]] * feat_value(&fl, f, qT)", _feature_form_pins),
    # feature form: alpha_p dropped from the query side
    "drop_alpha": ("a[fl.deg[f]] * (double)fl.cnt[f] * feat_value(&fl, f, qT)",
                   "(double)fl.cnt[f] * feat_value(&fl, f, qT)", _feature_form_pins),
    # feature form: the normaliser column accumulates 1 instead of phi(k)
    "normaliser": ("S[f * cols + dV] += phik;", "S[f * cols + dV] += 1.0;",
                   _feature_form_pins),
    # gradient: the normaliser's term h_T dropped
    "grad_drop_h": ("            hT /= den;\n", "            hT = 0.0;\n", _grad_pins),
    # gradient: w' with the power and the coefficient one term apart
    "grad_wprime": ("if (p + 1 < P) wp += (p + 1) * a[p + 1] * xp;",
                    "if (p + 1 < P) wp += (p + 1) * a[p] * xp;", _grad_pins),
    # gradient: dk takes the key instead of the query (a transposed operand)
    "grad_dk_operand": ("dkh[t * dK + i] += c * wp * qT[i];", "dkh[t * dK + i] += c * wp * kt[i];",
                        _grad_pins),
    # gradient: dv scaled by dy instead of dy / D
    "grad_dv_scale": ("dvh[t * dV + j] += w * gT[j];", "dvh[t * dV + j] += w * dyT[j];", _grad_pins),
    # feature form: a transposed operand (v indexed by the wrong token)
    "v_index": ("S[f * cols + j] += phik * vt[j];",
                "S[f * cols + j] += phik * v[((T + 1) % n) * dV + j];", _feature_form_pins),
}


@pytest.fixture()
def mutant_lib(tmp_path, monkeypatch):
    def make(name):
        old, new, _ = MUTANTS[name]
        text = open(SRC).read()
        assert text.count(old) == 1, "mutation anchor for %s must occur once" % name
        src = tmp_path / ("oracle_%s.c" % name)
        src.write_text(text.replace(old, new))
        so = tmp_path / ("liboracle_%s.so" % name)
        subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                        "-ffp-contract=off", "-o", str(so), str(src), "-lm"], check=True)
        monkeypatch.setattr(oracle, "_LIB", str(so))
        monkeypatch.setattr(oracle, "_lib", None)
        oracle._load()
    return make


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(name, mutant_lib):
    check = MUTANTS[name][2]
    mutant_lib(name)
    with pytest.raises((AssertionError, ValueError, RuntimeError)):
        with np.errstate(all="ignore"):
            check()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_pass_on_original(name):
    MUTANTS[name][2]()
