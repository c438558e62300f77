"""Plant plausible mistakes in copies of the oracle (on the CPU) and check
that each one fails at least one pin.  This is what makes the pins worth
trusting: a dropped term, a wrong sign, a transposed operand or a wrong
index anywhere in the oracle is caught."""
import os

import numpy as np
import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

MUTANTS = {
    "no_decay": ("S[(size_t)i * dv + j] *= a[i];", "S[(size_t)i * dv + j] *= 1.0;"),
    "decay_on_value_axis": ("S[(size_t)i * dv + j] *= a[i];", "S[(size_t)i * dv + j] *= a[j % dk];"),
    "undecayed_error": ("p += S[(size_t)i * dv + j] * kk[i];", "p += S[(size_t)i * dv + j] * kk[i] / a[i];"),
    "error_sign": ("e[j] = vv[j] - p;", "e[j] = vv[j] + p;"),
    "no_beta": ("+= b * kk[i] * e[j];", "+= kk[i] * e[j];"),
    "readout_with_k": ("acc += S[(size_t)i * dv + j] * qq[i];", "acc += S[(size_t)i * dv + j] * kk[i];"),
    "gate_sign": ("return KDA_ORACLE_GMIN * s;", "return KDA_ORACLE_GMIN * (1.0 - s);"),
    "gate_no_exp_A": ("double x = exp(A_h) * z;", "double x = A_h * z;"),
    "h0_transposed": ("h0[(((size_t)n * H + h) * dv + j) * dk + i]", "h0[(((size_t)n * H + h) * dk + i) * dv + j]"),
    "h0_ignored": ("h0 ? h0[(((size_t)n * H + h) * dv + j) * dk + i] : 0.0;", "0.0;"),
    "last_token_dropped": ("for (int t = t0; t < t1; ++t) {", "for (int t = t0; t < t1 - 1; ++t) {"),
    "outer_product_transposed": ("+= b * kk[i] * e[j];", "+= b * kk[j % dk] * e[i % dv];"),
}


@pytest.fixture(scope="module")
def mutant_libs(tmp_path_factory):
    d = tmp_path_factory.mktemp("mutants")
    base = open(SRC).read()
    libs = {}
    for name, (old, new) in MUTANTS.items():
        assert base.count(old) >= 1, name
        src = d / (name + ".c")
        src.write_text(base.replace(old, new))
        libs[name] = oracle.build(str(src), str(d / ("lib" + name + ".so")))
    return libs


def _failures(lib_path):
    run = lambda q, k, v, z, A, beta, h0, cu: oracle.prefill(q, k, v, z, A, beta, h0, cu,
                                                             lib_path=lib_path)
    lib = oracle.load(lib_path)
    failed = []
    checks = [("gate", lambda: pins.check_gate_closed_forms(lambda a, z: lib.kda_oracle_gate(a, z)))]
    checks += [(c.__name__, (lambda c=c: c(run))) for c in pins.ALL_PREFILL_CHECKS]
    for name, fn in checks:
        try:
            with np.errstate(all="ignore"):
                fn()
        except AssertionError:
            failed.append(name)
    return failed


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(mutant_libs, name):
    failed = _failures(mutant_libs[name])
    assert failed, "mutant %s passes every pin" % name


def test_unmutated_copy_passes(tmp_path):
    lib = oracle.build(SRC, str(tmp_path / "libclean.so"))
    assert _failures(lib) == []
