"""Plant plausible mistakes in a copy of the oracle's C source (on the CPU)
and require each broken build to fail at least one pin.  This is what makes
the pins a check of the oracle rather than a restatement of it."""
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import oracle
from oracle import build as obuild
from tests import _pins

SRC = open(obuild.SRC).read()
READ_CALL = "    read_output(J, S, qt, row, j0, nc);\n"

MUTATIONS = {
    "correction_sign": [("S[c * nc + j] - bt * kt[c] * read[j]", "S[c * nc + j] + bt * kt[c] * read[j]")],
    "write_without_beta": [("+ bt * kt[c] * vt[j0 + j]", "+ kt[c] * vt[j0 + j]")],
    "read_with_query": [("acc += kt[c] * S[c * nc + j]", "acc += qt[c] * S[c * nc + j]")],
    "no_decay": [("S[c * nc + j] *= alpha[c];", "S[c * nc + j] *= 1.0;")],
    "decay_after_erase": [
        ("S[c * nc + j] *= alpha[c];", "S[c * nc + j] *= 1.0;"),
        ("S[c * nc + j] = S[c * nc + j] - bt * kt[c] * read[j] + bt * kt[c] * vt[j0 + j];",
         "S[c * nc + j] = alpha[c] * (S[c * nc + j] - bt * kt[c] * read[j]) + bt * kt[c] * vt[j0 + j];"),
    ],
    "read_before_update": [
        (READ_CALL, ""),
        ("    /* 1. decay:", READ_CALL + "    /* 1. decay:"),
    ],
    "sigmoid_sign": [("double s = 1.0 / (1.0 + exp(-x));", "double s = 1.0 / (1.0 + exp(x));")],
    "gate_without_exp_A": [("double x = exp(A) * z;", "double x = A * z;")],
    "chunk_reset_off_by_one": [("if (t % chunk == 0) run = 0.0;", "if (t % chunk == 1) run = 0.0;")],
    "state_in_ignored": [("if (J->S_in) {", "if (0) {")],
    "state_in_transposed": [("S[c * nc + (j - j0)] = Si[c * dv + j];", "S[c * nc + (j - j0)] = Si[j * dk + c];")],
    "scale_ignored": [("ot[j0 + j] = J->scale * acc;", "ot[j0 + j] = acc;")],
    "alpha_not_exponentiated": [("alpha[c] = exp(g);", "alpha[c] = 1.0 + g;")],
}


@pytest.fixture(scope="module")
def workdir():
    d = tempfile.mkdtemp(prefix="kda_oracle_mut_")
    shutil.copy(os.path.join(os.path.dirname(obuild.SRC), "kda_oracle.h"), d)
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, workdir):
    src = SRC
    for old, new in MUTATIONS[name]:
        assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
        src = src.replace(old, new)
    c = os.path.join(workdir, f"{name}.c")
    so = os.path.join(workdir, f"{name}.so")
    with open(c, "w") as f:
        f.write(src)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread", "-o", so, c, "-lm"], check=True)
    orc = oracle.Oracle(so)
    failed = []
    for pin in _pins.ALL_PINS:
        try:
            pin(orc)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"


# The prologue is numpy code (oracle.l2_normalise, oracle.sigmoid): plant its
# plausible mistakes by swapping the function, on the CPU, and require a pin
# to fail.
PROLOGUE_MUTATIONS = {
    "eps_outside_root": ("l2_normalise", lambda x: x / (np.sqrt(np.sum(x * x, axis=-1, keepdims=True)) + 1e-6)),
    "eps_1e-3": ("l2_normalise", lambda x: x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + 1e-3)),
    "no_root": ("l2_normalise", lambda x: x / (np.sum(x * x, axis=-1, keepdims=True) + 1e-6)),
    "norm_over_tokens": ("l2_normalise", lambda x: x / np.sqrt(np.sum(x * x, axis=-3, keepdims=True) + 1e-6)),
    "no_normalisation": ("l2_normalise", lambda x: np.asarray(x, float) * 1.0),
    "sigmoid_sign": ("sigmoid", lambda x: 1.0 / (1.0 + np.exp(np.asarray(x, float)))),
    "beta_tanh": ("sigmoid", lambda x: 0.5 * (1.0 + np.tanh(np.asarray(x, float)))),
}


@pytest.mark.parametrize("name", sorted(PROLOGUE_MUTATIONS))
def test_prologue_mutation_is_caught(name, monkeypatch):
    attr, fn = PROLOGUE_MUTATIONS[name]
    monkeypatch.setattr(oracle, attr, fn)
    failed = []
    for pin in _pins.ALL_PINS:
        if not pin.__name__.startswith("pin_prologue"):
            continue
        try:
            pin(oracle.default())
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"prologue mutation {name} passed every prologue pin"


# The backward oracle (oracle/backward.py) is numpy code: plant its plausible
# mistakes in a copy of its source text, load that copy in place of the module's
# backward_z, and require a backward pin to fail.
import oracle.backward as _OB  # noqa: E402

BWD_SRC = open(_OB.__file__).read()
BACKWARD_MUTATIONS = {
    "dq_without_scale": [("dq[:, t] = scale * np.einsum", "dq[:, t] = np.einsum")],
    "dq_reads_old_state": [('np.einsum("bhcj,bhj->bhc", St, do[:, t])', 'np.einsum("bhcj,bhj->bhc", Sp, do[:, t])')],
    "dk_without_erase_term": [('        dkt = dkt - np.einsum("bhcj,bhj->bhc", D, de)\n', "")],
    "dD_sign": [("dD = dS - kt[:, :, :, None]", "dD = dS + kt[:, :, :, None]")],
    "dS_without_decay": [("dS = alpha[:, t, :, :, None] * dD", "dS = dD")],
    "dbeta_without_e": [('np.einsum("bhc,bhcj,bhj->bh", kt, dS, e)', 'np.einsum("bhc,bhcj->bh", kt, dS)')],
    "sigmoid_prime_missing": [("sig[:, t] * (1.0 - sig[:, t]) * dg", "sig[:, t] * dg")],
    "dA_without_z": [('np.einsum("bthc,bthc->hc", dx, z) * eA', "np.sum(dx, axis=(0, 1)) * eA")],
    "dv_sign": [("dv_[:, t] = de", "dv_[:, t] = -de")],
}


@pytest.mark.parametrize("name", sorted(BACKWARD_MUTATIONS))
def test_backward_mutation_is_caught(name, monkeypatch):
    src = BWD_SRC
    for old, new in BACKWARD_MUTATIONS[name]:
        assert src.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
        src = src.replace(old, new)
    ns = {"__name__": "oracle_backward_mutant"}
    exec(compile(src, f"<{name}>", "exec"), ns)
    monkeypatch.setattr(_OB, "backward_z", ns["backward_z"])
    failed = []
    for pin in _pins.ALL_PINS:
        if not pin.__name__.startswith("pin_backward"):
            continue
        try:
            pin(oracle.default())
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"backward mutation {name} passed every backward pin"
