"""The backward-oracle pins must catch plausible mistakes in it: each mutant
is a copy of oracle/backward.py with one planted mistake (a dropped term, a
wrong sign, a transposed operand, a wrong state in a product, a missing
factor), loaded as a separate module; at least one pin must fail on it."""
import importlib.util
import os
import tempfile

import pytest

from oracle import backward as ORACLE
import test_oracle_backward_pins as pins

SRC = open(ORACLE.__file__).read()

MUTANTS = {
    "read-out gradient dropped": ("                dS += np.outer(q[r, h], do[r, h])\n", ""),
    "dq from the old state": ("dq[r, h] = S[t + 1] @ do[r, h]", "dq[r, h] = S[t] @ do[r, h]"),
    "du transposed": ("du = dS.T @ k[r, h]", "du = dS @ k[r, h]"),
    "dk write term dropped": ("dk[r, h] = dS @ Uu[t]", "dk[r, h] = 0.0 * Uu[t][:1]"),
    "dbeta sign": ("db[r, h] = du @ (v[r, h] - P[t])", "db[r, h] = du @ (v[r, h] + P[t])"),
    "dv without beta": ("dv[r, h] = b[r, h] * du", "dv[r, h] = du"),
    "dp sign": ("dp = -b[r, h] * du", "dp = b[r, h] * du"),
    "erase term dropped from dS'": ("dSp = dS + np.outer(k[r, h], dp)", "dSp = dS.copy()"),
    "dk retrieval term dropped": ("                dk[r, h] += Sp[t] @ dp\n", ""),
    "dk retrieval from the undecayed state": ("dk[r, h] += Sp[t] @ dp",
                                             "dk[r, h] += S[t] @ dp"),
    "dlog_alpha without alpha": ("dg[r, h] = a * np.sum(dSp * S[t], axis=1)",
                                 "dg[r, h] = np.sum(dSp * S[t], axis=1)"),
    "dlog_alpha over the wrong axis": ("dg[r, h] = a * np.sum(dSp * S[t], axis=1)",
                                       "dg[r, h] = a * np.sum(dSp * S[t], axis=0)[:a.shape[0]]"),
    "decay not applied to dS": ("dS = a[:, None] * dSp", "dS = dSp"),
    "final-state gradient ignored": ("dS = np.zeros((Dk, Dv)) if dhT is None else dhT[n, h].copy()",
                                     "dS = np.zeros((Dk, Dv))"),
}


def _load(src):
    d = tempfile.mkdtemp()
    path = os.path.join(d, "backward_mutant.py")
    with open(path, "w") as f:
        f.write(src)
    spec = importlib.util.spec_from_file_location("backward_mutant", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_backward_mutant(name):
    old, new = MUTANTS[name]
    assert SRC.count(old) == 1, f"mutation anchor not found once: {old!r}"
    mod = _load(SRC.replace(old, new))
    caught = []
    for p in pins.PINS:
        try:
            p(mod)
        except Exception as e:
            caught.append((p.__name__, type(e).__name__))
    assert caught, f"no pin caught the mutant {name!r}"
